// prep_nv.hip -- the SharQ activation preparation for NVFP4 on gfx950.
//
// Same decomposition as the MXFP4 preparation (SharQ, arXiv 2606.26587: abstract and
// "Core claim"; the pages name NVFP4 as a supported format and Figure 2 shows the
// NVFP4 dataflow), with NVFP4's scale hierarchy: one E4M3 scale per 16 elements and
// one fp32 scale per tensor.  The pages do not fix the tensor scales; each path
// (backbone, residual) gets its own, S = amax / (6 * 448), from its own tensor
// maximum.  The residual's maximum is only known after the backbone has been
// quantized everywhere, so the preparation is three passes over X:
//   pass 0  amax|X|                      (= amax of the kept values: every group's
//                                         largest element is kept)
//   pass 1  mask, backbone, R; amax|R|
//   pass 2  mask, backbone, R again; write backbone and residual codes and scales
// The maximum passes leave one partial per work-group in the caller's workspace and a
// one-work-group kernel reduces them (no contended atomics); a final one-thread
// kernel writes both tensor scales.
//
// Arithmetic per 16-element block, each step one correctly rounded fp32 operation:
//   q = amax_blk / (6*S);  s = E4M3(q) (nearest-even, saturating at 448);
//   d = s * S;  code = E2M1(x / d) (all 0x0 when d == 0);  Bhat = value * d;
//   R = x - Bhat.
// E2M1 rounding uses the gfx950 scaled conversion with a unit scale (nearest-even,
// saturating, sign kept -- checked bit-for-bit against the format definition).
//
// Work mapping: lane = 8 consecutive elements (16-byte load) of the flat element
// sequence; an NVFP4 block is a lane pair, a mask group never straddles a lane.
#include "sharq_internal.h"

namespace sharq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 2;
constexpr float kUnitScale = 1.0f;
// workspace (uint32): [0] max|X|, [1] max|R|, partial maxima from kPartialBase on
constexpr int kPartialBase = 16;
constexpr int kMaxPartials = 2048;
static_assert((kPartialBase + 2 * kMaxPartials) * 4 <= (int)kNvPrepWorkspace, "workspace too small");

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// max over a lane pair (DPP quad_perm [1,0,3,2])
__device__ __forceinline__ uint32_t pair_max(uint32_t v) {
  return umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = umax(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ void cswap(uint32_t& a, uint32_t& b) {
  uint32_t hi = umax(a, b), lo = umin(a, b);
  a = hi;
  b = lo;
}

// top-n-of-m keep bits of a lane's 8 elements (see the MXFP4 preparation)
template <int SPM>
__device__ __forceinline__ uint32_t keep_bits(const uint32_t w[4]) {
  uint32_t ck[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t key = (j & 1) ? (w[j >> 1] >> 16) & 0x7FFFu : w[j >> 1] & 0x7FFFu;
    ck[j] = SPM == 4 ? (key << 2) | (3u - (j & 3)) : (key << 3) | (7u - j);
  }
  uint32_t bits = 0;
  if constexpr (SPM == 4) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t* c = ck + 4 * g;
      uint32_t hi1 = umax(c[0], c[1]), lo1 = umin(c[0], c[1]);
      uint32_t hi2 = umax(c[2], c[3]), lo2 = umin(c[2], c[3]);
      uint32_t second = umax(umin(hi1, hi2), umax(lo1, lo2));
#pragma unroll
      for (int j = 0; j < 4; ++j) bits |= (c[j] >= second ? 1u : 0u) << (4 * g + j);
    }
  } else {
    uint32_t a0 = ck[0], a1 = ck[1], a2 = ck[2], a3 = ck[3];
    uint32_t b0 = ck[4], b1 = ck[5], b2 = ck[6], b3 = ck[7];
    cswap(a0, a1); cswap(a2, a3); cswap(a0, a2); cswap(a1, a3); cswap(a1, a2);
    cswap(b0, b1); cswap(b2, b3); cswap(b0, b2); cswap(b1, b3); cswap(b1, b2);
    uint32_t fourth = umin(umin(umax(a0, b3), umax(a1, b2)), umin(umax(a2, b1), umax(a3, b0)));
#pragma unroll
    for (int j = 0; j < 8; ++j) bits |= (ck[j] >= fourth ? 1u : 0u) << j;
  }
  return bits;
}

// OCP E4M3 code of q >= 0: nearest value, ties to the even code, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  if (!(q > 0.0f)) return 0;
  if (q >= 448.0f) return 0x7E;
  if (q < 0.015625f) return (uint32_t)__builtin_rintf(q * 512.0f);  // subnormal step 2^-9 (exact scaling)
  const uint32_t u = __float_as_uint(q);
  const uint32_t ef = (u >> 23) - 120;  // E4M3 exponent field: (e - 127) + 7
  uint32_t code = (ef << 3) | ((u >> 20) & 7u);
  const uint32_t rem = u & 0xFFFFFu, half = 0x80000u;
  if (rem > half || (rem == half && (code & 1u))) code += 1;  // a carry moves into the exponent
  return code;
}

__device__ __forceinline__ float e4m3_value(uint32_t s) {
  const uint32_t ef = s >> 3, m = s & 7u;
  if (ef == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((ef + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ float tensor_scale_of(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 2688.0f);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) {
  bf16x2_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// Quantize 8 values of one lane (half of a 16-element block whose maximum magnitude
// is amax) with tensor scale S: returns 8 codes packed in a dword, the scale byte and
// the dequantized values.
__device__ __forceinline__ uint32_t nv_quant8(const float v[8], float amax, float S, uint32_t& sbyte,
                                              float deq[8]) {
  const float q = __fdiv_rn(amax, __fmul_rn(6.0f, S));
  sbyte = e4m3_encode(q);
  const float d = __fmul_rn(e4m3_value(sbyte), S);
  float t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = d == 0.0f ? 0.0f : __fdiv_rn(v[j], d);
  uint32_t packed = 0;
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[0], t[1], kUnitScale, 0);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[2], t[3], kUnitScale, 1);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[4], t[5], kUnitScale, 2);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[6], t[7], kUnitScale, 3);
  if (d == 0.0f) packed = 0;  // every code of a zero-scale block is 0x0
  auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 0);
  auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 1);
  auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 2);
  auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 3);
  const float val[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
  for (int j = 0; j < 8; ++j) deq[j] = __fmul_rn(val[j], d);
  return packed;
}

// Gather the scale bytes of the 32 blocks of a wave into 8 dwords held by lanes
// 0, 8, ..., 56 (block 4k+i is the lane pair starting at lane 8k+2i).
__device__ __forceinline__ uint32_t gather_scales(uint32_t byte) {
  uint32_t b1 = __shfl_down(byte, 2, 64);
  uint32_t b2 = __shfl_down(byte, 4, 64);
  uint32_t b3 = __shfl_down(byte, 6, 64);
  return byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// PASS 0: amax|X| -> work[0].  PASS 1: amax|R| -> work[1].  PASS 2: write outputs.
// MODE 0: SharQ preparation; MODE 1: plain NVFP4 quantization into (rcodes, rscales)
// with work[0] as its tensor maximum (passes 0 and 2 only).
template <int PASS, int MODE, int SPM, bool DENSE_ROWS, bool WRITE_MASK>
__global__ __launch_bounds__(kThreads) void prep_nv_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t chunks_per_row, int64_t nchunks,
    uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales, uint8_t* __restrict__ rcodes,
    uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask, uint32_t* __restrict__ work) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  // the maximum passes walk the chunks grid-stride with a bounded grid; the emitting
  // pass covers everything with one iteration per wave
  const int64_t stride = PASS <= 1 ? (int64_t)gridDim.x * (kThreads / 64) * 64 * kUnroll : nchunks;

  float Sb = 1.0f, Sr = 1.0f;
  if constexpr (PASS >= 1) Sb = tensor_scale_of(work[0]);
  if constexpr (PASS == 2 && MODE == 0) Sr = tensor_scale_of(work[1]);

  uint32_t run_max = 0;
  for (int64_t base = wave * 64 * kUnroll; base < nchunks; base += stride) {
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * 64 + lane;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (c < nchunks) {
      int64_t off;
      if constexpr (DENSE_ROWS) {
        off = c * 8;
      } else {
        const int64_t row = c / chunks_per_row;
        off = row * ldx + (c - row * chunks_per_row) * 8;
      }
      v[u] = *reinterpret_cast<const u32x4*>(x + off);
    }
  }

#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = base + u * 64 + lane;
    const bool valid = c < nchunks;
    const uint32_t w[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
    uint32_t kmax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) kmax = umax(kmax, umax(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    if constexpr (PASS == 0) {
      run_max = umax(run_max, kmax << 16);  // bf16 magnitude bits as fp32 bits
      continue;
    }
    float xf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[2 * i] = __uint_as_float(w[i] << 16);
      xf[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    const float bamax = __uint_as_float(pair_max(kmax) << 16);

    uint32_t keep = 0xFFu, bbyte = 0, bpacked = 0;
    float r[8];
    if constexpr (MODE == 0) {
      keep = keep_bits<SPM>(w);
      float kv[8], bh[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) kv[j] = (keep >> j) & 1 ? xf[j] : 0.0f;
      bpacked = nv_quant8(kv, bamax, Sb, bbyte, bh);
      // dropped positions: code 0x0 (kv = +0 -> code 0 and value +0)
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = __fsub_rn(xf[j], bh[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = xf[j];
    }

    uint32_t rmax = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) rmax = umax(rmax, __float_as_uint(r[j]) & 0x7FFFFFFFu);
    if constexpr (PASS == 1) {
      run_max = umax(run_max, rmax);
      continue;
    }
    // PASS 2: quantize R (or X in MODE 1) with its own block and tensor scales
    uint32_t rbyte = 0;
    float rdeq[8];
    const float rS = MODE == 0 ? Sr : Sb;
    const uint32_t rpacked = nv_quant8(r, __uint_as_float(pair_max(rmax)), rS, rbyte, rdeq);

    const int64_t g0 = (base + u * 64 + 8 * (lane >> 3)) >> 1;  // first block of this lane's dword
    const int64_t nblocks = nchunks >> 1;
    const uint32_t rpk = gather_scales(rbyte);
    uint32_t bpk = 0;
    if constexpr (MODE == 0) bpk = gather_scales(bbyte);
    if (valid) {
      *reinterpret_cast<uint32_t*>(rcodes + c * 4) = rpacked;
      if constexpr (MODE == 0) {
        *reinterpret_cast<uint32_t*>(bcodes + c * 4) = bpacked;
        if constexpr (WRITE_MASK) mask[c] = (uint8_t)keep;
      }
    }
    if ((lane & 7) == 0) {
      if (g0 + 3 < nblocks) {
        *reinterpret_cast<uint32_t*>(rscales + g0) = rpk;
        if constexpr (MODE == 0) *reinterpret_cast<uint32_t*>(bscales + g0) = bpk;
      } else {
        for (int i = 0; i < 4; ++i)
          if (g0 + i < nblocks) {
            rscales[g0 + i] = (uint8_t)(rpk >> (8 * i));
            if constexpr (MODE == 0) bscales[g0 + i] = (uint8_t)(bpk >> (8 * i));
          }
      }
    }
  }
  }
  if constexpr (PASS <= 1) {
    // work-group maximum -> one partial per work-group (no contended atomics)
    __shared__ uint32_t red[kThreads / 64];
    run_max = wave_max(run_max);
    if (lane == 0) red[threadIdx.x >> 6] = run_max;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = 0;
      for (int i = 0; i < kThreads / 64; ++i) m = umax(m, red[i]);
      work[kPartialBase + PASS * kMaxPartials + blockIdx.x] = m;
    }
  }
}

// work[slot] = max of the `n` partials of a maximum pass (one work-group).
__global__ void nv_reduce_kernel(uint32_t* work, int slot, int n) {
  __shared__ uint32_t red[256];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += 256) m = umax(m, work[kPartialBase + slot * kMaxPartials + i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = umax(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) work[slot] = red[0];
}

__global__ void nv_reset_kernel(uint32_t* work) {
  if (threadIdx.x < 2) work[threadIdx.x] = 0;
}

__global__ void nv_tensor_scales_kernel(const uint32_t* work, float* t0, float* t1) {
  if (threadIdx.x == 0) {
    if (t0) *t0 = tensor_scale_of(work[0]);
    if (t1) *t1 = tensor_scale_of(work[1]);
  }
}

template <int MODE, int SPM, bool DENSE, bool WRITE_MASK>
hipError_t run_passes(const uint16_t* x, int64_t ldx, int64_t cpr, int64_t nchunks, uint8_t* bcodes,
                      uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales, uint8_t* mask, uint32_t* work,
                      hipStream_t st) {
  const int64_t per_wg = (kThreads / 64) * 64 * kUnroll;
  const unsigned grid = (unsigned)((nchunks + per_wg - 1) / per_wg);
  const unsigned rgrid = grid < (unsigned)kMaxPartials ? grid : (unsigned)kMaxPartials;
  prep_nv_kernel<0, MODE, SPM, DENSE, WRITE_MASK><<<rgrid, kThreads, 0, st>>>(
      x, ldx, cpr, nchunks, bcodes, bscales, rcodes, rscales, mask, work);
  nv_reduce_kernel<<<1, 256, 0, st>>>(work, 0, (int)rgrid);
  if constexpr (MODE == 0) {
    prep_nv_kernel<1, MODE, SPM, DENSE, WRITE_MASK><<<rgrid, kThreads, 0, st>>>(
        x, ldx, cpr, nchunks, bcodes, bscales, rcodes, rscales, mask, work);
    nv_reduce_kernel<<<1, 256, 0, st>>>(work, 1, (int)rgrid);
  }
  prep_nv_kernel<2, MODE, SPM, DENSE, WRITE_MASK><<<grid, kThreads, 0, st>>>(
      x, ldx, cpr, nchunks, bcodes, bscales, rcodes, rscales, mask, work);
  return hipGetLastError();
}

template <int MODE, int SPM, bool WRITE_MASK>
hipError_t run_nv(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes, uint8_t* bscales,
                  float* bts, uint8_t* rcodes, uint8_t* rscales, float* rts, uint8_t* mask, uint32_t* work,
                  hipStream_t st) {
  nv_reset_kernel<<<1, 64, 0, st>>>(work);
  const int64_t cpr = K / 8;
  const int64_t nchunks = M * cpr;
  hipError_t e = hipSuccess;
  if (nchunks > 0) {
    e = ldx == K ? run_passes<MODE, SPM, true, WRITE_MASK>(x, ldx, cpr, nchunks, bcodes, bscales, rcodes,
                                                          rscales, mask, work, st)
                 : run_passes<MODE, SPM, false, WRITE_MASK>(x, ldx, cpr, nchunks, bcodes, bscales, rcodes,
                                                           rscales, mask, work, st);
    if (e != hipSuccess) return e;
  }
  nv_tensor_scales_kernel<<<1, 64, 0, st>>>(work, bts, rts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_nv(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                          uint8_t* bcodes, uint8_t* bscales, float* btscale, uint8_t* rcodes,
                          uint8_t* rscales, float* rtscale, uint8_t* mask, uint32_t* work,
                          hipStream_t stream) {
  (void)sp_n;
  if (sp_m == 4)
    return mask ? run_nv<0, 4, true>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale, mask,
                                     work, stream)
                : run_nv<0, 4, false>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale,
                                      mask, work, stream);
  return mask ? run_nv<0, 8, true>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale, mask,
                                   work, stream)
              : run_nv<0, 8, false>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale, mask,
                                    work, stream);
}

hipError_t launch_quant_nv(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, float* tscale, uint32_t* work, hipStream_t stream) {
  return run_nv<1, 4, false>(x, rows, K, ldx, nullptr, nullptr, tscale, codes, scales, nullptr, nullptr,
                             work, stream);
}

}  // namespace sharq
