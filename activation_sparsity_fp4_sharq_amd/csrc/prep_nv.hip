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
//   pass 1  mask, backbone -> written; R = X - Bhat; amax|R|
//   pass 2  R again from X and the written backbone; residual -> written
// The maximum passes leave one partial per work-group in the caller's workspace; every
// work-group of the pass after a maximum pass reduces those partials itself (a few KiB
// of L2-resident words, no atomics and no launch in between), and its work-group 0
// writes that path's tensor scale.
//
// Arithmetic per 16-element block, each step one correctly rounded fp32 operation:
//   q = amax_blk / (6*S);  s = E4M3(q) (nearest-even, saturating at 448);
//   d = s * S;  code = E2M1(x / d) (all 0x0 when d == 0);  Bhat = value * d;
//   R = x - Bhat.
// The quotients share their divisor (6*S per tensor, d per block), so each divisor's
// correctly rounded reciprocal y is formed once and every quotient takes one
// remainder step (Markstein): q0 = x*y, r = x - q0*d (fma), q = q0 + r*y (fma), which
// returns the correctly rounded x / d, the sign of a zero included (div_step), while the
// intermediates stay in the normal range (divisors below 2^-90 use the full division).
// E2M1 rounding uses the gfx950 scaled conversion with a unit scale (nearest-even,
// saturating, sign kept -- checked bit-for-bit against the format definition); the
// E4M3 block scale is coded and decoded with the fp8 conversions (e4m3_encode_hw and
// e4m3_value_hw, checked against the definition on every operand the block scale can
// take).
//
// Work mapping: lane = 8 consecutive elements (16-byte load) of the flat element
// sequence; an NVFP4 block is a lane pair, a mask group never straddles a lane.
#include "fp4_codec.h"
#include "sharq_internal.h"

namespace sharq {
namespace {

using namespace codec;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 2;  // chunks per lane and loop step
// Bounded grid of pass 2 (grid-stride beyond it): each work-group's prologue -- both
// tensor scales, the partial maxima of pass 1, the divisor tables -- is then paid a few
// times per lane instead of once per two chunks.
constexpr int kLastGroups = 2048;
constexpr int kMaxGroups = 2048;  // bounded grid of the maximum passes: at most this many partials each
constexpr float kUnitScale = 1.0f;
// workspace (uint32): [0] max|X| (written by pass 1 for pass 2), [1] max|R| (fp32 bits
// of non-negative values, so integer maxima order them), then one partial maximum per
// work-group of each maximum pass from kPartialBase on
constexpr int kPartialBase = 16;
static_assert((kPartialBase + 2 * kMaxGroups) * 4 <= (int)kNvPrepWorkspace, "workspace too small");


// max over a lane pair (DPP quad_perm [1,0,3,2])
__device__ __forceinline__ uint32_t pair_max(uint32_t v) {
  return umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = umax(v, __shfl_xor(v, off, 64));
  return v;
}

// Maximum of the n (1 <= n <= kMaxGroups) partials at p, by the whole work-group of TPB
// threads (every thread gets it, so every thread must call it).  Every load is issued
// before any is used: indices past n re-read partial n-1 (a maximum is unchanged by a
// repeated element), so no load sits under a branch that would have to wait for it.
template <int TPB>
__device__ __forceinline__ uint32_t group_max_of(const uint32_t* __restrict__ p, int n, uint32_t* red) {
  constexpr int kPer = kMaxGroups / TPB;
  uint32_t v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = j * TPB + (int)threadIdx.x;
    v[j] = p[i < n ? i : n - 1];
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) m = umax(m, v[j]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < TPB / 64; ++w) r = umax(r, red[w]);
  return r;
}

__device__ __forceinline__ float tensor_scale_of(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 2688.0f);
}

// The remainder step needs normal-range intermediates: it is used for divisors of at
// least 2^-90 (with quotients of magnitude 2^-4..2^4, where E2M1 rounding is decided,
// x*y, r and r*y then stay normal); smaller divisors take the full division.
constexpr float kFastDivisorMin = 0x1p-90f;

// Correctly rounded 1/d for the remainder step (0 when the step is not used).
__device__ __forceinline__ float recip_rn(float d) { return d >= kFastDivisorMin ? __fdiv_rn(1.0f, d) : 0.0f; }

// x / d correctly rounded, from y = RN(1/d): one remainder step.  The remainder is
// formed negated, t = q0*d - x = -r (exact), and the correction is q0 + (-t)*y: where
// the remainder is zero, -t is -0 and leaves q0's sign alone, so x = -0 gives -0 as the
// division does (x - q0*d itself would be +0 there, and +0 + -0 = +0 would drop the
// sign that E2M1 keeps as code 0x8).
__device__ __forceinline__ float div_step(float x, float d, float y) {
  const float q0 = __fmul_rn(x, y);
  const float t = __builtin_fmaf(q0, d, -x);
  return __builtin_fmaf(-t, y, q0);
}

__device__ __forceinline__ float div_rn(float x, float d, float y) {
  return d >= kFastDivisorMin ? div_step(x, d, y) : __fdiv_rn(x, d);
}

// Per-tensor constants of one path: S, 6*S and RN(1/(6*S)).
struct PathScale {
  float S, S6, yS6;
};

__device__ __forceinline__ PathScale path_scale(uint32_t amax_bits) {
  PathScale p;
  p.S = tensor_scale_of(amax_bits);
  p.S6 = __fmul_rn(6.0f, p.S);
  p.yS6 = recip_rn(p.S6);
  return p;
}

// A path's block divisors by scale code: {d(s), y(s)} with d(s) = fp32(value(s) * S) and
// y(s) = RN(1/d(s)) (recip_rn), for every E4M3 code s.  Each work-group fills its own
// copy in LDS once (one entry per thread) -- a block then looks its divisor up instead
// of decoding its scale and dividing for the reciprocal.
constexpr int kDivCodes = 128;

__device__ __forceinline__ float2 divisor_entry(uint32_t s, const PathScale& ps) {
  const float d = __fmul_rn(e4m3_value_hw(s), ps.S);
  return float2{d, recip_rn(d)};
}

// Block divisor d = E4M3(amax_blk / (6S)) * S, its reciprocal and its scale byte.
__device__ __forceinline__ float block_divisor(float amax_blk, const PathScale& ps, const float2* tab,
                                               uint32_t& sbyte, float& y) {
  sbyte = e4m3_encode_hw(div_rn(amax_blk, ps.S6, ps.yS6));
  const float2 e = tab[sbyte];
  y = e.y;
  return e.x;
}

// 8 values -> 8 E2M1 codes of v / d (one dword; 0 when d == 0); y = recip_rn(d).
__device__ __forceinline__ uint32_t nv_codes(const float v[8], float d, float y) {
  float t[8];
  if (d >= kFastDivisorMin) {
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = div_step(v[j], d, y);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = d == 0.0f ? 0.0f : __fdiv_rn(v[j], d);
  }
  uint32_t packed = __float_as_uint(t[0]);  // all four bytes are written below
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[0], t[1], kUnitScale, 0);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[2], t[3], kUnitScale, 1);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[4], t[5], kUnitScale, 2);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, t[6], t[7], kUnitScale, 3);
  return d == 0.0f ? 0u : packed;  // every code of a zero-scale block is 0x0
}

// Dequantized values value(code) * d of 8 codes.
__device__ __forceinline__ void nv_dequant(uint32_t packed, float d, float deq[8]) {
  auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 0);
  auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 1);
  auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 2);
  auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, kUnitScale, 3);
  const float val[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
  for (int j = 0; j < 8; ++j) deq[j] = __fmul_rn(val[j], d);
}

// Gather the scale bytes of the 32 blocks of a wave into 8 dwords held by lanes
// 0, 8, ..., 56 (block 4k+i is the lane pair starting at lane 8k+2i).  Lanes 8k+2,
// 8k+4 and 8k+6 lie in lane 8k's row of 16, so row shifts (DPP row_shl, lane i reads
// lane i+n of its row) bring the three bytes in without an LDS permute.
__device__ __forceinline__ uint32_t gather_scales(uint32_t byte) {
  const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x102, 0xF, 0xF, true);
  const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x104, 0xF, 0xF, true);
  const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)byte, 0x106, 0xF, 0xF, true);
  return byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

__device__ __forceinline__ void store_scale_words(uint8_t* dst, int64_t g0, int64_t nblocks, int lane, uint32_t pk) {
  if ((lane & 7) != 0) return;
  if (g0 + 3 < nblocks) {
    *reinterpret_cast<uint32_t*>(dst + g0) = pk;
  } else {
    for (int i = 0; i < 4; ++i)
      if (g0 + i < nblocks) dst[g0 + i] = (uint8_t)(pk >> (8 * i));
  }
}

__device__ __forceinline__ void unpack8(const u32x4& v, float xf[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xf[2 * i] = __uint_as_float(v[i] << 16);
    xf[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint32_t abs_max8_bits(const float v[8]) {
  const float m0 = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  const float m1 = fmaxf(fmaxf(fabsf(v[3]), fabsf(v[4])), fabsf(v[5]));
  const float m2 = fmaxf(fmaxf(fabsf(v[6]), fabsf(v[7])), m0);
  return __float_as_uint(fmaxf(m1, m2));
}

// Work-group shape of a pass.  The plain preparation's maximum passes over dense rows
// run 1024-thread work-groups held to 64 registers (two per CU: 8 waves per SIMD), so a
// pass leaves at most 512 partials for the next one to reduce; every other variant
// (its pass 1 needs more registers) keeps 256-thread work-groups.
template <int PASS, int MODE, bool DENSE_ROWS, bool WRITE_MASK, int XF>
struct NvShape {
  static constexpr bool kWide = PASS <= 1 && DENSE_ROWS && MODE == 0 && !WRITE_MASK && XF == kXfNone;
  static constexpr int kTpb = kWide ? 1024 : kThreads;
  static constexpr int kMinWaves = kWide ? 8 : 1;
  static constexpr int kGroups = kWide ? 512 : kMaxGroups;  // bounded grid of a maximum pass
};

// PASS 0: amax|X| partials.  PASS 1 (MODE 0): backbone written, amax|R| partials.
// PASS 2: MODE 0 writes the residual from X and the written backbone; MODE 1 (plain
// NVFP4 quantization, used for weights) quantizes X into (rcodes, rscales).  MODEs
// 2-4 are the ablations of the method's choices: 2 = residual against the
// unquantized sparse values (R = X - X*mask), 3 = a static mask (the first n of
// every m positions; the backbone maxima are then those of the kept values), 4 = no
// residual (all-zero residual payload, tensor scale 1).  The pass after a maximum pass
// reduces that pass's `nparts` partials in every work-group; work-group 0 writes the
// path's tensor scale (backbone or plain: bts, residual: rts) and pass 1's also
// max|X| into work[0] for pass 2.
// static mask of the lane's 8 elements (they start at a multiple of 8, so element j
// sits at position j % SPM of its group)
template <int SPM>
__device__ __forceinline__ void static_mask(bool kept[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) kept[j] = (j % SPM) < SPM / 2;
}

template <int PASS, int MODE, int SPM, bool DENSE_ROWS, bool WRITE_MASK, int XF>
__global__ __launch_bounds__((NvShape<PASS, MODE, DENSE_ROWS, WRITE_MASK, XF>::kTpb))
__attribute__((amdgpu_waves_per_eu(NvShape<PASS, MODE, DENSE_ROWS, WRITE_MASK, XF>::kMinWaves, 8))) void prep_nv_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t chunks_per_row, int64_t nchunks,
    uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales, uint8_t* __restrict__ rcodes,
    uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask, uint32_t* __restrict__ work,
    float* __restrict__ bts, float* __restrict__ rts, const float* __restrict__ rnorm,
    const uint16_t* __restrict__ gamma, int nparts) {
  const int lane = threadIdx.x & 63;
  constexpr int TPB = NvShape<PASS, MODE, DENSE_ROWS, WRITE_MASK, XF>::kTpb;  // threads per work-group
  const int64_t wave = (int64_t)blockIdx.x * (TPB / 64) + (threadIdx.x >> 6);
  // every pass walks the chunks grid-stride over a bounded grid
  constexpr int U = kUnroll;
  const int64_t stride = (int64_t)gridDim.x * (TPB / 64) * 64 * U;
  const int64_t nblocks = nchunks >> 1;

  PathScale pb{}, pr{};
  __shared__ uint32_t pred[TPB / 64];
  if constexpr (PASS == 1 || (PASS == 2 && MODE == 1)) {
    // the pass right after pass 0: max|X| from its partials
    const uint32_t amax = group_max_of<TPB>(work + kPartialBase, nparts, pred);
    pb = path_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      if (bts) *bts = pb.S;
      if constexpr (PASS == 1) work[0] = amax;
    }
  }
  if constexpr (PASS == 2 && MODE != 1) {
    pb = path_scale(work[0]);
    const uint32_t rmax = group_max_of<TPB>(work + kPartialBase + kMaxGroups, nparts, pred);
    pr = path_scale(rmax);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      work[1] = rmax;
      if (rts) *rts = pr.S;
    }
  }
  // the block-divisor tables of the backbone path [0] and the residual path [1]
  __shared__ float2 dtab[2][kDivCodes];
  if constexpr (PASS >= 1) {
    static_assert(TPB >= 2 * kDivCodes, "one table entry per thread");
    if (threadIdx.x < 2 * kDivCodes) {
      const uint32_t s = threadIdx.x & (kDivCodes - 1);
      dtab[threadIdx.x / kDivCodes][s] = divisor_entry(s, threadIdx.x < kDivCodes ? pb : pr);
    }
    __syncthreads();
  }

  uint32_t run_max = 0;
  for (int64_t base = wave * 64 * U; base < nchunks; base += stride) {
    u32x4 v[U];
    uint32_t bpk_in[U], bsb_in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * 64 + lane;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      bpk_in[u] = 0;
      bsb_in[u] = 0;
      if (c < nchunks) {
        int64_t off;
        if constexpr (DENSE_ROWS) {
          off = c * 8;
        } else {
          const int64_t row = c / chunks_per_row;
          off = row * ldx + (c - row * chunks_per_row) * 8;
        }
        v[u] = *reinterpret_cast<const u32x4*>(x + off);
        if constexpr (XF == kXfSwiglu) {  // gate at off, up K columns further in the same row
          const u32x4 up = *reinterpret_cast<const u32x4*>(x + off + chunks_per_row * 8);
          v[u] = u32x4{swiglu_pair(v[u][0], up[0]), swiglu_pair(v[u][1], up[1]), swiglu_pair(v[u][2], up[2]),
                       swiglu_pair(v[u][3], up[3])};
        }
        if constexpr (XF == kXfRms) {
          // RMS normalization folded in: bf16(fp32(fp32(x * r_row) * g_col))
          const int64_t row = c / chunks_per_row;
          const float rr = rnorm[row];
          const u32x4 g = *reinterpret_cast<const u32x4*>(gamma + (c - row * chunks_per_row) * 8);
          v[u] = u32x4{rms_scale_pair(v[u][0], g[0], rr), rms_scale_pair(v[u][1], g[1], rr),
                       rms_scale_pair(v[u][2], g[2], rr), rms_scale_pair(v[u][3], g[3], rr)};
        }
        if constexpr (PASS == 2 && (MODE == 0 || MODE == 3)) {
          bpk_in[u] = *reinterpret_cast<const uint32_t*>(bcodes + c * 4);
          bsb_in[u] = bscales[c >> 1];
        }
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * 64 + lane;
      const bool valid = c < nchunks;
      float xf[8];
      unpack8(v[u], xf);
      uint32_t xmax = abs_max8_bits(xf);
      if constexpr (MODE == 3 && PASS <= 1) {
        // static mask: the backbone's maxima are those of the kept values
        bool kept[8];
        static_mask<SPM>(kept);
        float kv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[j] = kept[j] ? xf[j] : 0.0f;
        xmax = abs_max8_bits(kv);
      }
      if constexpr (PASS == 0) {
        run_max = umax(run_max, xmax);
        continue;
      }
      const int64_t g0 = (base + u * 64 + 8 * (lane >> 3)) >> 1;  // first block of this lane's scale word

      if constexpr (MODE == 1) {
        // plain quantization of X with its own tensor scale (PASS 2 only)
        uint32_t sbyte;
        float y;
        const float d = block_divisor(__uint_as_float(pair_max(xmax)), pb, dtab[0], sbyte, y);
        const uint32_t packed = nv_codes(xf, d, y);
        const uint32_t pk = gather_scales(sbyte);
        if (valid) *reinterpret_cast<uint32_t*>(rcodes + c * 4) = packed;
        store_scale_words(rscales, g0, nblocks, lane, pk);
        continue;
      } else {
        float r[8], bh[8];
        bool kept[8];
        if constexpr (PASS == 1) {
          // mask and backbone (with the top-|x| mask the block maximum of the kept
          // values is that of X; the static mask's xmax is already the kept one)
          if constexpr (MODE == 3) static_mask<SPM>(kept);
          else keep_mask<SPM>(xf, kept);
          float kv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) kv[j] = kept[j] ? xf[j] : 0.0f;  // dropped: +0 -> code 0x0
          uint32_t bbyte;
          float y;
          const float d = block_divisor(__uint_as_float(pair_max(xmax)), pb, dtab[0], bbyte, y);
          const uint32_t bpacked = nv_codes(kv, d, y);
          nv_dequant(bpacked, d, bh);
          const uint32_t pk = gather_scales(bbyte);
          if (valid) {
            *reinterpret_cast<uint32_t*>(bcodes + c * 4) = bpacked;
            if constexpr (WRITE_MASK) {
              uint32_t keep = 0;
#pragma unroll
              for (int j = 0; j < 8; ++j) keep |= (kept[j] ? 1u : 0u) << j;
              mask[c] = (uint8_t)keep;
            }
          }
          store_scale_words(bscales, g0, nblocks, lane, pk);
        } else if constexpr (MODE == 0 || MODE == 3) {
          // the backbone as written by pass 1
          const float d = dtab[0][bsb_in[u] & (kDivCodes - 1)].x;  // a code pass 1 wrote: <= 0x7E
          nv_dequant(bpk_in[u], d, bh);
        } else if constexpr (MODE == 2) {
          keep_mask<SPM>(xf, kept);  // the same mask as pass 1's
        }
        if constexpr (MODE == 2) {
#pragma unroll
          for (int j = 0; j < 8; ++j) r[j] = kept[j] ? 0.0f : xf[j];  // x - x*mask, exact
        } else if constexpr (MODE == 4) {
#pragma unroll
          for (int j = 0; j < 8; ++j) r[j] = 0.0f;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) r[j] = __fsub_rn(xf[j], bh[j]);
        }
        const uint32_t rmax = abs_max8_bits(r);
        if constexpr (PASS == 1) {
          run_max = umax(run_max, rmax);
          continue;
        } else {
          uint32_t rbyte;
          float y;
          const float d = block_divisor(__uint_as_float(pair_max(rmax)), pr, dtab[1], rbyte, y);
          const uint32_t rpacked = nv_codes(r, d, y);
          const uint32_t pk = gather_scales(rbyte);
          if (valid) *reinterpret_cast<uint32_t*>(rcodes + c * 4) = rpacked;
          store_scale_words(rscales, g0, nblocks, lane, pk);
        }
      }
    }
  }
  if constexpr (PASS <= 1) {
    // work-group maximum -> one partial per work-group.  (Atomic maxima on one word
    // from every work-group serialize across the chip's separate L2s: a reduction
    // launch is far cheaper.)
    __shared__ uint32_t red[TPB / 64];
    run_max = wave_max(run_max);
    if (lane == 0) red[threadIdx.x >> 6] = run_max;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = 0;
      for (int i = 0; i < TPB / 64; ++i) m = umax(m, red[i]);
      work[kPartialBase + PASS * kMaxGroups + blockIdx.x] = m;
    }
  }
}

// Empty tensors: both maxima 0, tensor scales 1.
__global__ void nv_empty_kernel(uint32_t* work, float* t0, float* t1) {
  if (threadIdx.x == 0) {
    work[0] = 0;
    work[1] = 0;
    if (t0) *t0 = tensor_scale_of(0);
    if (t1) *t1 = tensor_scale_of(0);
  }
}

template <int MODE, int SPM, bool DENSE, bool WRITE_MASK, int XF>
hipError_t run_passes(const uint16_t* x, int64_t ldx, int64_t cpr, int64_t nchunks, uint8_t* bcodes,
                      uint8_t* bscales, float* bts, uint8_t* rcodes, uint8_t* rscales, float* rts, uint8_t* mask,
                      uint32_t* work, const float* rnorm, const uint16_t* gamma, hipStream_t st) {
  const int64_t per_wg = (kThreads / 64) * 64 * kUnroll;
  using S0 = NvShape<0, MODE, DENSE, WRITE_MASK, XF>;
  using S1 = NvShape<1, MODE, DENSE, WRITE_MASK, XF>;
  static_assert(S0::kTpb == S1::kTpb && S0::kGroups == S1::kGroups, "both maximum passes share a shape");
  const int64_t per_wg_max = (S0::kTpb / 64) * 64 * kUnroll;
  const int64_t grid = (nchunks + per_wg - 1) / per_wg;
  const int64_t mgrid = (nchunks + per_wg_max - 1) / per_wg_max;
  const unsigned rgrid = (unsigned)(mgrid < S0::kGroups ? mgrid : S0::kGroups);
  const int np = (int)rgrid;  // partials per maximum pass
  prep_nv_kernel<0, MODE, SPM, DENSE, WRITE_MASK, XF><<<dim3(rgrid), S0::kTpb, 0, st>>>(
      x, ldx, cpr, nchunks, bcodes, bscales, rcodes, rscales, mask, work, bts, rts, rnorm, gamma, np);
  if constexpr (MODE != 1)
    prep_nv_kernel<1, MODE, SPM, DENSE, WRITE_MASK, XF><<<dim3(rgrid), S1::kTpb, 0, st>>>(
        x, ldx, cpr, nchunks, bcodes, bscales, rcodes, rscales, mask, work, bts, rts, rnorm, gamma, np);
  const unsigned lgrid = (unsigned)(grid < kLastGroups ? grid : kLastGroups);
  prep_nv_kernel<2, MODE, SPM, DENSE, WRITE_MASK, XF><<<dim3(lgrid), kThreads, 0, st>>>(
      x, ldx, cpr, nchunks, bcodes, bscales, rcodes, rscales, mask, work, bts, rts, rnorm, gamma, np);
  return hipGetLastError();
}

template <int MODE, int SPM, bool WRITE_MASK, int XF>
hipError_t run_nv(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes, uint8_t* bscales,
                  float* bts, uint8_t* rcodes, uint8_t* rscales, float* rts, uint8_t* mask, uint32_t* work,
                  const float* rnorm, const uint16_t* gamma, hipStream_t st) {
  const int64_t cpr = K / 8;
  const int64_t nchunks = M * cpr;
  if (nchunks == 0) {
    nv_empty_kernel<<<1, 64, 0, st>>>(work, bts, rts);
    return hipGetLastError();
  }
  return ldx == K ? run_passes<MODE, SPM, true, WRITE_MASK, XF>(x, ldx, cpr, nchunks, bcodes, bscales, bts, rcodes,
                                                                  rscales, rts, mask, work, rnorm, gamma, st)
                  : run_passes<MODE, SPM, false, WRITE_MASK, XF>(x, ldx, cpr, nchunks, bcodes, bscales, bts,
                                                                   rcodes, rscales, rts, mask, work, rnorm, gamma, st);
}

template <int SPM, bool WRITE_MASK>
hipError_t run_prep(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes, uint8_t* bscales,
                    float* bts, uint8_t* rcodes, uint8_t* rscales, float* rts, uint8_t* mask, uint32_t* work,
                    const float* rnorm, const uint16_t* gamma, int xf, hipStream_t st) {
  if (xf == kXfRms)
    return run_nv<0, SPM, WRITE_MASK, kXfRms>(x, M, K, ldx, bcodes, bscales, bts, rcodes, rscales, rts, mask, work,
                                              rnorm, gamma, st);
  if (xf == kXfSwiglu)
    return run_nv<0, SPM, WRITE_MASK, kXfSwiglu>(x, M, K, ldx, bcodes, bscales, bts, rcodes, rscales, rts, mask,
                                                 work, nullptr, nullptr, st);
  return run_nv<0, SPM, WRITE_MASK, kXfNone>(x, M, K, ldx, bcodes, bscales, bts, rcodes, rscales, rts, mask, work,
                                             nullptr, nullptr, st);
}

}  // namespace

hipError_t launch_prep_nv(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                          uint8_t* bcodes, uint8_t* bscales, float* btscale, uint8_t* rcodes,
                          uint8_t* rscales, float* rtscale, uint8_t* mask, uint32_t* work,
                          const float* rnorm, const uint16_t* gamma, int swiglu, hipStream_t stream) {
  (void)sp_n;
  const int xf = swiglu ? kXfSwiglu : rnorm ? kXfRms : kXfNone;
  if (sp_m == 4)
    return mask ? run_prep<4, true>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale, mask, work,
                                    rnorm, gamma, xf, stream)
                : run_prep<4, false>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale, mask, work,
                                     rnorm, gamma, xf, stream);
  return mask ? run_prep<8, true>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale, mask, work,
                                  rnorm, gamma, xf, stream)
              : run_prep<8, false>(x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale, mask, work,
                                   rnorm, gamma, xf, stream);
}

namespace {
template <int SPM, bool WRITE_MASK>
hipError_t run_ablation(int variant, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes,
                        uint8_t* bscales, float* bts, uint8_t* rcodes, uint8_t* rscales, float* rts, uint8_t* mask,
                        uint32_t* work, hipStream_t st) {
  switch (variant) {
    case SHARQ_ABLATE_RESIDUAL_UNQUANTIZED:
      return run_nv<2, SPM, WRITE_MASK, kXfNone>(x, M, K, ldx, bcodes, bscales, bts, rcodes, rscales, rts, mask, work,
                                               nullptr, nullptr, st);
    case SHARQ_ABLATE_STATIC_MASK:
      return run_nv<3, SPM, WRITE_MASK, kXfNone>(x, M, K, ldx, bcodes, bscales, bts, rcodes, rscales, rts, mask, work,
                                               nullptr, nullptr, st);
    default:  // SHARQ_ABLATE_NO_RESIDUAL
      return run_nv<4, SPM, WRITE_MASK, kXfNone>(x, M, K, ldx, bcodes, bscales, bts, rcodes, rscales, rts, mask, work,
                                               nullptr, nullptr, st);
  }
}

}  // namespace

hipError_t launch_prep_nv_ablation(int variant, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_m,
                                   uint8_t* bcodes, uint8_t* bscales, float* btscale, uint8_t* rcodes,
                                   uint8_t* rscales, float* rtscale, uint8_t* mask, uint32_t* work,
                                   hipStream_t stream) {
  if (sp_m == 4)
    return mask ? run_ablation<4, true>(variant, x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale,
                                        mask, work, stream)
                : run_ablation<4, false>(variant, x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale,
                                         mask, work, stream);
  return mask ? run_ablation<8, true>(variant, x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale,
                                      mask, work, stream)
              : run_ablation<8, false>(variant, x, M, K, ldx, bcodes, bscales, btscale, rcodes, rscales, rtscale,
                                       mask, work, stream);
}

hipError_t launch_quant_nv(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, float* tscale, uint32_t* work, hipStream_t stream) {
  return run_nv<1, 4, false, kXfNone>(x, rows, K, ldx, nullptr, nullptr, tscale, codes, scales, nullptr, nullptr,
                                    work, nullptr, nullptr, stream);
}

}  // namespace sharq
