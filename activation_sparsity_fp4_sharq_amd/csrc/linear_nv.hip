// linear_nv.hip -- the two SharQ GEMMs over one NVFP4 weight payload on gfx950.
//
// Y = S_w (S_b * Bhat' W'^T + S_r * Rhat' W'^T), where a primed operand is the
// payload's E2M1 value times its E4M3 block scale and S_* are the per-tensor scales
// (SharQ, arXiv 2606.26587: abstract -- backbone and residual GEMMs share one FP4
// weight payload with path-specific scales; NVFP4 is one of the named formats).
//
// gfx950's block-scaled FP4 matrix instructions take power-of-two (E8M0) block
// scales only, and an E2M1 value times an E4M3 scale needs up to 6 significant bits,
// more than FP8 holds.  The product is, however, exact in fp16 (|v*s| <= 2688,
// >= 2^-10), so the operands are decoded once per work-group into fp16 while they are
// staged into LDS, and the contraction runs on v_mfma_f32_32x32x16_f16: every
// product is exact and only the fp32 summation order differs from exact arithmetic.
// The two paths keep separate accumulators because their tensor scales differ; the
// weight tile in LDS is shared by both.
//
// Tiling: 256 threads (4 waves, 2x2) own a 128x128 output tile (64x64 per wave =
// 2x2 instructions per path); per 64-element K-step the block decodes A_b, A_r and
// W (128 rows x 64 fp16 each, rows padded to 144 B) into LDS, double-buffered.
#include <atomic>

#include "sharq_internal.h"

namespace sharq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kRowPitch = BK * 2 + 16;       // bytes per LDS row (64 fp16 + pad)
constexpr int kTileBytes = BM * kRowPitch;   // 18432
constexpr int kStageBytes = 3 * kTileBytes;
constexpr int kXcds = 8;

struct Args {
  const uint8_t* bc; const uint8_t* bs; const float* bt;
  const uint8_t* rc; const uint8_t* rs; const float* rt;
  const uint8_t* wc; const uint8_t* ws; const float* wt;
  void* y;
  int64_t M, N, K, ldy;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E4M3 byte -> its value (both forms computed and selected: no branch in the decode)
__device__ __forceinline__ float e4m3_value(uint32_t s) {
  const uint32_t ef = (s >> 3) & 15u, m = s & 7u;
  const float normal = __uint_as_float(((ef + 120u) << 23) | (m << 20));
  const float subnormal = (float)m * 0.001953125f;  // m * 2^-9
  return ef == 0 ? subnormal : normal;
}

__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int logical = id;
  if (total % kXcds == 0) logical = (id % kXcds) * (total / kXcds) + id / kXcds;
  constexpr int G = 4;
  const int group = logical / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(tiles_m - first_m, G);
  const int in_group = logical - group * G * tiles_n;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// 16 E2M1 codes (8 bytes) times an E4M3 block scale -> 16 exact fp16 values.
__device__ __forceinline__ void decode16(u32x2 codes, uint32_t sbyte, v2h out[8]) {
  const _Float16 sh = (_Float16)e4m3_value(sbyte);  // exact: E4M3 lies inside fp16's range
  const v2h s2 = {sh, sh};
  v2h p[8];
  p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[0], 1.0f, 0);
  p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[0], 1.0f, 1);
  p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[0], 1.0f, 2);
  p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[0], 1.0f, 3);
  p[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[1], 1.0f, 0);
  p[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[1], 1.0f, 1);
  p[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[1], 1.0f, 2);
  p[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[1], 1.0f, 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = p[i] * s2;  // <= 6 significant bits: exact
}

template <bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void linear_nv_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = a.K / 2;    // code bytes per row
  const int64_t nbk = a.K / 16;  // scale bytes per row
  const int nk = (int)((a.K + BK - 1) / BK);

  // thread t stages chunk (row t/2, 32-element half t%2) of each of the three tiles
  const int srow = tid >> 1, scc = tid & 1;
  u32x2 gcodes[3][2];
  uint32_t gscale[3][2];

  auto gload = [&](int ks) {
#pragma unroll
    for (int which = 0; which < 3; ++which) {
      const uint8_t* c = which == 0 ? a.bc : which == 1 ? a.rc : a.wc;
      const uint8_t* s = which == 0 ? a.bs : which == 1 ? a.rs : a.ws;
      const int64_t grow = (which == 2 ? n0 : m0) + srow;
      const bool row_ok = grow < (which == 2 ? a.N : a.M);
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const int64_t blk = (int64_t)ks * 4 + scc * 2 + bi;  // 16-element block index along K
        gcodes[which][bi] = u32x2{0u, 0u};
        gscale[which][bi] = 0u;
        if (row_ok && blk < nbk) {
          gcodes[which][bi] = *reinterpret_cast<const u32x2*>(c + grow * kb + blk * 8);
          gscale[which][bi] = s[grow * nbk + blk];
        }
      }
    }
  };

  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * kStageBytes;
#pragma unroll
    for (int which = 0; which < 3; ++which)
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        v2h d[8];
        decode16(gcodes[which][bi], gscale[which][bi], d);
        uint8_t* dst = base + which * kTileBytes + srow * kRowPitch + (scc * 32 + bi * 16) * 2;
        u32x4 lo, hi;
        __builtin_memcpy(&lo, &d[0], 16);
        __builtin_memcpy(&hi, &d[4], 16);
        *reinterpret_cast<u32x4*>(dst) = lo;
        *reinterpret_cast<u32x4*>(dst + 16) = hi;
      }
  };

  v16f accb[2][2], accr[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      accb[i][j] = v16f{};
      accr[i][j] = v16f{};
    }

  gload(0);
  sstore(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* base = smem + buf * kStageBytes;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int col = (16 * s + 8 * h) * 2;
      v8h ab[2], ar[2], wf[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = wm * 64 + mt * 32 + r32;
        ab[mt] = *reinterpret_cast<const v8h*>(base + row * kRowPitch + col);
        ar[mt] = *reinterpret_cast<const v8h*>(base + kTileBytes + row * kRowPitch + col);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = wn * 64 + nt * 32 + r32;
        wf[nt] = *reinterpret_cast<const v8h*>(base + 2 * kTileBytes + row * kRowPitch + col);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          accb[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ab[mt], wf[nt], accb[mt][nt], 0, 0, 0);
          accr[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ar[mt], wf[nt], accr[mt][nt], 0, 0, 0);
        }
    }
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  const float sb = *a.bt, sr = *a.rt, sw = *a.wt;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t col = n0 + wn * 64 + nt * 32 + r32;
      if (col >= a.N) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t row = m0 + wm * 64 + mt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
        if (row < a.M) {
          const float v = __fmul_rn(sw, __fadd_rn(__fmul_rn(sb, accb[mt][nt][j]), __fmul_rn(sr, accr[mt][nt][j])));
          if constexpr (OUT_F32)
            reinterpret_cast<float*>(a.y)[row * a.ldy + col] = v;
          else
            reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + col] = f32_to_bf16_rne(v);
        }
      }
    }
}

// ---------------------------------------------------------------------------------
// Streaming variant for K % 64 == 0 (the usual case).  The raw payload -- 32 code
// bytes and 4 scale bytes per row and 64-element K-step -- goes global -> LDS by
// LDS-DMA into a 3-slot ring, two K-steps ahead, with no registers in flight; each
// K-step is then decoded cooperatively (every element once per work-group) into the
// fp16 tile the matrix instructions read, while the previous tile is consumed.
// One barrier per K-step:
//   iteration ks:  DMA of step ks+3 into raw slot ks%3 (decoded in iteration ks-1)
//                  decode raw step ks+1 -> fp16 buffer (ks+1)%2 | MFMA on buffer ks%2
//                  own loads of step ks+2 landed (vmcnt 5); barrier
// Per stage each wave issues 5 loads: 3 of the 12 code pieces (32 rows x 32 B) and 2
// of the 6 scale pieces (64 rows x 4 B; wave 3 repeats wave 2's), so every wave's
// count is the same.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kRawCodeBytes = 3 * BM * 32;                  // 12 KiB
constexpr int kRawStageBytes = kRawCodeBytes + 3 * BM * 4;  // + 1.5 KiB of scales
constexpr int kRawStages = 3;
constexpr int kRawBytes = kRawStages * kRawStageBytes;
#define SHARQ_NV_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void linear_nv_stream_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* raw = smem;               // kRawStages x [codes: 3 tiles x 128 rows x 32 B][scales: 3 x 128 x 4 B]
  uint8_t* half = smem + kRawBytes;  // 2 x 3 fp16 tiles
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = a.K / 2, nbk = a.K / 16;
  const int nk = (int)(a.K / BK);

  // this wave's loads: 3 code pieces and 2 scale pieces per stage (rows past the
  // operand's end re-read its last row; their results are never stored)
  const uint8_t* csrc[3];
  int cdst[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int piece = 3 * wave + j, t = piece >> 2, part = piece & 3;
    const uint8_t* base = t == 0 ? a.bc : t == 1 ? a.rc : a.wc;
    const int64_t rows = t == 2 ? a.N : a.M;
    int64_t row = (t == 2 ? n0 : m0) + 32 * part + (lane >> 1);
    row = row < rows ? row : rows - 1;
    csrc[j] = base + row * kb + (lane & 1) * 16;
    cdst[j] = t * BM * 32 + part * 1024;
  }
  const uint8_t* ssrc[2];
  int sdst[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int piece = 2 * (wave < 3 ? wave : 2) + j, t = piece >> 1, part = piece & 1;
    const uint8_t* base = t == 0 ? a.bs : t == 1 ? a.rs : a.ws;
    const int64_t rows = t == 2 ? a.N : a.M;
    int64_t row = (t == 2 ? n0 : m0) + 64 * part + lane;
    row = row < rows ? row : rows - 1;
    ssrc[j] = base + row * nbk;
    sdst[j] = kRawCodeBytes + t * BM * 4 + part * 256;
  }
  auto dma = [&](int ks) {
    uint8_t* st = raw + (ks % kRawStages) * kRawStageBytes;
    const int64_t kc = ks < nk ? ks : nk - 1;  // past the end: re-load into a slot nobody decodes
#pragma unroll
    for (int j = 0; j < 3; ++j)
      __builtin_amdgcn_global_load_lds(csrc[j] + kc * 32, (lds_void_t*)(st + cdst[j]), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(ssrc[j] + kc * 4, (lds_void_t*)(st + sdst[j]), 4, 0, 0);
  };

  // cooperative decode: thread t owns row t/2, 32-element half t%2 of each tile; a
  // step is 6 units (tile, 16-element block) over raw bytes read up front
  const int srow = tid >> 1, scc = tid & 1;
  u32x4 rcodes[3];
  uint32_t rsc[3];
  auto read_raw = [&](int ks) {
    const uint8_t* st = raw + (ks % kRawStages) * kRawStageBytes;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      rcodes[t] = *reinterpret_cast<const u32x4*>(st + t * BM * 32 + srow * 32 + scc * 16);
      rsc[t] = *reinterpret_cast<const uint16_t*>(st + kRawCodeBytes + t * BM * 4 + srow * 4 + scc * 2);
    }
  };
  auto decode_unit = [&](int u, int buf) {
    const int t = u >> 1, bi = u & 1;
    v2h d[8];
    decode16(u32x2{rcodes[t][2 * bi], rcodes[t][2 * bi + 1]}, (rsc[t] >> (8 * bi)) & 0xFFu, d);
    uint8_t* dst = half + buf * kStageBytes + t * kTileBytes + srow * kRowPitch + (scc * 32 + bi * 16) * 2;
    u32x4 lo, hi;
    __builtin_memcpy(&lo, &d[0], 16);
    __builtin_memcpy(&hi, &d[4], 16);
    *reinterpret_cast<u32x4*>(dst) = lo;
    *reinterpret_cast<u32x4*>(dst + 16) = hi;
  };
  auto decode = [&](int ks, int buf) {
    read_raw(ks);
#pragma unroll
    for (int u = 0; u < 6; ++u) decode_unit(u, buf);
  };

  v16f accb[2][2], accr[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      accb[i][j] = v16f{};
      accr[i][j] = v16f{};
    }
  // fp16 fragments of one 16-element sub-step, double-buffered in registers
  v8h fab[2][2], far[2][2], fw[2][2];
  auto read_frags = [&](int buf, int s, int slot) {
    const uint8_t* base = half + buf * kStageBytes;
    const int col = (16 * s + 8 * h) * 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int row = wm * 64 + mt * 32 + r32;
      fab[slot][mt] = *reinterpret_cast<const v8h*>(base + row * kRowPitch + col);
      far[slot][mt] = *reinterpret_cast<const v8h*>(base + kTileBytes + row * kRowPitch + col);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = wn * 64 + nt * 32 + r32;
      fw[slot][nt] = *reinterpret_cast<const v8h*>(base + 2 * kTileBytes + row * kRowPitch + col);
    }
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        accb[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fab[slot][mt], fw[slot][nt], accb[mt][nt], 0, 0, 0);
        accr[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(far[slot][mt], fw[slot][nt], accr[mt][nt], 0, 0, 0);
      }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_sched_barrier(0);
  };

  dma(0);
  dma(1);
  dma(2);
  SHARQ_NV_WAIT_VMCNT(10);  // step 0 landed
  barrier();
  decode(0, 0);
  SHARQ_NV_WAIT_VMCNT(5);   // step 1 landed
  barrier();
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1, nxt = cur ^ 1;
    dma(ks + 3);
    // (in the last iteration this decodes the clamped re-load of the last step into
    // the idle buffer: wasted once, but the body stays branch-free)
    read_raw(ks + 1);
    read_frags(cur, 0, 0);
    // each sub-step's 8 matrix instructions are issued, then a share of the next
    // step's decode runs on the vector ALU while they execute
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) read_frags(cur, s + 1, (s + 1) & 1);
      mma(s & 1);
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0 || s == 2) {
        decode_unit(s == 0 ? 0 : 3, nxt);
        decode_unit(s == 0 ? 1 : 4, nxt);
      } else {
        decode_unit(s == 1 ? 2 : 5, nxt);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    SHARQ_NV_WAIT_VMCNT(5);  // this wave's loads of step ks+2 landed
    barrier();
  }
  SHARQ_NV_WAIT_VMCNT(0);

  const float sb = *a.bt, sr = *a.rt, sw = *a.wt;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t col = n0 + wn * 64 + nt * 32 + r32;
      if (col >= a.N) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t row = m0 + wm * 64 + mt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
        if (row < a.M) {
          const float v = __fmul_rn(sw, __fadd_rn(__fmul_rn(sb, accb[mt][nt][j]), __fmul_rn(sr, accr[mt][nt][j])));
          if constexpr (OUT_F32)
            reinterpret_cast<float*>(a.y)[row * a.ldy + col] = v;
          else
            reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + col] = f32_to_bf16_rne(v);
        }
      }
    }
}

template <bool OUT_F32>
hipError_t launch_stream(const Args& a, hipStream_t stream) {
  constexpr int kLds = kRawBytes + 2 * kStageBytes;
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_nv_stream_kernel<OUT_F32>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  linear_nv_stream_kernel<OUT_F32><<<dim3(a.tiles_m * a.tiles_n), dim3(kThreads), kLds, stream>>>(a);
  return hipGetLastError();
}

template <bool OUT_F32>
hipError_t launch(const Args& a, hipStream_t stream) {
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_nv_kernel<OUT_F32>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStageBytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  linear_nv_kernel<OUT_F32><<<dim3(a.tiles_m * a.tiles_n), dim3(kThreads), 2 * kStageBytes, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

size_t linear_nv_workspace(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_linear_nv(const sharq_fp4& b, const sharq_fp4& r, int64_t M, const sharq_fp4& w,
                            int64_t N, int64_t K, void* y, int64_t ldy, int out_fp32, void*, size_t,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  Args a{b.codes, b.scales, b.tensor_scale, r.codes, r.scales, r.tensor_scale, w.codes, w.scales,
         w.tensor_scale, y, M, N, K, ldy, (int)((M + BM - 1) / BM), (int)((N + BN - 1) / BN)};
  if (K % BK == 0) return out_fp32 ? launch_stream<true>(a, stream) : launch_stream<false>(a, stream);
  return out_fp32 ? launch<true>(a, stream) : launch<false>(a, stream);
}

}  // namespace sharq
