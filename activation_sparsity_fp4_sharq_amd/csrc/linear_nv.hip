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
// >= 2^-10), so the operands are decoded into fp16 and the contraction runs on
// v_mfma_f32_32x32x16_f16: every product is exact and only the fp32 summation order
// differs from exact arithmetic.  The two paths keep separate accumulators because
// their tensor scales differ; the decoded weight operand is shared by both.
//
// Tiling: 256 threads (4 waves, 2x2).  For K % 64 == 0 the raw payload is staged
// through LDS and each wave decodes its operands in registers: with both paths and at
// least 256 output tiles of 128x256, linear_nv_wide_kernel (64x128 per wave, one wave
// per SIMD); otherwise linear_nv_stream_kernel (128x128 tiles, 64x64 per wave, two
// work-groups per CU).  Other K take linear_nv_kernel, which decodes each 64-element
// K-step cooperatively into fp16 LDS tiles (rows padded to 144 B), double-buffered.
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

// Epilogue: Y = S_w (S_b acc_b + S_r acc_r) in fp32, each operation rounded to nearest
// (with one activation operand: Y = S_w (S_r acc_r), the same value as with a zero
// backbone); lane holds column r32 of each 32x32 tile and rows 8*(j/4) + 4*h + j%4.
// row0 / col0: the wave's first output row and column (2 x NT instruction tiles).
template <bool OUT_F32, bool DUAL, int NT>
__device__ __forceinline__ void store_tile(const Args& a, const v16f (&accb)[2][NT], const v16f (&accr)[2][NT],
                                           int64_t row0, int64_t col0, int r32, int h) {
  const float sb = DUAL ? *a.bt : 0.f, sr = *a.rt, sw = *a.wt;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t col = col0 + nt * 32 + r32;
      if (col >= a.N) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t row = row0 + mt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
        if (row < a.M) {
          const float pr = __fmul_rn(sr, accr[mt][nt][j]);
          const float v = __fmul_rn(sw, DUAL ? __fadd_rn(__fmul_rn(sb, accb[mt][nt][j]), pr) : pr);
          if constexpr (OUT_F32)
            reinterpret_cast<float*>(a.y)[row * a.ldy + col] = v;
          else
            reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + col] = f32_to_bf16_rne(v);
        }
      }
    }
}

template <bool OUT_F32, bool DUAL>
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
    for (int which = DUAL ? 0 : 1; which < 3; ++which) {  // 0: A_b (absent for one operand), 1: A_r, 2: W
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
    for (int which = DUAL ? 0 : 1; which < 3; ++which)
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
        if constexpr (DUAL) ab[mt] = *reinterpret_cast<const v8h*>(base + row * kRowPitch + col);
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
          if constexpr (DUAL)
            accb[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ab[mt], wf[nt], accb[mt][nt], 0, 0, 0);
          accr[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ar[mt], wf[nt], accr[mt][nt], 0, 0, 0);
        }
    }
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  store_tile<OUT_F32, DUAL, 2>(a, accb, accr, m0 + wm * 64, n0 + wn * 64, r32, h);
}

// ---------------------------------------------------------------------------------
// Streaming variant for K % 64 == 0 (the usual case).  The raw payload -- 32 code
// bytes and 4 scale bytes per row and 64-element stage -- goes global -> LDS by
// LDS-DMA into a 3-slot ring, three stages ahead, with no registers in flight.  Each
// wave then reads the raw bytes of its own 64 A rows and 64 W rows straight into
// registers and decodes them into matrix-instruction operands there: no fp16 tile in
// LDS, one barrier per stage, and the decode's vector work of one wave runs beside the
// matrix instructions of the other wave on its SIMD (two work-groups per CU).
//
// K order inside a stage: the matrix instruction's k-slot 8*h + j (h = lane / 32) of
// sub-step i stands for stage element 32*h + 8*i + j, for A and W alike -- a dot
// product does not depend on the order of its terms -- so that a lane's four
// sub-steps read one contiguous 16-byte run of codes (elements 32*h .. 32*h + 31,
// NVFP4 blocks 2*h and 2*h + 1).
//   stage s:  raw bytes of stage s+1 -> registers;  16 sub-step pairs of matrix
//             instructions on stage s (decoded from registers);  own loads of stage
//             s+2 landed (vmcnt 5);  barrier;  DMA of stage s+4 into slot (s+1)%3
// Per stage each wave issues 5 loads: 3 of the 12 code pieces (32 rows x 32 B) and 2
// of the 6 scale pieces (64 rows x 4 B; wave 3 repeats wave 2's), so every wave's
// count is the same.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kRawCodeBytes = 3 * BM * 32;                  // 12 KiB
constexpr int kRawStageBytes = kRawCodeBytes + 3 * BM * 4;  // + 1.5 KiB of scales
constexpr int kRawStages = 3;
constexpr int kStreamLds = kRawStages * kRawStageBytes;     // 40.5 KiB
#define SHARQ_NV_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Two E4M3 scale bytes (low two bytes of w) -> their exact values as two fp16.  The
// byte's low seven bits shifted left by seven form an fp16 with the same exponent and
// mantissa fields, valued at 2^-8 of the E4M3 value (subnormals included: m * 2^-17),
// and the scaling by 2^8 is exact.
__device__ __forceinline__ v2h scale_pair(uint32_t w) {
  const uint32_t bits = ((w & 0x7Fu) << 7) | ((w & 0x7F00u) << 15);
  v2h s;
  __builtin_memcpy(&s, &bits, 4);
  return s * v2h{(_Float16)256.0f, (_Float16)256.0f};
}

// 8 E2M1 codes (one dword) times a block scale -> one matrix-instruction operand
__device__ __forceinline__ v8h decode8(uint32_t codes, _Float16 sc) {
  const v2h s2 = {sc, sc};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;  // <= 6 significant bits: exact
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <bool OUT_F32, bool DUAL>
__global__ __launch_bounds__(kThreads, 2) void linear_nv_stream_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* raw = smem;  // kRawStages x [codes: 3 tiles x 128 rows x 32 B][scales: 3 x 128 x 4 B]
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

  // this wave's loads per stage: 3 code pieces and 2 scale pieces (2 and 1 without
  // A_b; rows past the operand's end re-read its last row, never stored)
  constexpr int kT0 = DUAL ? 0 : 1;            // first tile present
  constexpr int kCodeLoads = DUAL ? 3 : 2, kScaleLoads = DUAL ? 2 : 1;
  constexpr int kLoads = kCodeLoads + kScaleLoads;
  const uint8_t* csrc[3];  // (fixed extents: template-dependent ones drop the host launch stub)
  int cdst[3];
#pragma unroll
  for (int j = 0; j < kCodeLoads; ++j) {
    const int piece = kCodeLoads * wave + j, t = kT0 + (piece >> 2), part = piece & 3;
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
  for (int j = 0; j < kScaleLoads; ++j) {
    // DUAL: 6 pieces, wave 3 repeats wave 2's; else 4 pieces, one per wave
    const int piece = DUAL ? 2 * (wave < 3 ? wave : 2) + j : wave, t = kT0 + (piece >> 1), part = piece & 1;
    const uint8_t* base = t == 0 ? a.bs : t == 1 ? a.rs : a.ws;
    const int64_t rows = t == 2 ? a.N : a.M;
    int64_t row = (t == 2 ? n0 : m0) + 64 * part + lane;
    row = row < rows ? row : rows - 1;
    ssrc[j] = base + row * nbk;
    sdst[j] = kRawCodeBytes + t * BM * 4 + part * 256;
  }
  auto dma = [&](int ks) {
    uint8_t* st = raw + (ks % kRawStages) * kRawStageBytes;
    const int64_t kc = ks < nk ? ks : nk - 1;  // past the end: re-load into a slot nobody reads
#pragma unroll
    for (int j = 0; j < kCodeLoads; ++j)
      __builtin_amdgcn_global_load_lds(csrc[j] + kc * 32, (lds_void_t*)(st + cdst[j]), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < kScaleLoads; ++j)
      __builtin_amdgcn_global_load_lds(ssrc[j] + kc * 4, (lds_void_t*)(st + sdst[j]), 4, 0, 0);
  };

  // this lane's six operand rows: A_b and A_r of rows wm*64 + 32*mt + r32, W of rows
  // wn*64 + 32*nt + r32; raw bytes: 16 code bytes at offset 16*h, two scale bytes
  int roff[6];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    roff[2 * mt] = wm * 64 + mt * 32 + r32;             // tile 0 (A_b)
    roff[2 * mt + 1] = BM + wm * 64 + mt * 32 + r32;    // tile 1 (A_r)
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) roff[4 + nt] = 2 * BM + wn * 64 + nt * 32 + r32;
  struct Raw {
    u32x4 codes[6];
    uint32_t scales[6];
  };
  auto read_raw = [&](Raw& r, int ks) {
    const uint8_t* st = raw + (ks % kRawStages) * kRawStageBytes;
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      if (!DUAL && q < 4 && (q & 1) == 0) continue;  // A_b absent
      r.codes[q] = *reinterpret_cast<const u32x4*>(st + roff[q] * 32 + h * 16);
      r.scales[q] = *reinterpret_cast<const uint32_t*>(st + kRawCodeBytes + roff[q] * 4) >> (16 * h);
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
  auto compute = [&](const Raw& r) {
    v2h sc[6];
#pragma unroll
    for (int q = 0; q < 6; ++q)
      if (DUAL || q >= 4 || (q & 1)) sc[q] = scale_pair(r.scales[q]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8h f[6];
#pragma unroll
      for (int q = 0; q < 6; ++q)
        if (DUAL || q >= 4 || (q & 1)) f[q] = decode8(r.codes[q][i], sc[q][i >> 1]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          if constexpr (DUAL)
            accb[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f[2 * mt], f[4 + nt], accb[mt][nt], 0, 0, 0);
          accr[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f[2 * mt + 1], f[4 + nt], accr[mt][nt], 0, 0, 0);
        }
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's raw reads have returned
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_sched_barrier(0);
  };

  dma(0);
  dma(1);
  dma(2);
  SHARQ_NV_WAIT_VMCNT(kLoads);  // this wave's loads of stages 0 and 1 landed
  barrier();
  Raw cur, nxt;
  read_raw(cur, 0);
  barrier();  // every wave has stage 0 in registers: its slot is free
  dma(3);
  for (int ks = 0; ks < nk; ++ks) {
    read_raw(nxt, ks + 1);   // past the last stage: a loaded slot, never used
    __builtin_amdgcn_sched_barrier(0);  // issue the reads first: their latency hides under compute
    compute(cur);
    __builtin_amdgcn_sched_barrier(0);
    SHARQ_NV_WAIT_VMCNT(kLoads);  // this wave's loads of stage ks+2 landed
    barrier();               // ... everyone's; everyone has stage ks+1 in registers
    dma(ks + 4);             // into the slot of stage ks+1
    cur = nxt;
  }
  SHARQ_NV_WAIT_VMCNT(0);

  store_tile<OUT_F32, DUAL, 2>(a, accb, accr, m0 + wm * 64, n0 + wn * 64, r32, h);
}

// ---------------------------------------------------------------------------------
// Wide variant (both activation paths, K % 64 == 0, enough output tiles to fill the
// chip).  The same raw-payload streaming and register decode as the streaming kernel,
// with a 64x128 tile per wave (2 x 4 instructions per path) and one wave per SIMD: a
// wave decodes 2 x 64 activation rows and 128 weight rows per stage for 64 matrix
// instructions, a third less vector work per instruction than at 64x64, and its 256
// accumulators sit in the accumulation registers, so the wave's decode of the next
// sub-step issues between its own matrix instructions.  4 waves (2 x 2) own a
// 128 x 256 output tile; the ring holds 4 stages of 18 KiB.
//
// Stage layout (rows of 32 code bytes, then one scale word per row, same row order):
// rows 0-127 A_b, 128-255 A_r, 256-511 W.  Per stage each wave loads 4 of the 16
// code pieces (32 rows, 1 KiB) and 2 of the 8 scale pieces (64 rows, 256 B).
constexpr int kWideBM = 128, kWideBN = 256;
constexpr int kWideRows = 2 * kWideBM + kWideBN;                 // 512
constexpr int kWideCodeBytes = kWideRows * 32;                   // 16 KiB
constexpr int kWideStageBytes = kWideCodeBytes + kWideRows * 4;  // + 2 KiB of scales
constexpr int kWideStages = 4;
constexpr int kWideLds = kWideStages * kWideStageBytes;          // 72 KiB
constexpr int kWideMinTiles = 256;
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3: raw (unswizzled) 32-bit data

template <bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void linear_nv_wide_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kWideBM, n0 = (int64_t)tn * kWideBN;
  const int64_t kb = a.K / 2, nbk = a.K / 16;
  const int nk = (int)(a.K / BK);

  // this wave's loads per stage (rows past an operand's end re-read its last row,
  // never stored)
  constexpr int kCodeLoads = 4, kScaleLoads = 2, kLoads = kCodeLoads + kScaleLoads;
  // sources as buffer resources (base, byte extent) and per-lane offsets: with buffer
  // loads the compiler tracks the LDS-read counter in order, so a use of one LDS read
  // waits for that read only (after global_load_lds it waits for all of them)
  const uint8_t* cbase[kCodeLoads];
  uint32_t cbytes[kCodeLoads], coff[kCodeLoads];
  int cdst[kCodeLoads];
#pragma unroll
  for (int j = 0; j < kCodeLoads; ++j) {
    const int piece = kCodeLoads * wave + j;    // 0..15, 32 stage rows each
    const int srow = 32 * piece + (lane >> 1);  // stage row of this lane's 16 bytes
    const int t = srow < kWideBM ? 0 : srow < 2 * kWideBM ? 1 : 2;
    const uint8_t* base = t == 0 ? a.bc : t == 1 ? a.rc : a.wc;
    const int64_t rows = t == 2 ? a.N : a.M;
    int64_t row = t == 2 ? n0 + (srow - 2 * kWideBM) : m0 + (srow - t * kWideBM);
    row = row < rows ? row : rows - 1;
    cbase[j] = base;
    cbytes[j] = (uint32_t)(rows * kb);
    coff[j] = (uint32_t)(row * kb + (lane & 1) * 16);
    cdst[j] = piece * 1024;
  }
  const uint8_t* sbase[kScaleLoads];
  uint32_t sbytes[kScaleLoads], soff[kScaleLoads];
  int sdst[kScaleLoads];
#pragma unroll
  for (int j = 0; j < kScaleLoads; ++j) {
    const int piece = kScaleLoads * wave + j;  // 0..7, 64 stage rows each
    const int srow = 64 * piece + lane;
    const int t = srow < kWideBM ? 0 : srow < 2 * kWideBM ? 1 : 2;
    const uint8_t* base = t == 0 ? a.bs : t == 1 ? a.rs : a.ws;
    const int64_t rows = t == 2 ? a.N : a.M;
    int64_t row = t == 2 ? n0 + (srow - 2 * kWideBM) : m0 + (srow - t * kWideBM);
    row = row < rows ? row : rows - 1;
    sbase[j] = base;
    sbytes[j] = (uint32_t)(rows * nbk);
    soff[j] = (uint32_t)(row * nbk);
    sdst[j] = kWideCodeBytes + piece * 256;
  }
  // load j (< kLoads) of stage ks (past the end: re-load into a slot nobody reads)
  auto dma_one = [&](int j, int ks) {
    uint8_t* st = smem + (ks % kWideStages) * kWideStageBytes;
    const int64_t kc = ks < nk ? ks : nk - 1;
    if (j < kCodeLoads) {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cbase[j]), 0, cbytes[j], kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(st + cdst[j]), 16, coff[j] + (uint32_t)kc * 32, 0, 0,
                                               0);
    } else {
      const int t = j - kCodeLoads;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sbase[t]), 0, sbytes[t], kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(st + sdst[t]), 4, soff[t] + (uint32_t)kc * 4, 0, 0, 0);
    }
  };
  auto dma = [&](int ks) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) dma_one(j, ks);
  };

  // this lane's eight operand rows in the stage: A_b / A_r rows wm*64 + 32*mt + r32
  // (q = 2*mt + path), W rows wn*128 + 32*nt + r32 (q = 4 + nt)
  int roff[8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    roff[2 * mt] = wm * 64 + mt * 32 + r32;
    roff[2 * mt + 1] = kWideBM + wm * 64 + mt * 32 + r32;
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) roff[4 + nt] = 2 * kWideBM + wn * 128 + nt * 32 + r32;
  struct Raw {
    u32x4 codes[8];
    uint32_t scales[8];
  };
  auto read_one = [&](Raw& r, int q, int ks) {
    const uint8_t* st = smem + (ks % kWideStages) * kWideStageBytes;
    r.codes[q] = *reinterpret_cast<const u32x4*>(st + roff[q] * 32 + h * 16);
    r.scales[q] = *reinterpret_cast<const uint32_t*>(st + kWideCodeBytes + roff[q] * 4);  // 4 blocks
  };
  auto read_raw = [&](Raw& r, int ks) {
#pragma unroll
    for (int q = 0; q < 8; ++q) read_one(r, q, ks);
  };

  // accumulators [mt][nt] hold W-tile x A-tile products (weights as the instruction's A
  // operand): lane (r32, h) holds output row 32*mt + r32 and the 4 consecutive columns
  // 32*nt + 8*g + 4*h + {0..3} in elements 4g..4g+3
  v16f accb[2][4], accr[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      accb[i][j] = v16f{};
      accr[i][j] = v16f{};
    }
  // Sub-step i of a stage: 16 instructions on operands decoded during sub-step i-1 (for
  // sub-step 0, during the previous stage's sub-step 3).  After every instruction the
  // wave issues half of the decode of one of the next sub-step's eight operands (two
  // conversions and two scale products: vector work that fits under one instruction);
  // during sub-step 0 also this stage's share of the ring loads (stage ks+4).  One set
  // of raw registers serves all stages: operand q's bytes of stage ks are last used by
  // the decode in sub-step 2, right after which the same registers receive stage ks+1's
  // bytes from LDS; sub-step 3 turns them into the next stage's block scales and its
  // first operands.
  v8h f[2][8];
  v2h sc[8], scn[8];
  auto compute = [&](Raw& r, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v8h(&c)[8] = f[i & 1];
      v8h(&n)[8] = f[(i + 1) & 1];
      if (i == 3) scn[0] = scale_pair(r.scales[0] >> (16 * h));  // blocks 2h, 2h+1 of stage ks+1
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int mt = j >> 3, path = (j >> 2) & 1, nt = j & 3;
        if (path == 0)
          accb[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(c[4 + nt], c[2 * mt], accb[mt][nt], 0, 0, 0);
        else
          accr[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(c[4 + nt], c[2 * mt + 1], accr[mt][nt], 0, 0, 0);
        // half (two dwords) of operand q of the next sub-step (sub-step 3: of stage ks+1)
        const int q = j >> 1, half = j & 1;
        const uint32_t codes = r.codes[q][(i + 1) & 3];
        const _Float16 s1 = i < 3 ? sc[q][(i + 1) >> 1] : scn[q][0];
        const v2h s2 = {s1, s1};
        // (the byte selector must be a literal)
        const v2h p0 = (half ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2)
                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0)) * s2;  // exact
        const v2h p1 = (half ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3)
                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1)) * s2;
        n[q][4 * half] = p0[0];
        n[q][4 * half + 1] = p0[1];
        n[q][4 * half + 2] = p1[0];
        n[q][4 * half + 3] = p1[1];
        if (i == 0 && j < kLoads) dma_one(j, ks + kWideStages);  // into the slot of stage ks
        // stage ks+1 replaces stage ks in operand q's registers once q's last decode is issued
        if (i == 2 && half) read_one(r, q, ks + 1);
        if (i == 3 && half && q < 7) scn[q + 1] = scale_pair(r.scales[q + 1] >> (16 * h));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 3) {
#pragma unroll
        for (int q = 0; q < 8; ++q) sc[q] = scn[q];
      }
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's raw reads have returned
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_sched_barrier(0);
  };
  // one K-step: stage ks in `r` on entry, stage ks+1 on exit (past the last stage: a
  // loaded slot, decoded and never used)
  auto step = [&](Raw& r, int ks) {
    compute(r, ks);
    __builtin_amdgcn_sched_barrier(0);
    SHARQ_NV_WAIT_VMCNT((kWideStages - 2) * kLoads);  // this wave's loads of stage ks+2 landed
    barrier();  // ... everyone's; everyone has stage ks+1 in registers (its slot is free)
  };

  // at the top of step ks: stages ks and ks+1 landed and visible to all waves, stage
  // ks in registers with its sub-step 0 decoded and its slot free, this wave's loads
  // of stages ks+2 and ks+3 in flight (step ks adds those of stage ks+4)
#pragma unroll
  for (int s = 0; s < kWideStages; ++s) dma(s);
  SHARQ_NV_WAIT_VMCNT((kWideStages - 2) * kLoads);  // this wave's loads of stages 0 and 1 landed
  barrier();
  Raw ra;
  read_raw(ra, 0);
  barrier();  // every wave has stage 0 in registers: its slot is free
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    sc[q] = scale_pair(ra.scales[q] >> (16 * h));
    f[0][q] = decode8(ra.codes[q][0], sc[q][0]);
  }
  for (int ks = 0; ks < nk; ++ks) step(ra, ks);
  SHARQ_NV_WAIT_VMCNT(0);
  __syncthreads();  // the ring is free: the epilogue stages the output tile in it

  // Epilogue: Y = S_w (S_b acc_b + S_r acc_r), each operation rounded to nearest.  A
  // wave whose 64x128 tile lies inside Y (bf16, 16-byte aligned rows) writes it to its
  // own LDS region and stores whole 16-byte row runs; others store element by element.
  const float sb = *a.bt, sr = *a.rt, sw = *a.wt;
  const int64_t row0 = m0 + wm * 64, col0 = n0 + wn * 128;
  const bool fast = !OUT_F32 && row0 + 64 <= a.M && col0 + 128 <= a.N &&
                    (reinterpret_cast<uintptr_t>(a.y) & 15u) == 0 && a.ldy % 8 == 0;
  if (fast) {
    constexpr int pitch = 128 * 2 + 16;
    uint8_t* lds = smem + wave * (64 * pitch);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint16_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * g + i;
            o[i] = f32_to_bf16_rne(
                __fmul_rn(sw, __fadd_rn(__fmul_rn(sb, accb[mt][nt][e]), __fmul_rn(sr, accr[mt][nt][e]))));
          }
          *reinterpret_cast<u32x2*>(lds + (mt * 32 + r32) * pitch + (nt * 32 + 8 * g + 4 * h) * 2) =
              u32x2{o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16)};
        }
    const int lr = lane >> 4, lc = lane & 15;  // 16 lanes per 256-byte row, 4 rows per pass
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = 4 * it + lr;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * pitch + lc * 16);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.y) + (row0 + row) * a.ldy + col0 + lc * 8) = v;
    }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = row0 + mt * 32 + r32;
        const int64_t col = col0 + nt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row >= a.M || col >= a.N) continue;
        const float v =
            __fmul_rn(sw, __fadd_rn(__fmul_rn(sb, accb[mt][nt][e]), __fmul_rn(sr, accr[mt][nt][e])));
        if constexpr (OUT_F32)
          reinterpret_cast<float*>(a.y)[row * a.ldy + col] = v;
        else
          reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + col] = f32_to_bf16_rne(v);
      }
}

// The dynamic-LDS limit is a per-device function attribute, set once per device and
// kernel instantiation (setting it twice is harmless).
template <const void* (*KERNEL)()>
hipError_t configure(int lds_bytes) {
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(KERNEL(), hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  return hipSuccess;
}
template <bool OUT_F32, bool DUAL>
const void* stream_kernel() { return reinterpret_cast<const void*>(&linear_nv_stream_kernel<OUT_F32, DUAL>); }
template <bool OUT_F32, bool DUAL>
const void* generic_kernel() { return reinterpret_cast<const void*>(&linear_nv_kernel<OUT_F32, DUAL>); }
template <bool OUT_F32>
const void* wide_kernel() { return reinterpret_cast<const void*>(&linear_nv_wide_kernel<OUT_F32>); }

template <bool OUT_F32, bool DUAL>
hipError_t launch(const Args& a, hipStream_t stream) {
  const dim3 grid(a.tiles_m * a.tiles_n);
  hipError_t e;
  if constexpr (DUAL) {
    // the wide tiles when they still give every CU one
    const int64_t wtm = (a.M + kWideBM - 1) / kWideBM, wtn = (a.N + kWideBN - 1) / kWideBN;
    // (buffer offsets are 32-bit: every payload below 2 GiB)
    const bool small = (a.M > a.N ? a.M : a.N) * (a.K / 2) < ((int64_t)1 << 31);
    if (a.K % BK == 0 && wtm * wtn >= kWideMinTiles && small) {
      Args w = a;
      w.tiles_m = (int)wtm;
      w.tiles_n = (int)wtn;
      if ((e = configure<wide_kernel<OUT_F32>>(kWideLds)) != hipSuccess) return e;
      linear_nv_wide_kernel<OUT_F32><<<dim3((unsigned)(wtm * wtn)), dim3(kThreads), kWideLds, stream>>>(w);
      return hipGetLastError();
    }
  }
  if (a.K % BK == 0) {
    if ((e = configure<stream_kernel<OUT_F32, DUAL>>(kStreamLds)) != hipSuccess) return e;
    linear_nv_stream_kernel<OUT_F32, DUAL><<<grid, dim3(kThreads), kStreamLds, stream>>>(a);
  } else {
    if ((e = configure<generic_kernel<OUT_F32, DUAL>>(2 * kStageBytes)) != hipSuccess) return e;
    linear_nv_kernel<OUT_F32, DUAL><<<grid, dim3(kThreads), 2 * kStageBytes, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

size_t linear_nv_workspace(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_linear_nv(const sharq_fp4* b, const sharq_fp4& r, int64_t M, const sharq_fp4& w,
                            int64_t N, int64_t K, void* y, int64_t ldy, int out_fp32, void*, size_t,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  Args a{b ? b->codes : nullptr, b ? b->scales : nullptr, b ? b->tensor_scale : nullptr,
         r.codes, r.scales, r.tensor_scale, w.codes, w.scales,
         w.tensor_scale, y, M, N, K, ldy, (int)((M + BM - 1) / BM), (int)((N + BN - 1) / BN)};
  if (b) return out_fp32 ? launch<true, true>(a, stream) : launch<false, true>(a, stream);
  return out_fp32 ? launch<true, false>(a, stream) : launch<false, false>(a, stream);
}

}  // namespace sharq
