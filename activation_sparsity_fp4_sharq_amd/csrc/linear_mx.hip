// linear_mx.hip -- the two SharQ GEMMs over one MXFP4 weight payload on gfx950.
//
// Y = Bhat W^T + Rhat W^T (SharQ, arXiv 2606.26587: abstract -- a sparse FP4 GEMM
// for the backbone and a dense FP4 GEMM for the residual share a single FP4 weight
// payload).  Both products run on the block-scaled FP4 matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 and accumulate into the SAME fp32 registers, and
// every weight tile staged in LDS is used by both paths, so the pair costs one
// weight stream and one accumulator tile.  gfx950 has no sparse (SMFMAC) form of
// the FP4 instruction, so the backbone runs zero-filled: its dropped positions hold
// code 0x0 and contribute exact zeros.
//
// Operand layout of the 32x32x64 FP4 instruction (checked on the device): lane l
// holds row (l % 32) and 32 consecutive K-elements of half (l / 32); its 16 bytes
// are those elements in the canonical nibble order (element 2c low nibble of byte
// c), and its E8M0 scale applies to exactly those 32 elements -- one MX block.  So a
// lane's operand is one 16-byte run of a row of the canonical payload, and its
// scale is the byte of that block.  The K order inside one instruction is free as
// long as A and B agree: lane half h at sub-step s takes block 2h+s of the 4-block
// (128-element) K-step, so a lane reads 32 contiguous bytes per K-step and the
// scale byte for sub-step s is byte s of (row's 4 scale bytes >> 16h), selected by
// the instruction's op_sel.
//
// Three kernels share the instruction and the 256x256 output tile: the pipelined
// LDS-DMA kernel for tiled payloads (the layout the preparation writes), a small-M
// kernel for tiled payloads with M <= 32 (decode: a weight stream), and a generic
// register-staged kernel for row-major payloads.  The generic kernel: 512 threads (8
// waves, 2 per SIMD) form a 4 (M) x 2 (N) grid of 64x128 wave tiles = 2x4
// instructions per path and sub-step; per 128-element K-step the block stages A_b,
// A_r, W tiles (256 rows x 64 B each, rows padded to 80 B so that 16-byte LDS reads of
// 32 consecutive rows hit distinct banks) and their scale dwords, double-buffered; one
// barrier per K-step.  Work-groups are renumbered so that consecutive tiles share an
// XCD (and its L2).  With one activation operand (sharq_linear_dense) every kernel
// skips the backbone path.
#include <atomic>
#include <type_traits>

#include "sharq_internal.h"

namespace sharq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BKB = 64;  // tile rows, tile cols, bytes of K per step (128 elements)
constexpr int kThreads = 512;
constexpr int kRowPitch = BKB + 16;          // padded LDS row (bytes)
constexpr int kTileBytes = BM * kRowPitch;   // 20480
constexpr int kStageBytes = 3 * kTileBytes + 3 * BM * 4;
constexpr int kXcds = 8;

struct Args {
  const uint8_t* bc; const uint8_t* bs;
  const uint8_t* rc; const uint8_t* rs;
  const uint8_t* wc; const uint8_t* ws;
  void* y;
  int64_t M, N, K, ldy;
  int tiles_m, tiles_n;
  int64_t Mp, Np, Kp;  // padded extents of the tiled layout
  bool y_aligned;      // y 16-byte aligned and ldy a multiple of 8 elements
  int splits;          // K split across this many work-groups per tile (1: none)
  float* part;         // fp32 partial sums [splits][M][N] when splits > 1
  int64_t wsp;         // row pitch of the weight's tiled scale words (its whole payload's padded rows)
};

// An FP4 operand is the low 4 dwords of the instruction's 8-dword operand; the upper
// half is ignored, so it is left undefined (no register copies).
__device__ __forceinline__ v8i widen(v4i a) {
  return __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values to two bf16 (a in the low half) in one gfx950 packed conversion
// (v_cvt_pk_bf16_f32): round to nearest even, so on every finite fp32 value the same
// bits as f32_to_bf16_rne (sharq_bf16_rounding_probe runs all 2^32 patterns through the
// same conversion on the device).  One instruction per pair against about six.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  const f32x2_t p = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
}

// The hardware hands work-group id to XCD id % 8; renumber the ids so that each XCD's
// share of the `total` ids is one contiguous run.
__device__ __forceinline__ int xcd_contiguous(int id, int total) {
  return total % kXcds == 0 ? (id % kXcds) * (total / kXcds) + id / kXcds : id;
}

// Tile of a contiguous id: runs of ids walk the tiles in groups of 4 tile-rows.
__device__ __forceinline__ void tile_of_run(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int G = 4;
  const int group = logical / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(tiles_m - first_m, G);
  const int in_group = logical - group * G * tiles_n;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Map the hardware work-group id to a tile so that the ids one XCD receives
// (id % 8 == x) form a contiguous run of tiles, walked in groups of 4 tile-rows.
__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  tile_of_run(xcd_contiguous(id, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// Epilogue shared by both kernels: lane holds column r32 of each 32x32 tile and rows
// 8*(j/4) + 4*h + j%4 of it (the 32x32 accumulator layout); bf16 is rounded to nearest-even.
template <bool OUT_F32>
__device__ __forceinline__ void store_tile(const Args& a, const v16f (&acc)[2][4], int64_t m0, int64_t n0,
                                           int wm, int wn, int r32, int h) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t col = n0 + wn * 128 + nt * 32 + r32;
      if (col >= a.N) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t row = m0 + wm * 64 + mt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
        if (row < a.M) {
          if constexpr (OUT_F32)
            reinterpret_cast<float*>(a.y)[row * a.ldy + col] = acc[mt][nt][j];
          else
            reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + col] = f32_to_bf16_rne(acc[mt][nt][j]);
        }
      }
    }
}

template <bool K_ALIGNED>
__device__ __forceinline__ uint32_t load_scale_dword(const uint8_t* s, int64_t row, int64_t nbk, int kstep) {
  if constexpr (K_ALIGNED) {
    return *reinterpret_cast<const uint32_t*>(s + row * nbk + (int64_t)kstep * 4);
  } else {
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i) {
      const int64_t blk = (int64_t)kstep * 4 + i;
      if (blk < nbk) v |= (uint32_t)s[row * nbk + blk] << (8 * i);
    }
    return v;
  }
}

template <bool OUT_F32, bool K_ALIGNED, bool DUAL>
__global__ __launch_bounds__(kThreads, 1) void linear_mx_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;   // 0..3
  const int wn = wave & 1;    // 0..1
  const int r32 = lane & 31;
  const int h = lane >> 5;

  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = a.K / 2;      // bytes per row
  const int64_t nbk = a.K / 32;    // scale bytes per row
  const int nk = (int)((a.K + 127) / 128);

  // ---- global -> register staging assignments (6 code chunks + 2 scale dwords per thread)
  u32x4 stage[6];
  uint32_t sstage[2];

  auto gload = [&](int kstep) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int c = tid + kThreads * (i & 1);  // chunk 0..1023 within its tile
      const int row = c >> 2, col = c & 3;
      const int which = i >> 1;              // 0: A_b, 1: A_r, 2: W
      if (!DUAL && which == 0) continue;     // one activation operand: A_b absent
      const uint8_t* src = which == 0 ? a.bc : which == 1 ? a.rc : a.wc;
      const int64_t grow = (which == 2 ? n0 : m0) + row;
      const int64_t glim = which == 2 ? a.N : a.M;
      const int64_t kbyte = (int64_t)kstep * BKB + col * 16;
      stage[i] = u32x4{0u, 0u, 0u, 0u};
      if (grow < glim && kbyte < kb)
        stage[i] = *reinterpret_cast<const u32x4*>(src + grow * kb + kbyte);
    }
    // scale dwords: thread t < 256 -> A_b row t, < 512 -> A_r row t-256; second: W row t (t < 256)
    {
      const int row = tid & 255;
      const uint8_t* s = tid < 256 ? a.bs : a.rs;
      const int64_t grow = m0 + row;
      sstage[0] = grow < a.M && (DUAL || tid >= 256) ? load_scale_dword<K_ALIGNED>(s, grow, nbk, kstep) : 0u;
      const int64_t wrow = n0 + row;
      sstage[1] = (tid < 256 && wrow < a.N) ? load_scale_dword<K_ALIGNED>(a.ws, wrow, nbk, kstep) : 0u;
    }
  };

  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int c = tid + kThreads * (i & 1);
      const int row = c >> 2, col = c & 3;
      const int which = i >> 1;
      if (!DUAL && which == 0) continue;
      *reinterpret_cast<u32x4*>(base + which * kTileBytes + row * kRowPitch + col * 16) = stage[i];
    }
    uint32_t* sc = reinterpret_cast<uint32_t*>(base + 3 * kTileBytes);
    sc[tid] = sstage[0];                      // [0,256): A_b scales, [256,512): A_r scales
    if (tid < 256) sc[512 + tid] = sstage[1]; // [512,768): W scales
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  gload(0);
  sstore(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);

    const uint8_t* base = smem + buf * kStageBytes;
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(base + 3 * kTileBytes);
    // fragments for both sub-steps: lane reads 32 contiguous bytes of its row
    v4i af[2][2][2];  // [path][mt][substep]
    uint32_t as[2][2];
#pragma unroll
    for (int p = DUAL ? 0 : 1; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = wm * 64 + mt * 32 + r32;
        const uint8_t* src = base + p * kTileBytes + row * kRowPitch + 32 * h;
        af[p][mt][0] = *reinterpret_cast<const v4i*>(src);
        af[p][mt][1] = *reinterpret_cast<const v4i*>(src + 16);
        as[p][mt] = sc[p * 256 + row] >> (16 * h);
      }
    v4i wf[4][2];
    uint32_t ws[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int row = wn * 128 + nt * 32 + r32;
      const uint8_t* src = base + 2 * kTileBytes + row * kRowPitch + 32 * h;
      wf[nt][0] = *reinterpret_cast<const v4i*>(src);
      wf[nt][1] = *reinterpret_cast<const v4i*>(src + 16);
      ws[nt] = sc[512 + row] >> (16 * h);
    }
#pragma unroll
    for (int p = DUAL ? 0 : 1; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              widen(af[p][mt][0]), widen(wf[nt][0]), acc[mt][nt], 4, 4, 0, (int)as[p][mt], 0, (int)ws[nt]);
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              widen(af[p][mt][1]), widen(wf[nt][1]), acc[mt][nt], 4, 4, 1, (int)as[p][mt], 1, (int)ws[nt]);
        }

    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  store_tile<OUT_F32>(a, acc, m0, n0, wm, wn, r32, h);
}

// ---------------------------------------------------------------------------------
// Pipelined kernel for tiled payloads (K padded to 128 by the layout).
//
// Same tiling and instruction as above, but the operands travel global -> LDS by
// LDS-DMA (buffer_load_dwordx4 ... lds) instead of through registers, into a 3-deep
// ring of stages, so the loads of later K-steps are in flight while a K-step
// computes (the schedule is described at the loop).  Each operand tile is stored in LDS in *fragment order*:
// 16 fragments of 1 KiB (8 row-tiles of 32 rows x 2 sub-steps), fragment byte
// 16*lane holding exactly the 16 bytes lane `lane` feeds the instruction.  A DMA
// load writes 64 lanes x 16 B contiguously, so one load fills one fragment (each
// lane fetches the global bytes its slot needs), and one ds_read_b128 at
// 16*lane reads it back with no bank conflicts.  Sub-step s, lane half h takes the
// 16-byte chunk 2s+h of the row's 64-byte K-step, so a load reads 32 contiguous
// bytes per row; the scale byte of chunk 2s+h is byte 2s of (row scale word >> 8h),
// op_sel 0 or 2.  Row tiles past the padded extent are clamped to the last one and
// scale words past it read as zero: loaded and computed, never stored.
constexpr int kFragBytes = 1024;
constexpr int kOpTileBytes = 16 * kFragBytes;                   // 256 rows x 128 K
constexpr int kDmaStageBytes = 3 * kOpTileBytes + 3 * 256 * 4;  // + scale words
constexpr int kDmaStages = 3;

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS-DMA through a buffer resource (buffer_load_dwordx4 ... lds): each lane's 16 bytes
// at `base + voffset` (base wave-uniform) land at LDS `dst + 16 * lane`.  Bytes past
// `bytes` read as zero.  The buffer form, unlike global_load_lds, leaves the compiler's
// LDS-read counter exact, so fragment reads that follow are waited for one by one
// instead of all at once.  Descriptor word 3 is the gfx9-family raw-buffer setting
// (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ void buffer_lds16(const uint8_t* base, uint32_t bytes, uint8_t* dst, uint32_t voffset) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voffset, 0, 0, 0);
}

// Epilogue of the tiled kernels.  The weights are the instruction's A operand, so in
// accumulator acc[mt][nt] lane (r32, h) holds output row (row0 + 32mt + r32) and
// columns col0 + 32nt + 8g + 4h + {0,1,2,3} in elements 4g..4g+3 -- four consecutive
// outputs.  A wave whose tile lies inside Y (and a 16-byte aligned Y) stages its bf16
// tile through its private LDS region (rows padded to 16 bytes past the tile width)
// and writes whole 16-byte runs, 16 lanes per row; other waves, and fp32 output,
// store the 4-value runs directly with bounds checks.
constexpr int kEpiPad = 16;

template <bool OUT_F32, int MT, int NT>
__device__ __forceinline__ void store_swapped(const Args& a, const v16f (&acc)[MT][NT], int64_t row0,
                                              int64_t col0, int lane, uint8_t* lds, bool y_aligned) {
  const int r32 = lane & 31, h = lane >> 5;
  const bool inside = row0 + 32 * MT <= a.M && col0 + 32 * NT <= a.N;
  if constexpr (!OUT_F32) {
    if (inside && y_aligned) {
      constexpr int pitch = 32 * NT * 2 + kEpiPad;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t lo = f32x2_to_bf16x2_rne(acc[mt][nt][4 * g], acc[mt][nt][4 * g + 1]);
            const uint32_t hi = f32x2_to_bf16x2_rne(acc[mt][nt][4 * g + 2], acc[mt][nt][4 * g + 3]);
            *reinterpret_cast<uint2*>(lds + (mt * 32 + r32) * pitch + (nt * 32 + 8 * g + 4 * h) * 2) = make_uint2(lo, hi);
          }
      constexpr int lanes_per_row = 32 * NT * 2 / 16;
      constexpr int rows_per_iter = 64 / lanes_per_row;
      const int lr = lane / lanes_per_row, lc = lane % lanes_per_row;
#pragma unroll
      for (int it = 0; it < 32 * MT / rows_per_iter; ++it) {
        const int row = it * rows_per_iter + lr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * pitch + lc * 16);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.y) + (row0 + row) * a.ldy + col0 + lc * 8) = v;
      }
      return;
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t row = row0 + mt * 32 + r32;
        const int64_t col = col0 + nt * 32 + 8 * g + 4 * h;
        if (row >= a.M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (col + i < a.N) {
            if constexpr (OUT_F32)
              reinterpret_cast<float*>(a.y)[row * a.ldy + col + i] = acc[mt][nt][4 * g + i];
            else
              reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + col + i] = f32_to_bf16_rne(acc[mt][nt][4 * g + i]);
          }
      }
}

// The fp32 partial tile of a wave (64 rows x 128 columns, accumulator layout as above)
// into part (row pitch N): staged through the wave's LDS region 32 rows at a time, so
// that each store instruction writes two whole 512-byte row runs.  A tile reaching past
// M or N, or rows that are not 16-byte aligned (N % 4 != 0), store element runs directly.
__device__ __forceinline__ void store_partial(float* part, int64_t M, int64_t N, const v16f (&acc)[2][4],
                                              int64_t row0, int64_t col0, int lane, uint8_t* lds) {
  const int r32 = lane & 31, h = lane >> 5;
  if (row0 + 64 > M || col0 + 128 > N || (N & 3) != 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t row = row0 + mt * 32 + r32;
          const int64_t col = col0 + nt * 32 + 8 * g + 4 * h;
          if (row >= M) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (col + i < N) part[row * N + col + i] = acc[mt][nt][4 * g + i];
        }
    return;
  }
  constexpr int pitch = 128 * 4 + 16;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(lds + r32 * pitch + (nt * 32 + 8 * g + 4 * h) * 4) =
            f32x4{acc[mt][nt][4 * g], acc[mt][nt][4 * g + 1], acc[mt][nt][4 * g + 2], acc[mt][nt][4 * g + 3]};
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave-private region is written
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = 2 * it + (lane >> 5), c = lane & 31;
      *reinterpret_cast<f32x4*>(part + (row0 + mt * 32 + row) * N + col0 + 4 * c) =
          *reinterpret_cast<const f32x4*>(lds + row * pitch + c * 16);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // every read of the region done before it is rewritten
    __builtin_amdgcn_wave_barrier();
  }
}

// s_waitcnt with only the vector-memory counter constrained (expcnt/lgkmcnt left free).
#define SHARQ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// SPLIT: work-group s of a tile sums the K-steps
// [s*steps/splits, (s+1)*steps/splits) and stores its fp32 tile into part[s]; the
// partials are summed in order by reduce_splits_kernel.  TN: tile columns, 256 or 128
// (each wave then owns 64 x TN/2 outputs: TN/64 instructions across per path and row tile).
template <bool OUT_F32, bool DUAL, bool SPLIT, int TN = BN>
__global__ __launch_bounds__(kThreads, 1) void linear_mx_dma_kernel(Args a) {
  static_assert(TN == 256 || TN == 128, "tile columns");
  static_assert(!SPLIT || TN == 256, "the K split runs 256-column tiles");
  constexpr int NT = TN / 64;  // 32-column instruction tiles per wave
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

  int tm, tn;
  int split = 0;
  if constexpr (SPLIT) {
    // each XCD gets a contiguous run of (split, tile) ids, split-major, so that the tiles
    // it holds at once share activation and weight panels as in the unsplit order
    const int tiles = a.tiles_m * a.tiles_n;
    const int id = xcd_contiguous((int)blockIdx.x, tiles * a.splits);
    split = id / tiles;
    tile_of_run(id - split * tiles, a.tiles_m, a.tiles_n, tm, tn);
  } else {
    tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * TN;
  int nk = (int)(a.Kp / 128);
  int k0 = 0;  // first K-step
  if constexpr (SPLIT) {
    const int steps = nk;
    k0 = split * steps / a.splits;
    nk = (split + 1) * steps / a.splits - k0;
  }

  // Each wave fills 6 of the 48 fragments of a stage (A_b, A_r x 16, W x TN/16; 4 of 32
  // without A_b; 5 of 40 and 3 of 24 with 128 columns): one contiguous 1 KiB fragment of
  // the tiled payload per load.  Row tiles past the padded extent are clamped to the last
  // one (computed, never stored).
  constexpr int kFragLoads = ((DUAL ? 32 : 16) + TN / 16) / 8;
  constexpr int kOp0 = DUAL ? 0 : 1;  // first activation operand present
  const uint8_t* fsrc[6];  // (fixed extent: a template-dependent one drops the host launch stub)
  int fdst[6];
#pragma unroll
  for (int j = 0; j < kFragLoads; ++j) {
    const int f = wave * kFragLoads + j;
    const int op = kOp0 + (f >> 4), fi = f & 15, rt = fi >> 1, sub = fi & 1;
    const uint8_t* base = op == 0 ? a.bc : op == 1 ? a.rc : a.wc;
    const int64_t ntiles = (op == 2 ? a.Np : a.Mp) / 32;
    int64_t t = (op == 2 ? n0 : m0) / 32 + rt;
    t = t < ntiles ? t : ntiles - 1;
    fsrc[j] = base + (t * (a.Kp / 64) + sub) * kFragBytes;  // wave-uniform; lane adds 16 * lane
    if constexpr (SPLIT) fsrc[j] += 2 * (int64_t)k0 * kFragBytes;
    fdst[j] = op * kOpTileBytes + fi * kFragBytes;
  }
  // Scale words: one operand's 256 words per K-step are 1 KiB contiguous; the first
  // waves load one operand each and the others repeat the weight's load (identical
  // bytes to the same place), so every wave issues the same loads per stage and no
  // branch sits between them -- the compiler's vmcnt bookkeeping then never degrades
  // to a full wait.
  // (rows past the padded extent read as zero: the load is bounded to the rows that exist)
  const uint8_t* ssrc;
  int64_t sstep;
  uint32_t sbytes;
  int sdst;
  {
    const int op = (kOp0 + wave < 3) ? kOp0 + wave : 2;
    const uint8_t* base = op == 0 ? a.bs : op == 1 ? a.rs : a.ws;
    const int64_t rp = op == 2 ? a.Np : a.Mp;
    const int64_t row0 = op == 2 ? n0 : m0;
    ssrc = base + row0 * 4;  // wave-uniform; lane adds 16 * lane (4 rows)
    sstep = (op == 2 ? a.wsp : rp) * 4;
    if constexpr (SPLIT) ssrc += k0 * sstep;
    sbytes = (uint32_t)((rp - row0) * 4 < 1024 ? (rp - row0) * 4 : 1024);
    sdst = 3 * kOpTileBytes + op * 1024;
  }
  constexpr int kLoads = kFragLoads + 1;  // per wave and stage
  // load j of stage ks (a stage past the last K-step -- only the prologue's, when K has
  // fewer than three steps -- re-loads the last one into a slot nobody reads)
  // the fragment loads go through loop-invariant resources over the tile's whole K range
  // (the K-step is the scalar offset), the scale block through one per K-step
  __amdgpu_buffer_rsrc_t frsrc[6];
#pragma unroll
  for (int j = 0; j < kFragLoads; ++j)
    frsrc[j] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(fsrc[j]), 0,
                                                 (uint32_t)nk * 2u * (uint32_t)kFragBytes, kRsrcWord3);
  auto issue_one = [&](int j, int ks, int slot) {
    uint8_t* st = smem + slot * kDmaStageBytes;
    const int64_t kc = ks < nk ? ks : nk - 1;
    if (j < kFragLoads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(frsrc[j], (lds_void_t*)(st + fdst[j]), 16, 16 * lane,
                                               (int)(kc * 2 * kFragBytes), 0, 0);
    else
      buffer_lds16(ssrc + kc * sstep, sbytes, st + sdst, 16 * lane);
  };

  v16f acc[2][NT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = v16f{};

  // Software pipeline across the K-steps, one barrier per step placed between its two
  // sub-steps, so the LDS latency of every fragment read hides under matrix work:
  //   [A] read sub-step 1 fragments of stage ks  |  16 MFMA on sub-step 0 of ks
  //   [B] own loads of stage ks+1 landed; all reads of stage ks done (lgkmcnt 0);
  //       barrier: stage ks+1 visible, slot ks%3 free
  //   [C] read scales + sub-step 0 fragments of ks+1  |  16 MFMA on sub-step 1 of ks,
  //       with the DMA of stage ks+3 into slot ks%3 spread between them
  // (the last three K-steps issue no loads: the stages they read are already in flight)
  auto read_frags = [&](v4i (&af)[2][2], v4i (&wf)[NT], const uint8_t* st, int sub) {
#pragma unroll
    for (int p = kOp0; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[p][mt] = *reinterpret_cast<const v4i*>(st + p * kOpTileBytes + ((wm * 2 + mt) * 2 + sub) * kFragBytes +
                                                  lane * 16);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wf[nt] = *reinterpret_cast<const v4i*>(st + 2 * kOpTileBytes + ((wn * NT + nt) * 2 + sub) * kFragBytes +
                                             lane * 16);
  };
  // Fragment j of sub-step 0 in read_frags' order (the activation fragments, then the weight's)
  constexpr int kReads = 2 * (2 - kOp0) + NT;
  auto read_one = [&](v4i (&af)[2][2], v4i (&wf)[NT], const uint8_t* st, int j) {
    constexpr int na = 2 * (2 - kOp0);
    if (j < na) {
      const int p = kOp0 + j / 2, mt = j % 2;
      af[p][mt] = *reinterpret_cast<const v4i*>(st + p * kOpTileBytes + ((wm * 2 + mt) * 2) * kFragBytes + lane * 16);
    } else {
      const int nt = j - na;
      wf[nt] = *reinterpret_cast<const v4i*>(st + 2 * kOpTileBytes + ((wn * NT + nt) * 2) * kFragBytes + lane * 16);
    }
  };
  auto read_scales = [&](uint32_t (&as)[2][2], uint32_t (&ws)[NT], const uint8_t* st) {
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + 3 * kOpTileBytes);
#pragma unroll
    for (int p = kOp0; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) as[p][mt] = sc[p * 256 + wm * 64 + mt * 32 + r32];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ws[nt] = sc[512 + wn * (TN / 2) + nt * 32 + r32];
  };
  // The matrix instructions of one sub-step (16 with both paths and 256 columns).  With
  // ISSUE, the loads of stage ld spread between them (one per kEvery instructions), and
  // the LDS stage rst's sub-step-0 fragments (into raf / rwf, one after each of the first
  // kReads instructions) and scale words (ras / rws, after the next one) are read between
  // them instead of all ahead of them, so that the LDS issue queue never holds the wave
  // back before its first matrix instruction.
  auto mma = [&](const v4i (&af)[2][2], const v4i (&wf)[NT], const uint32_t (&as)[2][2], const uint32_t (&ws)[NT],
                 auto sub_c, auto issue_c, int ld, int slot, v4i (&raf)[2][2], v4i (&rwf)[NT], const uint8_t* rst,
                 uint32_t (&ras)[2][2], uint32_t (&rws)[NT]) {
    constexpr int SUB = decltype(sub_c)::value;
    constexpr bool ISSUE = decltype(issue_c)::value;
    static_assert(2 * NT * (2 - kOp0) >= kReads, "one fragment read per matrix instruction");
    constexpr int kPerSub = 2 * NT * (2 - kOp0), kEvery = kPerSub / kLoads;
    static_assert(kEvery >= 1 && kPerSub / kEvery >= kLoads, "every load of a stage must be issued");
#pragma unroll
    for (int p = kOp0; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          // weights as the instruction's A operand: each lane's accumulators are then
          // 4 consecutive output columns of one output row (see store_swapped)
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              widen(wf[nt]), widen(af[p][mt]), acc[mt][nt], 4, 4, 2 * SUB, (int)(ws[nt] >> (8 * h)), 2 * SUB,
              (int)(as[p][mt] >> (8 * h)));
          if constexpr (ISSUE) {
            const int i = ((p - kOp0) * 2 + mt) * NT + nt;
            if (i < kReads) read_one(raf, rwf, rst, i);
            if (i == kReads) read_scales(ras, rws, rst);
            if (i % kEvery == kEvery - 1 && i / kEvery < kLoads) {
              issue_one(i / kEvery, ld, slot);
              __builtin_amdgcn_sched_barrier(0);  // keep the loads spread between the instructions
            }
          }
        }
  };

#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue_one(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue_one(j, 1, 1);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue_one(j, 2, 2);
  SHARQ_WAIT_VMCNT(2 * kLoads);  // this wave's loads of stage 0 landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  v4i af0[2][2], wf0[NT], af1[2][2], wf1[NT];
  uint32_t as[2][2], ws[NT], asn[2][2], wsn[NT];
  read_scales(as, ws, smem);
  read_frags(af0, wf0, smem, 0);
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using NoIssue = std::integral_constant<bool, false>;
  using Issue = std::integral_constant<bool, true>;
  // One K-step.  ISSUE: the loads of stage ks+3 go out during it; WAIT: the loads this
  // wave may leave in flight at the barrier (the stage after ks has landed then); slot:
  // ks % 3, the ring slot it reads and refills.  The loop runs whole rounds of the ring, so
  // the slots -- and every LDS address -- are compile-time constants there.
  auto kstep = [&](int ks, auto issue_c, auto wait_c, auto slot_c) {
    constexpr int WAIT = decltype(wait_c)::value;
    const int S = slot_c;  // ks % 3: a constant in the unrolled loop
    const uint8_t* st = smem + S * kDmaStageBytes;
    const uint8_t* nx = smem + (S == kDmaStages - 1 ? 0 : S + 1) * kDmaStageBytes;
    // [A]
    // sub-step 1's fragments, one read after each of the first sub-step-0 instructions (the
    // scheduling groups: 1 matrix instruction, 1 LDS read, ..., then the remaining ones)
    read_frags(af1, wf1, st, 1);
    mma(af0, wf0, as, ws, C0{}, NoIssue{}, 0, 0, af0, wf0, st, asn, wsn);  // (no ISSUE: reads nothing)
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NT * (2 - kOp0) - kReads, 0);
    // [B]
    __builtin_amdgcn_sched_barrier(0);
    SHARQ_WAIT_VMCNT(WAIT);              // this wave's loads of stage ks+1 landed
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage ks are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_sched_barrier(0);
    // [C]
    // the next stage's sub-step-0 fragments and scale words: inside the mma when it issues
    // loads, ahead of it otherwise
    if constexpr (!decltype(issue_c)::value) {
      read_scales(asn, wsn, nx);
      read_frags(af0, wf0, nx, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(af1, wf1, as, ws, C1{}, issue_c, ks + 3, S, af0, wf0, nx, asn, wsn);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) as[p][mt] = asn[p][mt];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ws[nt] = wsn[nt];
  };
  using Keep = std::integral_constant<int, kLoads>;
  using None = std::integral_constant<int, 0>;
  // every K-step but the last three loads a stage three ahead; those three load nothing
  // (all the stages they read are in flight), so no stage past the last is fetched
  const int nmain = nk > 3 ? nk - 3 : 0;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  int ks = 0;
  for (; ks + 3 <= nmain; ks += 3) {  // one round of the stage ring: slots known at compile time
    kstep(ks, Issue{}, Keep{}, S0{});
    kstep(ks + 1, Issue{}, Keep{}, S1{});
    kstep(ks + 2, Issue{}, Keep{}, S2{});
  }
  if (ks < nmain) kstep(ks++, Issue{}, Keep{}, S0{});
  if (ks < nmain) kstep(ks++, Issue{}, Keep{}, S1{});
  if (nk >= 3) kstep(nk - 3, NoIssue{}, Keep{}, (nk - 3) % kDmaStages);
  if (nk >= 2) kstep(nk - 2, NoIssue{}, None{}, (nk - 2) % kDmaStages);
  kstep(nk - 1, NoIssue{}, None{}, (nk - 1) % kDmaStages);
  SHARQ_WAIT_VMCNT(0);  // trailing loads land before the stage ring is reused

  __syncthreads();  // every wave is done with the stage ring; reuse it for the epilogue
  if constexpr (SPLIT) {
    store_partial(a.part + (int64_t)split * a.M * a.N, a.M, a.N, acc, m0 + wm * 64, n0 + wn * 128, lane,
                  smem + wave * (32 * (128 * 4 + 16)));
  } else {
    store_swapped<OUT_F32, 2, NT>(a, acc, m0 + wm * 64, n0 + wn * (TN / 2), lane,
                                  smem + wave * (64 * (NT * 64 + kEpiPad)), a.y_aligned);
  }
}

// y = sum over s of part[s], in order s = 0, 1, ... (one fp32 rounding per addition,
// the same order every call), rounded to bf16 or stored as fp32.  Four consecutive
// outputs per thread: 16-byte partial loads when N is a multiple of 4 (part is 16-byte
// aligned), one 8- or 16-byte store when y allows it (vec_y), element by element
// otherwise and in a row's last partial quad.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                            int64_t N, void* __restrict__ y, int64_t ldy,
                                                            bool vec_y) {
  const int64_t nq = (N + 3) / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * nq) return;
  const int64_t row = i / nq, c0 = (i - row * nq) * 4;
  const int64_t plane = M * N;
  const float* p = part + row * N + c0;
  if ((N & 3) == 0) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(p);
    for (int s = 1; s < splits; ++s) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(p + s * plane);
      acc = f32x4{__fadd_rn(acc[0], t[0]), __fadd_rn(acc[1], t[1]), __fadd_rn(acc[2], t[2]), __fadd_rn(acc[3], t[3])};
    }
    if (vec_y) {
      if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + row * ldy + c0) = acc;
      } else {
        const uint32_t lo = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + row * ldy + c0) = make_uint2(lo, hi);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (OUT_F32)
        reinterpret_cast<float*>(y)[row * ldy + c0 + j] = acc[j];
      else
        reinterpret_cast<uint16_t*>(y)[row * ldy + c0 + j] = f32_to_bf16_rne(acc[j]);
    }
    return;
  }
  const int cn = N - c0 < 4 ? (int)(N - c0) : 4;
  for (int j = 0; j < cn; ++j) {
    float acc = p[j];
    for (int s = 1; s < splits; ++s) acc = __fadd_rn(acc, p[j + s * plane]);
    if constexpr (OUT_F32)
      reinterpret_cast<float*>(y)[row * ldy + c0 + j] = acc;
    else
      reinterpret_cast<uint16_t*>(y)[row * ldy + c0 + j] = f32_to_bf16_rne(acc);
  }
}

// The dynamic-LDS limit is a per-device function attribute, set once per kernel and device
// (setting it twice is harmless).
template <bool OUT_F32, bool DUAL, bool SPLIT, int TN = BN>
hipError_t configure_dma() {
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_mx_dma_kernel<OUT_F32, DUAL, SPLIT, TN>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kDmaStages * kDmaStageBytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  return hipSuccess;
}

// Columns of 256-wide tiles to run as a tail of 128-wide tiles (0: none): when the tiles
// overflow whole waves of work-groups (one per compute unit) by at most half a wave and
// that overflow is whole tile columns, so the tail's 256 x 128 tiles fill at most one wave.
constexpr int kWave = 256;  // work-groups of this kernel resident at once (one per compute unit)

int tail_columns(int tiles_m, int tiles_n) {
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  const int64_t rem = tiles % kWave;
  if (tiles <= kWave || rem == 0 || rem % tiles_m != 0 || 2 * rem > kWave) return 0;
  return (int)(rem / tiles_m);
}

template <bool OUT_F32, bool DUAL>
hipError_t launch_dma(const Args& a, hipStream_t stream) {
  const int tiles = a.tiles_m * a.tiles_n;
  if (a.splits > 1) {
    hipError_t e = configure_dma<true, DUAL, true>();
    if (e != hipSuccess) return e;
    linear_mx_dma_kernel<true, DUAL, true>
        <<<dim3(tiles * a.splits), dim3(kThreads), kDmaStages * kDmaStageBytes, stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t quads = a.M * ((a.N + 3) / 4);
    const uintptr_t ya = reinterpret_cast<uintptr_t>(a.y);
    const bool vec_y = a.N % 4 == 0 && a.ldy % 4 == 0 && (ya & (OUT_F32 ? 15u : 7u)) == 0;
    reduce_splits_kernel<OUT_F32><<<dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream>>>(
        a.part, a.splits, a.M, a.N, a.y, a.ldy, vec_y);
    return hipGetLastError();
  }
  // A last wave of work-groups that would run at most half full (tiles % 256 <= 128,
  // whole tile columns) is run instead as one wave of 256 x 128 tiles over those columns,
  // after the whole waves: the head and tail are two products over disjoint column
  // ranges of W and Y (the weight's scale words keep the whole payload's pitch).
  const int tail_cols = tail_columns(a.tiles_m, a.tiles_n);
  hipError_t e = configure_dma<OUT_F32, DUAL, false>();
  if (e != hipSuccess) return e;
  if (tail_cols == 0) {
    linear_mx_dma_kernel<OUT_F32, DUAL, false><<<dim3(tiles), dim3(kThreads), kDmaStages * kDmaStageBytes, stream>>>(a);
    return hipGetLastError();
  }
  Args head = a, tail = a;
  const int64_t n1 = (int64_t)(a.tiles_n - tail_cols) * BN;  // first column of the tail
  head.N = n1;
  head.Np = n1;
  head.tiles_n = a.tiles_n - tail_cols;
  linear_mx_dma_kernel<OUT_F32, DUAL, false>
      <<<dim3(head.tiles_m * head.tiles_n), dim3(kThreads), kDmaStages * kDmaStageBytes, stream>>>(head);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  tail.N = a.N - n1;
  tail.Np = a.Np - n1;
  tail.tiles_n = (int)((tail.N + 127) / 128);
  tail.wc = a.wc + (n1 / 32) * (a.Kp / 64) * kFragBytes;  // row tiles n1/32 onwards
  tail.ws = a.ws + n1 * 4;                                // scale word (ks, n1 + r) at ks * wsp + n1 + r
  tail.y = static_cast<uint8_t*>(a.y) + n1 * (OUT_F32 ? 4 : 2);
  tail.y_aligned = a.y_aligned;  // n1 is a multiple of 256 columns
  if ((e = configure_dma<OUT_F32, DUAL, false, 128>()) != hipSuccess) return e;
  linear_mx_dma_kernel<OUT_F32, DUAL, false, 128>
      <<<dim3(tail.tiles_m * tail.tiles_n), dim3(kThreads), kDmaStages * kDmaStageBytes, stream>>>(tail);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Small-M kernel (M <= 32, the decode shape).  The product is a stream of the weight
// payload, so the design goal is bytes in flight, not matrix throughput.  A work-group
// owns NT 32-row weight tiles (32*NT output columns) and its 8 waves split K; each
// wave issues every load of a chunk of CH K-steps straight into registers before its
// first instruction uses one (a tiled fragment is an instruction operand: 1 KiB of
// contiguous codes), so a wave keeps CH*NT*2 KiB of weights in flight.  The activation
// fragments of a K-step are shared by the NT tiles.  Trailing steps of a chunk load
// clamped (valid) addresses and multiply zeroed weights, so the load sequence has no
// branches.  The 8 partial tiles are summed through LDS.
constexpr int kSmallWaves = 8;
constexpr int kSmallThreads = 64 * kSmallWaves;

template <bool OUT_F32, int NT, int CH, bool DUAL>
__global__ __launch_bounds__(kSmallThreads, 1) void linear_mx_small_kernel(Args a) {
  // partial tiles, [wave][tile][group g][lane]: lane's accumulators 4g..4g+3 as one float4
  __shared__ f32x4 part[kSmallWaves][NT][4][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t tn0 = (int64_t)blockIdx.x * NT;
  const int nk = (int)(a.Kp / 128);
  const int64_t kc_per_rt = a.Kp / 64;
  const int k0 = (int)((int64_t)nk * wave / kSmallWaves);
  const int k1 = (int)((int64_t)nk * (wave + 1) / kSmallWaves);

  const uint8_t* wsrc[NT];
  const uint32_t* wssrc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // a tile past the last one (odd tile count) re-reads the last tile; its result is
    // not stored
    const int64_t tn = tn0 + t < a.Np / 32 ? tn0 + t : a.Np / 32 - 1;
    wsrc[t] = a.wc + tn * kc_per_rt * kFragBytes + lane * 16;
    wssrc[t] = reinterpret_cast<const uint32_t*>(a.ws) + tn * 32 + r32;
  }
  const bool arow = r32 < a.M;
  const uint8_t* bsrc = a.bc + lane * 16;  // activation row tile 0
  const uint8_t* rsrc = a.rc + lane * 16;
  const uint32_t* bssrc = reinterpret_cast<const uint32_t*>(a.bs) + r32;
  const uint32_t* rssrc = reinterpret_cast<const uint32_t*>(a.rs) + r32;

  v16f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v16f{};
  for (int c = k0; c < k1; c += CH) {
    v4i wf[CH][NT][2], bf[CH][2], rf[CH][2];
    uint32_t wsw[CH][NT], bsw[CH], rsw[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t ks = c + j < k1 ? c + j : k1 - 1;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          wf[j][t][sub] = *reinterpret_cast<const v4i*>(wsrc[t] + (2 * ks + sub) * kFragBytes);
        // activation rows past M are zero padding in the payload: those lanes load nothing
        if constexpr (DUAL) bf[j][sub] = arow ? *reinterpret_cast<const v4i*>(bsrc + (2 * ks + sub) * kFragBytes) : v4i{};
        rf[j][sub] = arow ? *reinterpret_cast<const v4i*>(rsrc + (2 * ks + sub) * kFragBytes) : v4i{};
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) wsw[j][t] = wssrc[t][ks * a.Np];
      if constexpr (DUAL) bsw[j] = bssrc[ks * a.Mp];
      rsw[j] = rssrc[ks * a.Mp];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the chunk ahead of the math
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool live = c + j < k1;
      const int bs = DUAL ? (int)(bsw[j] >> (8 * h)) : 0, rs = (int)(rsw[j] >> (8 * h));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int ws = (int)(wsw[j][t] >> (8 * h));
        const v4i w0 = live ? wf[j][t][0] : v4i{0, 0, 0, 0};
        const v4i w1 = live ? wf[j][t][1] : v4i{0, 0, 0, 0};
        if constexpr (DUAL)
          acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(w0), widen(bf[j][0]), acc[t], 4, 4, 0, ws, 0, bs);
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(w0), widen(rf[j][0]), acc[t], 4, 4, 0, ws, 0, rs);
        if constexpr (DUAL)
          acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(w1), widen(bf[j][1]), acc[t], 4, 4, 2, ws, 2, bs);
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(w1), widen(rf[j][1]), acc[t], 4, 4, 2, ws, 2, rs);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      part[wave][t][g][lane] = f32x4{acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2], acc[t][4 * g + 3]};
  __syncthreads();
  // reduction over the 8 waves: one float4 (4 consecutive outputs of one row) per thread
  // and pass, consecutive threads on consecutive 16-byte LDS words (no bank conflicts).
  // Accumulator element 4g+i of lane (r32, h) is output row r32, column 8g + 4h + i.
  for (int q = tid; q < NT * 4 * 64; q += kSmallThreads) {
    const int t = q >> 8, g = (q >> 6) & 3, l = q & 63;
    const int row = l & 31;
    const int64_t col = (tn0 + t) * 32 + 8 * g + 4 * (l >> 5);
    if (row >= a.M || col >= a.N) continue;
    f32x4 v = part[0][t][g][l];
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w) v += part[w][t][g][l];
    if constexpr (OUT_F32) {
      float* yp = reinterpret_cast<float*>(a.y) + row * a.ldy + col;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (col + i < a.N) yp[i] = v[i];
    } else {
      uint16_t* yp = reinterpret_cast<uint16_t*>(a.y) + row * a.ldy + col;
      if (a.y_aligned && col + 4 <= a.N) {  // 16-byte aligned Y, ldy % 8 == 0, col % 4 == 0: an 8-byte store
        const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(yp) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (col + i < a.N) yp[i] = f32_to_bf16_rne(v[i]);
      }
    }
  }
}

template <bool OUT_F32, bool DUAL>
hipError_t launch_small(const Args& a, hipStream_t stream) {
  constexpr int NT = 2, CH = 4;
  const int64_t tiles = a.Np / 32;
  linear_mx_small_kernel<OUT_F32, NT, CH, DUAL>
      <<<dim3((unsigned)((tiles + NT - 1) / NT)), dim3(kSmallThreads), 0, stream>>>(a);
  return hipGetLastError();
}

template <bool OUT_F32, bool K_ALIGNED, bool DUAL>
hipError_t launch(const Args& a, hipStream_t stream) {
  // The dynamic-LDS limit is a per-device function attribute; setting it twice is harmless.
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_mx_kernel<OUT_F32, K_ALIGNED, DUAL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStageBytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  const int grid = a.tiles_m * a.tiles_n;
  linear_mx_kernel<OUT_F32, K_ALIGNED, DUAL><<<dim3(grid), dim3(kThreads), 2 * kStageBytes, stream>>>(a);
  return hipGetLastError();
}

template <bool DUAL>
hipError_t dispatch(const Args& a, bool tiled, bool out_fp32, hipStream_t stream) {
  if (tiled) {  // all payloads are tiled (checked by the caller)
    if (a.M <= 32) return out_fp32 ? launch_small<true, DUAL>(a, stream) : launch_small<false, DUAL>(a, stream);
    return out_fp32 ? launch_dma<true, DUAL>(a, stream) : launch_dma<false, DUAL>(a, stream);
  }
  if (a.K % 128 == 0)
    return out_fp32 ? launch<true, true, DUAL>(a, stream) : launch<false, true, DUAL>(a, stream);
  return out_fp32 ? launch<true, false, DUAL>(a, stream) : launch<false, false, DUAL>(a, stream);
}

// K split of the tiled GEMM: a shape with fewer 256x256 output tiles than the part has
// compute units splits each tile's K-steps over up to kMaxSplits work-groups, as many as
// fill the compute units, each keeping at least kMinSplitSteps K-steps (128 elements each).
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kMinSplitSteps = 16;
constexpr int64_t kMaxSplits = 4;

int mx_splits(int64_t M, int64_t N, int64_t K) {
  if (M <= 32) return 1;  // the small-M kernel
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int64_t s = kComputeUnits / tiles;
  s = s < round_up(K, 128) / 128 / kMinSplitSteps ? s : round_up(K, 128) / 128 / kMinSplitSteps;
  s = s < kMaxSplits ? s : kMaxSplits;
  return s >= 2 ? (int)s : 1;
}

}  // namespace

size_t linear_mx_workspace(int64_t, int64_t, int64_t) { return 0; }

size_t linear_mx_split_workspace(int64_t M, int64_t N, int64_t K) {
  const int s = mx_splits(M, N, K);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_linear_mx(const sharq_fp4* b, const sharq_fp4& r, int64_t M, const sharq_fp4& w,
                            int64_t N, int64_t K, void* y, int64_t ldy, int out_fp32, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const bool tiled = r.layout == SHARQ_LAYOUT_TILED;
  // the K split runs only when the workspace holds its partial sums
  int splits = tiled ? mx_splits(M, N, K) : 1;
  if (splits > 1 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u) ||
                     workspace_bytes < linear_mx_split_workspace(M, N, K)))
    splits = 1;
  Args a{b ? b->codes : nullptr, b ? b->scales : nullptr, r.codes, r.scales, w.codes, w.scales, y, M, N, K, ldy,
         (int)((M + BM - 1) / BM), (int)((N + BN - 1) / BN), round_up(M, 32), round_up(N, 32), round_up(K, 128),
         (reinterpret_cast<uintptr_t>(y) & 15u) == 0 && ldy % 8 == 0, splits,
         splits > 1 ? reinterpret_cast<float*>(workspace) : nullptr, round_up(N, 32)};
  return b ? dispatch<true>(a, tiled, out_fp32, stream) : dispatch<false>(a, tiled, out_fp32, stream);
}

}  // namespace sharq
