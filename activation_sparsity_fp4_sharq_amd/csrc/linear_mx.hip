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
// Tiling: 512 threads (8 waves, 2 per SIMD) own a 256x256 output tile; waves form a
// 4 (M) x 2 (N) grid of 64x128 wave tiles = 2x4 instructions per path and sub-step.
// Per 128-element K-step the block stages A_b, A_r, W tiles (256 rows x 64 B each,
// rows padded to 80 B so that 16-byte LDS reads of 32 consecutive rows hit
// distinct banks) and their scale dwords, double-buffered; one barrier per K-step.
// Work-groups are renumbered so that consecutive tiles share an XCD (and its L2).
#include <atomic>

#include "sharq_internal.h"

namespace sharq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
};

__device__ __forceinline__ v8i widen(v4i a) {
  return __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Map the hardware work-group id to a tile so that the ids one XCD receives
// (id % 8 == x) form a contiguous run of tiles, walked in groups of 4 tile-rows.
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

template <bool OUT_F32, bool K_ALIGNED>
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
      sstage[0] = grow < a.M ? load_scale_dword<K_ALIGNED>(s, grow, nbk, kstep) : 0u;
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
    for (int p = 0; p < 2; ++p)
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
    for (int p = 0; p < 2; ++p)
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
// Pipelined kernel for K % 128 == 0 (every shape the benchmarks use).
//
// Same tiling and instruction as above, but the operands travel global -> LDS by the
// gfx950 LDS-DMA loads (global_load_lds_dwordx4 / _dword) instead of through
// registers, into a 3-deep ring of stages, so the loads for K-step i+2 are in flight
// while K-step i computes.  Each operand tile is stored in LDS in *fragment order*:
// 16 fragments of 1 KiB (8 row-tiles of 32 rows x 2 sub-steps), fragment byte
// 16*lane holding exactly the 16 bytes lane `lane` feeds the instruction.  A DMA
// load writes 64 lanes x 16 B contiguously, so one load fills one fragment (each
// lane fetches the global bytes its slot needs), and one ds_read_b128 at
// 16*lane reads it back with no bank conflicts.  Sub-step s, lane half h takes the
// 16-byte chunk 2s+h of the row's 64-byte K-step, so a load reads 32 contiguous
// bytes per row; the scale byte of chunk 2s+h is byte 2s of (row scale word >> 8h),
// op_sel 0 or 2.  Rows past M (or N) are clamped to the last row: they are loaded
// and computed but never stored.
constexpr int kFragBytes = 1024;
constexpr int kOpTileBytes = 16 * kFragBytes;                   // 256 rows x 128 K
constexpr int kDmaStageBytes = 3 * kOpTileBytes + 3 * 256 * 4;  // + scale words
constexpr int kDmaStages = 3;

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector-memory counter constrained (expcnt/lgkmcnt left free).
#define SHARQ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void linear_mx_dma_kernel(Args a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int nk = (int)(a.Kp / 128);

  // Each wave fills 6 of the 48 fragments of a stage (A_b, A_r, W x 16): one
  // contiguous 1 KiB fragment of the tiled payload per load.  Row tiles past the
  // padded extent are clamped to the last one (computed, never stored).
  const uint8_t* fsrc[6];
  int fdst[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int f = wave * 6 + j;
    const int op = f >> 4, fi = f & 15, rt = fi >> 1, sub = fi & 1;
    const uint8_t* base = op == 0 ? a.bc : op == 1 ? a.rc : a.wc;
    const int64_t ntiles = (op == 2 ? a.Np : a.Mp) / 32;
    int64_t t = (op == 2 ? n0 : m0) / 32 + rt;
    t = t < ntiles ? t : ntiles - 1;
    fsrc[j] = base + (t * (a.Kp / 64) + sub) * kFragBytes + lane * 16;
    fdst[j] = op * kOpTileBytes + fi * kFragBytes;
  }
  // Scale words: one operand's 256 words per K-step are 1 KiB contiguous -> waves 0..2
  // load one operand each.
  const bool scale_wave = wave < 3;
  const uint8_t* ssrc;
  int64_t sstep;
  {
    const int op = scale_wave ? wave : 0;
    const uint8_t* base = op == 0 ? a.bs : op == 1 ? a.rs : a.ws;
    const int64_t rp = op == 2 ? a.Np : a.Mp;
    int64_t row = (op == 2 ? n0 : m0) + 4 * lane;
    row = row < rp - 4 ? row : rp - 4;
    ssrc = base + row * 4;
    sstep = rp * 4;
  }
  const int sdst = 3 * kOpTileBytes + (scale_wave ? wave : 0) * 1024;

  auto issue = [&](int ks, int stage) {
    uint8_t* st = smem + stage * kDmaStageBytes;
#pragma unroll
    for (int j = 0; j < 6; ++j)
      __builtin_amdgcn_global_load_lds(fsrc[j] + (int64_t)ks * 2 * kFragBytes, (lds_void_t*)(st + fdst[j]), 16, 0, 0);
    if (scale_wave)
      __builtin_amdgcn_global_load_lds(ssrc + (int64_t)ks * sstep, (lds_void_t*)(st + sdst), 16, 0, 0);
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  issue(0, 0);
  if (nk > 1) issue(1, 1);

  for (int ks = 0; ks < nk; ++ks) {
    // this wave's loads for stage ks are done once at most one stage's loads remain
    if (ks + 1 < nk) {
      if (scale_wave) SHARQ_WAIT_VMCNT(7); else SHARQ_WAIT_VMCNT(6);
    } else {
      SHARQ_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();  // every wave's stage-ks data is in LDS; stage ks-1 is free
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (ks + 2 < nk) issue(ks + 2, (ks + 2) % kDmaStages);

    const uint8_t* st = smem + (ks % kDmaStages) * kDmaStageBytes;
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + 3 * kOpTileBytes);
    uint32_t as[2][2], ws[4];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) as[p][mt] = sc[p * 256 + wm * 64 + mt * 32 + r32] >> (8 * h);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) ws[nt] = sc[512 + wn * 128 + nt * 32 + r32] >> (8 * h);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      v4i af[2][2], wf[4];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          af[p][mt] = *reinterpret_cast<const v4i*>(st + p * kOpTileBytes +
                                                    ((wm * 2 + mt) * 2 + sub) * kFragBytes + lane * 16);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        wf[nt] = *reinterpret_cast<const v4i*>(st + 2 * kOpTileBytes + ((wn * 4 + nt) * 2 + sub) * kFragBytes +
                                               lane * 16);
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            if (sub == 0)
              acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  widen(af[p][mt]), widen(wf[nt]), acc[mt][nt], 4, 4, 0, (int)as[p][mt], 0, (int)ws[nt]);
            else
              acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  widen(af[p][mt]), widen(wf[nt]), acc[mt][nt], 4, 4, 2, (int)as[p][mt], 2, (int)ws[nt]);
          }
    }
  }

  store_tile<OUT_F32>(a, acc, m0, n0, wm, wn, r32, h);
}

template <bool OUT_F32>
hipError_t launch_dma(const Args& a, hipStream_t stream) {
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_mx_dma_kernel<OUT_F32>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kDmaStages * kDmaStageBytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  const int grid = a.tiles_m * a.tiles_n;
  linear_mx_dma_kernel<OUT_F32><<<dim3(grid), dim3(kThreads), kDmaStages * kDmaStageBytes, stream>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Software-pipelined kernel: 4 waves (one per SIMD), each owning a 128x128 wave tile
// (4x4 instructions per path and sub-step, 256 fp32 accumulators per lane), so every
// fragment read from LDS feeds 4 (A) or 8 (W, both paths) instructions.  The fragment
// reads of the next sub-step are issued while the current sub-step's 32 instructions
// run, and the next K-step's first fragments are read right after the mid-step
// barrier, so the matrix pipe never waits on LDS latency.  LDS holds a 3-slot ring
// of stages in fragment order (as above); a stage's DMA is issued two K-steps ahead.
//   iteration i:  [A] read sub-step-1 fragments of stage i | 32 MFMA on sub-step 0
//                 [B] wait own DMA of stage i+1; barrier; DMA stage i+3 into slot i%3
//                 [C] read sub-step-0 fragments + scales of stage i+1 | 32 MFMA on sub-step 1
constexpr int kPipeThreads = 256;

struct Frags {
  v4i a[2][4];  // [path][mt]
  v4i w[4];     // [nt]
};

__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* st, int sub, int wm, int wn, int lane) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      f.a[p][mt] = *reinterpret_cast<const v4i*>(st + p * kOpTileBytes + ((wm * 4 + mt) * 2 + sub) * kFragBytes +
                                                 lane * 16);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
    f.w[nt] = *reinterpret_cast<const v4i*>(st + 2 * kOpTileBytes + ((wn * 4 + nt) * 2 + sub) * kFragBytes +
                                            lane * 16);
}

struct Scales {
  uint32_t a[2][4], w[4];
};

__device__ __forceinline__ void read_scales(Scales& sc, const uint8_t* st, int wm, int wn, int r32, int h) {
  const uint32_t* s = reinterpret_cast<const uint32_t*>(st + 3 * kOpTileBytes);
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sc.a[p][mt] = s[p * 256 + wm * 128 + mt * 32 + r32] >> (8 * h);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) sc.w[nt] = s[512 + wn * 128 + nt * 32 + r32] >> (8 * h);
}

template <int SUB>
__device__ __forceinline__ void mma_substep(v16f (&acc)[4][4], const Frags& f, const Scales& sc) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            widen(f.a[p][mt]), widen(f.w[nt]), acc[mt][nt], 4, 4, 2 * SUB, (int)sc.a[p][mt], 2 * SUB,
            (int)sc.w[nt]);
}

template <bool OUT_F32>
__device__ __forceinline__ void store_tile_4x4(const Args& a, const v16f (&acc)[4][4], int64_t m0, int64_t n0,
                                               int wm, int wn, int r32, int h) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t col = n0 + wn * 128 + nt * 32 + r32;
      if (col >= a.N) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t row = m0 + wm * 128 + mt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
        if (row < a.M) {
          if constexpr (OUT_F32)
            reinterpret_cast<float*>(a.y)[row * a.ldy + col] = acc[mt][nt][j];
          else
            reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + col] = f32_to_bf16_rne(acc[mt][nt][j]);
        }
      }
    }
}

template <bool OUT_F32>
__global__ __launch_bounds__(kPipeThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void linear_mx_pipe_kernel(Args a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int nk = (int)(a.Kp / 128);

  // Each wave fills 12 of the 48 fragments of a stage; waves 0..2 also load one
  // operand's 1 KiB of scale words.
  const uint8_t* fsrc[12];
  int fdst[12];
#pragma unroll
  for (int j = 0; j < 12; ++j) {
    const int f = wave * 12 + j;
    const int op = f >> 4, fi = f & 15, rt = fi >> 1, sub = fi & 1;
    const uint8_t* base = op == 0 ? a.bc : op == 1 ? a.rc : a.wc;
    const int64_t ntiles = (op == 2 ? a.Np : a.Mp) / 32;
    int64_t t = (op == 2 ? n0 : m0) / 32 + rt;
    t = t < ntiles ? t : ntiles - 1;
    fsrc[j] = base + (t * (a.Kp / 64) + sub) * kFragBytes + lane * 16;
    fdst[j] = op * kOpTileBytes + fi * kFragBytes;
  }
  const bool scale_wave = wave < 3;
  const uint8_t* ssrc;
  int64_t sstep;
  {
    const int op = scale_wave ? wave : 0;
    const uint8_t* base = op == 0 ? a.bs : op == 1 ? a.rs : a.ws;
    const int64_t rp = op == 2 ? a.Np : a.Mp;
    int64_t row = (op == 2 ? n0 : m0) + 4 * lane;
    row = row < rp - 4 ? row : rp - 4;
    ssrc = base + row * 4;
    sstep = rp * 4;
  }
  const int sdst = 3 * kOpTileBytes + (scale_wave ? wave : 0) * 1024;
  auto issue = [&](int ks) {
    uint8_t* st = smem + (ks % kDmaStages) * kDmaStageBytes;
#pragma unroll
    for (int j = 0; j < 12; ++j)
      __builtin_amdgcn_global_load_lds(fsrc[j] + (int64_t)ks * 2 * kFragBytes, (lds_void_t*)(st + fdst[j]), 16, 0, 0);
    if (scale_wave)
      __builtin_amdgcn_global_load_lds(ssrc + (int64_t)ks * sstep, (lds_void_t*)(st + sdst), 16, 0, 0);
  };
  auto stage_ptr = [&](int ks) { return smem + (ks % kDmaStages) * kDmaStageBytes; };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  // prologue: three stages in flight, wait for the first
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  // a wave issues L = 12 or 13 loads per stage
  if (nk > 2) { if (scale_wave) SHARQ_WAIT_VMCNT(26); else SHARQ_WAIT_VMCNT(24); }
  else if (nk > 1) { if (scale_wave) SHARQ_WAIT_VMCNT(13); else SHARQ_WAIT_VMCNT(12); }
  else SHARQ_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  Frags f0, f1;
  Scales sc, scn;
  read_frags(f0, stage_ptr(0), 0, wm, wn, lane);
  read_scales(sc, stage_ptr(0), wm, wn, r32, h);

  for (int ks = 0; ks < nk; ++ks) {
    const uint8_t* st = stage_ptr(ks);
    // [A]
    read_frags(f1, st, 1, wm, wn, lane);
    mma_substep<0>(acc, f0, sc);
    // [B] stage ks+1 complete for every wave; slot ks%3 free for stage ks+3
    if (ks + 2 < nk) { if (scale_wave) SHARQ_WAIT_VMCNT(13); else SHARQ_WAIT_VMCNT(12); }
    else SHARQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (ks + 3 < nk) issue(ks + 3);
    // [C]
    if (ks + 1 < nk) {
      read_frags(f0, stage_ptr(ks + 1), 0, wm, wn, lane);
      read_scales(scn, stage_ptr(ks + 1), wm, wn, r32, h);
    }
    mma_substep<1>(acc, f1, sc);
    sc = scn;
  }

  store_tile_4x4<OUT_F32>(a, acc, m0, n0, wm, wn, r32, h);
}

template <bool OUT_F32>
hipError_t launch_pipe(const Args& a, hipStream_t stream) {
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_mx_pipe_kernel<OUT_F32>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kDmaStages * kDmaStageBytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  const int grid = a.tiles_m * a.tiles_n;
  linear_mx_pipe_kernel<OUT_F32><<<dim3(grid), dim3(kPipeThreads), kDmaStages * kDmaStageBytes, stream>>>(a);
  return hipGetLastError();
}

template <bool OUT_F32, bool K_ALIGNED>
hipError_t launch(const Args& a, hipStream_t stream) {
  // The dynamic-LDS limit is a per-device function attribute; setting it twice is harmless.
  static std::atomic<bool> configured[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !configured[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_mx_kernel<OUT_F32, K_ALIGNED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStageBytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) configured[dev].store(true, std::memory_order_release);
  }
  const int grid = a.tiles_m * a.tiles_n;
  linear_mx_kernel<OUT_F32, K_ALIGNED><<<dim3(grid), dim3(kThreads), 2 * kStageBytes, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

size_t linear_mx_workspace(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_linear_mx(const sharq_fp4& b, const sharq_fp4& r, int64_t M, const sharq_fp4& w,
                            int64_t N, int64_t K, void* y, int64_t ldy, int out_fp32, void*, size_t,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  Args a{b.codes, b.scales, r.codes, r.scales, w.codes, w.scales, y, M, N, K, ldy,
         (int)((M + BM - 1) / BM), (int)((N + BN - 1) / BN), round_up(M, 32), round_up(N, 32), round_up(K, 128)};
  if (b.layout == SHARQ_LAYOUT_TILED)  // all three are tiled (checked by the caller)
    return out_fp32 ? launch_dma<true>(a, stream) : launch_dma<false>(a, stream);
  const bool k_aligned = K % 128 == 0;
  if (out_fp32) return k_aligned ? launch<true, true>(a, stream) : launch<true, false>(a, stream);
  return k_aligned ? launch<false, true>(a, stream) : launch<false, false>(a, stream);
}

}  // namespace sharq
