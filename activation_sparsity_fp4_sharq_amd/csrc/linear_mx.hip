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
         (int)((M + BM - 1) / BM), (int)((N + BN - 1) / BN)};
  const bool k_aligned = K % 128 == 0;
  if (out_fp32) return k_aligned ? launch<true, true>(a, stream) : launch<true, false>(a, stream);
  return k_aligned ? launch<false, true>(a, stream) : launch<false, false>(a, stream);
}

}  // namespace sharq
