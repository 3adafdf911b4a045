// rmsnorm.hip -- per-row factors of the RMS normalization that sharq_prep_rmsnorm
// folds into the preparation (SharQ, arXiv 2606.26587: "Core claim" and abstract --
// the fused preparation also takes over the layer normalization):
//   r_i = fp32( 1 / sqrt( S_i / K + eps ) ),
// S_i the row's sum of squares in fp64 in a fixed order: each square exact, each run of
// 8 consecutive elements summed in index order, the run sums added in a balanced
// binary tree over the run index (zero-padded to a power of two).  One wave per row:
// lane l holds run 64j + l of block j, so a 6-level xor butterfly gives every lane the
// tree over the block's 64 runs, and a binary counter over the blocks (an aligned
// block of 2^l blocks is merged as soon as it is complete, the rest combined from the
// smallest piece up) finishes the same tree -- bit-identical to any other aligned
// evaluation of it.  Used by the row-major layouts and NVFP4; the tiled MXFP4 path
// folds the sum into its one-read preparation kernel instead.
#include "sharq_internal.h"

namespace sharq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

constexpr int kLevels = 24;  // blocks of 64 runs per row below 2^24 (K < 2^33)

__global__ __launch_bounds__(kThreads) void row_rms_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                           int64_t ldx, double eps, float* __restrict__ r_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= M) return;  // whole waves only
  const uint16_t* xr = x + row * ldx;
  const int64_t nruns = (K + 7) / 8;  // K is a multiple of 16 here: whole runs
  double acc[kLevels];
  uint32_t occ = 0;
  // ordinary (temporal) loads: the preparation re-reads X right after, ideally from
  // the Infinity Cache; four 16-byte loads in flight per lane
  constexpr int kUnroll = 4;
  for (int64_t j0 = 0; j0 * 64 < nruns; j0 += kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = (j0 + u) * 64 + lane;
      v[u] = c < nruns ? *reinterpret_cast<const u32x4*>(xr + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if ((j0 + u) * 64 >= nruns) break;  // uniform
      // the run's squares in index order (each exact)
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = (double)__uint_as_float(v[u][i] << 16), b = (double)__uint_as_float(v[u][i] & 0xFFFF0000u);
        s = __dadd_rn(s, __dmul_rn(a, a));
        s = __dadd_rn(s, __dmul_rn(b, b));
      }
      // the tree over the block's 64 runs (fp64 addition is commutative: every lane
      // gets the same value)
#pragma unroll
      for (int off = 1; off <= 32; off <<= 1) s = __dadd_rn(s, __shfl_xor(s, off, 64));
      // binary counter over the blocks: merge with completed aligned pieces
      bool placed = false;
#pragma unroll
      for (int l = 0; l < kLevels; ++l) {
        if (!placed) {
          if (occ & (1u << l)) {
            s = __dadd_rn(acc[l], s);
            occ &= ~(1u << l);
          } else {
            acc[l] = s;
            occ |= 1u << l;
            placed = true;
          }
        }
      }
    }
  }
  // the padded tree's top: the remaining pieces from the smallest up
  double t = 0.0;
  bool have = false;
#pragma unroll
  for (int l = 0; l < kLevels; ++l)
    if (occ & (1u << l)) {
      t = have ? __dadd_rn(acc[l], t) : acc[l];
      have = true;
    }
  if (lane == 0) r_out[row] = (float)(1.0 / sqrt(t / (double)K + eps));
}

}  // namespace

hipError_t launch_row_rms(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float eps, float* r_out,
                          hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t grid = (M + kThreads / 64 - 1) / (kThreads / 64);
  row_rms_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(x, M, K, ldx, (double)eps, r_out);
  return hipGetLastError();
}

}  // namespace sharq
