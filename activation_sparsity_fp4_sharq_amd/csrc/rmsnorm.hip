// rmsnorm.hip -- per-row factors of the RMS normalization that sharq_prep_rmsnorm
// folds into the preparation (SharQ, arXiv 2606.26587: "Core claim" and abstract --
// the fused preparation also takes over the layer normalization):
//   r_i = fp32( 1 / sqrt( (sum_k x_ik^2) / K + eps ) )
// The squares of bf16 values are exact in fp64 and so is their sum to ~K * 2^-53, so
// the fp64 result depends on the summation order only in its last bits, and the
// rounding to fp32 is the same as an exact evaluation's except on a measure-zero set
// of inputs.  One wave per row; X is read once (and, at LLM sizes, stays resident in
// the 256 MB Infinity Cache for the preparation that follows).
#include "sharq_internal.h"

namespace sharq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void row_rms_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                           int64_t ldx, double eps, float* __restrict__ r_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= M) return;  // whole waves only
  const uint16_t* xr = x + row * ldx;
  double ss = 0.0;
  // ordinary (temporal) loads: the preparation re-reads X right after, ideally from
  // the Infinity Cache; four 16-byte loads in flight per lane
  constexpr int kUnroll = 4;
  for (int64_t k0 = (int64_t)lane * 8; k0 < K; k0 += 64 * 8 * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t k = k0 + (int64_t)u * 64 * 8;
      v[u] = k < K ? *reinterpret_cast<const u32x4*>(xr + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = (double)__uint_as_float(v[u][i] << 16), b = (double)__uint_as_float(v[u][i] & 0xFFFF0000u);
        ss = __fma_rn(a, a, ss);
        ss = __fma_rn(b, b, ss);
      }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) r_out[row] = (float)(1.0 / sqrt(ss / (double)K + eps));
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
