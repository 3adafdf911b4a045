// layout_mx.hip -- MXFP4 payload re-layout between the row-major layout and the tiled
// layout the fused GEMM loads (both defined in sharq.h).  One thread moves one
// 32-element block of one row: its 16 code bytes and its scale byte.  Used once per
// weight payload that arrives row-major, and by tests; never on the hot path.
#include "sharq_internal.h"

namespace sharq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t tiled_code_offset(int64_t r, int64_t b, int64_t Kp) {
  return ((r >> 5) * (Kp / 64) + (b >> 1)) * 1024 + ((r & 31) + 32 * (b & 1)) * 16;
}

__device__ __forceinline__ int64_t tiled_scale_offset(int64_t r, int64_t b, int64_t Rp) {
  return ((b >> 2) * Rp + r) * 4 + (b & 3);
}

// SRC_TILED / DST_TILED select the layouts.  Units cover the destination's rows and
// blocks (padded extents for a tiled destination); a unit outside the source's real
// extent writes zeros.
template <bool SRC_TILED, bool DST_TILED>
__global__ __launch_bounds__(256) void convert_kernel(const uint8_t* __restrict__ sc, const uint8_t* __restrict__ ss,
                                                      uint8_t* __restrict__ dc, uint8_t* __restrict__ ds,
                                                      int64_t rows, int64_t K, int64_t Rp, int64_t Kp) {
  const int64_t nb_dst = (DST_TILED ? Kp : K) / 32;
  const int64_t rows_dst = DST_TILED ? Rp : rows;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= rows_dst * nb_dst) return;
  const int64_t r = u / nb_dst, b = u - r * nb_dst;
  const int64_t nbk = K / 32;
  u32x4 codes = u32x4{0u, 0u, 0u, 0u};
  uint8_t scale = 0;
  if (r < rows && b < nbk) {
    const int64_t co = SRC_TILED ? tiled_code_offset(r, b, Kp) : r * (K / 2) + b * 16;
    const int64_t so = SRC_TILED ? tiled_scale_offset(r, b, Rp) : r * nbk + b;
    codes = *reinterpret_cast<const u32x4*>(sc + co);
    scale = ss[so];
  }
  const int64_t co = DST_TILED ? tiled_code_offset(r, b, Kp) : r * (K / 2) + b * 16;
  const int64_t so = DST_TILED ? tiled_scale_offset(r, b, Rp) : r * nbk + b;
  *reinterpret_cast<u32x4*>(dc + co) = codes;
  ds[so] = scale;
}

template <bool S, bool D>
hipError_t run(const sharq_fp4& src, const sharq_fp4& dst, int64_t rows, int64_t K, hipStream_t stream) {
  const int64_t Rp = round_up(rows, 32), Kp = round_up(K, 128);
  const int64_t units = (D ? Rp : rows) * ((D ? Kp : K) / 32);
  if (units == 0) return hipSuccess;
  convert_kernel<S, D><<<dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream>>>(
      src.codes, src.scales, dst.codes, dst.scales, rows, K, Rp, Kp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_convert_mx(const sharq_fp4& src, const sharq_fp4& dst, int64_t rows, int64_t K,
                             hipStream_t stream) {
  const bool s = src.layout == SHARQ_LAYOUT_TILED, d = dst.layout == SHARQ_LAYOUT_TILED;
  if (s && d) return run<true, true>(src, dst, rows, K, stream);
  if (s) return run<true, false>(src, dst, rows, K, stream);
  if (d) return run<false, true>(src, dst, rows, K, stream);
  return run<false, false>(src, dst, rows, K, stream);
}

}  // namespace sharq
