// dequant.hip -- the values an FP4 payload encodes, as fp32 (for checking
// reconstructions X ~ Bhat + Rhat; not on the linear layer's path).
//
// One thread per 8 consecutive elements (4 code bytes): it finds its code dword and
// block scale in the payload's layout, converts with the gfx950 scaled conversion
// (E2M1 -> fp32 times 2^E for MXFP4), or for NVFP4 multiplies the E2M1 value by the
// E4M3 block scale (exact, <= 6 significant bits) and then by the tensor scale (one
// rounding), and writes 8 fp32.
#include "sharq_internal.h"

namespace sharq {
namespace {

__device__ __forceinline__ float e4m3_value(uint32_t s) {
  const uint32_t ef = (s >> 3) & 15u, m = s & 7u;
  const float normal = __uint_as_float(((ef + 120u) << 23) | (m << 20));
  const float subnormal = (float)m * 0.001953125f;  // m * 2^-9
  return ef == 0 ? subnormal : normal;
}

template <int FMT, bool TILED>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ tscale, int64_t rows, int64_t K,
                                                      float* __restrict__ out, int64_t ldo) {
  const int64_t chunks_per_row = K / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= rows * chunks_per_row) return;
  const int64_t r = c / chunks_per_row, k0 = (c - r * chunks_per_row) * 8;
  uint32_t code_dword, sbyte;
  if constexpr (TILED) {
    const int64_t Rp = (rows + 31) / 32 * 32, Kp = (K + 127) / 128 * 128;
    const int64_t b = k0 / 32, kc = b >> 1, cc = b & 1;
    const int64_t frag = ((r >> 5) * (Kp / 64) + kc) * 1024;
    code_dword = *reinterpret_cast<const uint32_t*>(codes + frag + ((r & 31) + 32 * cc) * 16 + (k0 & 31) / 2);
    sbyte = scales[((b >> 2) * Rp + r) * 4 + (b & 3)];
  } else {
    code_dword = *reinterpret_cast<const uint32_t*>(codes + r * (K / 2) + k0 / 2);
    sbyte = scales[r * (K / (FMT == SHARQ_MXFP4 ? 32 : 16)) + k0 / (FMT == SHARQ_MXFP4 ? 32 : 16)];
  }
  // the conversion's byte selector must be an immediate: four explicit calls
  const float scale = FMT == SHARQ_MXFP4 ? __uint_as_float(sbyte << 23) : 1.0f;  // 2^(byte-127); 0 = 2^-127
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code_dword, scale, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code_dword, scale, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code_dword, scale, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code_dword, scale, 3);
  float v[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  if constexpr (FMT == SHARQ_NVFP4) {
    const float s = e4m3_value(sbyte), S = *tscale;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __fmul_rn(__fmul_rn(v[i], s), S);
  }
  float* dst = out + r * ldo + k0;
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = v[i];
}

}  // namespace

hipError_t launch_dequantize(const sharq_fp4& p, int64_t rows, int64_t K, int fmt, float* out, int64_t ldo,
                             hipStream_t stream) {
  const int64_t n = rows * (K / 8);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (fmt == SHARQ_MXFP4) {
    if (p.layout == SHARQ_LAYOUT_TILED)
      dequant_kernel<SHARQ_MXFP4, true><<<grid, block, 0, stream>>>(p.codes, p.scales, nullptr, rows, K, out, ldo);
    else
      dequant_kernel<SHARQ_MXFP4, false><<<grid, block, 0, stream>>>(p.codes, p.scales, nullptr, rows, K, out, ldo);
  } else {
    dequant_kernel<SHARQ_NVFP4, false><<<grid, block, 0, stream>>>(p.codes, p.scales, p.tensor_scale, rows, K, out,
                                                                  ldo);
  }
  return hipGetLastError();
}

}  // namespace sharq
