// clock.hip -- shader-clock probe for the measurement: the MFMA peak a kernel can
// reach is set by the clock the part holds under matrix load, which sits below the
// 2.4 GHz of the published peak.
//
// Every work-group (one per CU) runs four independent chains of scaled FP4 matrix
// instructions from registers for `iters` iterations per wave; wave 0 of work-group 0
// reads the shader-clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime) around its loop, so cycles / (ticks / 100 MHz) is the clock it ran at.
#include "sharq_internal.h"

namespace sharq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void clock_probe_kernel(int64_t iters, uint64_t* out) {
  const int lane = threadIdx.x & 63;
  const v8i a = {lane, 1, 2, 3, 4, 5, 6, 7};
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t s0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c0, 4, 4, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c1, 4, 4, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 4, 4, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c3, 4, 4, 0, 127, 0, 127);
  }
  const uint64_t s1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  const v16f s = c0 + c1 + c2 + c3;
  // the sum is never zero-tested by the host; writing it keeps the chains alive
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = s1 - s0;
    out[1] = r1 - r0;
    out[2] = (uint64_t)__float_as_uint(s[0]);
  }
}

}  // namespace

hipError_t launch_clock_probe(int64_t iters, uint64_t* out, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  clock_probe_kernel<<<dim3((unsigned)(cus > 0 ? cus : 1)), dim3(256), 0, stream>>>(iters, out);
  return hipGetLastError();
}

}  // namespace sharq
