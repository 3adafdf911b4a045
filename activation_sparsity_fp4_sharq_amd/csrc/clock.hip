// clock.hip -- measurement probes (none is on the SharQ path): the shader clock under
// matrix load (the MFMA peak a kernel can reach is set by the clock the part holds,
// which sits below the 2.4 GHz of the published peak), the rate of the two matrix
// instruction forms a sparse backbone can use, and the streaming ceiling of a plain
// read + write of the preparation's byte counts.
//
// Every work-group (one per CU) runs four independent chains of scaled FP4 matrix
// instructions from registers for `iters` iterations per wave; wave 0 of work-group 0
// reads the shader-clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime) around its loop, so cycles / (ticks / 100 MHz) is the clock it ran at.
#include "fp4_codec.h"
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

// Matrix-instruction rate of the two forms a sparse FP4 backbone can take on gfx950:
// form 0 the dense block-scaled FP4 32x32x64 instruction (a zero-filled backbone),
// form 1 the 2:4-sparse fp8 32x32x64 instruction (a compressed backbone; FP4 values
// are exact in fp8).  Both do 32 x 32 x 64 multiply-adds of the dense operand shape
// per instruction.  Every CU runs 4 waves, one per SIMD, each issuing eight
// independent accumulator chains from registers (enough to cover the instruction's
// latency), so the timed wave's loop is its SIMD's whole instruction stream.
typedef int v4i __attribute__((ext_vector_type(4)));

template <int FORM>
__device__ __forceinline__ v16f mfma_form(const v8i& a, const v4i& as, int idx, const v16f& c) {
  if constexpr (FORM == 0)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c, 4, 4, 0, 127, 0, 127);
  else
    return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(as, a, c, idx, 0, 0);
}

template <int FORM>
__global__ __launch_bounds__(256) void matrix_rate_kernel(int64_t iters, uint64_t* out) {
  const int lane = threadIdx.x & 63;
  const v8i a = {lane, 1, 2, 3, 4, 5, 6, 7};
  const v4i as = {lane, 1, 2, 3};
  const int idx = 0x44444444 ^ lane;  // sparsity index operand (any 2-of-4 selector)
  v16f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = v16f{};
  const uint64_t s0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = mfma_form<FORM>(a, as, idx, c[j]);
  }
  const uint64_t s1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  v16f s = c[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) s += c[j];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = s1 - s0;
    out[1] = r1 - r0;
    out[2] = (uint64_t)__float_as_uint(s[0]);
  }
}

// Streaming probe: a plain read of `nr` and write of `nw` 16-byte chunks with the
// preparation's access shape (each lane loads 4 chunks non-temporally, then stores
// 4), no arithmetic beyond an xor that keeps the loads alive -- the memory pattern's
// own ceiling at a given size.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamPerLane = 4;

__global__ __launch_bounds__(kStreamThreads) void stream_probe_kernel(const u32x4* __restrict__ src, int64_t nr,
                                                                      u32x4* __restrict__ dst, int64_t nw) {
  const int64_t base = (int64_t)blockIdx.x * kStreamThreads * kStreamPerLane + threadIdx.x;
  u32x4 v[kStreamPerLane];
#pragma unroll
  for (int u = 0; u < kStreamPerLane; ++u) {
    const int64_t c = base + u * kStreamThreads;
    v[u] = c < nr ? __builtin_nontemporal_load(src + c) : u32x4{(uint32_t)c, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kStreamPerLane; ++u) {
    const int64_t c = base + u * kStreamThreads;
    if (c < nw) dst[c] = v[u] ^ (uint32_t)c;
  }
}

// Rounding check of bf16x2_rne_hw against bf16_rne_bits over every fp32 pattern: lane
// i of the grid-stride loop converts the pair (2i, 2i+1); patterns with an all-ones
// exponent (infinities, NaN) are skipped.  out[0] += mismatches, out[1] = min pattern.
constexpr int kRoundThreads = 256;
constexpr int kRoundBlocks = 4096;

__global__ void rounding_init_kernel(unsigned long long* out) {
  out[0] = 0ull;
  out[1] = ~0ull;
}

__global__ __launch_bounds__(kRoundThreads) void rounding_probe_kernel(unsigned long long* out) {
  constexpr uint64_t kPairs = 1ull << 31;
  unsigned long long bad = 0, first = ~0ull;
  for (uint64_t i = (uint64_t)blockIdx.x * kRoundThreads + threadIdx.x; i < kPairs;
       i += (uint64_t)kRoundBlocks * kRoundThreads) {
    const uint32_t a = (uint32_t)(2 * i), b = a + 1u;
    const uint32_t hw = codec::bf16x2_rne_hw(__uint_as_float(a), __uint_as_float(b));
    const bool fa = (a & 0x7F800000u) != 0x7F800000u, fb = (b & 0x7F800000u) != 0x7F800000u;
    if (fa && (hw & 0xFFFFu) != codec::bf16_rne_bits(__uint_as_float(a))) {
      ++bad;
      first = first < a ? first : a;
    }
    if (fb && (hw >> 16) != codec::bf16_rne_bits(__uint_as_float(b))) {
      ++bad;
      first = first < b ? first : b;
    }
  }
  if (bad) {
    atomicAdd(&out[0], bad);
    atomicMin(&out[1], first);
  }
}

// Conversion check of e4m3_encode_hw against e4m3_encode_def over every fp32 pattern
// with the sign bit clear (the block-scale operand is a non-negative quotient; +inf and
// NaN included), and of e4m3_value_hw against e4m3_value_def on the codes 0..0x7E (the
// first 127 threads of work-group 0).  out[0] += mismatches, out[1] = min of the
// mismatching fp32 pattern, or 2^32 + code for a decode mismatch.
__global__ __launch_bounds__(kRoundThreads) void e4m3_probe_kernel(unsigned long long* out) {
  constexpr uint64_t kPatterns = 1ull << 31;
  unsigned long long bad = 0, first = ~0ull;
  for (uint64_t i = (uint64_t)blockIdx.x * kRoundThreads + threadIdx.x; i < kPatterns;
       i += (uint64_t)kRoundBlocks * kRoundThreads) {
    const float q = __uint_as_float((uint32_t)i);
    if (codec::e4m3_encode_hw(q) != codec::e4m3_encode_def(q)) {
      ++bad;
      first = first < i ? first : i;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x <= 0x7Eu) {
    const uint32_t s = threadIdx.x;
    if (__float_as_uint(codec::e4m3_value_hw(s)) != __float_as_uint(codec::e4m3_value_def(s))) {
      ++bad;
      const unsigned long long tag = (1ull << 32) | s;
      first = first < tag ? first : tag;
    }
  }
  if (bad) {
    atomicAdd(&out[0], bad);
    atomicMin(&out[1], first);
  }
}

}  // namespace

hipError_t launch_e4m3_probe(uint64_t* out, hipStream_t stream) {
  unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
  rounding_init_kernel<<<dim3(1), dim3(1), 0, stream>>>(o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e4m3_probe_kernel<<<dim3(kRoundBlocks), dim3(kRoundThreads), 0, stream>>>(o);
  return hipGetLastError();
}

hipError_t launch_rounding_probe(uint64_t* out, hipStream_t stream) {
  unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
  rounding_init_kernel<<<dim3(1), dim3(1), 0, stream>>>(o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  rounding_probe_kernel<<<dim3(kRoundBlocks), dim3(kRoundThreads), 0, stream>>>(o);
  return hipGetLastError();
}

hipError_t launch_matrix_rate_probe(int form, int64_t iters, uint64_t* out, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const dim3 grid((unsigned)(cus > 0 ? cus : 1));
  if (form == 0)
    matrix_rate_kernel<0><<<grid, dim3(256), 0, stream>>>(iters, out);
  else
    matrix_rate_kernel<1><<<grid, dim3(256), 0, stream>>>(iters, out);
  return hipGetLastError();
}

hipError_t launch_stream_probe(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                               hipStream_t stream) {
  const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
  const int64_t n = nr > nw ? nr : nw;
  if (n == 0) return hipSuccess;
  const int64_t per = (int64_t)kStreamThreads * kStreamPerLane;
  stream_probe_kernel<<<dim3((unsigned)((n + per - 1) / per)), dim3(kStreamThreads), 0, stream>>>(
      reinterpret_cast<const u32x4*>(src), nr, reinterpret_cast<u32x4*>(dst), nw);
  return hipGetLastError();
}

hipError_t launch_clock_probe(int64_t iters, uint64_t* out, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  clock_probe_kernel<<<dim3((unsigned)(cus > 0 ? cus : 1)), dim3(256), 0, stream>>>(iters, out);
  return hipGetLastError();
}

}  // namespace sharq
