// fp4_codec.h -- device helpers shared by the activation preparations (and the
// conversion self-checks): the top-n-of-m selection on a lane's 8 consecutive elements
// (SharQ's input-adaptive N:M mask: keep the n largest magnitudes of every group of m
// consecutive elements along K, lower index first on equal magnitude); bf16 rounding;
// E4M3 coding of NVFP4 block scales; the input transforms folded into the preparation
// (RMS normalization, SwiGLU) and the SiLU table of the SwiGLU form.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace sharq {
namespace codec {

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t umax3(uint32_t a, uint32_t b, uint32_t c) { return umax(umax(a, b), c); }
__device__ __forceinline__ uint32_t umin3(uint32_t a, uint32_t b, uint32_t c) { return umin(umin(a, b), c); }

// Median of three unsigned integers (one v_med3_u32; the compiler does not form it
// from min/max expressions).
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Second largest of four: with m = the median of (a, b, c), the second largest of
// all four is m unless d lies above m, in which case it is min(max(a, b, c), d).
__device__ __forceinline__ uint32_t second_of_4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return umax(umed3(a, b, c), umin(umax3(a, b, c), d));
}

// Descending sort of four (s0 >= s1 >= s2 >= s3) from the max, min and median of
// the first three and the fourth value.
__device__ __forceinline__ void sort4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t s[4]) {
  const uint32_t hi = umax3(a, b, c), lo = umin3(a, b, c), md = umed3(a, b, c);
  s[0] = umax(hi, d);
  s[1] = umax(md, umin(hi, d));
  s[2] = umin(md, umax(lo, d));
  s[3] = umin(lo, d);
}

// Fourth largest of eight: the top four of two descending runs a and b are
// max(a_i, b_{3-i}), so the fourth largest is the smallest of those four.
__device__ __forceinline__ uint32_t fourth_of_8(const uint32_t c[8]) {
  uint32_t a[4], b[4];
  sort4(c[0], c[1], c[2], c[3], a);
  sort4(c[4], c[5], c[6], c[7], b);
  return umin(umin3(umax(a[0], b[3]), umax(a[1], b[2]), umax(a[2], b[1])), umax(a[3], b[0]));
}

// Top-n-of-m selection on the lane's 8 elements.  Each element gets a compound key:
// its magnitude (the fp32 image of a bf16 value has 16 zero low bits) with a
// reversed in-group index in the low bits, so keys are distinct and "larger key"
// means "ranks earlier": bigger magnitude first, lower index first among equal
// magnitudes (+0 and -0 are equal).  An element is kept when its key is at or
// above the n-th largest key of its group.
template <int SPM>
__device__ __forceinline__ void keep_mask(const float xf[8], bool kept[8]) {
  uint32_t ck[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    ck[j] = (__float_as_uint(xf[j]) & 0x7FFF0000u) | (uint32_t)(SPM == 4 ? 3 - (j & 3) : 7 - j);
  if constexpr (SPM == 4) {
    const uint32_t t0 = second_of_4(ck[0], ck[1], ck[2], ck[3]);
    const uint32_t t1 = second_of_4(ck[4], ck[5], ck[6], ck[7]);
#pragma unroll
    for (int j = 0; j < 8; ++j) kept[j] = ck[j] >= (j < 4 ? t0 : t1);
  } else {
    const uint32_t t = fourth_of_8(ck);
#pragma unroll
    for (int j = 0; j < 8; ++j) kept[j] = ck[j] >= t;
  }
}

}  // namespace codec
}  // namespace sharq

namespace sharq {
namespace codec {

// RMS normalization folded into the preparation (SharQ's fused preparation takes over
// the layer normalization): each bf16 element x of row i becomes
// bf16_rne(fp32(fp32(x * r_i) * g_k)), r_i the row's factor, g_k the channel's bf16
// gain.  Applied to a dword of two bf16 values and the matching dword of gains.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite values (the contract)
}

// Two fp32 values to two bf16 (a in the low half) with the gfx950 packed conversion,
// which rounds to nearest even and keeps subnormals under the kernels' fp32 mode.  On
// every finite fp32 pattern it agrees with bf16_rne_bits (sharq_bf16_rounding_probe
// checks all 2^32 patterns on the device).
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne_hw(float a, float b) {
  const f32x2_cvt_t p = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_cvt_t));
}

// OCP E4M3 (the NVFP4 block-scale format: 4 exponent bits, bias 7, 3 mantissa bits, no
// infinities, 0x7F the NaN) of q >= 0 from the format's definition, worked on the fp32
// bits: nearest value, ties to the even code, saturating at 448 (0x7E); +0 and NaN give 0.
__device__ __forceinline__ uint32_t e4m3_encode_def(float q) {
  if (!(q > 0.0f)) return 0;
  if (q >= 448.0f) return 0x7E;
  if (q < 0.015625f) return (uint32_t)__builtin_rintf(q * 512.0f);  // subnormal step 2^-9 (exact scaling)
  const uint32_t u = __float_as_uint(q);
  const uint32_t ef = (u >> 23) - 120;  // E4M3 exponent field: (e - 127) + 7
  uint32_t code = (ef << 3) | ((u >> 20) & 7u);
  const uint32_t rem = u & 0xFFFFFu, half = 0x80000u;
  if (rem > half || (rem == half && (code & 1u))) code += 1;  // a carry moves into the exponent
  return code;
}

// The value of an E4M3 code 0..0x7E from the definition: m * 2^-9 when the exponent
// field is 0, else (1 + m/8) * 2^(e - 7).
__device__ __forceinline__ float e4m3_value_def(uint32_t s) {
  const uint32_t ef = (s >> 3) & 15u, m = s & 7u;
  const float normal = __uint_as_float(((ef + 120u) << 23) | (m << 20));
  const float subnormal = (float)m * 0.001953125f;  // m * 2^-9
  return ef == 0 ? subnormal : normal;
}

// The same two maps through gfx950's fp8 conversions (OCP E4M3, nearest-even).  The
// operand is first held to [0, 448] (NaN to 0), so no overflow or NaN rule of the
// instruction is relied on.  sharq_e4m3_conversion_probe checks both against the
// definition forms on the device: every fp32 pattern with the sign bit clear, and every
// code up to 0x7E.
__device__ __forceinline__ uint32_t e4m3_encode_hw(float q) {
  const float c = q > 0.0f ? (q < 448.0f ? q : 448.0f) : 0.0f;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

__device__ __forceinline__ float e4m3_value_hw(uint32_t s) { return __builtin_amdgcn_cvt_f32_fp8((int)s, 0); }

// rms_scale_pair for one dword of two bf16 x and one of two bf16 gains, returning the two
// bf16 results as fp32 values (rounded by bf16x2_rne_hw).
__device__ __forceinline__ void rms_scale_f2(uint32_t w, uint32_t gw, float r, float& y0, float& y1) {
  const uint32_t b = bf16x2_rne_hw(__fmul_rn(__fmul_rn(__uint_as_float(w << 16), r), __uint_as_float(gw << 16)),
                                   __fmul_rn(__fmul_rn(__uint_as_float(w & 0xFFFF0000u), r),
                                             __uint_as_float(gw & 0xFFFF0000u)));
  y0 = __uint_as_float(b << 16);
  y1 = __uint_as_float(b & 0xFFFF0000u);
}

__device__ __forceinline__ uint32_t rms_scale_pair(uint32_t w, uint32_t gw, float r) {
  const float y0 = __fmul_rn(__fmul_rn(__uint_as_float(w << 16), r), __uint_as_float(gw << 16));
  const float y1 = __fmul_rn(__fmul_rn(__uint_as_float(w & 0xFFFF0000u), r), __uint_as_float(gw & 0xFFFF0000u));
  return bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16);
}

// Input transforms the preparation kernels can apply to the loaded bf16 values.
constexpr int kXfNone = 0;    // X as given
constexpr int kXfRms = 1;     // RMS normalization with a bf16 gain (rms_scale_pair)
constexpr int kXfSwiglu = 2;  // SwiGLU of a gate/up pair (swiglu_pair)

// SwiGLU: h = bf16(fp32(silu(g) * u)), silu(g) = fp32(g / fp32(1 + e)), e = e^-g in
// fp32 by Cody and Waite's range reduction (t = -g clamped to [-150, 150],
// n = rint(t log2 e), r = (t - n ln2_hi) - n ln2_lo with a 15-bit ln2_hi so that
// n ln2_hi is exact) and the degree-7 Taylor polynomial of e^r, scaled by 2^n.  Every
// operation is one rounding in a fixed order, so the value is reproducible bit for bit.
__device__ __forceinline__ float silu_f32(float g) {
  float t = -g;
  t = t > 150.0f ? 150.0f : t;
  t = t < -150.0f ? -150.0f : t;
  const float n = __builtin_rintf(__fmul_rn(t, 0x1.715476p+0f));
  const float r = __fsub_rn(__fsub_rn(t, __fmul_rn(n, 0x1.62e4p-1f)), __fmul_rn(n, 0x1.7f7d1cp-20f));
  float p = 0x1.a01a02p-13f;                        // 1/7!
  p = __fadd_rn(__fmul_rn(p, r), 0x1.6c16c2p-10f);  // 1/6!
  p = __fadd_rn(__fmul_rn(p, r), 0x1.111112p-7f);   // 1/5!
  p = __fadd_rn(__fmul_rn(p, r), 0x1.555556p-5f);   // 1/4!
  p = __fadd_rn(__fmul_rn(p, r), 0x1.555556p-3f);   // 1/3!
  p = __fadd_rn(__fmul_rn(p, r), 0.5f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  const float e = ldexpf(p, (int)n);
  return __fdiv_rn(g, __fadd_rn(1.0f, e));
}

// Two bf16 gates and two bf16 ups (packed) -> two bf16 SwiGLU values (packed).
__device__ __forceinline__ uint32_t swiglu_pair(uint32_t gw, uint32_t uw) {
  const float h0 = __fmul_rn(silu_f32(__uint_as_float(gw << 16)), __uint_as_float(uw << 16));
  const float h1 = __fmul_rn(silu_f32(__uint_as_float(gw & 0xFFFF0000u)), __uint_as_float(uw & 0xFFFF0000u));
  return bf16_rne_bits(h0) | (bf16_rne_bits(h1) << 16);
}

// silu_f32 of a bf16 gate by lookup.  The gate is one of 2^16 patterns, so silu_f32 can
// be tabulated; only the patterns with exponent field 103..133 (|g| in [2^-24, 2^7))
// need the table (2 signs x 31 exponents x 128 mantissas).  Below that range e rounds
// to 1, the divisor is 2 and silu_f32(g) = g/2 exactly; above it silu_f32(g) is g for
// g > 0 (e is 0 or subnormal, the divisor rounds to 1) and -0 for g < 0 (e overflows
// to +inf).  Each rule equals silu_f32 on every finite bf16 it covers.  (Non-finite
// inputs are outside the preparation's contract; the rules send +inf to +inf and -inf
// to -0, NaN to itself or -0, and never index outside the table.)  A work-group fills
// its LDS copy of the table once (silu_table_fill) and reads it for every gate after.
constexpr uint32_t kSiluElo = 103, kSiluSpan = 31;        // exponent fields 103..133
constexpr uint32_t kSiluHalf = kSiluSpan * 128;           // entries per sign
constexpr int kSiluEntries = 2 * (int)kSiluHalf;          // 7936 floats = 31 KiB

__device__ __forceinline__ void silu_table_fill(float* tab, int tid, int nthreads) {
  for (int i = tid; i < kSiluEntries; i += nthreads) {
    const uint32_t sign = (uint32_t)i >= kSiluHalf ? 1u : 0u;
    const uint32_t b = (sign << 15) | ((kSiluElo << 7) + ((uint32_t)i - sign * kSiluHalf));
    tab[i] = silu_f32(__uint_as_float(b << 16));
  }
}

// b: a bf16 pattern in the low 16 bits.
__device__ __forceinline__ float silu_lookup(const float* tab, uint32_t b) {
  const uint32_t mag = b & 0x7FFFu, sign = b >> 15;
  const uint32_t off = mag - (kSiluElo << 7);  // wraps above the window's top for small gates
  const bool in = off < kSiluHalf;
  const float t = tab[in ? sign * kSiluHalf + off : 0u];
  const uint32_t gb = b << 16;
  const float small = __fmul_rn(__uint_as_float(gb), 0.5f);
  const float large = __uint_as_float(sign ? 0x80000000u : gb);
  return in ? t : (mag < (kSiluElo << 7) ? small : large);
}

// swiglu_pair with silu_f32 looked up.
__device__ __forceinline__ uint32_t swiglu_pair_tab(const float* tab, uint32_t gw, uint32_t uw) {
  const float h0 = __fmul_rn(silu_lookup(tab, gw & 0xFFFFu), __uint_as_float(uw << 16));
  const float h1 = __fmul_rn(silu_lookup(tab, gw >> 16), __uint_as_float(uw & 0xFFFF0000u));
  return bf16_rne_bits(h0) | (bf16_rne_bits(h1) << 16);
}

}  // namespace codec
}  // namespace sharq
