// prep_mx.hip -- the fused SharQ activation preparation for MXFP4 on gfx950.
//
// One pass over X (SharQ, arXiv 2606.26587: abstract and "Core claim"; Figure 2's
// fused preparation kernel): N:M top-|x| mask, MXFP4 backbone, residual against the
// dequantized backbone, MXFP4 residual with its own scales.
//
// Work mapping.  X is viewed as a flat sequence of 32-element blocks (block b is
// row b / (K/32), columns 32*(b % (K/32)) ..).  Four lanes of a quad own one block,
// 8 consecutive bf16 (one 16-byte load) each, so a wave covers 16 blocks and a
// load instruction reads 1 KiB of contiguous X when rows are dense.  Mask groups
// (4 or 8 elements) never straddle a lane; the block maxima are two DPP quad
// exchanges.  The E2M1 conversions use the gfx950 scaled-conversion instructions,
// whose rounding (nearest-even, saturating, sign kept, E8M0 byte 0 = 2^-127,
// subnormals kept) was checked bit-for-bit against the format definition.
//
// Outputs are dense: codes at b*16 bytes, scales at byte b, mask bits at b*4.
#include "sharq_internal.h"

namespace sharq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // blocks in flight per quad
constexpr int kBlocksPerWave = 16;

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Maximum over the 4 lanes of a quad (DPP quad_perm [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
  return v;
}

// Sort (a >= b).
__device__ __forceinline__ void cswap(uint32_t& a, uint32_t& b) {
  uint32_t hi = umax(a, b), lo = umin(a, b);
  a = hi;
  b = lo;
}

// Keep bits (bit j = element j of the lane's 8) for the top-n-of-m mask.  Every
// element gets a compound key (|x| bits, then a reversed index) so that keys are
// distinct and "larger key" means "ranks earlier": bigger magnitude first, lower
// index first among equal magnitudes.  The kept elements are those at or above
// the n-th largest compound key of their group.
template <int SPM>
__device__ __forceinline__ uint32_t keep_bits(const uint32_t w[4]) {
  uint32_t ck[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t key = (j & 1) ? (w[j >> 1] >> 16) & 0x7FFFu : w[j >> 1] & 0x7FFFu;
    ck[j] = SPM == 4 ? (key << 2) | (3u - (j & 3)) : (key << 3) | (7u - j);
  }
  uint32_t bits = 0;
  if constexpr (SPM == 4) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t* c = ck + 4 * g;
      uint32_t hi1 = umax(c[0], c[1]), lo1 = umin(c[0], c[1]);
      uint32_t hi2 = umax(c[2], c[3]), lo2 = umin(c[2], c[3]);
      uint32_t second = umax(umin(hi1, hi2), umax(lo1, lo2));  // 2nd largest of 4
#pragma unroll
      for (int j = 0; j < 4; ++j) bits |= (c[j] >= second ? 1u : 0u) << (4 * g + j);
    }
  } else {
    uint32_t a0 = ck[0], a1 = ck[1], a2 = ck[2], a3 = ck[3];
    uint32_t b0 = ck[4], b1 = ck[5], b2 = ck[6], b3 = ck[7];
    cswap(a0, a1); cswap(a2, a3); cswap(a0, a2); cswap(a1, a3); cswap(a1, a2);
    cswap(b0, b1); cswap(b2, b3); cswap(b0, b2); cswap(b1, b3); cswap(b1, b2);
    // top half of two descending runs: max(a_i, b_{3-i}); its minimum is the 4th largest
    uint32_t fourth = umin(umin(umax(a0, b3), umax(a1, b2)), umin(umax(a2, b1), umax(a3, b0)));
#pragma unroll
    for (int j = 0; j < 8; ++j) bits |= (ck[j] >= fourth ? 1u : 0u) << j;
  }
  return bits;
}

// E8M0 byte for a block whose largest magnitude has IEEE exponent field `e`
// (bf16 or fp32 alike): E = floor(log2 amax) - 2, clamped at -127; byte = E + 127.
__device__ __forceinline__ uint32_t e8m0_from_expfield(uint32_t e) { return e > 2 ? e - 2 : 0; }

// fp32 whose exponent bits are the E8M0 byte: the conversion instructions read
// the scale's exponent field, so byte 0 (bit pattern +0.0) means 2^-127.
__device__ __forceinline__ float scale_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) {
  bf16x2_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times 2^E.
__device__ __forceinline__ void dequant8(uint32_t packed, float scale, float out[8]) {
  auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, scale, 0);
  auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, scale, 1);
  auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, scale, 2);
  auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, scale, 3);
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
}

// Gather the scale bytes of the 16 blocks of a wave into 4 dwords held by lanes
// 0, 16, 32, 48 (the byte of block 4k+i comes from quad 4k+i = lane 16k+4i).
__device__ __forceinline__ uint32_t gather_scales(uint32_t byte) {
  uint32_t b1 = __shfl_down(byte, 4, 64);
  uint32_t b2 = __shfl_down(byte, 8, 64);
  uint32_t b3 = __shfl_down(byte, 12, 64);
  return byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

__device__ __forceinline__ void store_scales(uint8_t* dst, int64_t b, int64_t nblocks, int lane,
                                             uint32_t packed) {
  if ((lane & 15) != 0) return;
  if (b + 3 < nblocks) {
    *reinterpret_cast<uint32_t*>(dst + b) = packed;  // b is a multiple of 4 here
  } else {
    for (int i = 0; i < 4; ++i)
      if (b + i < nblocks) dst[b + i] = (uint8_t)(packed >> (8 * i));
  }
}

// The per-block codec of one lane: 8 consecutive bf16 of a 32-element block (the
// quad's other three lanes hold the rest).  MODE 0: mask, backbone codes and scale,
// residual against the dequantized backbone, residual codes and scale.  MODE 1:
// plain MXFP4 of the 8 values into (rbyte, rpacked).  Every lane of the quad must
// call it together (the block maxima are quad exchanges).
template <int MODE, int SPM>
__device__ __forceinline__ void codec_block(const uint32_t w[4], uint32_t& keep, uint32_t& bbyte,
                                            uint32_t& bpacked, uint32_t& rbyte, uint32_t& rpacked) {
  // x as fp32 (exact)
  float xf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xf[2 * i] = __uint_as_float(w[i] << 16);
    xf[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }

  float r[8];
  keep = 0xFFu; bbyte = 0; bpacked = 0;
  if constexpr (MODE == 0) {
    keep = keep_bits<SPM>(w);
    // Backbone block maximum: every group's largest element is kept and the
    // groups tile the block, so the kept maximum is the block maximum of |x|.
    uint32_t kmax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) kmax = umax(kmax, umax(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    kmax = quad_max(kmax);
    bbyte = e8m0_from_expfield(kmax >> 7);
    const float bscale = scale_operand(bbyte);
    // dropped positions become +0 (bf16 bits 0), which encodes as code 0x0
    uint32_t wm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wm[i] = w[i] & (((keep >> (2 * i)) & 1 ? 0x0000FFFFu : 0u) |
                      ((keep >> (2 * i + 1)) & 1 ? 0xFFFF0000u : 0u));
    bpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(bpacked, as_bf16x2(wm[0]), bscale, 0);
    bpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(bpacked, as_bf16x2(wm[1]), bscale, 1);
    bpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(bpacked, as_bf16x2(wm[2]), bscale, 2);
    bpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(bpacked, as_bf16x2(wm[3]), bscale, 3);
    // residual against the dequantized backbone: one fp32 subtraction each
    float bh[8];
    dequant8(bpacked, bscale, bh);
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = xf[j] - bh[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = xf[j];
  }

  // residual (or plain) quantization with its own block scale
  uint32_t rmax = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) rmax = umax(rmax, __float_as_uint(r[j]) & 0x7FFFFFFFu);
  rmax = quad_max(rmax);
  rbyte = e8m0_from_expfield(rmax >> 23);
  const float rscale = scale_operand(rbyte);
  rpacked = 0;
  rpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rpacked, r[0], r[1], rscale, 0);
  rpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rpacked, r[2], r[3], rscale, 1);
  rpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rpacked, r[4], r[5], rscale, 2);
  rpacked = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rpacked, r[6], r[7], rscale, 3);
}

// MODE 0: SharQ preparation (mask, backbone, residual).  MODE 1: plain MXFP4
// quantization of X into (rcodes, rscales) -- used for weight payloads.
template <int MODE, int SPM, bool DENSE_ROWS, bool WRITE_MASK>
__global__ __launch_bounds__(kThreads) void prep_mx_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t nbk, int64_t nblocks,
    uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales, uint8_t* __restrict__ rcodes,
    uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask) {
  const int lane = threadIdx.x & 63;
  const int q = lane & 3;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t base = wave * (kBlocksPerWave * kUnroll);

  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t b = base + u * kBlocksPerWave + (lane >> 2);
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (b < nblocks) {
      int64_t off;
      if constexpr (DENSE_ROWS) {
        off = b * 32 + q * 8;
      } else {
        const int64_t row = b / nbk;
        off = row * ldx + (b - row * nbk) * 32 + q * 8;
      }
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off));
    }
  }

#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t b = base + u * kBlocksPerWave + (lane >> 2);
    const bool valid = b < nblocks;
    const uint32_t w[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};

    uint32_t keep, bbyte, bpacked, rbyte, rpacked;
    codec_block<MODE, SPM>(w, keep, bbyte, bpacked, rbyte, rpacked);

    // scale bytes: gathered by every lane (wave-wide shuffles), stored by 4 lanes
    const int64_t b0 = base + u * kBlocksPerWave + 4 * (lane >> 4);
    const uint32_t rpk = gather_scales(rbyte);
    uint32_t bpk = 0;
    if constexpr (MODE == 0) bpk = gather_scales(bbyte);

    if (valid) {
      __builtin_nontemporal_store(rpacked, reinterpret_cast<uint32_t*>(rcodes + b * 16 + q * 4));
      if constexpr (MODE == 0) {
        __builtin_nontemporal_store(bpacked, reinterpret_cast<uint32_t*>(bcodes + b * 16 + q * 4));
        if constexpr (WRITE_MASK) mask[b * 4 + q] = (uint8_t)keep;
      }
    }
    store_scales(rscales, b0, nblocks, lane, rpk);
    if constexpr (MODE == 0) store_scales(bscales, b0, nblocks, lane, bpk);
  }
}

// Tiled-layout output (the layout the fused GEMM loads; see sharq.h).  A wave owns
// 16 consecutive rows x one 128-element K-step: quad k is row 16*rg + k and walks the
// step's 4 blocks (u = 0..3).  Each store instruction then writes the 16-byte slots of
// 16 consecutive rows of one fragment (256 contiguous bytes), and each quad leader
// ends with its row's 4 scale bytes = one scale word, so a wave's scale words are 64
// contiguous bytes.  Rows >= M and blocks >= K/32 are processed as zeros, which
// writes the layout's zero padding.
template <int MODE, int SPM, bool WRITE_MASK>
__global__ __launch_bounds__(kThreads) void prep_mx_tiled_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int64_t Mp, int64_t Kp,
    uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales, uint8_t* __restrict__ rcodes,
    uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask) {
  const int lane = threadIdx.x & 63;
  const int q = lane & 3, k = lane >> 2;
  const int64_t nks = Kp / 128;
  const int64_t task = (int64_t)blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (task >= (Mp / 16) * nks) return;  // whole waves only
  const int64_t rg = task / nks, ks = task - rg * nks;
  const int64_t r = rg * 16 + k;
  const int64_t nbk = K / 32;

  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t b = ks * 4 + u;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (r < M && b < nbk)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + r * ldx + b * 32 + q * 8));
  }
  const int64_t frag_row = (r >> 5) * (Kp / 64);
  const int slot_row = (int)(r & 31);
  uint32_t bword = 0, rword = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t b = ks * 4 + u;
    const uint32_t w[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
    uint32_t keep, bbyte, bpacked, rbyte, rpacked;
    codec_block<MODE, SPM>(w, keep, bbyte, bpacked, rbyte, rpacked);
    const int64_t off = (frag_row + (b >> 1)) * 1024 + (slot_row + 32 * (int)(b & 1)) * 16 + q * 4;
    __builtin_nontemporal_store(rpacked, reinterpret_cast<uint32_t*>(rcodes + off));
    rword |= rbyte << (8 * u);
    if constexpr (MODE == 0) {
      __builtin_nontemporal_store(bpacked, reinterpret_cast<uint32_t*>(bcodes + off));
      bword |= bbyte << (8 * u);
      if constexpr (WRITE_MASK)
        if (r < M && b < nbk) mask[r * (K / 8) + b * 4 + q] = (uint8_t)keep;
    }
  }
  if (q == 0) {
    reinterpret_cast<uint32_t*>(rscales)[ks * Mp + r] = rword;
    if constexpr (MODE == 0) reinterpret_cast<uint32_t*>(bscales)[ks * Mp + r] = bword;
  }
}

template <int MODE, int SPM, bool WRITE_MASK>
hipError_t launch_tiled(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes,
                        uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales, uint8_t* mask,
                        hipStream_t stream) {
  const int64_t Mp = (M + 31) / 32 * 32, Kp = (K + 127) / 128 * 128;
  const int64_t tasks = (Mp / 16) * (Kp / 128);
  if (tasks == 0) return hipSuccess;
  const int64_t grid = (tasks + kThreads / 64 - 1) / (kThreads / 64);
  prep_mx_tiled_kernel<MODE, SPM, WRITE_MASK><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      x, M, K, ldx, Mp, Kp, bcodes, bscales, rcodes, rscales, mask);
  return hipGetLastError();
}

template <int MODE, int SPM, bool WRITE_MASK>
hipError_t launch_dense_or_strided(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes,
                                   uint8_t* rscales, uint8_t* mask, hipStream_t stream) {
  const int64_t nbk = K / 32;
  const int64_t nblocks = M * nbk;
  if (nblocks == 0) return hipSuccess;
  const int64_t per_wg = (kThreads / 64) * kBlocksPerWave * kUnroll;
  const int64_t grid = (nblocks + per_wg - 1) / per_wg;
  if (ldx == K)
    prep_mx_kernel<MODE, SPM, true, WRITE_MASK><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        x, ldx, nbk, nblocks, bcodes, bscales, rcodes, rscales, mask);
  else
    prep_mx_kernel<MODE, SPM, false, WRITE_MASK><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        x, ldx, nbk, nblocks, bcodes, bscales, rcodes, rscales, mask);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                          uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales,
                          uint8_t* mask, int tiled, hipStream_t stream) {
  (void)sp_n;  // n = m/2 for both supported patterns
  if (tiled) {
    if (sp_m == 4)
      return mask ? launch_tiled<0, 4, true>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream)
                  : launch_tiled<0, 4, false>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream);
    return mask ? launch_tiled<0, 8, true>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream)
                : launch_tiled<0, 8, false>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream);
  }
  if (sp_m == 4) {
    if (mask)
      return launch_dense_or_strided<0, 4, true>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream);
    return launch_dense_or_strided<0, 4, false>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream);
  }
  if (mask)
    return launch_dense_or_strided<0, 8, true>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream);
  return launch_dense_or_strided<0, 8, false>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, stream);
}

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, int tiled, hipStream_t stream) {
  if (tiled)
    return launch_tiled<1, 4, false>(x, rows, K, ldx, nullptr, nullptr, codes, scales, nullptr, stream);
  return launch_dense_or_strided<1, 4, false>(x, rows, K, ldx, nullptr, nullptr, codes, scales, nullptr,
                                              stream);
}

}  // namespace sharq
