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
#include "fp4_codec.h"
#include "sharq_internal.h"

namespace sharq {
namespace {

using namespace codec;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // blocks in flight per quad
constexpr int kBlocksPerWave = 16;

// Maximum over the 4 lanes of a quad (DPP quad_perm [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
  return v;
}

// Scale-operand bits for a block whose largest magnitude has fp32 bits `amax_bits`:
// E = floor(log2 amax) - 2 clamped at -127, i.e. exponent field minus 2 saturating
// at 0; the E8M0 byte is that field.  The conversion instructions read the scale's
// exponent field, so field 0 (bit pattern +0.0) means 2^-127.
__device__ __forceinline__ uint32_t scale_bits_of(uint32_t amax_bits) {
  return __builtin_elementwise_sub_sat(amax_bits & 0x7F800000u, 0x01000000u);
}

// Largest |v| of the lane's 8 values, as fp32 bits (non-negative floats order like
// their bit patterns, so the quad exchange can use integer maxima).
__device__ __forceinline__ uint32_t abs_max8(const float v[8]) {
  const float m0 = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  const float m1 = fmaxf(fmaxf(fabsf(v[3]), fabsf(v[4])), fabsf(v[5]));
  const float m2 = fmaxf(fmaxf(fabsf(v[6]), fabsf(v[7])), m0);
  return __float_as_uint(fmaxf(m1, m2));
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

// Eight fp32 values to E2M1 codes with scale 2^E (round to nearest even, saturating).
__device__ __forceinline__ uint32_t quant8(const float v[8], float scale) {
  // the four conversions write all four bytes, so the initial contents do not matter
  uint32_t p = __float_as_uint(v[0]);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0], v[1], scale, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2], v[3], scale, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4], v[5], scale, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6], v[7], scale, 3);
  return p;
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
// plain MXFP4 of the 8 values into (rbyte, rpacked).  MODEs 2-4 are the ablations
// of the method's choices: 2 = residual against the unquantized sparse values
// (R = X - X*mask: the backbone's quantization error is left uncompensated), 3 = a
// static mask (the first n of every m positions, whatever the input), 4 = no
// residual (direct N:M sparsity + FP4; the residual payload is all zero).  Every
// lane of the quad must call it together (the block maxima are quad exchanges).
// `keep` (bit j = element j kept) is only computed when a caller uses it.
// codec_block_f takes the 8 values as fp32 (each a bf16 value, exactly).
template <int MODE, int SPM>
__device__ __forceinline__ void codec_block_f(const float xf[8], uint32_t& keep, uint32_t& bbyte,
                                              uint32_t& bpacked, uint32_t& rbyte, uint32_t& rpacked) {
  float r[8];
  keep = 0xFFu; bbyte = 0; bpacked = 0;
  if constexpr (MODE != 1) {
    bool kept[8];
    if constexpr (MODE == 3) {
      // static: the lane's 8 elements start at a multiple of 8, so element j sits
      // at position j % SPM of its group
#pragma unroll
      for (int j = 0; j < 8; ++j) kept[j] = (j % SPM) < SPM / 2;
    } else {
      keep_mask<SPM>(xf, kept);
    }
    keep = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) keep |= (kept[j] ? 1u : 0u) << j;
    // dropped positions become +0, which encodes as code 0x0
    float xm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xm[j] = kept[j] ? xf[j] : 0.0f;
    // Backbone block maximum: with the top-|x| mask every group's largest element is
    // kept and the groups tile the block, so the kept maximum is the block maximum
    // of |x|; a static mask needs the maximum of the kept values themselves.
    const uint32_t bsb = scale_bits_of(quad_max(abs_max8(MODE == 3 ? xm : xf)));
    bbyte = bsb >> 23;
    const float bscale = __uint_as_float(bsb);
    bpacked = quant8(xm, bscale);
    if constexpr (MODE == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = kept[j] ? 0.0f : xf[j];  // x - x*mask, exact
    } else if constexpr (MODE == 4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = 0.0f;
    } else {
      // residual against the dequantized backbone: one fp32 subtraction each
      float bh[8];
      dequant8(bpacked, bscale, bh);
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = xf[j] - bh[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = xf[j];
  }

  // residual (or plain) quantization with its own block scale
  const uint32_t rsb = scale_bits_of(quad_max(abs_max8(r)));
  rbyte = rsb >> 23;
  rpacked = quant8(r, __uint_as_float(rsb));
}

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
  codec_block_f<MODE, SPM>(xf, keep, bbyte, bpacked, rbyte, rpacked);
}

// Optional RMS normalization applied to the loaded bf16 values (XF == kXfRms): per-row
// factors r[M] and per-channel bf16 gains g[K] (see rms_scale_pair).
struct Norm {
  const float* r;
  const uint16_t* g;
};

__device__ __forceinline__ u32x4 swiglu8(const u32x4& g, const u32x4& u) {
  return u32x4{swiglu_pair(g[0], u[0]), swiglu_pair(g[1], u[1]), swiglu_pair(g[2], u[2]), swiglu_pair(g[3], u[3])};
}

// swiglu8 with the SiLU table (silu_lookup).
__device__ __forceinline__ u32x4 swiglu8_tab(const float* tab, const u32x4& g, const u32x4& u) {
  return u32x4{swiglu_pair_tab(tab, g[0], u[0]), swiglu_pair_tab(tab, g[1], u[1]), swiglu_pair_tab(tab, g[2], u[2]),
               swiglu_pair_tab(tab, g[3], u[3])};
}

__device__ __forceinline__ u32x4 rms_scale8(const u32x4& v, const Norm& nm, int64_t row, int64_t col) {
  const float r = nm.r[row];
  const u32x4 g = *reinterpret_cast<const u32x4*>(nm.g + col);
  return u32x4{rms_scale_pair(v[0], g[0], r), rms_scale_pair(v[1], g[1], r), rms_scale_pair(v[2], g[2], r),
               rms_scale_pair(v[3], g[3], r)};
}

// MODE 0: SharQ preparation (mask, backbone, residual).  MODE 1: plain MXFP4
// quantization of X into (rcodes, rscales) -- used for weight payloads.  MODEs 2-4:
// the ablations (see codec_block).
template <int MODE, int SPM, bool DENSE_ROWS, bool WRITE_MASK, int XF>
__global__ __launch_bounds__(kThreads) void prep_mx_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t nbk, int64_t nblocks,
    uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales, uint8_t* __restrict__ rcodes,
    uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask, Norm nm) {
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
      if constexpr (XF == kXfSwiglu) {  // gate at off, up K columns further in the same row
        v[u] = swiglu8(v[u], __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off + nbk * 32)));
      }
      if constexpr (XF == kXfRms) {
        const int64_t row = b / nbk;
        v[u] = rms_scale8(v[u], nm, row, (b - row * nbk) * 32 + q * 8);
      }
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
    if constexpr (MODE != 1) bpk = gather_scales(bbyte);

    if (valid) {
      __builtin_nontemporal_store(rpacked, reinterpret_cast<uint32_t*>(rcodes + b * 16 + q * 4));
      if constexpr (MODE != 1) {
        __builtin_nontemporal_store(bpacked, reinterpret_cast<uint32_t*>(bcodes + b * 16 + q * 4));
        if constexpr (WRITE_MASK) mask[b * 4 + q] = (uint8_t)keep;
      }
    }
    store_scales(rscales, b0, nblocks, lane, rpk);
    if constexpr (MODE != 1) store_scales(bscales, b0, nblocks, lane, bpk);
  }
}

// Tiled-layout output (the layout the fused GEMM loads; see sharq.h).  A wave owns
// 16 consecutive rows x one 128-element K-step (an item): quad k is row 16*rg + k and
// walks the step's 4 blocks (u = 0..3).  Each store instruction then writes the 16-byte
// slots of 16 consecutive rows of one fragment (256 contiguous bytes), and each quad
// leader ends with its row's 4 scale bytes = one scale word, so a wave's scale words are
// 64 contiguous bytes.  Rows >= M and blocks >= K/32 are processed as zeros, which
// writes the layout's zero padding.

// The item's 4 x 8 elements of this lane from the rows at x (row stride ldx): zeros
// outside X.  A wave wholly inside X loads unguarded.
__device__ __forceinline__ void tiled_load(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                                           int64_t ks, int64_t rg, u32x4 (&v)[4]) {
  const int lane = threadIdx.x & 63;
  const int q = lane & 3, k = lane >> 2;
  const int64_t r0 = rg * 16;
  const uint16_t* xrow = x + r0 * ldx + ks * 128;  // uniform base
  const int64_t lane_off = (int64_t)k * ldx + q * 8;
  if (r0 + 16 <= M && ks * 4 + 4 <= K / 32) {
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xrow + lane_off + u * 32));
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (r0 + k < M && ks * 4 + u < K / 32)
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xrow + lane_off + u * 32));
    }
  }
}

// Codes of the item's (transformed) elements v: mask, backbone, residual, through the
// wave's private LDS staging `my`, `myb` (2 x 1 KiB) so that every global store writes
// 16 B per lane: lane L then holds slot (row L%16, block u = L/16), and the four 256-byte
// row runs of the wave are fragment (r/32, 2ks + u/2), slots (r%32) + 32(u%2).
template <int MODE, int SPM, bool WRITE_MASK>
__device__ __forceinline__ void tiled_code(const u32x4 (&v)[4], int64_t M, int64_t K, int64_t Mp, int64_t Kp,
                                           int64_t ks, int64_t rg, uint8_t* __restrict__ bcodes,
                                           uint8_t* __restrict__ bscales, uint8_t* __restrict__ rcodes,
                                           uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask, uint32_t* my,
                                           uint32_t* myb) {
  const int lane = threadIdx.x & 63;
  const int q = lane & 3, k = lane >> 2;
  const int64_t r0 = rg * 16;
  const int64_t r = r0 + k;
  const int64_t nbk = K / 32;
  uint32_t bword = 0, rword = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t w[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
    uint32_t keep, bbyte, bpacked, rbyte, rpacked;
    codec_block<MODE, SPM>(w, keep, bbyte, bpacked, rbyte, rpacked);
    my[u * 64 + lane] = rpacked;  // = slot (u, k), dword q
    rword |= rbyte << (8 * u);
    if constexpr (MODE != 1) {
      myb[u * 64 + lane] = bpacked;
      bword |= bbyte << (8 * u);
      if constexpr (WRITE_MASK)
        if (r < M && ks * 4 + u < nbk) mask[r * (K / 8) + (ks * 4 + u) * 4 + q] = (uint8_t)keep;
    }
  }
  // the staging is wave-private: a wave-level wait on the LDS writes is enough
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  const int64_t frag0 = ((r0 >> 5) * (Kp / 64) + 2 * ks) * 1024;
  const int su = lane >> 4;
  const int off = (su >> 1) * 1024 + (su & 1) * 512 + (int)(((r0 & 31) + (lane & 15)) * 16);
  // ordinary (cached) stores: the GEMM reads these payloads next (measured: non-temporal
  // stores here cost the 32760x3072 preparation about 4 %)
  *reinterpret_cast<u32x4*>(rcodes + frag0 + off) = reinterpret_cast<const u32x4*>(my)[lane];
  if constexpr (MODE != 1)
    *reinterpret_cast<u32x4*>(bcodes + frag0 + off) = reinterpret_cast<const u32x4*>(myb)[lane];
  if (q == 0) {
    reinterpret_cast<uint32_t*>(rscales)[ks * Mp + r] = rword;
    if constexpr (MODE != 1) reinterpret_cast<uint32_t*>(bscales)[ks * Mp + r] = bword;
  }
}

// One item per wave, loads, codec and stores in one body (the same steps as tiled_load
// and tiled_code; written out here because the split form measured slower for this
// kernel: 11.9 against 11.2 us at 4096 x 4096).  The grid is (K-step groups of 4, row
// groups): a work-group's 4 waves take 4 consecutive K-steps of the same 16 rows.  XF:
// none or RMS normalization.
template <int MODE, int SPM, bool WRITE_MASK, int XF>
__global__ __launch_bounds__(kThreads) void prep_mx_tiled_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int64_t Mp, int64_t Kp,
    int64_t rg0, uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales,
    uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask, Norm nm) {
  static_assert(XF != kXfSwiglu, "the SwiGLU transform runs prep_mx_tiled_swiglu_kernel");
  const int lane = threadIdx.x & 63;
  const int q = lane & 3, k = lane >> 2;
  const int64_t nks = Kp / 128;
  const int64_t ks = (int64_t)blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (ks >= nks) return;  // whole waves only
  const int64_t rg = rg0 + blockIdx.y;
  const int64_t r0 = rg * 16;  // first row of the wave (uniform)
  const int64_t r = r0 + k;
  const int64_t nbk = K / 32;

  // loads: the 16 rows x 4 blocks; a wave wholly inside X loads unguarded
  u32x4 v[4];
  const uint16_t* xrow = x + r0 * ldx + ks * 128;  // uniform base
  const int64_t lane_off = (int64_t)k * ldx + q * 8;
  if (r0 + 16 <= M && ks * 4 + 4 <= nbk) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xrow + lane_off + u * 32));
      if constexpr (XF == kXfRms) v[u] = rms_scale8(v[u], nm, r, ks * 128 + u * 32 + q * 8);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (r < M && ks * 4 + u < nbk) {
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xrow + lane_off + u * 32));
        if constexpr (XF == kXfRms) v[u] = rms_scale8(v[u], nm, r, ks * 128 + u * 32 + q * 8);
      }
    }
  }

  // Codes go through a wave-private LDS tile so that every global store writes 16 B
  // per lane: lane L then holds slot (row L%16, block u = L/16), and the four 256-byte
  // row runs of the wave are fragment (r/32, 2ks + u/2), slots (r%32) + 32(u%2).
  __shared__ uint32_t tile[kThreads / 64][2][4 * 16 * 4];
  uint32_t* my = tile[threadIdx.x >> 6][0];
  uint32_t* myb = tile[threadIdx.x >> 6][1];
  uint32_t bword = 0, rword = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t w[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
    uint32_t keep, bbyte, bpacked, rbyte, rpacked;
    codec_block<MODE, SPM>(w, keep, bbyte, bpacked, rbyte, rpacked);
    my[u * 64 + lane] = rpacked;  // = slot (u, k), dword q
    rword |= rbyte << (8 * u);
    if constexpr (MODE != 1) {
      myb[u * 64 + lane] = bpacked;
      bword |= bbyte << (8 * u);
      if constexpr (WRITE_MASK)
        if (r < M && ks * 4 + u < nbk) mask[r * (K / 8) + (ks * 4 + u) * 4 + q] = (uint8_t)keep;
    }
  }
  // the tile is wave-private: a wave-level wait on the LDS writes is enough
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  const int64_t frag0 = ((r0 >> 5) * (Kp / 64) + 2 * ks) * 1024;
  const int su = lane >> 4;
  const int off = (su >> 1) * 1024 + (su & 1) * 512 + (int)(((r0 & 31) + (lane & 15)) * 16);
  // ordinary (cached) stores: the GEMM reads these payloads next (measured: non-temporal
  // stores here cost the 32760x3072 preparation about 4 %)
  *reinterpret_cast<u32x4*>(rcodes + frag0 + off) = reinterpret_cast<const u32x4*>(my)[lane];
  if constexpr (MODE != 1)
    *reinterpret_cast<u32x4*>(bcodes + frag0 + off) = reinterpret_cast<const u32x4*>(myb)[lane];
  if (q == 0) {
    reinterpret_cast<uint32_t*>(rscales)[ks * Mp + r] = rword;
    if constexpr (MODE != 1) reinterpret_cast<uint32_t*>(bscales)[ks * Mp + r] = bword;
  }
}

// The same tiled preparation of h = SwiGLU(gate, up) (gate in columns [0, K) of each row
// of x, up in [K, 2K)), with silu_f32 looked up: each work-group fills its 31 KiB SiLU
// table once, then its waves walk the (row group, K-step) items grid-stride -- K-steps
// fastest, so consecutive waves take consecutive K-steps of the same 16 rows.  A wave
// issues the loads of its next item before it codes the current one, and its first
// loads before the table fill, so the memory traffic runs under the arithmetic.  The
// bounded grid (kSwigluGroups work-groups of 1024 threads) pays for each table over
// several items per wave.  Outside X, gate and up load as zeros, so h is +0 there as
// the padding needs.
constexpr int kSwigluThreads = 1024;
constexpr int kSwigluGroups = 256;

template <int SPM, bool WRITE_MASK>
__global__ __launch_bounds__(kSwigluThreads) void prep_mx_tiled_swiglu_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int64_t Mp, int64_t Kp,
    uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales, uint8_t* __restrict__ rcodes,
    uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask) {
  __shared__ float stab[kSiluEntries];
  __shared__ uint32_t tile[kSwigluThreads / 64][2][4 * 16 * 4];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nks = Kp / 128, items = nks * (Mp / 16);
  const int64_t nwaves = (int64_t)gridDim.x * (kSwigluThreads / 64);
  int64_t it = (int64_t)blockIdx.x * (kSwigluThreads / 64) + wv;
  u32x4 g[4], up[4];
  if (it < items) {
    const int64_t rg = it / nks;
    tiled_load(x, M, K, ldx, it - rg * nks, rg, g);
    tiled_load(x + K, M, K, ldx, it - rg * nks, rg, up);
  }
  silu_table_fill(stab, (int)threadIdx.x, kSwigluThreads);
  __syncthreads();
  for (; it < items; it += nwaves) {
    const int64_t rg = it / nks, ks = it - rg * nks;
    const int64_t nx = it + nwaves;
    u32x4 gn[4], upn[4];
    if (nx < items) {  // uniform
      const int64_t nrg = nx / nks;
      tiled_load(x, M, K, ldx, nx - nrg * nks, nrg, gn);
      tiled_load(x + K, M, K, ldx, nx - nrg * nks, nrg, upn);
    }
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = swiglu8_tab(stab, g[u], up[u]);
    tiled_code<0, SPM, WRITE_MASK>(v, M, K, Mp, Kp, ks, rg, bcodes, bscales, rcodes, rscales, mask, tile[wv][0],
                                   tile[wv][1]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      g[u] = gn[u];
      up[u] = upn[u];
    }
  }
}

// fp64 value of another lane through a DPP pattern (both halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}

// RMS normalization and preparation in one read of X (tiled output).  A work-group owns
// R whole rows; L = 64/R lanes share a row, lane p of a row covering, in each step of
// 32L elements, the four consecutive 32-element blocks 4(p/4)..4(p/4)+3, elements
// 8(p%4)..8(p%4)+7 of each: a quad of lanes per block, as the codec wants, and the four
// scale bytes of one tiled scale word in one lane.  Wave w holds steps [w*KS, w*KS+KS)
// of the rows in registers.  The row's sum of squares is evaluated in the defined order
// (runs of 8 in index order, then a balanced tree over the run index): run
// c = 4L*step + 16(p/4) + 4u + p%4 of the row is lane p's block u, so the tree's two
// lowest levels are xor exchanges over p%4, the next two the lane's blocks u, then xor
// exchanges over p/4, then the lane's steps (KS a power of two: each wave's steps are an
// aligned power-of-two range of runs), and the top levels combine the waves' sums,
// zero-padded to 16.  The factor r, the gain and the codec then work from the same
// registers.  At one step per wave the kernel is held to 64 registers (8 waves per SIMD).
template <int R, int SPM, int KS, bool WRITE_MASK>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(KS == 1 ? 8 : 1, 8))) void prep_mx_rms_tiled_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int64_t Mp, int64_t Kp,
    const uint16_t* __restrict__ gamma, double eps, uint8_t* __restrict__ bcodes, uint8_t* __restrict__ bscales,
    uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales, uint8_t* __restrict__ mask) {
  constexpr int L = 64 / R;
  static_assert(R == 4 || R == 8 || R == 16, "rows per group");
  __shared__ double part[16][R];  // [wave][row]: each wave's share of the row sums
  __shared__ float rfac[R];
  extern __shared__ uint32_t tiles[];  // per wave: staging of the code stores, 2 x 64 slots of 16 B
  const int lane = threadIdx.x & 63;
  const int j = lane / L, p = lane % L;
  const int q = p & 3, g4 = p >> 2;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = (int)(blockDim.x >> 6);
  const int64_t r0 = (int64_t)blockIdx.x * R;  // first row of the group (uniform)
  const int64_t r = r0 + j;
  const int64_t nbk = K / 32, nbp = Kp / 32;
  const bool row_ok = r < M;
  // the group and the wave's steps wholly inside X (uniform): nothing to zero
  const bool interior = r0 + R <= M && ((int64_t)wave * KS + KS) * L <= nbk;

  // every load of X in flight first.  Loads are unconditional, from clamped (in-bounds)
  // addresses, and what lies outside X is zeroed afterwards: a load under a branch would
  // have to complete before the branch joins.  Addresses are a uniform base and a 32-bit
  // lane offset.  The gains are loaded per block in the coding loop (L2 hits shared by
  // every row group): holding them from the start would take 16 more registers.
  u32x4 v[KS][4];
  // rows past M read row M-1: the base is the group's first row clamped the same way,
  // so the lane's row offset is never negative
  const int64_t rb = r0 < M ? r0 : M - 1;
  const uint8_t* xg = reinterpret_cast<const uint8_t*>(x + rb * ldx);
  const uint32_t jc = (uint32_t)((row_ok ? r : M - 1) - rb);
  const uint32_t lane_x = jc * (uint32_t)ldx * 2u + (uint32_t)q * 16u;
  const uint32_t last_blk = (uint32_t)nbk - 1u;
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    const uint32_t ks = (uint32_t)(wave * KS + t);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t bc = min(ks * L + g4 * 4 + u, last_blk);
      v[t][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xg + lane_x + bc * 64u));
    }
  }
  // outside X the value (and, below, the gain) is zeroed: with r finite (rows past M
  // take r = 1), y = (0 r) 0 is +0 there
  if (!interior) {
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (!(row_ok && ((int64_t)wave * KS + t) * L + g4 * 4 + u < nbk)) v[t][u] = u32x4{0u, 0u, 0u, 0u};
  }

  // the row sums in the defined order; the partner lanes of the tree's lane levels are
  // DPP patterns: xor 1 and xor 2 within a quad, then (every quad, then every 8 lanes,
  // holding one value) the half-row and row mirrors
  double st[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    double su[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // a bf16 square is exact in fp64, so a fused multiply-add rounds exactly as the
      // addition of the square would
      const double a0 = (double)__uint_as_float(v[t][u][0] << 16);
      double s = __dmul_rn(a0, a0);
      const double b0 = (double)__uint_as_float(v[t][u][0] & 0xFFFF0000u);
      s = __fma_rn(b0, b0, s);
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        const double a = (double)__uint_as_float(v[t][u][i] << 16);
        const double b = (double)__uint_as_float(v[t][u][i] & 0xFFFF0000u);
        s = __fma_rn(a, a, s);
        s = __fma_rn(b, b, s);
      }
      s = __dadd_rn(s, dpp_f64<0xB1>(s));  // runs (q, q^1): quad_perm [1,0,3,2]
      s = __dadd_rn(s, dpp_f64<0x4E>(s));  // then pairs of those: quad_perm [2,3,0,1]
      su[u] = s;
    }
    double sg = __dadd_rn(__dadd_rn(su[0], su[1]), __dadd_rn(su[2], su[3]));
    if constexpr (L >= 8) sg = __dadd_rn(sg, dpp_f64<0x141>(sg));  // quads (0,1), (2,3): half-row mirror
    if constexpr (L >= 16) sg = __dadd_rn(sg, dpp_f64<0x140>(sg));  // then those pairs: row mirror
    st[t] = sg;
  }
#pragma unroll
  for (int w = KS; w > 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) st[i] = __dadd_rn(st[2 * i], st[2 * i + 1]);
  if (p == 0) part[wave][j] = st[0];
  // the normalization re-extracts the fp32 values from the bf16 pairs: keeping the sum's
  // extraction alive across the barriers would take 32 more registers per step, and at
  // one step per wave the kernel is held to 64 (8 waves per SIMD: every row group of a
  // prefill-sized X resident at once)
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(v[t][u]));
  __syncthreads();
  if (threadIdx.x < R) {
    double s[16];
#pragma unroll
    for (int w = 0; w < 16; ++w) s[w] = w < W ? part[w][threadIdx.x] : 0.0;
#pragma unroll
    for (int n = 16; n > 1; n /= 2)
#pragma unroll
      for (int i = 0; i < n / 2; ++i) s[i] = __dadd_rn(s[2 * i], s[2 * i + 1]);
    rfac[threadIdx.x] = r0 + threadIdx.x < M ? (float)(1.0 / sqrt(s[0] / (double)K + eps)) : 1.0f;
  }
  __syncthreads();
  const float rr = rfac[j];

  // normalize and code each step of the wave
  uint32_t* my = tiles + wave * 512;
  uint32_t* myb = my + 256;
  const int js = lane % R, bs = lane / R;  // the slot this lane stores: row js, block bs of the step
  // fragment (row/32, block/2), half block%2, row%32: 16 B per (row, block)
  uint8_t* rc_g = rcodes + (r0 >> 5) * (Kp / 64) * 1024;
  uint8_t* bc_g = bcodes + (r0 >> 5) * (Kp / 64) * 1024;
  const uint32_t lane_c = (uint32_t)((bs >> 1) * 1024 + (bs & 1) * 512 + (int)((r0 & 31) + js) * 16);
  uint32_t* rs_g = reinterpret_cast<uint32_t*>(rscales) + r0;
  uint32_t* bs_g = reinterpret_cast<uint32_t*>(bscales) + r0;
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    const int64_t ks = (int64_t)wave * KS + t;
    if (ks * L >= nbp) break;  // uniform: the step starts past the padded row
    uint32_t bword = 0, rword = 0;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the previous step's tile reads are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t blk = ks * L + g4 * 4 + u;
      u32x4 g = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(gamma) +
                                                min((uint32_t)blk, last_blk) * 64u + q * 16u);
      if (!interior && !(row_ok && blk < nbk)) g = u32x4{0u, 0u, 0u, 0u};
      // y = bf16(fp32(fp32(x r) g)), as fp32
      float y[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) rms_scale_f2(v[t][u][i], g[i], rr, y[2 * i], y[2 * i + 1]);
      uint32_t keep, bbyte, bpacked, rbyte, rpacked;
      codec_block_f<0, SPM>(y, keep, bbyte, bpacked, rbyte, rpacked);
      const int slot = (g4 * 4 + u) * R + j;
      my[slot * 4 + q] = rpacked;
      myb[slot * 4 + q] = bpacked;
      rword |= rbyte << (8 * u);
      bword |= bbyte << (8 * u);
      if constexpr (WRITE_MASK)
        if (row_ok && blk < nbk) mask[r * (K / 8) + blk * 4 + q] = (uint8_t)keep;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the tile is wave-private: a wave-level wait suffices
    __builtin_amdgcn_wave_barrier();
    if (ks * L + bs < nbp) {
      const uint32_t off = (uint32_t)(ks * L / 2) * 1024u + lane_c;  // ks * L is even
      *reinterpret_cast<u32x4*>(rc_g + off) = reinterpret_cast<const u32x4*>(my)[lane];
      *reinterpret_cast<u32x4*>(bc_g + off) = reinterpret_cast<const u32x4*>(myb)[lane];
    }
    const int64_t word = ks * (L / 4) + g4;  // blocks 4*word .. 4*word+3
    if (q == 0 && word < nbp / 4) {
      const uint32_t wo = (uint32_t)word * (uint32_t)Mp + (uint32_t)j;
      rs_g[wo] = rword;
      bs_g[wo] = bword;
    }
  }
}

template <int R, int SPM, int KS, bool WRITE_MASK>
hipError_t launch_rms_tiled_ks(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                               double eps, uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales,
                               uint8_t* mask, hipStream_t stream) {
  const int64_t Mp = (M + 31) / 32 * 32, Kp = (K + 127) / 128 * 128;
  const int64_t steps = (Kp / 32 + (64 / R) - 1) / (64 / R);
  const int waves = (int)((steps + KS - 1) / KS);
  prep_mx_rms_tiled_kernel<R, SPM, KS, WRITE_MASK>
      <<<dim3((unsigned)(Mp / R)), dim3(64 * waves), (size_t)waves * 2048, stream>>>(
          x, M, K, ldx, Mp, Kp, gamma, eps, bcodes, bscales, rcodes, rscales, mask);
  return hipGetLastError();
}

constexpr int kRmsRows = 4;  // rows per work-group of the one-read kernel

template <int SPM, bool WRITE_MASK>
hipError_t launch_rms_tiled(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma, double eps,
                            uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales, uint8_t* mask,
                            hipStream_t stream) {
  constexpr int64_t span = 32 * (64 / kRmsRows);
  const int64_t steps = ((K + 127) / 128 * 128 + span - 1) / span;
  // the smallest step depth per wave that covers the row with at most 16 waves; a depth
  // of 4 would need more than the 128 registers a lane has at 16 waves per group
  if (steps <= 16)
    return launch_rms_tiled_ks<kRmsRows, SPM, 1, WRITE_MASK>(x, M, K, ldx, gamma, eps, bcodes, bscales, rcodes,
                                                             rscales, mask, stream);
  return launch_rms_tiled_ks<kRmsRows, SPM, 2, WRITE_MASK>(x, M, K, ldx, gamma, eps, bcodes, bscales, rcodes, rscales,
                                                           mask, stream);
}

template <int MODE, int SPM, bool WRITE_MASK, int XF>
hipError_t launch_tiled(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes,
                        uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales, uint8_t* mask, Norm nm,
                        hipStream_t stream) {
  const int64_t Mp = (M + 31) / 32 * 32, Kp = (K + 127) / 128 * 128;
  const int64_t nks = Kp / 128, nrg = Mp / 16;
  if (nks == 0 || nrg == 0) return hipSuccess;
  if constexpr (XF == kXfSwiglu) {
    static_assert(MODE == 0, "SwiGLU is folded into the SharQ preparation only");
    const int64_t waves = nks * nrg;
    const int64_t groups = (waves + kSwigluThreads / 64 - 1) / (kSwigluThreads / 64);
    const unsigned grid = (unsigned)(groups < kSwigluGroups ? groups : kSwigluGroups);
    prep_mx_tiled_swiglu_kernel<SPM, WRITE_MASK><<<dim3(grid), dim3(kSwigluThreads), 0, stream>>>(
        x, M, K, ldx, Mp, Kp, bcodes, bscales, rcodes, rscales, mask);
    return hipGetLastError();
  } else {
    const int64_t gx = (nks + kThreads / 64 - 1) / (kThreads / 64);
    constexpr int64_t kMaxGridY = 65535;
    for (int64_t rg0 = 0; rg0 < nrg; rg0 += kMaxGridY) {
      const int64_t gy = nrg - rg0 < kMaxGridY ? nrg - rg0 : kMaxGridY;
      prep_mx_tiled_kernel<MODE, SPM, WRITE_MASK, XF><<<dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, stream>>>(
          x, M, K, ldx, Mp, Kp, rg0, bcodes, bscales, rcodes, rscales, mask, nm);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
}

template <int MODE, int SPM, bool WRITE_MASK, int XF>
hipError_t launch_dense_or_strided(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes,
                                   uint8_t* rscales, uint8_t* mask, Norm nm, hipStream_t stream) {
  const int64_t nbk = K / 32;
  const int64_t nblocks = M * nbk;
  if (nblocks == 0) return hipSuccess;
  const int64_t per_wg = (kThreads / 64) * kBlocksPerWave * kUnroll;
  const int64_t grid = (nblocks + per_wg - 1) / per_wg;
  if (ldx == K)
    prep_mx_kernel<MODE, SPM, true, WRITE_MASK, XF><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        x, ldx, nbk, nblocks, bcodes, bscales, rcodes, rscales, mask, nm);
  else
    prep_mx_kernel<MODE, SPM, false, WRITE_MASK, XF><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        x, ldx, nbk, nblocks, bcodes, bscales, rcodes, rscales, mask, nm);
  return hipGetLastError();
}


// Dispatch over the compile-time variants: pattern, mask output, normalization, layout.
template <int MODE, int SPM, bool WRITE_MASK, int XF>
hipError_t prep_variant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes, uint8_t* bscales,
                        uint8_t* rcodes, uint8_t* rscales, uint8_t* mask, Norm nm, int tiled, hipStream_t stream) {
  if (tiled)
    return launch_tiled<MODE, SPM, WRITE_MASK, XF>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, stream);
  return launch_dense_or_strided<MODE, SPM, WRITE_MASK, XF>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask,
                                                              nm, stream);
}

// The ablations (MODEs 2-4), without normalization.
template <int SPM>
hipError_t prep_ablation(int variant, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes,
                         uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales, uint8_t* mask, int tiled,
                         hipStream_t stream) {
  const Norm none{nullptr, nullptr};
  switch (variant) {
    case SHARQ_ABLATE_RESIDUAL_UNQUANTIZED:
      return mask ? prep_variant<2, SPM, true, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, none, tiled, stream)
                  : prep_variant<2, SPM, false, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, none, tiled, stream);
    case SHARQ_ABLATE_STATIC_MASK:
      return mask ? prep_variant<3, SPM, true, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, none, tiled, stream)
                  : prep_variant<3, SPM, false, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, none, tiled, stream);
    default:  // SHARQ_ABLATE_NO_RESIDUAL
      return mask ? prep_variant<4, SPM, true, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, none, tiled, stream)
                  : prep_variant<4, SPM, false, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, none, tiled, stream);
  }
}

template <int SPM>
hipError_t prep_pattern(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* bcodes, uint8_t* bscales,
                        uint8_t* rcodes, uint8_t* rscales, uint8_t* mask, Norm nm, int xf, int tiled,
                        hipStream_t stream) {
  if (xf == kXfRms)
    return mask ? prep_variant<0, SPM, true, kXfRms>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, tiled, stream)
                : prep_variant<0, SPM, false, kXfRms>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, tiled, stream);
  if (xf == kXfSwiglu)
    return mask ? prep_variant<0, SPM, true, kXfSwiglu>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, tiled, stream)
                : prep_variant<0, SPM, false, kXfSwiglu>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, tiled, stream);
  return mask ? prep_variant<0, SPM, true, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, tiled, stream)
              : prep_variant<0, SPM, false, kXfNone>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, tiled, stream);
}

}  // namespace

hipError_t launch_prep_mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                          uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales,
                          uint8_t* mask, const float* rnorm, const uint16_t* gamma, int swiglu, int tiled,
                          hipStream_t stream) {
  (void)sp_n;  // n = m/2 for both supported patterns
  const Norm nm{rnorm, gamma};
  const int xf = swiglu ? kXfSwiglu : rnorm ? kXfRms : kXfNone;
  if (sp_m == 4) return prep_pattern<4>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, xf, tiled, stream);
  return prep_pattern<8>(x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, nm, xf, tiled, stream);
}

bool prep_mx_rms_one_read(int64_t M, int64_t K, int64_t ldx) {
  constexpr int64_t span = 32 * (64 / kRmsRows);  // elements per wave step
  // rows that fit the group's registers; 32-bit lane offsets into X and the scale words
  return M > 0 && ((K + 127) / 128 * 128 + span - 1) / span <= 32 && kRmsRows * ldx * 2 < ((int64_t)1 << 31) &&
         M < ((int64_t)1 << 26);
}

hipError_t launch_prep_mx_rms_tiled(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                    float eps, int sp_m, uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes,
                                    uint8_t* rscales, uint8_t* mask, hipStream_t stream) {
  if (sp_m == 4)
    return mask ? launch_rms_tiled<4, true>(x, M, K, ldx, gamma, (double)eps, bcodes, bscales, rcodes, rscales, mask,
                                            stream)
                : launch_rms_tiled<4, false>(x, M, K, ldx, gamma, (double)eps, bcodes, bscales, rcodes, rscales, mask,
                                             stream);
  return mask ? launch_rms_tiled<8, true>(x, M, K, ldx, gamma, (double)eps, bcodes, bscales, rcodes, rscales, mask,
                                          stream)
              : launch_rms_tiled<8, false>(x, M, K, ldx, gamma, (double)eps, bcodes, bscales, rcodes, rscales, mask,
                                           stream);
}

hipError_t launch_prep_mx_ablation(int variant, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_m,
                                   uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales,
                                   uint8_t* mask, int tiled, hipStream_t stream) {
  if (sp_m == 4) return prep_ablation<4>(variant, x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, tiled, stream);
  return prep_ablation<8>(variant, x, M, K, ldx, bcodes, bscales, rcodes, rscales, mask, tiled, stream);
}

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, int tiled, hipStream_t stream) {
  const Norm none{nullptr, nullptr};
  if (tiled)
    return launch_tiled<1, 4, false, kXfNone>(x, rows, K, ldx, nullptr, nullptr, codes, scales, nullptr, none, stream);
  return launch_dense_or_strided<1, 4, false, kXfNone>(x, rows, K, ldx, nullptr, nullptr, codes, scales, nullptr, none,
                                                     stream);
}

}  // namespace sharq
