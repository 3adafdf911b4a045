/*
 * sharq.h -- C ABI of libsharq, the SharQ sparse-dense FP4 linear layer on AMD
 * MI355X (gfx950).
 *
 * The method (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
 * Inference, arXiv 2606.26587; abstract and "Core claim"): for each activation
 * tensor X[M,K], an input-adaptive N:M mask along K keeps the n largest |x| of
 * every m consecutive elements (the outlier-dominated sparse backbone); the
 * backbone is quantized to FP4; a dense residual R = X - dequant(backbone) is
 * formed against the *quantized* backbone and quantized to FP4 with its own
 * block scales; a sparse-backbone FP4 GEMM and a dense-residual FP4 GEMM share
 * one FP4 weight payload and their products are summed:
 *     Y[M,N] = Bhat * What^T + Rhat * What^T.
 * Figure 2 of the pages shows the preparation fused into one kernel ahead of the
 * two GEMMs; here the preparation is sharq_prep and both GEMMs are one kernel,
 * sharq_linear, accumulating into one fp32 tile.
 *
 * Conventions for every entry point
 *  - Pointers marked "device" are HIP device pointers on the current device;
 *    pointers marked "host" are host memory.  The caller owns every buffer.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and is asynchronous.  Nothing is allocated, freed or synchronized.
 *  - Arguments are validated before anything is launched; on error the status
 *    is returned and nothing has been enqueued or written.
 *  - Non-finite inputs are outside the contract: they produce unspecified codes
 *    but never an out-of-bounds access.
 *  - Thread-safe: the only global state is a per-device flag array for the one-time
 *    kernel attribute set-up (atomic) and a per-thread cache of the device check.
 *
 * FP4 payload (struct sharq_fp4) of a [rows, K] tensor.  A code is E2M1: bit 3
 * sign, bits 2..1 exponent (bias 1), bit 0 mantissa; magnitudes 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6.  Within 16 bytes holding 32 consecutive elements, element 2c sits in
 * the low nibble of byte c.  Block scales: MXFP4 one E8M0 byte (2^(byte-127)) per
 * 32 consecutive elements along K; NVFP4 one OCP E4M3 byte (bias 7, max 448) per
 * 16, times one fp32 tensor_scale (device; ignored for MXFP4).
 *
 * Two layouts (field `layout`):
 *  - SHARQ_LAYOUT_ROWMAJOR (both formats): codes [rows, K/2], scales [rows, K/B]
 *    (B = 32 or 16), both row-major and dense.  This is the plain MX/NV layout.
 *  - SHARQ_LAYOUT_TILED (MXFP4 only), the layout the gfx950 FP4 matrix
 *    instruction consumes directly.  Let Rp = rows rounded up to 32 and Kp = K
 *    rounded up to 128; padding holds code 0 and scale byte 0.
 *      codes: 1 KiB fragments, fragment (rt, kc) = rows 32rt..32rt+31, elements
 *        64kc..64kc+63, at byte ((rt * Kp/64) + kc) * 1024; inside it, the 16
 *        bytes of row r's block b (= 2kc + c, c in {0,1}) sit at slot
 *        (r % 32) + 32c, i.e. bytes 16*slot .. 16*slot+15.  Total Rp*Kp/2 bytes.
 *      scales: one 32-bit word per (row, 128-element K-step ks): byte (b % 4) of
 *        word (ks * Rp + r) is the scale of block b = 4ks + (b % 4).  Total
 *        Rp*Kp/32 bytes.
 *    sharq_payload_bytes gives the sizes; sharq_convert_layout converts.
 *  - codes and scales must be 16-byte aligned; an empty payload (0 rows) may
 *    pass NULL codes and scales, but an NVFP4 tensor_scale must always exist.
 */
#ifndef SHARQ_H_
#define SHARQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHARQ_ABI_VERSION 12

typedef enum sharq_status {
  SHARQ_OK = 0,
  SHARQ_E_NULL = 1,      /* a required pointer is NULL                                   */
  SHARQ_E_SHAPE = 2,     /* negative/zero size, K not a multiple of the block, ld < K     */
  SHARQ_E_PATTERN = 3,   /* n:m is not 2:4 or 4:8                                         */
  SHARQ_E_FORMAT = 4,    /* unknown block format or output dtype                          */
  SHARQ_E_ALIGN = 5,     /* pointer or leading dimension not aligned as required          */
  SHARQ_E_WORKSPACE = 6, /* workspace NULL or smaller than the *_workspace_bytes value    */
  SHARQ_E_LAUNCH = 7,    /* a kernel launch failed (hipGetLastError after the launch)     */
  SHARQ_E_DEVICE = 8     /* the current device is not a gfx950                            */
} sharq_status;

typedef enum sharq_format { SHARQ_MXFP4 = 0, SHARQ_NVFP4 = 1 } sharq_format;
typedef enum sharq_out_dtype { SHARQ_OUT_BF16 = 0, SHARQ_OUT_FP32 = 1 } sharq_out_dtype;

typedef enum sharq_layout { SHARQ_LAYOUT_ROWMAJOR = 0, SHARQ_LAYOUT_TILED = 1 } sharq_layout;

typedef struct sharq_fp4 {
  uint8_t* codes;      /* device, see the layouts above                          */
  uint8_t* scales;     /* device, see the layouts above                          */
  float* tensor_scale; /* device, 1 float (NVFP4); unused for MXFP4              */
  int32_t layout;      /* sharq_layout                                           */
  int32_t reserved;    /* must be 0                                              */
} sharq_fp4;

/* Version of this ABI (SHARQ_ABI_VERSION). */
int sharq_abi_version(void);

/* Static text for a status code; never NULL. */
const char* sharq_status_str(int status);

/* Sizes in bytes of the codes and scales arrays of a [rows, K] payload in the given
 * format and layout (writes *codes_bytes and *scales_bytes; either may be NULL).
 * Returns the total, or 0 when the combination is invalid (tiled NVFP4, K not a
 * multiple of the block, negative sizes).  Host-only. */
size_t sharq_payload_bytes(int64_t rows, int64_t K, int fmt, int layout, size_t* codes_bytes,
                           size_t* scales_bytes);

/* Re-lays out an MXFP4 payload [rows, K] from src->layout into dst->layout (row-major
 * <-> tiled; the same layout is a plain copy).  Values are unchanged; the tiled
 * padding is written as zeros.  Asynchronous on `stream`; src and dst must not
 * overlap.  Errors as for the other entry points; tiled NVFP4 is SHARQ_E_FORMAT. */
sharq_status sharq_convert_layout(const sharq_fp4* src, const sharq_fp4* dst, int64_t rows, int64_t K,
                                  int fmt, void* stream);

/* Bytes of device workspace sharq_prep / sharq_quantize need for these sizes
 * (0 for MXFP4; a few hundred bytes for NVFP4, which keeps its two running
 * tensor maxima there).  Host-only, launches nothing. */
size_t sharq_prep_workspace_bytes(int64_t rows, int64_t K, int fmt);

/* Bytes of device workspace sharq_linear needs for these sizes (the split-K
 * partial sums of small-M shapes; 0 when the shape runs without split-K). */
size_t sharq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt);

/* Bytes of workspace that let sharq_linear (and sharq_forward, sharq_linear_dense) split
 * K for these sizes: a tiled MXFP4 product with fewer 256 x 256 output tiles than the GPU
 * has compute units (256) and long rows gives each tile's K-steps to up to 4 work-groups,
 * which store fp32 partial sums [splits][M][N] in the workspace; a second kernel adds
 * them in split order and rounds Y.  0 when the shape does not split (NVFP4, row-major
 * payloads, M <= 32, enough tiles, or fewer than 2 x 2048 columns of K per split).  Any
 * smaller workspace (also none) is accepted: the call then runs unsplit.  A split call
 * sums in a different order than an unsplit one, so the two agree to the fp32 summation
 * bound, not bit for bit; each is deterministic. */
size_t sharq_linear_split_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt);

/* Plain FP4 quantization (no mask, no residual) of a bf16 matrix -- how a weight
 * payload W is produced (the pages quantize the weights once, and both GEMMs of the
 * abstract read that one FP4 weight payload).  Each block is quantized as the residual blocks
 * of sharq_prep are: MXFP4 E8M0 exponent floor(log2 amax) - 2 and E2M1
 * round-to-nearest-even with saturation; NVFP4 with a tensor scale amax/2688.
 *   x       device bf16 [rows, ldx], first K columns used; 16-byte aligned, ldx % 8 == 0
 *   rows    >= 0 (0 enqueues nothing for MXFP4; NVFP4 still writes tensor_scale = 1)
 *   K       > 0, multiple of 32 (MXFP4) or 16 (NVFP4)
 *   out     payload to write (codes, scales, and tensor_scale for NVFP4), in out->layout
 *   workspace / workspace_bytes: >= sharq_prep_workspace_bytes(rows, K, fmt), device
 */
sharq_status sharq_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx, int fmt,
                            const sharq_fp4* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/* The SharQ activation preparation (abstract; "Core claim"; Figure 2's fused
 * preparation kernel; sharq_prep_rmsnorm below adds the layer normalization):
 *   1. mask: in every group of m consecutive elements along K keep the n with the
 *      largest |x| (compared on the bf16 bits with the sign cleared; on equal
 *      magnitude the lower index wins), so exactly n are kept per group;
 *   2. backbone: FP4-quantize X with the dropped positions set to +0 (code 0x0);
 *      the block scale is taken over the kept values;
 *   3. residual: R = X - dequant(backbone), one fp32 subtraction per element;
 *   4. FP4-quantize R over all positions with its own scales (and, for NVFP4, its
 *      own tensor scale amax(R)/2688).
 *   x          device bf16 [M, ldx], first K columns used; 16-byte aligned, ldx % 8 == 0
 *   M          >= 0;  K > 0, multiple of 32 (MXFP4) or 16 (NVFP4)
 *   sp_n:sp_m  2:4 or 4:8
 *   backbone   output payload [M, K] (zero-filled dense: dropped positions hold code 0x0),
 *              in the layout its `layout` field names (tiled is MXFP4 only)
 *   residual   output payload [M, K], likewise
 *   mask_bits  device [M, K/8] or NULL: bit (k % 8) of byte k/8 set when element k is kept
 *   workspace  device, >= sharq_prep_workspace_bytes(M, K, fmt) bytes (NULL allowed when 0)
 * Masks, codes and scale bytes are deterministic and identical for every launch shape. */
sharq_status sharq_prep(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                        int fmt, const sharq_fp4* backbone, const sharq_fp4* residual,
                        uint8_t* mask_bits, void* workspace, size_t workspace_bytes,
                        void* stream);

/* The preparation of an MLP block's down projection with its SwiGLU activation
 * folded in: the input is h = SwiGLU(gate, up), formed from each row's gate and up
 * halves while they are loaded and never stored, then prepared exactly as
 * sharq_prep prepares X (SharQ, arXiv 2606.26587: Figure 2's fused preparation takes
 * over the element-wise work in front of the GEMMs; the benchmark's MLP block
 * workload chains two SharQ layers around it).
 *   h = bf16(fp32(silu(g) * u)), silu(g) = fp32(g / fp32(1 + e)), e = e^-g in fp32
 *   by Cody and Waite's range reduction (t = -g clamped to [-150, 150],
 *   n = rint(t log2 e), r = (t - n ln2_hi) - n ln2_lo with a 15-bit ln2_hi) and the
 *   degree-7 Taylor polynomial of e^r times 2^n -- every operation one fp32
 *   rounding in a fixed order, so h is reproducible bit for bit.  An h that rounds to
 *   an infinity (|silu(g) * u| beyond bf16's range) is outside the contract, as a
 *   non-finite input is.
 *   gate_up  device bf16 [M, ld]: gate in columns [0, I), up in [I, 2I) of each row
 *            (the output of one linear over the concatenated gate and up weights);
 *            16-byte aligned, ld % 8 == 0, ld >= 2I
 *   I        the intermediate size (the down projection's K): > 0, multiple of 32
 *            (MXFP4) or 16 (NVFP4)
 *   other arguments, outputs, workspace (sharq_prep_workspace_bytes(M, I, fmt)) and
 *   errors as for sharq_prep; ld < 2I -> SHARQ_E_SHAPE. */
sharq_status sharq_prep_swiglu(const void* gate_up, int64_t M, int64_t I, int64_t ld, int sp_n, int sp_m,
                               int fmt, const sharq_fp4* backbone, const sharq_fp4* residual,
                               uint8_t* mask_bits, void* workspace, size_t workspace_bytes, void* stream);

/* The ablations of the method's choices named by the pages' review ("What would
 * settle it": the residual against the unquantized sparse values; the referee's
 * third major comment on Table 2 and Section 5.1: a static mask, and direct N:M
 * sparsity on the unquantized activations), as preparation variants:
 *   SHARQ_ABLATE_RESIDUAL_UNQUANTIZED  residual R = X - X*mask (the dropped values
 *                                      only: the backbone's FP4 error is left in)
 *   SHARQ_ABLATE_STATIC_MASK           mask = the first n of every m positions for
 *                                      every row (backbone block scales over the kept
 *                                      values); residual against the dequantized backbone
 *   SHARQ_ABLATE_NO_RESIDUAL           direct N:M + FP4: backbone as sharq_prep, the
 *                                      residual payload all zero (codes 0x0, scale
 *                                      bytes 0, NVFP4 tensor scale 1) */
typedef enum sharq_ablation {
  SHARQ_ABLATE_RESIDUAL_UNQUANTIZED = 1,
  SHARQ_ABLATE_STATIC_MASK = 2,
  SHARQ_ABLATE_NO_RESIDUAL = 3
} sharq_ablation;

/* sharq_prep with one of the ablations above (arguments, layouts, workspace and
 * errors as for sharq_prep; a variant outside the enum -> SHARQ_E_FORMAT).  For
 * measurement and comparison only: the method itself is sharq_prep. */
sharq_status sharq_prep_ablation(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                                 int fmt, int variant, const sharq_fp4* backbone, const sharq_fp4* residual,
                                 uint8_t* mask_bits, void* workspace, size_t workspace_bytes, void* stream);

/* The values an FP4 payload encodes, as fp32: out[i * ldo + k] = E2M1(code) * 2^(E-127)
 * (MXFP4, exact) or E2M1(code) * E4M3(scale) * tensor_scale rounded once to fp32
 * (NVFP4; the first product is exact).  For checking reconstructions (X against
 * Bhat + Rhat).
 *   p        payload [rows, K] in either layout (tiled: MXFP4)
 *   out      device fp32 [rows, ldo], ldo >= K, 4-byte aligned
 * Errors as for sharq_quantize's shape and payload checks; out == NULL with
 * rows > 0 -> SHARQ_E_NULL. */
sharq_status sharq_dequantize(const sharq_fp4* p, int64_t rows, int64_t K, int fmt, float* out, int64_t ldo,
                              void* stream);

/* Bytes of device workspace sharq_prep_rmsnorm needs: the format's preparation
 * workspace plus one fp32 row factor per row (rounded up).  Host-only. */
size_t sharq_prep_rmsnorm_workspace_bytes(int64_t M, int64_t K, int fmt);

/* sharq_prep with the layer normalization folded in, as the pages' fused preparation
 * does ("Core claim"; abstract: the preparation also takes over the layer
 * normalization).  The pages do not spell the normalization out; it is read as RMS
 * normalization with a per-channel gain and no bias, producing the bf16 tensor that
 * the preparation then decomposes:
 *   r_i  = fp32( 1 / sqrt( S_i / K + eps ) )   (mean, sqrt, division in fp64)
 *   y_ik = bf16_rne( fp32( fp32(x_ik * r_i) * gamma_k ) )
 * where S_i, the fp64 sum of the row's squares, is evaluated in one fixed order: each
 * run of 8 consecutive squares added in index order, the run sums added in a balanced
 * binary tree over the run index (zero-padded to a power of two) -- so r_i is a single
 * defined number.  backbone / residual / mask_bits are exactly sharq_prep's outputs for y.
 * MXFP4 to the tiled layout with K <= 16384 reads X once (sums, factors and the
 * preparation from registers); other layouts, NVFP4 and longer rows launch a row-factor
 * kernel first and keep the factors in the workspace.
 *   x, M, K, ldx, sp_n, sp_m, fmt, backbone, residual, mask_bits: as for sharq_prep
 *   gamma      device bf16 [K] gains, 16-byte aligned (may be NULL only when M == 0)
 *   eps        >= 0 and finite, else SHARQ_E_SHAPE (a zero row with eps = 0 gives
 *              r_i = infinity and NaN values)
 *   workspace  device, >= sharq_prep_rmsnorm_workspace_bytes(M, K, fmt) bytes, 16-byte
 *              aligned; holds the row factors (and NVFP4's maxima) of the two-launch form */
sharq_status sharq_prep_rmsnorm(const void* x, int64_t M, int64_t K, int64_t ldx, const void* gamma,
                                float eps, int sp_n, int sp_m, int fmt, const sharq_fp4* backbone,
                                const sharq_fp4* residual, uint8_t* mask_bits, void* workspace,
                                size_t workspace_bytes, void* stream);

/* The two SharQ GEMMs over one weight payload (abstract: a sparse FP4 GEMM for the
 * backbone, a dense FP4 GEMM for the residual, one FP4 weight payload), summed in
 * one fp32 accumulator per output:  Y = Bhat W^T + Rhat W^T.
 *   backbone, residual  payloads [M, K] from sharq_prep (same format)
 *   weight              payload [N, K] (e.g. from sharq_quantize)
 *                       MXFP4 runs its fast pipelined kernel when all three payloads
 *                       are tiled (then K <= 2^27, else SHARQ_E_SHAPE: the kernel addresses
 *                       a row tile's K range with 32-bit offsets); any row-major payload
 *                       takes a slower generic kernel.
 *   y                   device [M, ldy] bf16 (round to nearest even) or fp32; ldy >= N;
 *                       aligned to its element size
 *   workspace           device, >= sharq_linear_workspace_bytes(M, N, K, fmt) bytes; with
 *                       sharq_linear_split_workspace_bytes(...) bytes (16-byte aligned) a
 *                       shape with few output tiles splits K (see there)
 * MXFP4 runs on the gfx950 block-scaled FP4 matrix cores, so every product of two
 * FP4 values and their scales is exact and only the fp32 summation order differs
 * from an exact result.  NVFP4 (E4M3 block scales, which the FP4 matrix cores
 * cannot apply) runs exactly on the fp16 matrix cores. */
sharq_status sharq_linear(const sharq_fp4* backbone, const sharq_fp4* residual, int64_t M,
                          const sharq_fp4* weight, int64_t N, int64_t K, int fmt, void* y,
                          int64_t ldy, int out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Plain FP4 linear layer without SharQ: Y = Ahat W^T over one activation payload
 * (e.g. from sharq_quantize) -- the kernels of sharq_linear with the backbone path
 * off.  It is the plain FP4 baseline the method is measured against (SharQ,
 * arXiv 2606.26587: Figure 4 normalizes prefill latency to plain NVFP4; the
 * summary's speed claims are against FP16 and FP8).
 *   a                   payload [M, K], same format and layout as weight
 *   weight, y, ldy, out_dtype, workspace, stream: as for sharq_linear
 *   NVFP4: Y = S_w (S_a acc) in fp32, each product rounded to nearest.
 * Errors as for sharq_linear (SHARQ_E_NULL for a NULL payload or y). */
sharq_status sharq_linear_dense(const sharq_fp4* a, int64_t M, const sharq_fp4* weight, int64_t N,
                                int64_t K, int fmt, void* y, int64_t ldy, int out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Measurement aid: the shader clock under matrix load.  Every CU runs iters x 4
 * register-only FP4 matrix instructions per wave; counters (device, 8-byte aligned,
 * >= 3 uint64) receive [0] the shader-clock cycles and [1] the 100 MHz reference
 * ticks of one wave's loop (clock = [0] / ([1] / 1e8) Hz) and [2] a value that keeps
 * the loop from being optimized away.  Errors: NULL counters -> SHARQ_E_NULL; iters
 * outside [1, 2^40] -> SHARQ_E_SHAPE; misaligned -> SHARQ_E_ALIGN. */
sharq_status sharq_clock_probe(int64_t iters, uint64_t* counters, void* stream);

/* Measurement aid: the issue rate of the two matrix-instruction forms a sparse FP4
 * backbone can take on gfx950 (the backbone form is chosen by this measurement; the
 * pages' backbone GEMM is sparse, and gfx950 has no sparse FP4 instruction):
 *   form 0  dense block-scaled FP4 32x32x64 (v_mfma_scale_f32_32x32x64_f8f6f4) on a
 *           zero-filled backbone
 *   form 1  2:4-sparse fp8 32x32x64 (v_smfmac_f32_32x32x64_fp8_fp8) on a compressed
 *           backbone (FP4 values are exact in fp8)
 * Both perform 32 x 32 x 64 multiply-adds of the dense operand shape per instruction.
 * Every CU runs 4 waves (one per SIMD) of iters x 8 register-only instructions in eight
 * independent chains; counters (device, 8-byte aligned, >= 3 uint64) receive [0] the
 * shader cycles and [1] the 100 MHz ticks of one wave's loop, [2] a value that keeps
 * the loop alive; cycles per instruction per SIMD = [0] / (iters * 8).  Errors: form not 0/1 -> SHARQ_E_FORMAT,
 * otherwise as for sharq_clock_probe. */
sharq_status sharq_matrix_rate_probe(int form, int64_t iters, uint64_t* counters, void* stream);

/* Measurement aid: the streaming ceiling of a memory pattern like the preparation's --
 * read read_bytes of src (non-temporal 16-byte loads) and write write_bytes of dst
 * (16-byte stores), four chunks per lane, no arithmetic.  Timing it at a preparation's
 * byte counts bounds what that preparation can reach.
 *   src, dst     device, 16-byte aligned (NULL allowed for a zero byte count)
 *   read_bytes, write_bytes  >= 0, multiples of 16, else SHARQ_E_SHAPE
 *   dst's contents afterwards are unspecified. */
sharq_status sharq_stream_probe(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, void* stream);

/* Self-check of the fp32 -> bf16 rounding the one-read normalized preparation uses (the
 * gfx950 packed conversion; reading R9 rounds y to nearest even): converts every fp32
 * bit pattern on the device and compares with round-to-nearest-even done on the bits.
 *   counters  device, 8-byte aligned, >= 2 uint64: [0] receives the number of finite
 *             patterns that differ, [1] the smallest such pattern (2^64 - 1 if none)
 * Errors: SHARQ_E_NULL, SHARQ_E_ALIGN, SHARQ_E_DEVICE, SHARQ_E_LAUNCH. */
sharq_status sharq_bf16_rounding_probe(uint64_t* counters, void* stream);

/* Self-check of the E4M3 conversions the NVFP4 preparation uses for its block scales
 * (the gfx950 fp8 conversions; reading R5 codes each block scale to the nearest E4M3
 * value, ties to the even code, saturating at 448): codes every fp32 pattern with the
 * sign bit clear and decodes every code 0..0x7E on the device, and compares both with
 * the format's definition worked on the bits.
 *   counters  device, 8-byte aligned, >= 2 uint64: [0] receives the number of
 *             mismatches, [1] the smallest mismatching fp32 pattern, or 2^32 + code for a
 *             decode mismatch (2^64 - 1 if none)
 * Errors: SHARQ_E_NULL, SHARQ_E_ALIGN, SHARQ_E_DEVICE, SHARQ_E_LAUNCH. */
sharq_status sharq_e4m3_conversion_probe(uint64_t* counters, void* stream);

/* One SharQ linear layer end to end (SharQ, arXiv 2606.26587: the abstract's
 * decomposition as one layer; Figure 2's dataflow of the fused preparation feeding the
 * sparse-backbone and dense-residual GEMMs over one weight payload): sharq_prep into
 * the caller's backbone and residual payloads, then sharq_linear, on one stream.
 * Arguments as above; the workspace must cover both calls (max of the two
 * *_workspace_bytes values).  Errors: every argument of both calls is validated before
 * the first launch, so on error nothing is enqueued. */
sharq_status sharq_forward(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                           int fmt, const sharq_fp4* backbone, const sharq_fp4* residual,
                           const sharq_fp4* weight, int64_t N, void* y, int64_t ldy,
                           int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): sharq_forward without a workspace
 * argument.  Its scratch (the NVFP4 preparation's partial and tensor maxima) is a fixed
 * array of SHARQ_NOALLOC_SCRATCH_BYTES bytes in the library's own device memory, one
 * copy per GPU, held until the process ends; the first call on a device resolves that
 * device's copy.  Nothing is allocated or freed, by the library or by any library it
 * calls.
 *   Arguments, outputs and errors as for sharq_forward; a shape whose workspace would
 *   exceed the scratch -> SHARQ_E_WORKSPACE (no shape does today: the preparation's
 *   workspace is a constant and the GEMMs need none); the scratch cannot be resolved on
 *   the current device -> SHARQ_E_DEVICE.
 *   Every call on one GPU shares that GPU's scratch, which keeps the last call's
 *   contents (a call writes every scratch word before it reads it): calls that overlap
 *   on one GPU, on any streams, race. */
#define SHARQ_NOALLOC_SCRATCH_BYTES 16640
sharq_status sharq_forward_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m,
                                   int fmt, const sharq_fp4* backbone, const sharq_fp4* residual,
                                   const sharq_fp4* weight, int64_t N, void* y, int64_t ldy, int out_dtype,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_H_ */
