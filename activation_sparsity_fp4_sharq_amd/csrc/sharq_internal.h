// sharq_internal.h -- declarations shared by the HIP sources of libsharq (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sharq.h"

namespace sharq {

// Launchers: each validates nothing (the C ABI layer does), enqueues its kernels on
// `stream` and returns hipGetLastError().
// `tiled` selects the output layout (SHARQ_LAYOUT_TILED when non-zero).
// rnorm / gamma: optional RMS normalization folded into the preparation (both NULL
// for none): per-row factors r[M] (from launch_row_rms) and per-channel bf16 gains g[K].
// swiglu != 0: the preparation's input is SwiGLU(gate, up) of x's rows, gate in
// columns [0, K) and up in [K, 2K) (ldx >= 2K).
hipError_t launch_prep_mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_n,
                          int sp_m, uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes,
                          uint8_t* rscales, uint8_t* mask, const float* rnorm, const uint16_t* gamma,
                          int swiglu, int tiled, hipStream_t stream);
// RMS normalization and MXFP4 preparation in one read of X, tiled output, for the row
// lengths whose rows fit one work-group's registers (prep_mx_rms_one_read tells).
bool prep_mx_rms_one_read(int64_t M, int64_t K, int64_t ldx);
hipError_t launch_prep_mx_rms_tiled(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                                    float eps, int sp_m, uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes,
                                    uint8_t* rscales, uint8_t* mask, hipStream_t stream);
// The ablation variants of the preparation (sharq_ablation), without normalization.
hipError_t launch_prep_mx_ablation(int variant, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_m,
                                   uint8_t* bcodes, uint8_t* bscales, uint8_t* rcodes, uint8_t* rscales,
                                   uint8_t* mask, int tiled, hipStream_t stream);
hipError_t launch_prep_nv_ablation(int variant, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_m,
                                   uint8_t* bcodes, uint8_t* bscales, float* btscale, uint8_t* rcodes,
                                   uint8_t* rscales, float* rtscale, uint8_t* mask, uint32_t* work,
                                   hipStream_t stream);
// fp32 values of a payload (row-major or tiled MXFP4; row-major NVFP4).
hipError_t launch_dequantize(const sharq_fp4& p, int64_t rows, int64_t K, int fmt, float* out, int64_t ldo,
                             hipStream_t stream);
hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, int tiled, hipStream_t stream);
hipError_t launch_convert_mx(const sharq_fp4& src, const sharq_fp4& dst, int64_t rows, int64_t K,
                             hipStream_t stream);

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

hipError_t launch_prep_nv(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_n,
                          int sp_m, uint8_t* bcodes, uint8_t* bscales, float* btscale,
                          uint8_t* rcodes, uint8_t* rscales, float* rtscale, uint8_t* mask,
                          uint32_t* work, const float* rnorm, const uint16_t* gamma, int swiglu,
                          hipStream_t stream);
// r_out[i] = fp32(1 / sqrt(sum_k x_ik^2 / K + eps)) for the M rows of x.
hipError_t launch_row_rms(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float eps, float* r_out,
                          hipStream_t stream);
hipError_t launch_quant_nv(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, float* tscale, uint32_t* work,
                           hipStream_t stream);

// Linear launchers: b == NULL runs one activation operand (Y = R W^T, the backbone path off).
hipError_t launch_linear_mx(const sharq_fp4* b, const sharq_fp4& r, int64_t M, const sharq_fp4& w,
                            int64_t N, int64_t K, void* y, int64_t ldy, int out_fp32,
                            void* work, size_t work_bytes, hipStream_t stream);
size_t linear_mx_workspace(int64_t M, int64_t N, int64_t K);
// Workspace bytes that let the tiled MXFP4 GEMM split K (0 when the shape does not split).
size_t linear_mx_split_workspace(int64_t M, int64_t N, int64_t K);

hipError_t launch_linear_nv(const sharq_fp4* b, const sharq_fp4& r, int64_t M, const sharq_fp4& w,
                            int64_t N, int64_t K, void* y, int64_t ldy, int out_fp32,
                            void* work, size_t work_bytes, hipStream_t stream);
size_t linear_nv_workspace(int64_t M, int64_t N, int64_t K);

// Shader-clock probe: out[0] = shader cycles, out[1] = 100 MHz ticks over one wave's
// loop of `iters` x 4 FP4 matrix instructions while every CU runs the same loop.
hipError_t launch_clock_probe(int64_t iters, uint64_t* out, hipStream_t stream);
hipError_t launch_matrix_rate_probe(int form, int64_t iters, uint64_t* out, hipStream_t stream);
hipError_t launch_rounding_probe(uint64_t* out, hipStream_t stream);
hipError_t launch_e4m3_probe(uint64_t* out, hipStream_t stream);
hipError_t launch_stream_probe(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                               hipStream_t stream);

constexpr size_t kNvPrepWorkspace = 16448;  // 16 + 2 * 2048 dwords: maxima and partials
static_assert(SHARQ_NOALLOC_SCRATCH_BYTES >= kNvPrepWorkspace, "the fixed scratch must cover the preparation");
constexpr int kMaxDevices = 64;

}  // namespace sharq
