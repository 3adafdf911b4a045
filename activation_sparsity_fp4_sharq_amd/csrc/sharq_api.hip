// sharq_api.hip -- the C ABI of libsharq (declared in include/sharq.h): argument
// validation, workspace sizing and dispatch to the gfx950 kernels.  Every check
// runs before anything is enqueued; no exception crosses the ABI.
#include <string.h>

#include <atomic>
#include <mutex>

#include "sharq_internal.h"

using namespace sharq;

// Scratch of sharq_forward_noalloc: file-scope device memory, one copy per GPU the
// library runs on, held until the process ends.  Host code never uses this name as an
// address: each device's copy is resolved once with hipGetSymbolAddress (below).
static __device__ __align__(256) uint8_t scratch[SHARQ_NOALLOC_SCRATCH_BYTES];

namespace {

// The device address of `scratch` on the current device (nullptr if it cannot be
// resolved).  Resolved once per device, with that device current; later calls read
// the cached address.
void* scratch_address(int dev) {
  static std::atomic<void*> cached[kMaxDevices];
  static std::mutex lock;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> guard(lock);
  p = cached[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error for the caller's next call
      return nullptr;
    }
    cached[dev].store(p, std::memory_order_release);
  }
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The tiled GEMM addresses a row tile's whole K range with 32-bit buffer offsets.
constexpr int64_t kMaxTiledGemmK = (int64_t)1 << 27;

int block_of(int fmt) { return fmt == SHARQ_MXFP4 ? 32 : 16; }

sharq_status check_format(int fmt) {
  return (fmt == SHARQ_MXFP4 || fmt == SHARQ_NVFP4) ? SHARQ_OK : SHARQ_E_FORMAT;
}

sharq_status check_pattern(int n, int m) {
  return ((n == 2 && m == 4) || (n == 4 && m == 8)) ? SHARQ_OK : SHARQ_E_PATTERN;
}

// A payload of `rows` rows; an empty one (rows == 0) may have NULL codes and scales,
// but an NVFP4 tensor scale is always written or read, so it must exist.
sharq_status check_payload(const sharq_fp4* p, int fmt, int64_t rows) {
  if (!p) return SHARQ_E_NULL;
  if (p->reserved != 0) return SHARQ_E_FORMAT;
  if (p->layout != SHARQ_LAYOUT_ROWMAJOR && p->layout != SHARQ_LAYOUT_TILED) return SHARQ_E_FORMAT;
  if (p->layout == SHARQ_LAYOUT_TILED && fmt != SHARQ_MXFP4) return SHARQ_E_FORMAT;
  if (rows > 0 && (!p->codes || !p->scales)) return SHARQ_E_NULL;
  if (fmt == SHARQ_NVFP4 && !p->tensor_scale) return SHARQ_E_NULL;
  if (!aligned16(p->codes) || !aligned16(p->scales)) return SHARQ_E_ALIGN;
  if (fmt == SHARQ_NVFP4 && (reinterpret_cast<uintptr_t>(p->tensor_scale) & 3u)) return SHARQ_E_ALIGN;
  return SHARQ_OK;
}

// The activation / bf16-input checks shared by sharq_prep and sharq_quantize.
sharq_status check_input(const void* x, int64_t rows, int64_t K, int64_t ldx, int fmt) {
  sharq_status s = check_format(fmt);
  if (s != SHARQ_OK) return s;
  if (rows < 0 || K <= 0 || K % block_of(fmt) || ldx < K) return SHARQ_E_SHAPE;
  if (rows > (int64_t)1 << 31 || K > (int64_t)1 << 30) return SHARQ_E_SHAPE;
  if (rows > 0 && !x) return SHARQ_E_NULL;
  if (x && (!aligned16(x) || ldx % 8)) return SHARQ_E_ALIGN;
  return SHARQ_OK;
}

sharq_status check_device() {
  static thread_local int cached_dev = -1;
  static thread_local bool cached_ok = false;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SHARQ_E_DEVICE;
  if (dev != cached_dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SHARQ_E_DEVICE;
    cached_ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    cached_dev = dev;
  }
  return cached_ok ? SHARQ_OK : SHARQ_E_DEVICE;
}

sharq_status launched(hipError_t e) { return e == hipSuccess ? SHARQ_OK : SHARQ_E_LAUNCH; }

// The preparation's launch for either format, optionally with the RMS normalization
// folded in (rnorm / gamma non-NULL).  Arguments were validated by the caller.
hipError_t enqueue_prep(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m, int fmt,
                        const sharq_fp4* backbone, const sharq_fp4* residual, uint8_t* mask_bits, void* workspace,
                        const float* rnorm, const uint16_t* gamma, int swiglu, hipStream_t st) {
  if (fmt == SHARQ_MXFP4)
    return launch_prep_mx(x, M, K, ldx, sp_n, sp_m, backbone->codes, backbone->scales, residual->codes,
                          residual->scales, mask_bits, rnorm, gamma, swiglu, backbone->layout == SHARQ_LAYOUT_TILED,
                          st);
  return launch_prep_nv(x, M, K, ldx, sp_n, sp_m, backbone->codes, backbone->scales, backbone->tensor_scale,
                        residual->codes, residual->scales, residual->tensor_scale, mask_bits,
                        reinterpret_cast<uint32_t*>(workspace), rnorm, gamma, swiglu, st);
}

// The row factors of sharq_prep_rmsnorm follow the format's own preparation workspace.
size_t rms_factor_offset(int fmt) { return fmt == SHARQ_NVFP4 ? round_up(kNvPrepWorkspace, 256) : 0; }

}  // namespace

// Every check of sharq_forward (both halves), before anything is enqueued; *need receives
// the workspace both halves need.
static sharq_status check_forward(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m, int fmt,
                                  const sharq_fp4* backbone, const sharq_fp4* residual, const sharq_fp4* weight,
                                  int64_t N, void* y, int64_t ldy, int out_dtype, size_t* need) {
  sharq_status s = check_input(x, M, K, ldx, fmt);
  if (s != SHARQ_OK) return s;
  if ((s = check_pattern(sp_n, sp_m)) != SHARQ_OK) return s;
  if (out_dtype != SHARQ_OUT_BF16 && out_dtype != SHARQ_OUT_FP32) return SHARQ_E_FORMAT;
  if (N <= 0 || ldy < N || N > (int64_t)1 << 30) return SHARQ_E_SHAPE;
  if ((s = check_payload(backbone, fmt, M)) != SHARQ_OK) return s;
  if ((s = check_payload(residual, fmt, M)) != SHARQ_OK) return s;
  if ((s = check_payload(weight, fmt, N)) != SHARQ_OK) return s;
  if (backbone->layout != residual->layout || backbone->layout != weight->layout) return SHARQ_E_FORMAT;
  if (backbone->layout == SHARQ_LAYOUT_TILED && K > kMaxTiledGemmK) return SHARQ_E_SHAPE;
  if (M > 0 && !y) return SHARQ_E_NULL;
  if (reinterpret_cast<uintptr_t>(y) & (out_dtype == SHARQ_OUT_FP32 ? 3u : 1u)) return SHARQ_E_ALIGN;
  const size_t np = sharq_prep_workspace_bytes(M, K, fmt);
  const size_t nl = sharq_linear_workspace_bytes(M, N, K, fmt);
  *need = np > nl ? np : nl;
  return SHARQ_OK;
}

// Shared by sharq_linear (backbone != NULL) and sharq_linear_dense (backbone == NULL:
// one activation payload, passed as `residual`).
static sharq_status linear_common(const sharq_fp4* backbone, const sharq_fp4* residual, int64_t M,
                           const sharq_fp4* weight, int64_t N, int64_t K, int fmt, void* y, int64_t ldy,
                           int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  sharq_status s = check_format(fmt);
  if (s != SHARQ_OK) return s;
  if (out_dtype != SHARQ_OUT_BF16 && out_dtype != SHARQ_OUT_FP32) return SHARQ_E_FORMAT;
  if (M < 0 || N <= 0 || K <= 0 || K % block_of(fmt) || ldy < N) return SHARQ_E_SHAPE;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30) return SHARQ_E_SHAPE;
  if ((s = check_payload(weight, fmt, N)) != SHARQ_OK) return s;
  if (backbone && (s = check_payload(backbone, fmt, M)) != SHARQ_OK) return s;
  if ((s = check_payload(residual, fmt, M)) != SHARQ_OK) return s;
  if (residual->layout != weight->layout || (backbone && backbone->layout != residual->layout))
    return SHARQ_E_FORMAT;
  if (residual->layout == SHARQ_LAYOUT_TILED && K > kMaxTiledGemmK) return SHARQ_E_SHAPE;
  if (M > 0) {
    if (!y) return SHARQ_E_NULL;
    if (reinterpret_cast<uintptr_t>(y) & (out_dtype == SHARQ_OUT_FP32 ? 3u : 1u)) return SHARQ_E_ALIGN;
  }
  const size_t need = sharq_linear_workspace_bytes(M, N, K, fmt);
  if (need && (!workspace || workspace_bytes < need)) return SHARQ_E_WORKSPACE;
  if (need && !aligned16(workspace)) return SHARQ_E_ALIGN;
  if ((s = check_device()) != SHARQ_OK) return s;
  if (M == 0) return SHARQ_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int f32 = out_dtype == SHARQ_OUT_FP32;
  if (fmt == SHARQ_MXFP4)
    return launched(launch_linear_mx(backbone, *residual, M, *weight, N, K, y, ldy, f32, workspace,
                                     workspace_bytes, st));
  return launched(launch_linear_nv(backbone, *residual, M, *weight, N, K, y, ldy, f32, workspace,
                                   workspace_bytes, st));
}

extern "C" {

int sharq_abi_version(void) { return SHARQ_ABI_VERSION; }

const char* sharq_status_str(int status) {
  switch (status) {
    case SHARQ_OK: return "ok";
    case SHARQ_E_NULL: return "required pointer is NULL";
    case SHARQ_E_SHAPE: return "invalid shape (size, block multiple or leading dimension)";
    case SHARQ_E_PATTERN: return "unsupported N:M pattern (2:4 and 4:8 are supported)";
    case SHARQ_E_FORMAT: return "unknown block format or output dtype";
    case SHARQ_E_ALIGN: return "pointer or leading dimension misaligned";
    case SHARQ_E_WORKSPACE: return "workspace missing or too small";
    case SHARQ_E_LAUNCH: return "kernel launch failed";
    case SHARQ_E_DEVICE: return "current device is not a gfx950";
    default: return "unknown status";
  }
}

size_t sharq_payload_bytes(int64_t rows, int64_t K, int fmt, int layout, size_t* codes_bytes,
                           size_t* scales_bytes) {
  if (check_format(fmt) != SHARQ_OK || rows < 0 || K <= 0 || K % block_of(fmt)) return 0;
  if (layout != SHARQ_LAYOUT_ROWMAJOR && layout != SHARQ_LAYOUT_TILED) return 0;
  if (layout == SHARQ_LAYOUT_TILED && fmt != SHARQ_MXFP4) return 0;
  size_t c, sc;
  if (layout == SHARQ_LAYOUT_TILED) {
    const int64_t Rp = round_up(rows, 32), Kp = round_up(K, 128);
    c = (size_t)(Rp * Kp / 2);
    sc = (size_t)(Rp * Kp / 32);
  } else {
    c = (size_t)(rows * K / 2);
    sc = (size_t)(rows * K / block_of(fmt));
  }
  if (codes_bytes) *codes_bytes = c;
  if (scales_bytes) *scales_bytes = sc;
  return c + sc;
}

sharq_status sharq_convert_layout(const sharq_fp4* src, const sharq_fp4* dst, int64_t rows, int64_t K, int fmt,
                                  void* stream) {
  sharq_status s = check_format(fmt);
  if (s != SHARQ_OK) return s;
  if (fmt != SHARQ_MXFP4) return SHARQ_E_FORMAT;
  if (rows < 0 || K <= 0 || K % 32 || rows > (int64_t)1 << 31 || K > (int64_t)1 << 30) return SHARQ_E_SHAPE;
  if ((s = check_payload(src, fmt, rows)) != SHARQ_OK) return s;
  if ((s = check_payload(dst, fmt, rows)) != SHARQ_OK) return s;
  if ((s = check_device()) != SHARQ_OK) return s;
  return launched(launch_convert_mx(*src, *dst, rows, K, reinterpret_cast<hipStream_t>(stream)));
}

size_t sharq_prep_workspace_bytes(int64_t, int64_t, int fmt) {
  return fmt == SHARQ_NVFP4 ? kNvPrepWorkspace : 0;
}

size_t sharq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return fmt == SHARQ_NVFP4 ? linear_nv_workspace(M, N, K) : linear_mx_workspace(M, N, K);
}

size_t sharq_linear_split_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt) {
  if (M <= 0 || N <= 0 || K <= 0 || fmt != SHARQ_MXFP4) return 0;
  return linear_mx_split_workspace(M, N, K);
}

sharq_status sharq_quantize(const void* x, int64_t rows, int64_t K, int64_t ldx, int fmt,
                            const sharq_fp4* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  sharq_status s = check_input(x, rows, K, ldx, fmt);
  if (s != SHARQ_OK) return s;
  if ((s = check_payload(out, fmt, rows)) != SHARQ_OK) return s;
  const size_t need = sharq_prep_workspace_bytes(rows, K, fmt);
  if (need && (!workspace || workspace_bytes < need)) return SHARQ_E_WORKSPACE;
  if (need && !aligned16(workspace)) return SHARQ_E_ALIGN;
  if ((s = check_device()) != SHARQ_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  if (fmt == SHARQ_MXFP4)
    return launched(launch_quant_mx(xb, rows, K, ldx, out->codes, out->scales,
                                    out->layout == SHARQ_LAYOUT_TILED, st));
  return launched(launch_quant_nv(xb, rows, K, ldx, out->codes, out->scales, out->tensor_scale,
                                  reinterpret_cast<uint32_t*>(workspace), st));
}

sharq_status sharq_prep(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m, int fmt,
                        const sharq_fp4* backbone, const sharq_fp4* residual, uint8_t* mask_bits,
                        void* workspace, size_t workspace_bytes, void* stream) {
  sharq_status s = check_input(x, M, K, ldx, fmt);
  if (s != SHARQ_OK) return s;
  if ((s = check_pattern(sp_n, sp_m)) != SHARQ_OK) return s;
  if ((s = check_payload(backbone, fmt, M)) != SHARQ_OK) return s;
  if ((s = check_payload(residual, fmt, M)) != SHARQ_OK) return s;
  if (backbone->layout != residual->layout) return SHARQ_E_FORMAT;
  if (mask_bits && (reinterpret_cast<uintptr_t>(mask_bits) & 3u)) return SHARQ_E_ALIGN;
  const size_t need = sharq_prep_workspace_bytes(M, K, fmt);
  if (need && (!workspace || workspace_bytes < need)) return SHARQ_E_WORKSPACE;
  if (need && !aligned16(workspace)) return SHARQ_E_ALIGN;
  if ((s = check_device()) != SHARQ_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  return launched(enqueue_prep(xb, M, K, ldx, sp_n, sp_m, fmt, backbone, residual, mask_bits, workspace, nullptr,
                               nullptr, 0, st));
}

sharq_status sharq_prep_swiglu(const void* gate_up, int64_t M, int64_t I, int64_t ld, int sp_n, int sp_m, int fmt,
                               const sharq_fp4* backbone, const sharq_fp4* residual, uint8_t* mask_bits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  sharq_status s = check_input(gate_up, M, I, ld, fmt);
  if (s != SHARQ_OK) return s;
  if (ld < 2 * I) return SHARQ_E_SHAPE;
  if ((s = check_pattern(sp_n, sp_m)) != SHARQ_OK) return s;
  if ((s = check_payload(backbone, fmt, M)) != SHARQ_OK) return s;
  if ((s = check_payload(residual, fmt, M)) != SHARQ_OK) return s;
  if (backbone->layout != residual->layout) return SHARQ_E_FORMAT;
  if (mask_bits && (reinterpret_cast<uintptr_t>(mask_bits) & 3u)) return SHARQ_E_ALIGN;
  const size_t need = sharq_prep_workspace_bytes(M, I, fmt);
  if (need && (!workspace || workspace_bytes < need)) return SHARQ_E_WORKSPACE;
  if (need && !aligned16(workspace)) return SHARQ_E_ALIGN;
  if ((s = check_device()) != SHARQ_OK) return s;
  return launched(enqueue_prep(reinterpret_cast<const uint16_t*>(gate_up), M, I, ld, sp_n, sp_m, fmt, backbone,
                               residual, mask_bits, workspace, nullptr, nullptr, 1,
                               reinterpret_cast<hipStream_t>(stream)));
}

sharq_status sharq_prep_ablation(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m, int fmt,
                                 int variant, const sharq_fp4* backbone, const sharq_fp4* residual,
                                 uint8_t* mask_bits, void* workspace, size_t workspace_bytes, void* stream) {
  sharq_status s = check_input(x, M, K, ldx, fmt);
  if (s != SHARQ_OK) return s;
  if ((s = check_pattern(sp_n, sp_m)) != SHARQ_OK) return s;
  if (variant != SHARQ_ABLATE_RESIDUAL_UNQUANTIZED && variant != SHARQ_ABLATE_STATIC_MASK &&
      variant != SHARQ_ABLATE_NO_RESIDUAL)
    return SHARQ_E_FORMAT;
  if ((s = check_payload(backbone, fmt, M)) != SHARQ_OK) return s;
  if ((s = check_payload(residual, fmt, M)) != SHARQ_OK) return s;
  if (backbone->layout != residual->layout) return SHARQ_E_FORMAT;
  if (mask_bits && (reinterpret_cast<uintptr_t>(mask_bits) & 3u)) return SHARQ_E_ALIGN;
  const size_t need = sharq_prep_workspace_bytes(M, K, fmt);
  if (need && (!workspace || workspace_bytes < need)) return SHARQ_E_WORKSPACE;
  if (need && !aligned16(workspace)) return SHARQ_E_ALIGN;
  if ((s = check_device()) != SHARQ_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  if (fmt == SHARQ_MXFP4)
    return launched(launch_prep_mx_ablation(variant, xb, M, K, ldx, sp_m, backbone->codes, backbone->scales,
                                            residual->codes, residual->scales, mask_bits,
                                            backbone->layout == SHARQ_LAYOUT_TILED, st));
  return launched(launch_prep_nv_ablation(variant, xb, M, K, ldx, sp_m, backbone->codes, backbone->scales,
                                          backbone->tensor_scale, residual->codes, residual->scales,
                                          residual->tensor_scale, mask_bits, reinterpret_cast<uint32_t*>(workspace),
                                          st));
}

sharq_status sharq_dequantize(const sharq_fp4* p, int64_t rows, int64_t K, int fmt, float* out, int64_t ldo,
                              void* stream) {
  sharq_status s = check_format(fmt);
  if (s != SHARQ_OK) return s;
  if (rows < 0 || K <= 0 || K % block_of(fmt) || ldo < K) return SHARQ_E_SHAPE;
  if (rows > (int64_t)1 << 31 || K > (int64_t)1 << 30 || rows * (K / 8) > ((int64_t)1 << 39)) return SHARQ_E_SHAPE;
  if ((s = check_payload(p, fmt, rows)) != SHARQ_OK) return s;
  if (rows > 0 && !out) return SHARQ_E_NULL;
  if (reinterpret_cast<uintptr_t>(out) & 3u) return SHARQ_E_ALIGN;
  if ((s = check_device()) != SHARQ_OK) return s;
  if (rows == 0) return SHARQ_OK;
  return launched(launch_dequantize(*p, rows, K, fmt, out, ldo, reinterpret_cast<hipStream_t>(stream)));
}

size_t sharq_prep_rmsnorm_workspace_bytes(int64_t M, int64_t K, int fmt) {
  if (M < 0) return 0;
  return rms_factor_offset(fmt) + (size_t)round_up(M > 0 ? M : 1, 64) * sizeof(float);
}

sharq_status sharq_prep_rmsnorm(const void* x, int64_t M, int64_t K, int64_t ldx, const void* gamma, float eps,
                                int sp_n, int sp_m, int fmt, const sharq_fp4* backbone, const sharq_fp4* residual,
                                uint8_t* mask_bits, void* workspace, size_t workspace_bytes, void* stream) {
  sharq_status s = check_input(x, M, K, ldx, fmt);
  if (s != SHARQ_OK) return s;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return SHARQ_E_SHAPE;  // negative, NaN or infinite
  if ((s = check_pattern(sp_n, sp_m)) != SHARQ_OK) return s;
  if ((s = check_payload(backbone, fmt, M)) != SHARQ_OK) return s;
  if ((s = check_payload(residual, fmt, M)) != SHARQ_OK) return s;
  if (backbone->layout != residual->layout) return SHARQ_E_FORMAT;
  if (M > 0 && !gamma) return SHARQ_E_NULL;
  if (gamma && !aligned16(gamma)) return SHARQ_E_ALIGN;
  if (mask_bits && (reinterpret_cast<uintptr_t>(mask_bits) & 3u)) return SHARQ_E_ALIGN;
  const size_t need = sharq_prep_rmsnorm_workspace_bytes(M, K, fmt);
  if (!workspace || workspace_bytes < need) return SHARQ_E_WORKSPACE;
  if (!aligned16(workspace)) return SHARQ_E_ALIGN;
  if ((s = check_device()) != SHARQ_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  // MXFP4 to the tiled layout: one read of X (row sums, factors and codec from registers)
  if (fmt == SHARQ_MXFP4 && backbone->layout == SHARQ_LAYOUT_TILED && prep_mx_rms_one_read(M, K, ldx))
    return launched(launch_prep_mx_rms_tiled(xb, M, K, ldx, reinterpret_cast<const uint16_t*>(gamma), eps, sp_m,
                                             backbone->codes, backbone->scales, residual->codes, residual->scales,
                                             mask_bits, st));
  float* rfac = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + rms_factor_offset(fmt));
  hipError_t e = launch_row_rms(xb, M, K, ldx, eps, rfac, st);
  if (e != hipSuccess) return SHARQ_E_LAUNCH;
  return launched(enqueue_prep(xb, M, K, ldx, sp_n, sp_m, fmt, backbone, residual, mask_bits, workspace, rfac,
                               reinterpret_cast<const uint16_t*>(gamma), 0, st));
}

sharq_status sharq_linear(const sharq_fp4* backbone, const sharq_fp4* residual, int64_t M,
                          const sharq_fp4* weight, int64_t N, int64_t K, int fmt, void* y, int64_t ldy,
                          int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!backbone) return SHARQ_E_NULL;  // the one-operand form is sharq_linear_dense
  return linear_common(backbone, residual, M, weight, N, K, fmt, y, ldy, out_dtype, workspace,
                       workspace_bytes, stream);
}

sharq_status sharq_linear_dense(const sharq_fp4* a, int64_t M, const sharq_fp4* weight, int64_t N, int64_t K,
                                int fmt, void* y, int64_t ldy, int out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return linear_common(nullptr, a, M, weight, N, K, fmt, y, ldy, out_dtype, workspace, workspace_bytes,
                       stream);
}

sharq_status sharq_clock_probe(int64_t iters, uint64_t* counters, void* stream) {
  if (!counters) return SHARQ_E_NULL;
  if (iters < 1 || iters > ((int64_t)1 << 40)) return SHARQ_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(counters) & 7u) return SHARQ_E_ALIGN;
  sharq_status s = check_device();
  if (s != SHARQ_OK) return s;
  return launched(launch_clock_probe(iters, counters, reinterpret_cast<hipStream_t>(stream)));
}

sharq_status sharq_matrix_rate_probe(int form, int64_t iters, uint64_t* counters, void* stream) {
  if (form != 0 && form != 1) return SHARQ_E_FORMAT;
  if (!counters) return SHARQ_E_NULL;
  if (iters < 1 || iters > ((int64_t)1 << 40)) return SHARQ_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(counters) & 7u) return SHARQ_E_ALIGN;
  sharq_status s = check_device();
  if (s != SHARQ_OK) return s;
  return launched(launch_matrix_rate_probe(form, iters, counters, reinterpret_cast<hipStream_t>(stream)));
}

sharq_status sharq_stream_probe(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, void* stream) {
  if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 || write_bytes % 16) return SHARQ_E_SHAPE;
  if ((read_bytes > 0 && !src) || (write_bytes > 0 && !dst)) return SHARQ_E_NULL;
  if (!aligned16(src) || !aligned16(dst)) return SHARQ_E_ALIGN;
  if (read_bytes / 16 > ((int64_t)1 << 40) || write_bytes / 16 > ((int64_t)1 << 40)) return SHARQ_E_SHAPE;
  sharq_status s = check_device();
  if (s != SHARQ_OK) return s;
  return launched(launch_stream_probe(src, read_bytes, dst, write_bytes, reinterpret_cast<hipStream_t>(stream)));
}

sharq_status sharq_bf16_rounding_probe(uint64_t* counters, void* stream) {
  if (!counters) return SHARQ_E_NULL;
  if (reinterpret_cast<uintptr_t>(counters) & 7u) return SHARQ_E_ALIGN;
  sharq_status s = check_device();
  if (s != SHARQ_OK) return s;
  return launched(launch_rounding_probe(counters, reinterpret_cast<hipStream_t>(stream)));
}

sharq_status sharq_e4m3_conversion_probe(uint64_t* counters, void* stream) {
  if (!counters) return SHARQ_E_NULL;
  if (reinterpret_cast<uintptr_t>(counters) & 7u) return SHARQ_E_ALIGN;
  sharq_status s = check_device();
  if (s != SHARQ_OK) return s;
  return launched(launch_e4m3_probe(counters, reinterpret_cast<hipStream_t>(stream)));
}

sharq_status sharq_forward(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m, int fmt,
                           const sharq_fp4* backbone, const sharq_fp4* residual, const sharq_fp4* weight,
                           int64_t N, void* y, int64_t ldy, int out_dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  size_t need = 0;
  sharq_status s = check_forward(x, M, K, ldx, sp_n, sp_m, fmt, backbone, residual, weight, N, y, ldy, out_dtype,
                                 &need);
  if (s != SHARQ_OK) return s;
  if (need && (!workspace || workspace_bytes < need)) return SHARQ_E_WORKSPACE;
  if (need && !aligned16(workspace)) return SHARQ_E_ALIGN;
  s = sharq_prep(x, M, K, ldx, sp_n, sp_m, fmt, backbone, residual, nullptr, workspace, workspace_bytes,
                 stream);
  if (s != SHARQ_OK) return s;
  return sharq_linear(backbone, residual, M, weight, N, K, fmt, y, ldy, out_dtype, workspace,
                      workspace_bytes, stream);
}

sharq_status sharq_forward_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx, int sp_n, int sp_m, int fmt,
                                   const sharq_fp4* backbone, const sharq_fp4* residual, const sharq_fp4* weight,
                                   int64_t N, void* y, int64_t ldy, int out_dtype, void* stream) {
  size_t need = 0;
  sharq_status s = check_forward(x, M, K, ldx, sp_n, sp_m, fmt, backbone, residual, weight, N, y, ldy, out_dtype,
                                 &need);
  if (s != SHARQ_OK) return s;
  if (need > SHARQ_NOALLOC_SCRATCH_BYTES) return SHARQ_E_WORKSPACE;  // beyond the fixed scratch
  if ((s = check_device()) != SHARQ_OK) return s;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SHARQ_E_DEVICE;
  void* ws = scratch_address(dev);
  if (!ws) return SHARQ_E_DEVICE;
  return sharq_forward(x, M, K, ldx, sp_n, sp_m, fmt, backbone, residual, weight, N, y, ldy, out_dtype, ws,
                       SHARQ_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
