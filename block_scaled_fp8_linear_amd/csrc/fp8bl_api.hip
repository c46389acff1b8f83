// C ABI of the block-scaled FP8 linear library (declared in include/fp8bl.h).
//
// Host-side only: argument validation (done first, before any HIP call),
// the gfx950 gate, path choice and workspace sizing. All device work is in
// the kernel files; nothing here touches tensor data.
#include "fp8bl.h"

#include <atomic>
#include <cstring>
#include <mutex>

#include "fp8bl_internal.h"

#define FP8BL_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxDim = (int64_t)1 << 31;     // every dimension fits int32
constexpr int64_t kMaxElems = (int64_t)1 << 35;   // N*K, M*K and M*N stay below this (8-element chunk index fits uint32)
constexpr int kSkinnyMaxM = 32;
// The GEMM kernels address a tile's rows with 32-bit buffer offsets.
constexpr int64_t kMaxLinearK = (int64_t)1 << 20;
// The large-tile kernel also stores 256 output rows (fp32 partials) through
// one buffer descriptor: 256 * N * 4 bytes must stay below 2^31.
constexpr int64_t kLargeMaxN = (int64_t)1 << 21;

// 0 = unknown, 1 = gfx950, 2 = other.
std::atomic<int> g_arch[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t grid_elems(int64_t n, int64_t k) {
  return (size_t)((n + FP8BL_BLOCK - 1) / FP8BL_BLOCK) * (size_t)((k + FP8BL_BLOCK - 1) / FP8BL_BLOCK);
}

int check_nk(int64_t n, int64_t k) {
  if (n < 0 || k <= 0 || (k % 16) != 0) return FP8BL_INVALID_ARG;
  if (n >= kMaxDim || k >= kMaxDim || (n > 0 && n * k >= kMaxElems)) return FP8BL_INVALID_ARG;
  if ((n + FP8BL_BLOCK - 1) / FP8BL_BLOCK > 65535) return FP8BL_INVALID_ARG;
  return FP8BL_OK;
}

// The current device must be a gfx950; the answer is cached per device.
int gate_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FP8BL_HIP_ERROR;
  if (dev < 0 || dev >= kMaxDevices) return FP8BL_UNSUPPORTED_DEVICE;
  int state = g_arch[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8BL_HIP_ERROR;
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? FP8BL_OK : FP8BL_UNSUPPORTED_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP8BL_OK : FP8BL_HIP_ERROR; }

int validate_linear(const uint16_t* x, const uint8_t* q, const float* s, const uint16_t* y,
                    int64_t m, int64_t n, int64_t k, int path) {
  if (path != FP8BL_PATH_AUTO && path != FP8BL_PATH_TILED && path != FP8BL_PATH_SKINNY &&
      path != FP8BL_PATH_LARGE)
    return FP8BL_INVALID_ARG;
  if (path == FP8BL_PATH_LARGE && n >= kLargeMaxN) return FP8BL_INVALID_ARG;
  if (m < 0 || m >= kMaxDim) return FP8BL_INVALID_ARG;
  int st = check_nk(n, k);
  if (st != FP8BL_OK) return st;
  if (k > kMaxLinearK) return FP8BL_INVALID_ARG;
  if (m > 0 && m * k >= kMaxElems) return FP8BL_INVALID_ARG;
  if (m > 0 && n > 0 && m * n >= kMaxElems) return FP8BL_INVALID_ARG;
  if (m == 0 || n == 0) return FP8BL_OK;
  if (!x || !q || !s || !y) return FP8BL_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(y, 16) || !aligned(s, 4))
    return FP8BL_ALIGNMENT;
  const size_t ybytes = (size_t)m * n * 2;
  if (overlap(y, ybytes, x, (size_t)m * k * 2) || overlap(y, ybytes, q, (size_t)n * k) ||
      overlap(y, ybytes, s, grid_elems(n, k) * 4))
    return FP8BL_INVALID_ARG;
  return FP8BL_OK;
}

size_t x_scale_elems(int64_t m, int64_t k) {
  return (size_t)((k + FP8BL_BLOCK - 1) / FP8BL_BLOCK) * (size_t)m;
}

// The W8A8 GEMMs address the activation scales through a 32-bit buffer
// range: at most 2^32 - 4 bytes of them (reached only with very small K and
// M near 2^31).
bool x_scale_fits(int64_t m, int64_t k) {
  return m <= 0 || k <= 0 || x_scale_elems(m, k) * 4 < ((size_t)1 << 32);
}

// Shape rules of the W8A8 GEMM (as the bf16 linear) plus the operands'
// alignment and the output's overlap with them.
int validate_w8a8(const uint8_t* xq, const float* xs, const uint8_t* q, const float* s,
                  const uint16_t* y, int64_t m, int64_t n, int64_t k) {
  if (m < 0 || m >= kMaxDim) return FP8BL_INVALID_ARG;
  int st = check_nk(n, k);
  if (st != FP8BL_OK) return st;
  if (k > kMaxLinearK) return FP8BL_INVALID_ARG;
  if (m > 0 && m * k >= kMaxElems) return FP8BL_INVALID_ARG;
  if (m > 0 && n > 0 && m * n >= kMaxElems) return FP8BL_INVALID_ARG;
  if (!x_scale_fits(m, k)) return FP8BL_INVALID_ARG;
  if (m == 0 || n == 0) return FP8BL_OK;
  if (!xq || !xs || !q || !s || !y) return FP8BL_INVALID_ARG;
  if (!aligned(xq, 16) || !aligned(q, 16) || !aligned(y, 16) || !aligned(xs, 4) || !aligned(s, 4))
    return FP8BL_ALIGNMENT;
  const size_t ybytes = (size_t)m * n * 2;
  if (overlap(y, ybytes, xq, (size_t)m * k) || overlap(y, ybytes, q, (size_t)n * k) ||
      overlap(y, ybytes, s, grid_elems(n, k) * 4) || overlap(y, ybytes, xs, x_scale_elems(m, k) * 4))
    return FP8BL_INVALID_ARG;
  return FP8BL_OK;
}

// Workspace of fp8_block_linear_w8a8_bf16: the quantized activation, its
// scales, then the GEMM's split-K partials, each 256-byte aligned.
size_t w8a8_act_bytes(int64_t m, int64_t k) {
  return fp8bl::round_up((size_t)m * k, fp8bl::kWorkspaceAlign) +
         fp8bl::round_up(x_scale_elems(m, k) * 4, fp8bl::kWorkspaceAlign);
}

}  // namespace

FP8BL_EXPORT int fp8_block_abi_version(void) { return FP8BL_ABI_VERSION; }

FP8BL_EXPORT const char* fp8_block_status_string(int status) {
  switch (status) {
    case FP8BL_OK: return "FP8BL_OK";
    case FP8BL_INVALID_ARG: return "FP8BL_INVALID_ARG: null pointer, bad size, K % 16 != 0, bad path or overlapping output";
    case FP8BL_ALIGNMENT: return "FP8BL_ALIGNMENT: data pointers must be 16-byte aligned (scales 4-byte)";
    case FP8BL_WORKSPACE: return "FP8BL_WORKSPACE: workspace missing or smaller than fp8_block_linear_workspace_size";
    case FP8BL_UNSUPPORTED_DEVICE: return "FP8BL_UNSUPPORTED_DEVICE: the current HIP device is not gfx950";
    case FP8BL_HIP_ERROR: return "FP8BL_HIP_ERROR: a HIP runtime call failed";
    default: return "FP8BL_UNKNOWN_STATUS";
  }
}

FP8BL_EXPORT int fp8_block_device_supported(int device) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) return 0;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

FP8BL_EXPORT int fp8_block_dequant(const uint8_t* q, const float* scale_inv, uint16_t* w_bf16,
                                   int64_t n, int64_t k, hipStream_t stream) {
  int st = check_nk(n, k);
  if (st != FP8BL_OK) return st;
  if (n == 0) return FP8BL_OK;
  if (!q || !scale_inv || !w_bf16) return FP8BL_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(w_bf16, 16) || !aligned(scale_inv, 4)) return FP8BL_ALIGNMENT;
  const size_t wbytes = (size_t)n * k * 2;
  if (overlap(w_bf16, wbytes, q, (size_t)n * k) ||
      overlap(w_bf16, wbytes, scale_inv, grid_elems(n, k) * 4))
    return FP8BL_INVALID_ARG;
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  return hip_status(fp8bl::launch_dequant(q, scale_inv, w_bf16, n, k, stream));
}

FP8BL_EXPORT size_t fp8_block_linear_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || (k % 16) != 0) return 0;
  if (m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return 0;
  size_t a = fp8bl::tiled_workspace_bytes(m, n, k);
  const size_t b = fp8bl::skinny_workspace_bytes(m, n, k);
  if (n < kLargeMaxN) {
    const size_t c = fp8bl::large_workspace_bytes(m, n, k);
    a = a > c ? a : c;
  }
  return a > b ? a : b;
}

namespace {

// The kernel a call runs: the forced one, or the library's choice for AUTO:
// the weight-streaming kernel up to 32 rows, otherwise whichever of the two
// fused kernels the planners' cost models (same units, fitted to MI355X
// measurements) expect to finish first. The 256x256 persistent kernel wins
// on large shapes (16384 x 12288 x 3072: 945 against 1062 us) and on 512-row
// shapes whose units fill the CUs once (512 x 25600 x 5120: 131 against 158
// us; 512 x 5120 x 25600 with 6 K splits: 126 against 143 us).
int resolve_path(int path, int64_t m, int64_t n, int64_t k) {
  if (path != FP8BL_PATH_AUTO) return path;
  if (m <= kSkinnyMaxM) return FP8BL_PATH_SKINNY;
  if (n < kLargeMaxN && fp8bl::plan_large(m, n, k).cost < fp8bl::tiled_cost(m, n, k))
    return FP8BL_PATH_LARGE;
  return FP8BL_PATH_TILED;
}

// Split-K partial bytes of one (resolved) path on one shape.
size_t path_workspace_bytes(int path, int64_t m, int64_t n, int64_t k) {
  return path == FP8BL_PATH_SKINNY ? fp8bl::skinny_workspace_bytes(m, n, k)
       : path == FP8BL_PATH_LARGE  ? fp8bl::large_workspace_bytes(m, n, k)
                                   : fp8bl::tiled_workspace_bytes(m, n, k);
}

hipError_t launch_linear(int path, const uint16_t* x, const uint8_t* q, const float* s, uint16_t* y,
                         int64_t m, int64_t n, int64_t k, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  return path == FP8BL_PATH_SKINNY
             ? fp8bl::launch_gemm_skinny(x, q, s, y, m, n, k, ws, ws_bytes, stream)
         : path == FP8BL_PATH_LARGE
             ? fp8bl::launch_gemm_large(x, q, s, y, m, n, k, ws, ws_bytes, stream)
             : fp8bl::launch_gemm_tiled(x, q, s, y, m, n, k, ws, ws_bytes, stream);
}

// ---- Library-held scratch for fp8_block_linear_noalloc.
// One copy of this array per device (the code object's global), kept until
// the process ends. Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, looked up once per device on
// the first call there, with that device current.
constexpr size_t kScratchBytes = (size_t)FP8BL_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FP8BL_HIP_ERROR;
  if (dev < 0 || dev >= kMaxDevices) return FP8BL_UNSUPPORTED_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return FP8BL_HIP_ERROR;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8BL_OK;
}

}  // namespace

FP8BL_EXPORT int fp8_block_linear_ex(const uint16_t* x, const uint8_t* q, const float* scale_inv,
                                     uint16_t* y, int64_t m, int64_t n, int64_t k,
                                     void* workspace, size_t workspace_bytes, int path,
                                     hipStream_t stream) {
  int st = validate_linear(x, q, scale_inv, y, m, n, k, path);
  if (st != FP8BL_OK) return st;
  if (m == 0 || n == 0) return FP8BL_OK;
  path = resolve_path(path, m, n, k);
  const size_t need = path_workspace_bytes(path, m, n, k);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FP8BL_WORKSPACE;
    if (!aligned(workspace, fp8bl::kWorkspaceAlign)) return FP8BL_ALIGNMENT;
    if (overlap(workspace, need, y, (size_t)m * n * 2) ||
        overlap(workspace, need, x, (size_t)m * k * 2) ||
        overlap(workspace, need, q, (size_t)n * k) ||
        overlap(workspace, need, scale_inv, grid_elems(n, k) * 4))
      return FP8BL_INVALID_ARG;
  }
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  return hip_status(launch_linear(path, x, q, scale_inv, y, m, n, k, workspace, workspace_bytes, stream));
}

FP8BL_EXPORT int fp8_block_linear_noalloc(const uint16_t* x, const uint8_t* q,
                                          const float* scale_inv, uint16_t* y, int64_t m,
                                          int64_t n, int64_t k, hipStream_t stream) {
  int st = validate_linear(x, q, scale_inv, y, m, n, k, FP8BL_PATH_AUTO);
  if (st != FP8BL_OK) return st;
  if (m == 0 || n == 0) return FP8BL_OK;
  const int path = resolve_path(FP8BL_PATH_AUTO, m, n, k);
  const size_t need = path_workspace_bytes(path, m, n, k);
  if (need > kScratchBytes) return FP8BL_WORKSPACE;
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = current_scratch(&ws);
    if (st != FP8BL_OK) return st;
  }
  // The partials of every split are written in full before the reduce reads
  // them, so the scratch needs no clearing between calls.
  return hip_status(launch_linear(path, x, q, scale_inv, y, m, n, k, ws, need > 0 ? kScratchBytes : 0,
                                  stream));
}

FP8BL_EXPORT int fp8_block_linear(const uint16_t* x, const uint8_t* q, const float* scale_inv,
                                  uint16_t* y, int64_t m, int64_t n, int64_t k,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fp8_block_linear_ex(x, q, scale_inv, y, m, n, k, workspace, workspace_bytes,
                             FP8BL_PATH_AUTO, stream);
}

FP8BL_EXPORT int fp8_block_mlp_gate_up_ex(const uint16_t* x, const uint8_t* q_gate,
                                          const float* scale_inv_gate, const uint8_t* q_up,
                                          const float* scale_inv_up, uint16_t* h, int64_t m,
                                          int64_t n, int64_t k, int path, hipStream_t stream) {
  if (path != FP8BL_PATH_AUTO && path != FP8BL_PATH_TILED && path != FP8BL_PATH_LARGE)
    return FP8BL_INVALID_ARG;
  if (path == FP8BL_PATH_LARGE && (n % 8 != 0 || n >= kLargeMaxN)) return FP8BL_INVALID_ARG;
  int st = validate_linear(x, q_gate, scale_inv_gate, h, m, n, k, FP8BL_PATH_AUTO);
  if (st != FP8BL_OK) return st;
  st = validate_linear(x, q_up, scale_inv_up, h, m, n, k, FP8BL_PATH_AUTO);
  if (st != FP8BL_OK) return st;
  if (m == 0 || n == 0) return FP8BL_OK;
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  if (path == FP8BL_PATH_AUTO)
    path = (n % 8 == 0 && n < kLargeMaxN &&
            fp8bl::large_gated_cost(m, n, k) < fp8bl::mlp_tiled_cost(m, n, k))
               ? FP8BL_PATH_LARGE
               : FP8BL_PATH_TILED;
  if (path == FP8BL_PATH_LARGE)
    return hip_status(fp8bl::launch_gemm_large_gated(x, q_gate, scale_inv_gate, q_up,
                                                     scale_inv_up, h, m, n, k, stream));
  return hip_status(fp8bl::launch_mlp_gate_up(x, q_gate, scale_inv_gate, q_up, scale_inv_up, h,
                                              m, n, k, stream));
}

FP8BL_EXPORT int fp8_block_mlp_gate_up(const uint16_t* x, const uint8_t* q_gate,
                                       const float* scale_inv_gate, const uint8_t* q_up,
                                       const float* scale_inv_up, uint16_t* h, int64_t m,
                                       int64_t n, int64_t k, hipStream_t stream) {
  return fp8_block_mlp_gate_up_ex(x, q_gate, scale_inv_gate, q_up, scale_inv_up, h, m, n, k,
                                  FP8BL_PATH_AUTO, stream);
}

FP8BL_EXPORT int fp8_act_quantize(const uint16_t* x, uint8_t* xq, float* x_scale, int64_t m,
                                  int64_t k, hipStream_t stream) {
  if (m < 0 || k <= 0 || (k % 16) != 0 || m >= kMaxDim || k >= kMaxDim) return FP8BL_INVALID_ARG;
  if (m > 0 && m * k >= kMaxElems) return FP8BL_INVALID_ARG;
  if ((k + FP8BL_BLOCK - 1) / FP8BL_BLOCK > 65535) return FP8BL_INVALID_ARG;
  if (m == 0) return FP8BL_OK;
  if (!x || !xq || !x_scale) return FP8BL_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4)) return FP8BL_ALIGNMENT;
  const size_t sbytes = x_scale_elems(m, k) * 4;
  if (overlap(xq, (size_t)m * k, x, (size_t)m * k * 2) || overlap(x_scale, sbytes, x, (size_t)m * k * 2) ||
      overlap(xq, (size_t)m * k, x_scale, sbytes))
    return FP8BL_INVALID_ARG;
  int st = gate_current_device();
  if (st != FP8BL_OK) return st;
  return hip_status(fp8bl::launch_act_quantize(x, xq, x_scale, m, k, stream));
}

FP8BL_EXPORT size_t fp8_block_linear_w8a8_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || (k % 16) != 0) return 0;
  if (m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return 0;
  return w8a8_act_bytes(m, k) + fp8bl::w8a8_partials_bytes(m, n, k);
}

FP8BL_EXPORT int fp8_block_linear_w8a8_ex(const uint8_t* xq, const float* x_scale,
                                          const uint8_t* q, const float* scale_inv, uint16_t* y,
                                          int64_t m, int64_t n, int64_t k, void* workspace,
                                          size_t workspace_bytes, int path, hipStream_t stream) {
  if (path != FP8BL_PATH_AUTO && path != FP8BL_PATH_TILED && path != FP8BL_PATH_LARGE)
    return FP8BL_INVALID_ARG;
  if (path == FP8BL_PATH_LARGE && (n % 8 != 0 || n >= kLargeMaxN)) return FP8BL_INVALID_ARG;
  int st = validate_w8a8(xq, x_scale, q, scale_inv, y, m, n, k);
  if (st != FP8BL_OK) return st;
  if (m == 0 || n == 0) return FP8BL_OK;
  const size_t need = fp8bl::w8a8_partials_bytes(m, n, k);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FP8BL_WORKSPACE;
    if (!aligned(workspace, fp8bl::kWorkspaceAlign)) return FP8BL_ALIGNMENT;
    if (overlap(workspace, need, y, (size_t)m * n * 2) || overlap(workspace, need, xq, (size_t)m * k) ||
        overlap(workspace, need, q, (size_t)n * k) ||
        overlap(workspace, need, scale_inv, grid_elems(n, k) * 4) ||
        overlap(workspace, need, x_scale, x_scale_elems(m, k) * 4))
      return FP8BL_INVALID_ARG;
  }
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  const int kind = path == FP8BL_PATH_AUTO    ? (n < kLargeMaxN ? fp8bl::w8a8_choose(m, n, k) : 0)
                   : path == FP8BL_PATH_LARGE ? 1
                                              : 0;
  return hip_status(fp8bl::launch_gemm_w8a8(xq, x_scale, q, scale_inv, y, m, n, k, workspace,
                                            workspace_bytes, stream, kind));
}

FP8BL_EXPORT int fp8_block_linear_w8a8(const uint8_t* xq, const float* x_scale, const uint8_t* q,
                                       const float* scale_inv, uint16_t* y, int64_t m, int64_t n,
                                       int64_t k, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  return fp8_block_linear_w8a8_ex(xq, x_scale, q, scale_inv, y, m, n, k, workspace,
                                  workspace_bytes, FP8BL_PATH_AUTO, stream);
}

FP8BL_EXPORT int fp8_block_linear_w8a8_bf16(const uint16_t* x, const uint8_t* q,
                                            const float* scale_inv, uint16_t* y, int64_t m,
                                            int64_t n, int64_t k, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  int st = validate_linear(x, q, scale_inv, y, m, n, k, FP8BL_PATH_AUTO);
  if (st != FP8BL_OK) return st;
  if (!x_scale_fits(m, k)) return FP8BL_INVALID_ARG;
  if (m == 0 || n == 0) return FP8BL_OK;
  const size_t need = fp8_block_linear_w8a8_workspace_size(m, n, k);
  if (workspace == nullptr || workspace_bytes < need) return FP8BL_WORKSPACE;
  if (!aligned(workspace, fp8bl::kWorkspaceAlign)) return FP8BL_ALIGNMENT;
  if (overlap(workspace, need, y, (size_t)m * n * 2) || overlap(workspace, need, x, (size_t)m * k * 2) ||
      overlap(workspace, need, q, (size_t)n * k) ||
      overlap(workspace, need, scale_inv, grid_elems(n, k) * 4))
    return FP8BL_INVALID_ARG;
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xq = ws;
  float* xs = reinterpret_cast<float*>(ws + fp8bl::round_up((size_t)m * k, fp8bl::kWorkspaceAlign));
  uint8_t* part = ws + w8a8_act_bytes(m, k);
  hipError_t e = fp8bl::launch_act_quantize(x, xq, xs, m, k, stream);
  if (e != hipSuccess) return FP8BL_HIP_ERROR;
  return hip_status(fp8bl::launch_gemm_w8a8(xq, xs, q, scale_inv, y, m, n, k, part,
                                            need - w8a8_act_bytes(m, k), stream,
                                            n < kLargeMaxN ? fp8bl::w8a8_choose(m, n, k) : 0));
}

FP8BL_EXPORT int fp8_block_quantize(const float* w, uint8_t* q, float* scale_inv,
                                    int64_t n, int64_t k, hipStream_t stream) {
  int st = check_nk(n, k);
  if (st != FP8BL_OK) return st;
  if (n == 0) return FP8BL_OK;
  if ((k + FP8BL_BLOCK - 1) / FP8BL_BLOCK > 65535 * 4) return FP8BL_INVALID_ARG;
  if (!w || !q || !scale_inv) return FP8BL_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scale_inv, 4)) return FP8BL_ALIGNMENT;
  const size_t sbytes = grid_elems(n, k) * 4;
  if (overlap(q, (size_t)n * k, w, (size_t)n * k * 4) || overlap(scale_inv, sbytes, w, (size_t)n * k * 4) ||
      overlap(q, (size_t)n * k, scale_inv, sbytes))
    return FP8BL_INVALID_ARG;
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  return hip_status(fp8bl::launch_quantize(w, q, scale_inv, n, k, stream));
}

FP8BL_EXPORT int fp8_block_quantize_bf16(const uint16_t* w_bf16, uint8_t* q, float* scale_inv,
                                         int64_t n, int64_t k, hipStream_t stream) {
  int st = check_nk(n, k);
  if (st != FP8BL_OK) return st;
  if (n == 0) return FP8BL_OK;
  if ((k + FP8BL_BLOCK - 1) / FP8BL_BLOCK > 65535 * 4) return FP8BL_INVALID_ARG;
  if (!w_bf16 || !q || !scale_inv) return FP8BL_INVALID_ARG;
  if (!aligned(w_bf16, 16) || !aligned(q, 16) || !aligned(scale_inv, 4)) return FP8BL_ALIGNMENT;
  const size_t sbytes = grid_elems(n, k) * 4;
  if (overlap(q, (size_t)n * k, w_bf16, (size_t)n * k * 2) ||
      overlap(scale_inv, sbytes, w_bf16, (size_t)n * k * 2) || overlap(q, (size_t)n * k, scale_inv, sbytes))
    return FP8BL_INVALID_ARG;
  st = gate_current_device();
  if (st != FP8BL_OK) return st;
  return hip_status(fp8bl::launch_quantize_bf16(w_bf16, q, scale_inv, n, k, stream));
}

FP8BL_EXPORT int fp8_block_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                                       hipStream_t stream) {
  if (bytes == 0) return FP8BL_OK;
  if (!buf || !sink || blocks < 1 || blocks > 65536 || (bytes % 16) != 0) return FP8BL_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return FP8BL_ALIGNMENT;
  if (overlap(sink, (size_t)blocks * 256 * 4, buf, bytes)) return FP8BL_INVALID_ARG;
  const int st = gate_current_device();
  if (st != FP8BL_OK) return st;
  return hip_status(fp8bl::launch_stream_read(buf, bytes, sink, blocks, stream));
}
