// Internal (non-exported) launchers behind the C ABI. Every launcher assumes
// its arguments were validated by the ABI layer (sizes, alignment, K % 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8bl {

hipError_t launch_dequant(const uint8_t* q, const float* s, uint16_t* w,
                          int64_t n, int64_t k, hipStream_t stream);

hipError_t launch_quantize(const float* w, uint8_t* q, float* s,
                           int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_quantize_bf16(const uint16_t* w, uint8_t* q, float* s,
                                int64_t n, int64_t k, hipStream_t stream);

// W8A8 route: per-token 1x128 activation quantizer (scales [GK, M]) and the
// FP8 x FP8 block-scaled GEMM.
hipError_t launch_act_quantize(const uint16_t* x, uint8_t* xq, float* xs, int64_t m, int64_t k,
                               hipStream_t stream);
// W8A8 kernels: `kind` 0 = 128x128 tiles, 1 = 256x256 tiles (N % 8 == 0),
// -1 = the cost models' choice. w8a8_partials_bytes covers either kernel.
size_t w8a8_partials_bytes(int64_t m, int64_t n, int64_t k);
int w8a8_choose(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_w8a8(const uint8_t* xq, const float* xs, const uint8_t* q, const float* s,
                            uint16_t* y, int64_t m, int64_t n, int64_t k, void* ws,
                            size_t ws_bytes, hipStream_t stream, int kind = -1);
struct W8a8LargePlan {
  int bm;           // X rows per tile: 192 or 128
  int splits, kb_per_split;
  double cost;      // time estimate, microseconds
};
W8a8LargePlan plan_w8a8_large(int64_t m, int64_t n, int64_t k);
size_t w8a8_large_partials_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_w8a8_large(const uint8_t* xq, const float* xs, const uint8_t* q,
                                  const float* s, uint16_t* y, int64_t m, int64_t n, int64_t k,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

// Tile-planned fused GEMM (E4M3 tiles decoded to bf16 in registers, bf16
// MFMA); tiled_cost is its planner's time estimate for the chosen plan.
size_t tiled_workspace_bytes(int64_t m, int64_t n, int64_t k);
double tiled_cost(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_tiled(const uint16_t* x, const uint8_t* q, const float* s,
                             uint16_t* y, int64_t m, int64_t n, int64_t k,
                             void* ws, size_t ws_bytes, hipStream_t stream);

// Large-M fused GEMM: 256x256 tiles of four waves, X through a three-stage
// direct-to-LDS ring, codes decoded one sub-step ahead of the MFMAs.
struct LargePlan {
  int splits, kt_per_split;
  double cost;      // planner's time estimate, the units of tiled_cost
};
LargePlan plan_large(int64_t m, int64_t n, int64_t k);
size_t large_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_large(const uint16_t* x, const uint8_t* q, const float* s,
                             uint16_t* y, int64_t m, int64_t n, int64_t k,
                             void* ws, size_t ws_bytes, hipStream_t stream);
// Its gated form (gate/up pair, SwiGLU epilogue; N % 8 == 0, N < 2^21) and
// that form's time estimate in the same units.
double large_gated_cost(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_large_gated(const uint16_t* x, const uint8_t* qg, const float* sg,
                                   const uint8_t* qu, const float* su, uint16_t* h, int64_t m,
                                   int64_t n, int64_t k, hipStream_t stream);

// MLP gate/up pair with the SwiGLU epilogue: h = swiglu(x Wg^T, x Wu^T), on
// the tile-planned kernels; mlp_tiled_cost is their planner's estimate.
double mlp_tiled_cost(int64_t m, int64_t n, int64_t k);
hipError_t launch_mlp_gate_up(const uint16_t* x, const uint8_t* qg, const float* sg,
                              const uint8_t* qu, const float* su, uint16_t* h,
                              int64_t m, int64_t n, int64_t k, hipStream_t stream);

// Skinny-M (M <= 32 rows per pass) weight-streaming GEMM.
size_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_skinny(const uint16_t* x, const uint8_t* q, const float* s,
                              uint16_t* y, int64_t m, int64_t n, int64_t k,
                              void* ws, size_t ws_bytes, hipStream_t stream);

// Deterministic sum of `splits` fp32 partial [M,N] slabs (in split order,
// slab stride partial_slab(M, N)) and one bf16 rounding into y.
hipError_t launch_reduce_partials(const float* part, uint16_t* y, int splits,
                                  int64_t m, int64_t n, hipStream_t stream);

// Streaming read of `bytes` (a multiple of 16) by `blocks` workgroups of 256
// threads; one XOR-folded word per thread into sink[blocks * 256].
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t stream);

constexpr size_t kWorkspaceAlign = 256;
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
// Split-K partial slabs ([M,N] fp32 each) start every 64 floats, so every
// slab is 256-byte aligned inside the workspace.
__host__ __device__ inline size_t partial_slab(size_t m, size_t n) { return (m * n + 63) & ~(size_t)63; }

}  // namespace fp8bl
