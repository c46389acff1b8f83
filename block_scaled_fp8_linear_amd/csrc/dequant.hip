// Standalone block dequant: Q[N,K] E4M3 + S[GN,GK] fp32 -> bf16 W_hat[N,K].
//
// FastVideo PR #1829, "Purpose": the block-scaled weight is dequantized to
// BF16 right before a plain matmul (the transient weight of the Hopper route,
// "Checklist": at most ~0.26 GB for the largest layer). "Changes", tests
// bullet: bit-exact against the reference broadcast.
//
// HBM-bound: 1 byte read and 2 bytes written per element (+ the scale grid,
// which stays in cache). Each thread moves 16-byte chunks (16 codes in, 32
// bytes out); a chunk never straddles a scale block because K % 16 == 0 and
// 128 % 16 == 0. The flat chunk index doubles as the output offset, so the
// only index arithmetic is one 32-bit division for the scale lookup.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

constexpr int kDqThreads = 256;
constexpr int kDqChunksPerThread = 4;

__global__ __launch_bounds__(kDqThreads)
void dequant_kernel(const u32x4* __restrict__ q, const float* __restrict__ s,
                    u32x4* __restrict__ w, uint32_t chunks_per_row,
                    uint32_t total_chunks, uint32_t gk) {
  const uint32_t base = blockIdx.x * (kDqThreads * kDqChunksPerThread) + threadIdx.x;
  u32x4 codes[kDqChunksPerThread];
#pragma unroll
  for (int i = 0; i < kDqChunksPerThread; ++i) {
    const uint32_t c = base + i * kDqThreads;
    if (c < total_chunks) codes[i] = __builtin_nontemporal_load(q + c);
  }
#pragma unroll
  for (int i = 0; i < kDqChunksPerThread; ++i) {
    const uint32_t c = base + i * kDqThreads;
    if (c >= total_chunks) continue;
    const uint32_t row = c / chunks_per_row;
    const uint32_t col = (c - row * chunks_per_row) * 16u;
    const float sc = s[(row / kBlock) * gk + col / kBlock];
    u32x4 o0, o1;
    u32x2 t;
    t = dequant4(codes[i][0], sc); o0[0] = canon_nan_bf16x2(t[0]); o0[1] = canon_nan_bf16x2(t[1]);
    t = dequant4(codes[i][1], sc); o0[2] = canon_nan_bf16x2(t[0]); o0[3] = canon_nan_bf16x2(t[1]);
    t = dequant4(codes[i][2], sc); o1[0] = canon_nan_bf16x2(t[0]); o1[1] = canon_nan_bf16x2(t[1]);
    t = dequant4(codes[i][3], sc); o1[2] = canon_nan_bf16x2(t[0]); o1[3] = canon_nan_bf16x2(t[1]);
    __builtin_nontemporal_store(o0, w + 2 * (size_t)c);
    __builtin_nontemporal_store(o1, w + 2 * (size_t)c + 1);
  }
}

hipError_t launch_dequant(const uint8_t* q, const float* s, uint16_t* w,
                          int64_t n, int64_t k, hipStream_t stream) {
  const uint64_t chunks_per_row = (uint64_t)k / 16;
  const uint64_t total = (uint64_t)n * chunks_per_row;
  const uint64_t gk = ((uint64_t)k + kBlock - 1) / kBlock;
  const uint64_t per_block = (uint64_t)kDqThreads * kDqChunksPerThread;
  const uint64_t blocks = (total + per_block - 1) / per_block;
  hipLaunchKernelGGL(dequant_kernel, dim3((uint32_t)blocks), dim3(kDqThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(q), s, reinterpret_cast<u32x4*>(w),
                     (uint32_t)chunks_per_row, (uint32_t)total, (uint32_t)gk);
  return hipGetLastError();
}

}  // namespace fp8bl
