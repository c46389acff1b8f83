// Standalone block dequant: Q[N,K] E4M3 + S[GN,GK] fp32 -> bf16 W_hat[N,K].
//
// FastVideo PR #1829, "Purpose": the Hopper route turns each block-scaled
// weight into BF16 just ahead of the layer's matmul ("Checklist": that
// temporary BF16 copy reaches about 0.26 GB for the biggest layer).
// "Changes", tests bullet: the output must match, bit for bit, decoding the
// codes and multiplying by the scale grid expanded over its blocks.
//
// HBM-bound: 1 byte read and 2 bytes written per element (+ the scale grid,
// which stays in cache). Each thread moves 8-code chunks (8 bytes in, 16
// bytes out), eight of them in flight. The flat chunk index doubles as the
// input and output offset, so the only index arithmetic is one 32-bit
// division for the scale lookup.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

constexpr int kDqThreads = 256;
constexpr int kDqChunksPerThread = 8;

// A chunk is 8 consecutive codes of one row: an 8-byte load per lane (512
// contiguous bytes per wave instruction) and a 16-byte store (1 KB
// contiguous per wave instruction), so every store fills whole cache lines.
// A chunk never straddles a scale block (K % 16 == 0, 128 % 8 == 0).
__global__ __launch_bounds__(kDqThreads)
void dequant_kernel(const u32x2* __restrict__ q, const float* __restrict__ s,
                    u32x4* __restrict__ w, uint32_t chunks_per_row,
                    uint32_t total_chunks, uint32_t gk) {
  const uint32_t base = blockIdx.x * (kDqThreads * kDqChunksPerThread) + threadIdx.x;
  u32x2 codes[kDqChunksPerThread];
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
    const uint32_t col = (c - row * chunks_per_row) * 8u;
    const float sc = s[(row / kBlock) * gk + col / kBlock];
    const u32x2 lo = dequant4(codes[i][0], sc);
    const u32x2 hi = dequant4(codes[i][1], sc);
    const u32x4 o = {canon_nan_bf16x2(lo[0]), canon_nan_bf16x2(lo[1]),
                     canon_nan_bf16x2(hi[0]), canon_nan_bf16x2(hi[1])};
    __builtin_nontemporal_store(o, w + c);
  }
}

hipError_t launch_dequant(const uint8_t* q, const float* s, uint16_t* w,
                          int64_t n, int64_t k, hipStream_t stream) {
  const uint64_t chunks_per_row = (uint64_t)k / 8;
  const uint64_t total = (uint64_t)n * chunks_per_row;
  const uint64_t gk = ((uint64_t)k + kBlock - 1) / kBlock;
  const uint64_t per_block = (uint64_t)kDqThreads * kDqChunksPerThread;
  const uint64_t blocks = (total + per_block - 1) / per_block;
  hipLaunchKernelGGL(dequant_kernel, dim3((uint32_t)blocks), dim3(kDqThreads), 0, stream,
                     reinterpret_cast<const u32x2*>(q), s, reinterpret_cast<u32x4*>(w),
                     (uint32_t)chunks_per_row, (uint32_t)total, (uint32_t)gk);
  return hipGetLastError();
}

}  // namespace fp8bl
