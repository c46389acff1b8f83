// A plain streaming read of a device buffer: the practical HBM ceiling that
// the bandwidth-bound kernels (dequant, skinny GEMM, activation quantizer)
// are measured against. Not part of the linear layer.
//
// Grid-stride loop of 16-byte non-temporal loads: in each round the whole
// grid reads one contiguous window, each wave 1 KB of it. Every thread folds
// its words by XOR into one 32-bit value written to `sink`, so the loads
// cannot be dropped and the sink's XOR equals the XOR of every 32-bit word
// of the buffer.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

__global__ __launch_bounds__(256)
void stream_read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace fp8bl
