// Block quantizer: fp32 W[N,K] -> E4M3 codes Q[N,K] + fp32 weight_scale_inv
// S[GN,GK], the format the converter writes (FastVideo PR #1829, "Changes",
// converter bullet: E4M3 weight plus [N/128, K/128] weight_scale_inv).
//
// Per 128x128 block (present elements only, for partial edge blocks):
//   amax = max |w|;  S = fl32(amax / 448), or 1 when amax == 0;
//   code = nearest finite E4M3 to fl32(w / S), ties to the even code,
//          saturating at 448, sign kept.
// One workgroup of eight waves per block, each lane holding 32 elements in
// registers between the amax and the encode; offline work, so every element
// takes an IEEE division. The input is fp32, or bf16 widened exactly to fp32
// (a checkpoint stored in bf16). Wave loads cover whole block rows: lanes
// that each took one row's 64-column half (a wave load touching 64 separate
// lines) measured 4-6x slower on MI355X.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

constexpr int kThreads = 256;

// Two fp32 values -> their E4M3FN codes in bytes 0 and 1 (HI false) or 2
// and 3 (HI) of `old`, by the gfx950 conversion v_cvt_pk_fp8_f32: nearest
// code, ties to even, sign kept (-0 -> 0x80). It gives the same codes as an
// integer nearest-even encoder that saturates at 448 on every input the GPU
// tests feed it: each bf16-valued fp32 up to 448 and each fp32 within 4096
// ulp of every code and of every midpoint between neighbouring codes, both
// signs, plus subnormal inputs. The quotients w / S and x / S of both
// quantizers stay below 448 * (1 + 2^-23), where saturation and rounding to
// 448 coincide.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_hw(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Four consecutive inputs as fp32: fp32 loads as they are; bf16 widens
// exactly (its 16 bits are the high half of the fp32 pattern).
__device__ __forceinline__ f32x4 load4(const float* w, size_t i) {
  return *reinterpret_cast<const f32x4*>(w + i);
}
__device__ __forceinline__ f32x4 load4(const uint16_t* w, size_t i) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(w + i);
  return f32x4{__builtin_bit_cast(float, v[0] << 16), __builtin_bit_cast(float, v[0] & 0xFFFF0000u),
               __builtin_bit_cast(float, v[1] << 16), __builtin_bit_cast(float, v[1] & 0xFFFF0000u)};
}

constexpr int kQThreads = 512;

template <typename T>
__global__ __launch_bounds__(kQThreads)
void quantize_kernel(const T* __restrict__ w, uint8_t* __restrict__ q,
                     float* __restrict__ s, int N, int K, int gk) {
  __shared__ float wave_max[kQThreads / 64];
  const int bi = blockIdx.y, bj = blockIdx.x;
  const int tid = threadIdx.x;
  // Wave w covers block rows 16 w .. 16 w + 15; pass i of its lane l takes
  // row 16 w + 2 i + (l >> 5), columns 4 (l & 31) .. +4, so each wave load
  // reads two whole 128-column block rows (contiguous runs).
  const int row0 = bi * kBlock + (tid >> 6) * 16 + ((tid >> 5) & 1);
  const int col = bj * kBlock + (tid & 31) * 4;
  // K % 16 == 0 and col % 4 == 0: a group of four is wholly inside or outside K
  const bool col_ok = col < K;

  f32x4 v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + 2 * i;
    if (col_ok && row < N) {
      v[i] = load4(w, (size_t)row * K + col);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])),
                               fmaxf(fabsf(v[i][2]), fabsf(v[i][3]))));
    } else {
      v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) wave_max[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3])),
               fmaxf(fmaxf(wave_max[4], wave_max[5]), fmaxf(wave_max[6], wave_max[7])));
  const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  if (tid == 0) s[bi * gk + bj] = sc;
  if (!col_ok) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + 2 * i;
    if (row >= N) break;
    const f32x4 t = v[i];
    *reinterpret_cast<uint32_t*>(q + (size_t)row * K + col) =
        e4m3x2_hw<true>(__fdiv_rn(t[2], sc), __fdiv_rn(t[3], sc),
                        e4m3x2_hw<false>(__fdiv_rn(t[0], sc), __fdiv_rn(t[1], sc), 0u));
  }
}

// Activation quantizer of the W8A8 route: per token, per 1x128 K group,
// the same arithmetic as the weight blocks (S = fl32(amax / 448), 1 for an
// all-zero group; code = nearest E4M3 of fl32(x / S)). A 256-thread block
// covers 16 consecutive rows of one K group: 16 lanes per row, 8 bf16 each
// (one 16-byte load), the group maximum by a 16-lane butterfly. Scales are
// written K-block-major, xs[kb * M + row], so a block's 16 scales are one
// contiguous 64-byte run.
//
// The quotient: with y = fl32(1 / S) (one IEEE division per group),
// q0 = fl32(x * y), r = fma(-q0, S, x), q = fma(r, y, q0) carrying the sign
// of x (for x = -0 the fma sum is +0). Over every finite bf16 x with
// |x| <= amax and every bf16 amax whose S >= 2^-64, this gives the same E4M3
// code as the IEEE quotient (a GPU test runs every such pair, both signs,
// against a plain CPU reference); smaller scales take the IEEE division.
__global__ __launch_bounds__(kThreads)
void act_quantize_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                         float* __restrict__ xs, int M, int K) {
  const int kb = blockIdx.y;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int col = kb * kBlock + sub * 8;
  // K % 16 == 0 and col % 8 == 0, so a chunk is wholly inside or outside K
  const bool ok = row < M && col < K;
  float v[8];
  float amax = 0.0f;
  if (ok) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(x + (size_t)row * K + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
      v[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const float sc = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  if (ok) {
    float qv[8];
    if (sc >= 0x1p-64f) {
      const float y = __fdiv_rn(1.0f, sc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = __fmul_rn(v[i], y);
        const float r = __builtin_fmaf(-q0, sc, v[i]);
        qv[i] = __builtin_copysignf(__builtin_fmaf(r, y, q0), v[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = __fdiv_rn(v[i], sc);
    }
    u32x2 out;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      out[h] = e4m3x2_hw<true>(qv[4 * h + 2], qv[4 * h + 3], e4m3x2_hw<false>(qv[4 * h], qv[4 * h + 1], 0u));
    *reinterpret_cast<u32x2*>(xq + (size_t)row * K + col) = out;
  }
  if (sub == 0 && row < M) xs[(size_t)kb * M + row] = sc;
}

}  // namespace

hipError_t launch_act_quantize(const uint16_t* x, uint8_t* xq, float* xs, int64_t m, int64_t k,
                               hipStream_t stream) {
  const int gk = (int)((k + kBlock - 1) / kBlock);
  const uint64_t rows = ((uint64_t)m + 15) / 16;
  hipLaunchKernelGGL(act_quantize_kernel, dim3((uint32_t)rows, (uint32_t)gk), dim3(kThreads), 0,
                     stream, x, xq, xs, (int)m, (int)k);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, uint8_t* q, float* s, int64_t n, int64_t k,
                           hipStream_t stream) {
  const int gn = (int)((n + kBlock - 1) / kBlock);
  const int gk = (int)((k + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(quantize_kernel<float>, dim3((uint32_t)gk, (uint32_t)gn), dim3(kQThreads), 0,
                     stream, w, q, s, (int)n, (int)k, gk);
  return hipGetLastError();
}

hipError_t launch_quantize_bf16(const uint16_t* w, uint8_t* q, float* s, int64_t n, int64_t k,
                                hipStream_t stream) {
  const int gn = (int)((n + kBlock - 1) / kBlock);
  const int gk = (int)((k + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(quantize_kernel<uint16_t>, dim3((uint32_t)gk, (uint32_t)gn), dim3(kQThreads), 0,
                     stream, w, q, s, (int)n, (int)k, gk);
  return hipGetLastError();
}

}  // namespace fp8bl
