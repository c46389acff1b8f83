// Device-side building blocks shared by the gfx950 kernels: vector types,
// the E4M3 -> fp32 -> bf16 dequant of packed codes, and small helpers.
//
// Dequant of one element (FastVideo PR #1829, "Purpose"):
//   bf16_rne( fl32( e4m3(code) * scale ) )
// The E4M3 decode uses the gfx950 hardware conversion (v_cvt_pk_f32_fp8,
// OCP E4M3FN on this architecture: every finite code is exact in fp32), the
// product is one IEEE fp32 multiply (no contraction: nothing is added to
// it), and v_cvt_pk_bf16_f32 rounds two results to nearest-even at once.
// fp32 denormals are kept (the library is built without flush-to-zero).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bl {

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kBlock = 128;  // scale-block edge

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Four E4M3 codes (byte i of `codes` is element i) -> two packed bf16 pairs,
// each element scaled by `s` in fp32 first.
__device__ __forceinline__ u32x2 dequant4(uint32_t codes, float s) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);  // bytes 0,1
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);   // bytes 2,3
  u32x2 r;
  r[0] = pack_bf16x2(__fmul_rn(lo[0], s), __fmul_rn(lo[1], s));
  r[1] = pack_bf16x2(__fmul_rn(hi[0], s), __fmul_rn(hi[1], s));
  return r;
}

// Eight codes (two dwords) -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 dequant8(uint32_t c0, uint32_t c1, float s) {
  u32x2 a = dequant4(c0, s);
  u32x2 b = dequant4(c1, s);
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// bf16 NaN (exponent all ones, mantissa non-zero) -> the canonical 0x7FC0,
// applied to both halves of a packed pair.
__device__ __forceinline__ uint32_t canon_nan_bf16x2(uint32_t v) {
  uint32_t lo = v & 0xFFFFu, hi = v >> 16;
  lo = ((lo & 0x7FFFu) > 0x7F80u) ? 0x7FC0u : lo;
  hi = ((hi & 0x7FFFu) > 0x7F80u) ? 0x7FC0u : hi;
  return lo | (hi << 16);
}

// bf16 SwiGLU of two fp32 accumulators, rounded where eager bf16 ops round
// (FastVideo fasth3_omniref_b200 README, "What --lossless-accel turns on"):
// g and u each to bf16, silu(g) = g / (1 + e^-g) in fp32 then to bf16, and
// the product of the two bf16 values (exact in fp32) rounded once.
// e^-g is 2^(-g log2 e) on the hardware exp2 and the quotient a hardware
// reciprocal times g: the fp32 silu is off by a relative (|g| + 4) 2^-23 at
// most (the rounding of the exponent argument grows with |g|), far inside
// the half-ulp of the bf16 rounding that follows (2^-9), so only values
// within that distance of a bf16 rounding boundary can round the other way.
// Past g < -88.7 the exponential overflows and silu(g) comes out -0 (exactly:
// a negative number below 1e-36 in size); -inf gives NaN, as g / (1 + e^-g).
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}
__device__ __forceinline__ uint16_t swiglu_bf16(float acc_g, float acc_u) {
  const float g = (float)(__bf16)acc_g;
  const float u = (float)(__bf16)acc_u;
  const float sl = (float)(__bf16)silu_f32(g);
  const __bf16 h = (__bf16)(sl * u);
  return __builtin_bit_cast(uint16_t, h);
}
// The same on two packed bf16 pairs (low half first): g and u already bf16.
__device__ __forceinline__ uint32_t swiglu_bf16x2(uint32_t g2, uint32_t u2) {
  const uint32_t s2 = pack_bf16x2(silu_f32(__uint_as_float(g2 << 16)),
                                  silu_f32(__uint_as_float(g2 & 0xFFFF0000u)));
  return pack_bf16x2(__uint_as_float(s2 << 16) * __uint_as_float(u2 << 16),
                     __uint_as_float(s2 & 0xFFFF0000u) * __uint_as_float(u2 & 0xFFFF0000u));
}

}  // namespace fp8bl
