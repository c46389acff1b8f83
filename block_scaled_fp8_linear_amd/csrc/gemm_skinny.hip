// Skinny-M block-FP8 linear (M <= 32 per pass): the run is bound by the HBM
// bytes of the E4M3 weight, so the kernel is organised around streaming W
// once, at full bandwidth, with as many 16-byte loads in flight as possible.
//
// Same arithmetic as the tiled path (FastVideo PR #1829, "Purpose": the
// weight goes to BF16, then an ordinary matmul; fp32 accumulation, one bf16
// rounding per output).
//
// Work unit: a workgroup of W waves owns 16*NT weight rows and one K range
// (its split; normally all of K). The range is cut into 256-wide
// super-steps dealt round-robin to the waves; each wave prefetches its next
// super-step while it computes the current one.
//
// Load shape. HBM streams well when each load instruction reads a few long
// runs: 4 rows x 256 contiguous bytes per 64-lane instruction reaches ~95%
// of a plain sequential read on MI355X, while the MFMA operand shape (16
// rows x 64 bytes) reaches ~60%. So codes are loaded 4 rows x 256 bytes at a
// time, written to a small per-wave LDS slab (XOR-permuted by row so writes
// and reads are bank-conflict-free) and read back in the MFMA layout; no
// barrier is needed because each wave only reads what it wrote. Rows past N
// and the K tail read as zero through the buffer descriptors.
//
// The k order inside a super-step is permuted (the MFMA sums over k, so A
// and B only have to agree): MFMA 2h+e gives lane group g the codes
// k = 16*(g + 4h) + 8e .. +8, and X is loaded with the same k. X (rows past
// M read as zero) is tiny and stays in L2; the NT tiles of a wave share each
// X fragment. At the end the waves' partial sums meet in LDS and are added
// in wave order; with one split the result is rounded to bf16 directly,
// otherwise fp32 partials go to the workspace and are summed in split order
// by the reduce kernel (no atomics anywhere).
//
// v_mfma_f32_16x16x32_bf16: lane l gives 8 consecutive-k values of row
// (l % 16) of A and of column (l % 16) of B; lane group l / 16 picks the
// k chunk. Output: lane l holds rows (l/16)*4 + r, r = 0..3, column l % 16.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

constexpr int kSuper = 256;               // K per super-step (16 chunks of 16 codes per row)
constexpr uint32_t kOob = 0x80000000u;    // buffer offset past every valid range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: raw (untyped) buffer descriptor of the gfx9
  // family; offsets at or past `bytes` read as zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The weight is read once: its loads carry the non-temporal cache policy
// (bit 1 of the buffer instruction's cache field on gfx950), which on MI355X
// streams an 8000 x 8192 weight 5-10% faster than default-policy loads.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}

template <int MT, int NT, int WAVES>
__global__ __launch_bounds__(WAVES * 64)
void gemm_skinny_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                        const float* __restrict__ s, uint16_t* __restrict__ y,
                        float* __restrict__ part, int M, int N, int K, int gk,
                        int ss_per_split) {
  // Per-wave staging of one super-step of codes: NT tiles x 16 rows x 256 B.
  __shared__ __attribute__((aligned(16))) uint8_t wl[WAVES][NT][16 * kSuper];
  __shared__ f32x4 red[WAVES][MT * NT][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * (16 * NT);
  const int nss = (K + kSuper - 1) / kSuper;
  const int ss0 = blockIdx.y * ss_per_split;
  const int ss1 = min(ss0 + ss_per_split, nss);

  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(q + (size_t)n0 * K, (uint32_t)(min(N - n0, 16 * NT) * K));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)(M * K * 2));

  // Loads: instruction r (0..3) of tile j brings rows 4r..4r+3 of the tile,
  // 256 contiguous bytes each (lane >> 4 picks the row, lane & 15 the
  // 16-byte chunk). Lane i lands at byte 16*i of that instruction's 1 KB
  // slab in LDS; it fetches the logical chunk (i & 15) ^ row, so the slab
  // holds each row's chunks XOR-permuted by the row index.
  const int lrow4 = lane >> 4;
  const int lchk = lane & 15;
  uint32_t woff[NT][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * r + lrow4;
    const int c = lchk ^ row;
#pragma unroll
    for (int j = 0; j < NT; ++j) woff[j][r] = (uint32_t)((j * 16 + row) * K + c * 16);
  }
  // MFMA operands: lane l is weight row n = l & 15 and k group g = l >> 4.
  // For h = 0..3 it reads logical chunk g + 4h (16 codes = 2 MFMAs), stored
  // at physical chunk (g + 4h) ^ n: the 16 lanes of a read phase hit 16
  // distinct 16-byte bank groups. MFMA 2h+e of a super-step covers, for
  // lane group g, k = 16*(g + 4h) + 8e .. +8; X follows the same k.
  const int bn = lane & 15;
  const int bg = lane >> 4;
  uint32_t xoff[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) xoff[i] = (uint32_t)(((i * 16 + bn) * K + bg * 16) * 2);

  int srow[NT];
  bool tile_live[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    tile_live[j] = (n0 + j * 16) < N;
    srow[j] = tile_live[j] ? (n0 + j * 16) / kBlock : 0;
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wv[NT][4], xv[MT][4][2];
  auto issue = [&](int ss, u32x4 (&w)[NT][4], u32x4 (&xa)[MT][4][2]) {
    const bool live = ss < ss1;
    const uint32_t kb = (uint32_t)(ss * kSuper);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * r + lrow4;
      const bool kin = live && (int)kb + ((lchk ^ row) * 16) < K;
#pragma unroll
      for (int j = 0; j < NT; ++j) w[j][r] = buf_load16_nt(wrs, kin ? woff[j][r] + kb : kOob);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const bool kin = live && (int)kb + (bg + 4 * h) * 16 < K;
        const uint32_t o = xoff[i] + (kb + (uint32_t)(64 * h)) * 2;
        xa[i][h][0] = buf_load16(xrs, kin ? o : kOob);
        xa[i][h][1] = buf_load16(xrs, kin ? o + 16 : kOob);
      }
  };

  // Every workgroup walks its K range from a different starting super-step
  // (rotated by its index), so at any moment the GPU reads many K offsets at
  // once instead of all rows at one offset: with rows a power-of-two apart
  // the latter concentrates traffic on a few HBM channels. The order is
  // fixed per workgroup, so results stay run-to-run identical.
  const int count = ss1 - ss0;
  const int rot = count > 0 ? (int)(blockIdx.x % (unsigned)count) : 0;
  auto ss_of = [&](int i) {            // i-th super-step of the range, rotated
    if (i >= count) return ss1;        // past the end: loads read nothing
    const int r = i + rot;
    return ss0 + (r >= count ? r - count : r);
  };
  int it = wave;
  issue(ss_of(it), wv, xv);
  for (; it < count; it += WAVES) {
    const int ss = ss_of(it);
    u32x4 wn[NT][4], xn[MT][4][2];
    issue(ss_of(it + WAVES), wn, xn);          // next super-step in flight
    const int kb = (ss * kSuper) / kBlock;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      uint8_t* slab = &wl[wave][j][0];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4*>(slab + r * 1024 + lane * 16) = wv[j][r];
      // A super-step spans two 128-column scale blocks: logical chunks 0..7
      // (h = 0, 1) take the first, chunks 8..15 (h = 2, 3) the second. A K
      // tail never reads the second block's scale unless it exists.
      const float sc0 = tile_live[j] ? s[srow[j] * gk + kb] : 0.0f;
      const float sc1 = (tile_live[j] && kb + 1 < gk) ? s[srow[j] * gk + kb + 1] : 0.0f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float sc = h < 2 ? sc0 : sc1;
        const u32x4 c = *reinterpret_cast<const u32x4*>(slab + bn * kSuper + (((bg + 4 * h) ^ bn) << 4));
        const bf16x8 b0 = dequant8(c[0], c[1], sc);
        const bf16x8 b1 = dequant8(c[2], c[3], sc);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, xv[i][h][0]), b0, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, xv[i][h][1]), b1, acc[i][j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[j][r] = wn[j][r];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) { xv[i][h][0] = xn[i][h][0]; xv[i][h][1] = xn[i][h][1]; }
  }

  // Cross-wave sum in wave order.
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[wave][i * NT + j][lane] = acc[i][j];
  __syncthreads();
  // Each of the first MT*NT waves finishes one (m-tile, n-tile) pair.
  const int pair = wave;
  if (pair >= MT * NT) return;
  const int i = pair / NT, j = pair % NT;
  f32x4 t = red[0][pair][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    const f32x4 o = red[w][pair][lane];
    t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
  }
  const int col = n0 + j * 16 + (lane & 15);
  if (col >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = i * 16 + (lane >> 4) * 4 + r;
    if (row >= M) continue;
    if (gridDim.y == 1) {
      const __bf16 v = (__bf16)t[r];
      y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, v);
    } else {
      part[(size_t)blockIdx.y * partial_slab(M, N) + (size_t)row * N + col] = t[r];
    }
  }
}

// Sum of split-K partials, 8 outputs per thread (two 16-byte loads per
// split), added in split order and rounded once; a scalar tail handles
// M*N not divisible by 8. With the split count fixed at compile time every
// load is in flight before the first add (bit-identical; 1-5% faster than
// the run-time loop on MI355X, which waits for each split's loads in turn).
// S > 0: exactly S splits, every load issued before the first add; S == 0:
// `splits` at run time.
template <int S>
__global__ __launch_bounds__(256)
void reduce_partials_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                            int splits, size_t mn, size_t slab) {
  const size_t i8 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if constexpr (S == 0) {
    if (i8 + 8 <= mn) {
      f32x4 a = *reinterpret_cast<const f32x4*>(part + i8);
      f32x4 b = *reinterpret_cast<const f32x4*>(part + i8 + 4);
      for (int sp = 1; sp < splits; ++sp) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(part + (size_t)sp * slab + i8);
        const f32x4 d = *reinterpret_cast<const f32x4*>(part + (size_t)sp * slab + i8 + 4);
        a[0] += c[0]; a[1] += c[1]; a[2] += c[2]; a[3] += c[3];
        b[0] += d[0]; b[1] += d[1]; b[2] += d[2]; b[3] += d[3];
      }
      u32x4 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                 pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
      *reinterpret_cast<u32x4*>(y + i8) = o;
      return;
    }
  } else if (i8 + 8 <= mn) {
    f32x4 c[S], d[S];
#pragma unroll
    for (int sp = 0; sp < S; ++sp) {
      c[sp] = *reinterpret_cast<const f32x4*>(part + (size_t)sp * slab + i8);
      d[sp] = *reinterpret_cast<const f32x4*>(part + (size_t)sp * slab + i8 + 4);
    }
    f32x4 a = c[0], b = d[0];
#pragma unroll
    for (int sp = 1; sp < S; ++sp) {
      a[0] += c[sp][0]; a[1] += c[sp][1]; a[2] += c[sp][2]; a[3] += c[sp][3];
      b[0] += d[sp][0]; b[1] += d[sp][1]; b[2] += d[sp][2]; b[3] += d[sp][3];
    }
    u32x4 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
               pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
    *reinterpret_cast<u32x4*>(y + i8) = o;
    return;
  }
  if (i8 < mn) {
    for (size_t i = i8; i < mn; ++i) {
      float t = part[i];
      for (int sp = 1; sp < (S > 0 ? S : splits); ++sp) t += part[(size_t)sp * slab + i];
      const __bf16 v = (__bf16)t;
      y[i] = __builtin_bit_cast(uint16_t, v);
    }
  }
}

constexpr int kWaves = 4;

struct SkinnyPlan {
  int mt, nt, splits, ss_per_split;
};

// From measurements on MI355X (N=8000, K=8192): 4 waves per workgroup; 32
// weight rows per workgroup (two 16-row tiles sharing each X fragment)
// except for M <= 4, where X costs nothing and 16 rows per workgroup give
// twice the workgroups.
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k) {
  SkinnyPlan p;
  p.mt = m > 16 ? 2 : 1;
  p.nt = m > 4 ? 2 : 1;
  const int nss = (int)((k + kSuper - 1) / kSuper);
  const int64_t groups = (n + 16 * p.nt - 1) / (16 * p.nt);
  int splits = 1;
  // Split K only when there are too few row groups to occupy the GPU,
  // keeping >= 2 super-steps per wave.
  while (groups * splits < 192 && nss / (splits * 2) >= kWaves * 2) splits *= 2;
  p.ss_per_split = (nss + splits - 1) / splits;
  p.splits = (nss + p.ss_per_split - 1) / p.ss_per_split;
  return p;
}

}  // namespace

hipError_t launch_reduce_partials(const float* part, uint16_t* y, int splits,
                                  int64_t m, int64_t n, hipStream_t stream) {
  const size_t mn = (size_t)m * (size_t)n;
  const size_t blocks = (mn + 256 * 8 - 1) / (256 * 8);
  const size_t slab = partial_slab((size_t)m, (size_t)n);
  const dim3 grid((uint32_t)blocks);
  switch (splits) {
    case 2: hipLaunchKernelGGL(reduce_partials_kernel<2>, grid, dim3(256), 0, stream, part, y, splits, mn, slab); break;
    case 3: hipLaunchKernelGGL(reduce_partials_kernel<3>, grid, dim3(256), 0, stream, part, y, splits, mn, slab); break;
    case 4: hipLaunchKernelGGL(reduce_partials_kernel<4>, grid, dim3(256), 0, stream, part, y, splits, mn, slab); break;
    case 5: hipLaunchKernelGGL(reduce_partials_kernel<5>, grid, dim3(256), 0, stream, part, y, splits, mn, slab); break;
    case 6: hipLaunchKernelGGL(reduce_partials_kernel<6>, grid, dim3(256), 0, stream, part, y, splits, mn, slab); break;
    case 7: hipLaunchKernelGGL(reduce_partials_kernel<7>, grid, dim3(256), 0, stream, part, y, splits, mn, slab); break;
    case 8: hipLaunchKernelGGL(reduce_partials_kernel<8>, grid, dim3(256), 0, stream, part, y, splits, mn, slab); break;
    default: hipLaunchKernelGGL(reduce_partials_kernel<0>, grid, dim3(256), 0, stream, part, y, splits, mn, slab);
  }
  return hipGetLastError();
}

size_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  // Passes of up to 32 rows of X run one after another through the same
  // workspace; size for the widest pass.
  const int64_t rows = m < 32 ? m : 32;
  if (rows == 0) return 0;
  const SkinnyPlan p = plan_skinny(rows, n, k);
  if (p.splits <= 1) return 0;
  return round_up((size_t)p.splits * partial_slab(rows, n) * sizeof(float), kWorkspaceAlign);
}

hipError_t launch_gemm_skinny(const uint16_t* x, const uint8_t* q, const float* s,
                              uint16_t* y, int64_t m, int64_t n, int64_t k,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  const int gk = (int)((k + kBlock - 1) / kBlock);
  for (int64_t r0 = 0; r0 < m; r0 += 32) {
    const int64_t rows = (m - r0) < 32 ? (m - r0) : 32;
    const SkinnyPlan p = plan_skinny(rows, n, k);
    float* part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    if (p.splits > 1 && (ws == nullptr || ws_bytes < (size_t)p.splits * partial_slab(rows, n) * sizeof(float)))
      return hipErrorInvalidValue;
    const dim3 grid((uint32_t)((n + 16 * p.nt - 1) / (16 * p.nt)), (uint32_t)p.splits);
    const uint16_t* xp = x + (size_t)r0 * k;
    uint16_t* yp = y + (size_t)r0 * n;
    const dim3 block(kWaves * 64);
    if (p.mt == 1 && p.nt == 1)
      hipLaunchKernelGGL((gemm_skinny_kernel<1, 1, kWaves>), grid, block, 0, stream, xp, q, s, yp,
                         part, (int)rows, (int)n, (int)k, gk, p.ss_per_split);
    else if (p.mt == 1)
      hipLaunchKernelGGL((gemm_skinny_kernel<1, 2, kWaves>), grid, block, 0, stream, xp, q, s, yp,
                         part, (int)rows, (int)n, (int)k, gk, p.ss_per_split);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<2, 2, kWaves>), grid, block, 0, stream, xp, q, s, yp,
                         part, (int)rows, (int)n, (int)k, gk, p.ss_per_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.splits > 1) {
      e = launch_reduce_partials(part, yp, p.splits, rows, n, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace fp8bl
