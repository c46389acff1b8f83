// Skinny-M block-FP8 linear (M <= 32 per pass): the run is bound by the HBM
// bytes of the E4M3 weight, so the kernel is organised around streaming W
// once, at full bandwidth, with as many 16-byte loads in flight as possible.
//
// Same arithmetic as the tiled path (FastVideo PR #1829, "Purpose":
// dequantize to BF16 then a plain matmul; fp32 accumulation, one bf16
// rounding per output).
//
// Work unit: a workgroup owns 16*NT weight rows and one K range (its split);
// its 4 waves interleave over that range in 64-wide K steps, wave w taking
// steps w, w+4, w+8, ... so that at any moment the workgroup reads adjacent
// 64-byte pieces of the same rows. Each lane loads 16 codes (one row, 16
// consecutive k) per 16-row tile per step, dequantizes them in registers and
// feeds two v_mfma_f32_16x16x32_bf16 whose A operand is the matching X
// chunk (rows of X beyond M are zero). X is tiny and stays in L2; the NT
// tiles of a wave share each X fragment. At the end the 4 waves' partial
// sums meet in LDS and are added in wave order; with one split the result is
// rounded to bf16 directly, otherwise fp32 partials go to the workspace and
// are summed in split order by the reduce kernel (no atomics anywhere).
//
// v_mfma_f32_16x16x32_bf16: lane l gives 8 consecutive-k values of row
// (l % 16) of A and of column (l % 16) of B; lane group l / 16 picks the
// k chunk. Output: lane l holds rows (l/16)*4 + r, r = 0..3, column l % 16.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kStep = 64;       // K per MFMA pair
constexpr int kUnroll = 4;      // K steps a wave has in flight

template <int MT, int NT>
__global__ __launch_bounds__(kThreads)
void gemm_skinny_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                        const float* __restrict__ s, uint16_t* __restrict__ y,
                        float* __restrict__ part, int M, int N, int K, int gk,
                        int steps_per_split) {
  __shared__ f32x4 red[kWaves][MT * NT][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * (16 * NT);
  const int nsteps = (K + kStep - 1) / kStep;
  const int st0 = blockIdx.y * steps_per_split;
  const int st1 = min(st0 + steps_per_split, nsteps);

  const int lrow = lane & 15;           // row inside a 16-row tile
  const int lk = (lane >> 4) * 16;      // lane's 16-wide k chunk inside a step

  // Row pointers (rows past N read nothing).
  const uint8_t* wrow[NT];
  bool wok[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = n0 + j * 16 + lrow;
    wok[j] = r < N;
    wrow[j] = q + (size_t)(wok[j] ? r : 0) * K;
  }
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = i * 16 + lrow;
    xok[i] = r < M;
    xrow[i] = x + (size_t)(xok[i] ? r : 0) * K;
  }
  // Scale row of each 16-row tile (a tile never straddles a 128-row block).
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

  for (int st = st0 + wave; st < st1; st += kWaves * kUnroll) {
    u32x4 wv[kUnroll][NT];
    u32x4 xv[kUnroll][MT][2];
    // Issue every load of kUnroll steps before using any of them.
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int stu = st + u * kWaves;
      const int kk = stu * kStep + lk;
      const bool kin = stu < st1 && kk < K;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        wv[u][j] = (kin && wok[j]) ? __builtin_nontemporal_load(
                                         reinterpret_cast<const u32x4*>(wrow[j] + kk))
                                   : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (kin && xok[i]) {
          xv[u][i][0] = *reinterpret_cast<const u32x4*>(xrow[i] + kk);
          xv[u][i][1] = *reinterpret_cast<const u32x4*>(xrow[i] + kk + 8);
        } else {
          xv[u][i][0] = u32x4{0, 0, 0, 0};
          xv[u][i][1] = u32x4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int stu = st + u * kWaves;
      if (stu >= st1) break;
      const int kb = (stu * kStep) / kBlock;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sc = tile_live[j] ? s[srow[j] * gk + kb] : 0.0f;
        const bf16x8 b0 = dequant8(wv[u][j][0], wv[u][j][1], sc);
        const bf16x8 b1 = dequant8(wv[u][j][2], wv[u][j][3], sc);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, xv[u][i][0]), b0, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, xv[u][i][1]), b1, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // Cross-wave sum in wave order.
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[wave][i * NT + j][lane] = acc[i][j];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      f32x4 t = red[0][i * NT + j][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const f32x4 o = red[w][i * NT + j][lane];
        t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
      }
      const int col = n0 + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = i * 16 + (lane >> 4) * 4 + r;
        if (row >= M) continue;
        if (gridDim.y == 1) {
          const __bf16 v = (__bf16)t[r];
          y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, v);
        } else {
          part[((size_t)blockIdx.y * M + row) * N + col] = t[r];
        }
      }
    }
}

__global__ __launch_bounds__(256)
void reduce_partials_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                            int splits, size_t mn) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  float t = part[i];
  for (int sp = 1; sp < splits; ++sp) t += part[(size_t)sp * mn + i];
  const __bf16 v = (__bf16)t;
  y[i] = __builtin_bit_cast(uint16_t, v);
}

struct SkinnyPlan {
  int mt, nt, splits, steps_per_split;
};

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k) {
  SkinnyPlan p;
  p.mt = m > 16 ? 2 : 1;
  p.nt = 2;
  const int nsteps = (int)((k + kStep - 1) / kStep);
  const int64_t groups = (n + 16 * p.nt - 1) / (16 * p.nt);
  int splits = 1;
  // Aim for at least ~2 workgroups per CU; each split keeps >= 8 steps per wave.
  while (groups * splits < 480 && nsteps / (splits * 2) >= kWaves * 8) splits *= 2;
  p.steps_per_split = (nsteps + splits - 1) / splits;
  p.splits = (nsteps + p.steps_per_split - 1) / p.steps_per_split;
  return p;
}

}  // namespace

hipError_t launch_reduce_partials(const float* part, uint16_t* y, int splits,
                                  int64_t m, int64_t n, hipStream_t stream) {
  const size_t mn = (size_t)m * (size_t)n;
  const size_t blocks = (mn + 255) / 256;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     part, y, splits, mn);
  return hipGetLastError();
}

size_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  size_t total = 0;
  // Passes of up to 32 rows of X run one after another through the same
  // workspace; size for the widest pass.
  const int64_t rows = m < 32 ? m : 32;
  if (rows == 0) return 0;
  const SkinnyPlan p = plan_skinny(rows, n, k);
  if (p.splits > 1)
    total = round_up((size_t)p.splits * (size_t)rows * (size_t)n * sizeof(float), kWorkspaceAlign);
  return total;
}

hipError_t launch_gemm_skinny(const uint16_t* x, const uint8_t* q, const float* s,
                              uint16_t* y, int64_t m, int64_t n, int64_t k,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  const int gk = (int)((k + kBlock - 1) / kBlock);
  for (int64_t r0 = 0; r0 < m; r0 += 32) {
    const int64_t rows = (m - r0) < 32 ? (m - r0) : 32;
    const SkinnyPlan p = plan_skinny(rows, n, k);
    float* part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    if (p.splits > 1 && (ws == nullptr || ws_bytes < (size_t)p.splits * rows * n * sizeof(float)))
      return hipErrorInvalidValue;
    const dim3 grid((uint32_t)((n + 16 * p.nt - 1) / (16 * p.nt)), (uint32_t)p.splits);
    const uint16_t* xp = x + (size_t)r0 * k;
    uint16_t* yp = y + (size_t)r0 * n;
    if (p.mt == 1)
      hipLaunchKernelGGL((gemm_skinny_kernel<1, 2>), grid, dim3(kThreads), 0, stream,
                         xp, q, s, yp, part, (int)rows, (int)n, (int)k, gk, p.steps_per_split);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<2, 2>), grid, dim3(kThreads), 0, stream,
                         xp, q, s, yp, part, (int)rows, (int)n, (int)k, gk, p.steps_per_split);
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
