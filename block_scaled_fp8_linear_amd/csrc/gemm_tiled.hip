// Fused block-FP8 linear for large M: Y[M,N] = X[M,K] * W_hat[N,K]^T.
//
// FastVideo PR #1829, "Purpose": each linear dequantizes its block-scaled
// weight to BF16 right before a plain matmul. Here the BF16 weight never
// reaches memory: E4M3 codes go from HBM straight into the registers of the
// wave that consumes them, are dequantized there (fp32 multiply by the
// block's weight_scale_inv, RNE to bf16) and fed to bf16 MFMA with fp32
// accumulators (LightX2V PR #1657, "Walkthrough": FP32 accumulation).
//
// Workgroup tile BM x BN, 4 waves side by side along N: wave w owns the
// BN/4 weight rows [n0 + w*BN/4, ...) for all BM rows of X. So every weight
// element is decoded exactly once per workgroup (decode cost per MFMA flop
// falls as 1/BM), while the X tile is shared through LDS, staged with
// 16-byte loads into an XOR-swizzled layout that the MFMA operand reads hit
// without bank conflicts. A wave's rows lie inside one 128-row scale block
// and a 64-wide K step inside one 128-column block, so each wave needs one
// scalar scale per K step.
//
// MFMA v_mfma_f32_32x32x16_bf16 (gfx950): lane l supplies 8 consecutive-k
// bf16 of row (l % 32) for A and of column (l % 32) for B; the two half-waves
// (l / 32) take different 8-wide k chunks. Both operands are K-contiguous in
// memory (X row-major, W row-major [N,K]), so no transpose is needed. A
// 16-byte load of codes gives a lane the k chunks of two consecutive MFMAs;
// the matching X chunks are read from LDS with the same permutation of k.
//
// Split-K (gridDim.y > 1) writes fp32 partials that a second kernel sums in
// split order (deterministic) and rounds once to bf16.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

constexpr int kBK = 64;           // K per pipeline step
constexpr int kThreads = 256;     // 4 waves

// XOR swizzle of 16-byte chunks inside a 128-byte LDS row (64 bf16 of K).
__device__ __forceinline__ int xs_offset(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

template <int BM, int BN, int MINB>
__global__ __launch_bounds__(kThreads, MINB)
void gemm_tiled_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                       const float* __restrict__ s, uint16_t* __restrict__ y,
                       float* __restrict__ part, int M, int N, int K, int gk,
                       int tiles_m, int tiles_n, int kt_per_split) {
  constexpr int WN = BN / 4;            // weight rows per wave
  constexpr int NB = WN / 32;           // 32-wide MFMA column blocks per wave
  constexpr int MB = BM / 32;           // 32-tall MFMA row blocks
  constexpr int XCH = BM * kBK / 8 / kThreads;  // 16-byte X chunks per thread per step
  static_assert(WN % 32 == 0 && 128 % WN == 0, "wave rows must sit in one scale block");
  static_assert(XCH >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Tile order: consecutive workgroups are dealt round-robin to the 8 XCDs;
  // renumber so each XCD gets a contiguous run of tiles, then walk the run
  // in groups of 8 M-tiles so concurrently running tiles share X and W in
  // that XCD's L2.
  const int ntiles = tiles_m * tiles_n;
  int id = blockIdx.x;
  if ((ntiles & 7) == 0) id = (id & 7) * (ntiles >> 3) + (id >> 3);
  constexpr int GM = 8;
  const int group = id / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = id - group * GM * tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int nkt = (K + kBK - 1) / kBK;
  const int kt0 = blockIdx.y * kt_per_split;
  const int kt1 = min(kt0 + kt_per_split, nkt);

  // ---- X staging: thread handles chunk (tid & 7) of rows (tid >> 3) + 32 i.
  const int xc = tid & 7;
  const int xr0 = tid >> 3;
  u32x4 xreg[XCH];
  auto load_x = [&](int kt) {
    const int kk = kt * kBK + xc * 8;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int row = m0 + xr0 + 32 * i;
      if (row < M && kk < K)
        xreg[i] = *reinterpret_cast<const u32x4*>(x + (size_t)row * K + kk);
      else
        xreg[i] = u32x4{0, 0, 0, 0};
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      *reinterpret_cast<u32x4*>(&xs[buf][xs_offset(xr0 + 32 * i, xc)]) = xreg[i];
  };

  // ---- W codes: lane holds 16 codes of row (lane % 32) of each column
  // block, k chunk (lane / 32) of each 32-wide k slab.
  const int wrow0 = n0 + wave * WN + (lane & 31);
  const int wkoff = (lane >> 5) * 16;
  u32x4 wreg[NB][2];
  auto load_w = [&](int kt) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int row = wrow0 + nb * 32;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int kk = kt * kBK + sl * 32 + wkoff;
        if (row < N && kk < K)
          wreg[nb][sl] = *reinterpret_cast<const u32x4*>(q + (size_t)row * K + kk);
        else
          wreg[nb][sl] = u32x4{0, 0, 0, 0};
      }
    }
  };
  const int srow = (n0 + wave * WN) / kBlock;
  const bool wave_live = (n0 + wave * WN) < N;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (kt0 < kt1) {
    load_x(kt0);
    load_w(kt0);
    store_x(0);
  }
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    // Dequantize this step's codes into MFMA B operands.
    const float sc = wave_live ? s[srow * gk + (kt * kBK) / kBlock] : 0.0f;
    bf16x8 wb[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        wb[nb][sl * 2 + 0] = dequant8(wreg[nb][sl][0], wreg[nb][sl][1], sc);
        wb[nb][sl * 2 + 1] = dequant8(wreg[nb][sl][2], wreg[nb][sl][3], sc);
      }
    // Prefetch the next step while this one computes.
    const bool more = kt + 1 < kt1;
    if (more) {
      load_x(kt + 1);
      load_w(kt + 1);
    }
    // k16 step t = slab * 2 + half; lane reads X row (l % 32), k chunk
    // slab*32 + (l/32)*16 + half*8 -> 16-byte chunk index slab*4 + (l/32)*2 + half.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int chunk = (t >> 1) * 4 + (lane >> 5) * 2 + (t & 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = mb * 32 + (lane & 31);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[cur][xs_offset(row, chunk)]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wb[nb][t], acc[mb][nb], 0, 0, 0);
      }
    }
    if (more) store_x(cur ^ 1);
    __syncthreads();
  }

  // ---- Epilogue. acc[mb][nb][r] holds row mb*32 + (r/4)*8 + (l/32)*4 + r%4,
  // column nb*32 + l%32 of the wave's sub-tile.
  const int col_base = n0 + wave * WN + (lane & 31);
  const int row_base = m0 + (lane >> 5) * 4;
  if (gridDim.y == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = col_base + nb * 32;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_base + mb * 32 + (r >> 2) * 8 + (r & 3);
          if (row < M) {
            const __bf16 v = (__bf16)acc[mb][nb][r];
            y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, v);
          }
        }
      }
  } else {
    float* p = part + (size_t)blockIdx.y * M * N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = col_base + nb * 32;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_base + mb * 32 + (r >> 2) * 8 + (r & 3);
          if (row < M) p[(size_t)row * N + col] = acc[mb][nb][r];
        }
      }
  }
}

struct TiledPlan {
  int bm, bn, splits, kt_per_split;
};

TiledPlan plan_tiled(int64_t m, int64_t n, int64_t k) {
  const int nkt = (int)((k + kBK - 1) / kBK);
  TiledPlan p{256, 256, 1, nkt};
  const int64_t tiles_big = ((m + 255) / 256) * ((n + 255) / 256);
  if (tiles_big < 512) {
    p.bm = 128;
    p.bn = 128;
  }
  const int64_t tiles = ((m + p.bm - 1) / p.bm) * ((n + p.bn - 1) / p.bn);
  // Too few tiles to fill 256 CUs: split K (partials summed in order).
  int splits = 1;
  while (tiles * splits < 200 && splits < 8 && nkt / (splits * 2) >= 8) splits *= 2;
  p.splits = splits;
  p.kt_per_split = (nkt + splits - 1) / splits;
  p.splits = (nkt + p.kt_per_split - 1) / p.kt_per_split;
  return p;
}

}  // namespace

size_t tiled_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const TiledPlan p = plan_tiled(m, n, k);
  if (p.splits <= 1) return 0;
  return round_up((size_t)p.splits * (size_t)m * (size_t)n * sizeof(float), kWorkspaceAlign);
}

hipError_t launch_gemm_tiled(const uint16_t* x, const uint8_t* q, const float* s,
                             uint16_t* y, int64_t m, int64_t n, int64_t k,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  const TiledPlan p = plan_tiled(m, n, k);
  const int gk = (int)((k + kBlock - 1) / kBlock);
  const int tiles_m = (int)((m + p.bm - 1) / p.bm);
  const int tiles_n = (int)((n + p.bn - 1) / p.bn);
  float* part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
  if (p.splits > 1 && (ws == nullptr || ws_bytes < tiled_workspace_bytes(m, n, k)))
    return hipErrorInvalidValue;
  const dim3 grid((uint32_t)(tiles_m * tiles_n), (uint32_t)p.splits);
  if (p.bm == 256)
    hipLaunchKernelGGL((gemm_tiled_kernel<256, 256, 1>), grid, dim3(kThreads), 0, stream,
                       x, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                       p.kt_per_split);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<128, 128, 2>), grid, dim3(kThreads), 0, stream,
                       x, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                       p.kt_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_reduce_partials(part, y, p.splits, m, n, stream);
}

}  // namespace fp8bl
