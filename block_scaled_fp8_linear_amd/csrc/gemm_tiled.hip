// Fused block-FP8 linear for large M: Y[M,N] = X[M,K] * W_hat[N,K]^T.
//
// FastVideo PR #1829, "Purpose": the Hopper route converts every layer's
// block-scaled weight to BF16 just ahead of an ordinary matmul. Here the
// BF16 weight never reaches memory: E4M3 codes go from HBM straight into
// the registers of the wave that consumes them, are dequantized there (fp32
// multiply by the block's weight_scale_inv, RNE to bf16) and fed to bf16
// MFMA with fp32 accumulators (LightX2V PR #1657, "Walkthrough": FP32
// accumulation).
//
// Workgroup tile BM x BN, W waves side by side along N: wave w owns the
// BN/W weight rows [n0 + w*BN/W, ...) for all BM rows of X (W = 4, or 8 for
// the 128x256 and 256x256 tiles, where each wave keeps one 32-column block). Every weight
// element is therefore decoded exactly once per workgroup (decode VALU per
// MFMA flop falls as 1/BM), while the X tile is shared through LDS, staged
// with 16-byte loads into an XOR-swizzled layout that the MFMA operand reads
// hit without bank conflicts. A wave's rows lie inside one 128-row scale
// block and a 64-wide K step inside one 128-column block, so each wave needs
// one scalar scale per K step.
//
// Pipeline (one barrier per K step): a wave dequantizes the codes of step k
// (loaded one step earlier), issues the loads of X and codes for step k+1,
// runs step k's MFMAs from LDS and the decoded registers, then stages X for
// step k+1 into the other LDS buffer. Two or three workgroups share each CU
// (three with 128x128 tiles), so one workgroup's decode overlaps another's
// MFMAs. The 128x256 and 256x256 tiles run 8 waves of one 32-column block
// each (128x256: about 130 VGPRs, two workgroups per CU; 256x256: about 200
// VGPRs, one). For 128x256, per 128x128x64 step of work it moves
// 16 KB of X and codes through the CU's vector-memory path against 24 KB
// for two 128x128 workgroups, which measured 2-6% faster than both the
// 4-wave 128x256 tile and 128x128 on the shapes that choose it (the load
// path of a CU, not the matrix core, limits these kernels: the time to
// issue a step's loads grows with the workgroups sharing the CU). Loads go
// through buffer descriptors covering only the tile's valid rows: rows past
// M or N and the K tail read as zero without branches. (Measured alternatives that did not
// pay on MI355X: decoding step k+1 inside step k's MFMA stream with two
// operand sets, and prefetching two steps ahead.)
//
// MFMA v_mfma_f32_32x32x16_bf16 (gfx950): lane l supplies 8 consecutive-k
// bf16 of row (l % 32) for A and of column (l % 32) for B; the two half-waves
// (l / 32) take different 8-wide k chunks. Both operands are K-contiguous in
// memory (X row-major, W row-major [N,K]), so no transpose is needed. A
// 16-byte load of codes gives a lane the k chunks of two consecutive MFMAs;
// the matching X chunks are read from LDS with the same permutation of k.
//
// Split-K (gridDim.y > 1): every split writes an fp32 partial tile to the
// workspace and a second kernel adds the splits in split order
// (deterministic) and rounds once to bf16. (Finishing the sum inside the
// GEMM with a per-tile arrival counter needs a device-scope release/acquire
// per workgroup, which on this multi-XCD part means an L2 write-back and
// invalidate each time; measured about 3x slower than the second kernel.)
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

constexpr int kBK = 64;           // K per pipeline step
constexpr int kThreads = 256;     // 4 waves
constexpr uint32_t kOob = 0x80000000u;   // buffer offset past every valid range

// XOR swizzle of 16-byte chunks inside a 128-byte LDS row (64 bf16 of K).
// gfx950's LDS has 64 four-byte banks: two consecutive 128-byte rows fill
// all of them, and a 16-byte read is served 16 lanes at a time. The MFMA
// operand read has 16 lanes on 16 consecutive rows at one logical chunk;
// XOR-ing the chunk with (row / 2) % 8 gives those lanes 16 distinct
// 16-byte bank groups (row parity picks the half, the XOR the group), so
// reads and the row-wise staging writes are conflict-free.
__device__ __forceinline__ int xs_offset(int row, int chunk) {
  return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: raw (untyped) buffer, 32-bit data format, the
  // layout gfx9-family descriptors use; out-of-range reads return zero.
  // The size is wave-uniform, but without the readfirstlane the compiler
  // computed it in VALU for the weight descriptor and wrapped every weight
  // load in a waterfall loop.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Order of a step's MFMA phase: the X fragment reads (one ds_read_b128 per
// fragment, 4 * MB per step) run kReadsAhead fragments in front of the MFMAs
// that consume them, each fragment feeding PER_FRAG MFMAs. Left to itself
// the compiler issued each read pair right before its MFMAs and waited for
// it there, exposing the LDS latency every few MFMAs (measured 2-6% slower
// across the workloads).
template <int MB, int PER_FRAG>
__device__ __forceinline__ void schedule_operand_reads() {
  constexpr int kReadsAhead = 4;
  __builtin_amdgcn_sched_group_barrier(0x100, kReadsAhead, 0);     // DS reads
#pragma unroll
  for (int i = 0; i < 4 * MB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, PER_FRAG, 0);      // MFMAs
    if (i + kReadsAhead < 4 * MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// GATED: the MLP gate/up pair in one pass. The same X tile feeds two weights
// (q, s = gate; q2, s2 = up) into two accumulator sets and the epilogue
// writes swiglu(gate, up) instead of either product.
template <int BM, int BN, bool GATED, int WAVES, bool PAIRED = false>
__device__ __forceinline__
void tiled_body(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                const float* __restrict__ s, uint16_t* __restrict__ y,
                float* __restrict__ part, int M, int N, int K, int gk,
                int tiles_m, int tiles_n, int kt_per_split,
                const uint8_t* __restrict__ q2, const float* __restrict__ s2) {
  constexpr int kT = WAVES * 64;        // threads
  constexpr int WN = BN / WAVES;        // weight rows per wave
  constexpr int NB = WN / 32;           // 32-wide MFMA column blocks per wave
  constexpr int MB = BM / 32;           // 32-tall MFMA row blocks
  constexpr int XCH = BM * kBK / 8 / kT;  // 16-byte X chunks per thread per step
  static_assert(WN % 32 == 0 && 128 % WN == 0, "wave rows must sit in one scale block");
  static_assert(XCH >= 1, "tile too small");
  // PAIRED: the first WAVES/2 waves run weight (q, s) and the others weight
  // (q2, s2), over the same BN/2 output columns of the tile.
  constexpr int BNO = PAIRED ? BN / 2 : BN;   // output columns per tile
  static_assert(!(PAIRED && GATED), "one pairing mode at a time");
  static_assert(!PAIRED || 2 * kBK >= BNO, "the exchange tile must fit the X buffers");

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Work order: consecutive workgroups (in dispatch order, x fastest) are
  // dealt round-robin to the 8 XCDs; renumber so each XCD gets a contiguous
  // run of (split, tile) units, split-major, then walk the tiles in groups of
  // 8 M-tiles so concurrently running tiles share X and W in that XCD's L2.
  // Split-major keeps an XCD on one or two K ranges: with the splits of a
  // tile on one XCD (tile-major), every XCD read all of X over all of K
  // (512 x 5120 x 5120 in 3 splits: 74 MB fetched for 31 MB of X and W).
  const int ntiles = tiles_m * tiles_n;
  const int units = ntiles * (int)gridDim.y;
  int id = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
  if ((units & 7) == 0) id = (id & 7) * (units >> 3) + (id >> 3);
  const int split = id / ntiles;
  id -= split * ntiles;
  constexpr int GM = 8;
  const int group = id / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = id - group * GM * tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * BM;
  const int n0 = tn * BNO;

  const int nkt = (K + kBK - 1) / kBK;
  const int kt0 = split * kt_per_split;
  const int kt1 = min(kt0 + kt_per_split, nkt);

  // ---- X: thread moves chunk (tid & 7) of tile rows (tid >> 3) + (kT / 8) i.
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(x + (size_t)m0 * K, (uint32_t)(min(M - m0, BM) * K * 2));
  const int xc = tid & 7;
  const int xr0 = tid >> 3;
  const uint32_t xoff0 = (uint32_t)(xr0 * K * 2 + xc * 16);
  const uint32_t xrow_stride = (uint32_t)((kT / 8) * K * 2);

  // ---- W codes: lane holds 16 codes of row (lane % 32) of each column
  // block, k chunk (lane / 32) of each 32-wide k slab.
  const bool upper = PAIRED && wave >= WAVES / 2;
  const int wslot = upper ? wave - WAVES / 2 : wave;   // column slot of the wave's rows
  const uint8_t* __restrict__ qw = upper ? q2 : q;
  const float* __restrict__ sw = upper ? s2 : s;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(qw + (size_t)n0 * K, (uint32_t)(max(min(N - n0, BNO), 0) * K));
  const __amdgpu_buffer_rsrc_t wrs2 =
      make_rsrc((GATED ? q2 : q) + (size_t)n0 * K, (uint32_t)(max(min(N - n0, BN), 0) * K));
  const int wkoff = (lane >> 5) * 16;
  const uint32_t woff0 = (uint32_t)((wslot * WN + (lane & 31)) * K + wkoff);
  const uint32_t wnb_stride = (uint32_t)(32 * K);
  const int srow = (n0 + wslot * WN) / kBlock;
  const bool wave_live = (n0 + wslot * WN) < N;

  u32x4 xreg[XCH];
  auto load_x = [&](int kt) {
    const bool kin = kt < kt1 && kt * kBK + xc * 8 < K;
    const uint32_t base = kin ? xoff0 + (uint32_t)(kt * kBK * 2) : kOob;
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      xreg[i] = buf_load16(xrs, kin ? base + i * xrow_stride : kOob);
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      *reinterpret_cast<u32x4*>(&xs[buf][xs_offset(xr0 + (kT / 8) * i, xc)]) = xreg[i];
  };
  auto load_w = [&](u32x4 (&wr)[NB][2], int kt) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const bool kin = kt < kt1 && kt * kBK + sl * 32 + wkoff < K;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        wr[nb][sl] = buf_load16(wrs, kin ? woff0 + nb * wnb_stride + (uint32_t)(kt * kBK + sl * 32)
                                         : kOob);
    }
  };
  auto scale_of = [&](int kt) -> float {
    // always a valid address (clamped block column), zero for dead waves
    const int kb = min((kt * kBK) / kBlock, gk - 1);
    const float v = sw[(wave_live ? srow : 0) * gk + kb];
    return wave_live ? v : 0.0f;
  };
  // The same two for the second (up) weight of a gated tile.
  auto load_w2 = [&](u32x4 (&wr)[NB][2], int kt) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const bool kin = kt < kt1 && kt * kBK + sl * 32 + wkoff < K;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        wr[nb][sl] = buf_load16(wrs2, kin ? woff0 + nb * wnb_stride + (uint32_t)(kt * kBK + sl * 32)
                                          : kOob);
    }
  };
  auto scale2_of = [&](int kt) -> float {
    const int kb = min((kt * kBK) / kBlock, gk - 1);
    const float v = s2[(wave_live ? srow : 0) * gk + kb];
    return wave_live ? v : 0.0f;
  };
  // Dequantize the k16 step t of a code set into B operands.
  auto decode_t = [&](bf16x8 (&wb)[NB][4], const u32x4 (&wr)[NB][2], float sc, int t) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      wb[nb][t] = dequant8(wr[nb][t >> 1][(t & 1) * 2], wr[nb][t >> 1][(t & 1) * 2 + 1], sc);
  };

  constexpr int MB2 = GATED ? MB : 1, NB2 = GATED ? NB : 1;
  f32x16 acc[MB][NB];
  f32x16 acc2[MB2][NB2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if constexpr (GATED) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc2[i][j][r] = 0.0f;
  }

  auto mfma_step = [&](int cur, bf16x8 (&wb)[NB][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int chunk = (t >> 1) * 4 + (lane >> 5) * 2 + (t & 1);
      bf16x8 a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(&xs[cur][xs_offset(mb * 32 + (lane & 31), chunk)]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], wb[nb][t], acc[mb][nb], 0, 0, 0);
    }
    schedule_operand_reads<MB, NB>();
  };
  // Gated step: each X fragment read from LDS feeds both weights.
  auto mfma_step2 = [&](int cur, bf16x8 (&wb)[NB][4], bf16x8 (&wb2)[NB2][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int chunk = (t >> 1) * 4 + (lane >> 5) * 2 + (t & 1);
      bf16x8 a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(&xs[cur][xs_offset(mb * 32 + (lane & 31), chunk)]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], wb[nb][t], acc[mb][nb], 0, 0, 0);
          acc2[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], wb2[nb][t], acc2[mb][nb], 0, 0, 0);
        }
    }
    schedule_operand_reads<MB, 2 * NB>();
  };

  {
    // Decode this step's codes, prefetch the next step, then the MFMAs;
    // the other resident workgroup's waves cover the decode.
    u32x4 wr[NB][2], wr2[NB2][2];
    bf16x8 wb[NB][4], wb2[NB2][4];
    if (kt0 < kt1) {
      load_x(kt0);
      load_w(wr, kt0);
      if constexpr (GATED) load_w2(wr2, kt0);
      store_x(0);
    }
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const float sc = scale_of(kt);
#pragma unroll
      for (int t = 0; t < 4; ++t) decode_t(wb, wr, sc, t);
      if constexpr (GATED) {
        const float sc2 = scale2_of(kt);
#pragma unroll
        for (int t = 0; t < 4; ++t) decode_t(wb2, wr2, sc2, t);
      }
      // Branch-free step (one basic block for the scheduler): past the last
      // step these loads read zero and the staged tile goes unused. X is
      // issued first: its staging at the end of this step then waits only
      // for the X loads, and the code loads stay in flight across the
      // barrier until the next step's decode needs them.
      load_x(kt + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_w(wr, kt + 1);
      if constexpr (GATED) load_w2(wr2, kt + 1);
      // Raise this wave's issue priority while it feeds the matrix core, so
      // the other workgroup's decode fills VALU slots around it.
      __builtin_amdgcn_s_setprio(1);
      if constexpr (GATED)
        mfma_step2(cur, wb, wb2);
      else
        mfma_step(cur, wb);
      __builtin_amdgcn_s_setprio(0);
      store_x(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- Epilogue. acc[mb][nb][r] holds row mb*32 + (r/4)*8 + (l/32)*4 + r%4,
  // column nb*32 + l%32 of the wave's sub-tile.
  const int col_base = n0 + wslot * WN + (lane & 31);
  const int row_base = m0 + (lane >> 5) * 4;
  if constexpr (PAIRED) {
    // The upper waves hand their products, rounded to bf16 (the rounding the
    // SwiGLU applies to them first anyway), to the lower waves through the X
    // buffers: a BM x BNO bf16 tile.
    uint16_t* ex = &xs[0][0];
    const int exc = wslot * WN + (lane & 31);
    __syncthreads();
    if (upper) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = mb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            ex[rl * BNO + exc + nb * 32] = __builtin_bit_cast(uint16_t, (__bf16)acc[mb][nb][r]);
          }
    }
    __syncthreads();
    if (!upper) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = col_base + nb * 32;
          if (col >= N) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = mb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (m0 + rl < M) {
              const float u = __builtin_bit_cast(float, (uint32_t)ex[rl * BNO + exc + nb * 32] << 16);
              y[(size_t)(m0 + rl) * N + col] = swiglu_bf16(acc[mb][nb][r], u);
            }
          }
        }
    }
    return;
  }
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
            if constexpr (GATED) {
              y[(size_t)row * N + col] = swiglu_bf16(acc[mb][nb][r], acc2[mb][nb][r]);
            } else {
              const __bf16 v = (__bf16)acc[mb][nb][r];
              y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, v);
            }
          }
        }
      }
  } else {
    // Split-K: this split's fp32 partial tile; a second kernel adds the
    // splits in order and rounds once.
    float* p = part + (size_t)split * partial_slab(M, N);
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

template <int BM, int BN, int MINB, int WAVES>
__global__ __launch_bounds__(WAVES * 64, MINB)
void gemm_tiled_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                       const float* __restrict__ s, uint16_t* __restrict__ y,
                       float* __restrict__ part, int M, int N, int K, int gk,
                       int tiles_m, int tiles_n, int kt_per_split) {
  tiled_body<BM, BN, false, WAVES>(x, q, s, y, part, M, N, K, gk, tiles_m, tiles_n, kt_per_split,
                                   nullptr, nullptr);
}

template <int BM, int BN, int MINB>
__global__ __launch_bounds__(kThreads, MINB)
void gemm_gated_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ qg,
                       const float* __restrict__ sg, const uint8_t* __restrict__ qu,
                       const float* __restrict__ su, uint16_t* __restrict__ h, int M, int N,
                       int K, int gk, int tiles_m, int tiles_n) {
  tiled_body<BM, BN, true, 4>(x, qg, sg, h, nullptr, M, N, K, gk, tiles_m, tiles_n,
                              (K + kBK - 1) / kBK, qu, su);
}

template <int BM, int BN, int MINB>
__global__ __launch_bounds__(512, MINB)
void gemm_gated_paired_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ qg,
                              const float* __restrict__ sg, const uint8_t* __restrict__ qu,
                              const float* __restrict__ su, uint16_t* __restrict__ h, int M, int N,
                              int K, int gk, int tiles_m, int tiles_n) {
  tiled_body<BM, BN, false, 8, true>(x, qg, sg, h, nullptr, M, N, K, gk, tiles_m, tiles_n,
                                     (K + kBK - 1) / kBK, qu, su);
}

struct TiledPlan {
  int cfg;          // 0: 128x256, 1: 256x128, 2: 128x128, 3: 256x256
  int bm, bn, splits, kt_per_split;
};

// Tile and split choice from a cost model fitted to measurements on MI355X.
// Work is counted in 128x128x64 MFMA steps; a CU runs its workgroups one
// (256x256 of 8 waves, ~200 VGPRs), two (128x256 of 8 waves, 256x128 of 4
// waves with 210+ VGPRs) or three (128x128) at a time, and its throughput
// depends on how many it holds (steps per microsecond, below).
// The busiest CU sets the time: ceil(W / 256) workgroups of W, each taking
// ceil(nkt / splits) steps. K splits add the fp32 partials' round trip
// (4 bytes per output and split written and read back, 2 bytes of bf16
// out, at ~5 TB/s). Large shapes favour the 256x256 tile (each step moves
// 12 KB of X and codes per 128x128x64 of work through the CU, against 16 KB
// for 128x256 and 24 KB for 128x128); shapes whose 128x128 tiles fill the
// CUs more evenly (e.g. 2048x5120x5120, 3072^3) favour 128x128; 512-row
// text-encoder shapes with few tiles split K.
double cu_rate(int cfg, int64_t per_cu) {
  if (cfg == 2) return per_cu <= 1 ? 0.91 : per_cu == 2 ? 1.56 : 1.70;
  if (cfg == 0) return per_cu <= 1 ? 1.69 : 1.90;
  if (cfg == 3) return 2.00;   // one workgroup per CU at a time
  return per_cu <= 1 ? 1.44 : 1.90;
}

TiledPlan plan_tiled(int64_t m, int64_t n, int64_t k, double* cost_out = nullptr) {
  const int nkt = (int)((k + kBK - 1) / kBK);
  // evaluation order breaks ties: 256x128 first below 2048 rows
  const int order_small[4] = {1, 0, 2, 3}, order_large[4] = {3, 0, 1, 2};
  const int* order = m < 2048 ? order_small : order_large;
  TiledPlan best{2, 128, 128, 1, nkt};
  double best_cost = 1e30;
  for (int oi = 0; oi < 4; ++oi) {
    const int cfg = order[oi];
    const int bm = (cfg == 1 || cfg == 3) ? 256 : 128, bn = (cfg == 0 || cfg == 3) ? 256 : 128;
    const int units = cfg == 2 ? 1 : cfg == 3 ? 4 : 2;
    const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
    for (int sp = 1; sp <= 8; ++sp) {
      const int steps = (nkt + sp - 1) / sp;
      if (sp > 1 && steps < 8) break;
      const int64_t per_cu = (tiles * sp + 255) / 256;
      double cost = (double)per_cu * steps * units / cu_rate(cfg, per_cu);
      if (sp > 1) cost += (double)(6 * sp + 2) * (double)(m * n) / 5.0e6;
      if (cost < best_cost) {
        best_cost = cost;
        best = TiledPlan{cfg, bm, bn, sp, steps};
      }
    }
  }
  best.kt_per_split = best.splits > 1 ? (nkt + best.splits - 1) / best.splits : nkt;
  best.splits = (nkt + best.kt_per_split - 1) / best.kt_per_split;
  if (cost_out) *cost_out = best_cost;
  return best;
}

}  // namespace

double tiled_cost(int64_t m, int64_t n, int64_t k) {
  double c = 0.0;
  (void)plan_tiled(m, n, k, &c);
  return c;
}

// Workspace: the fp32 partials of every split.
size_t tiled_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const TiledPlan p = plan_tiled(m, n, k);
  if (p.splits <= 1) return 0;
  return round_up((size_t)p.splits * partial_slab(m, n) * sizeof(float), kWorkspaceAlign);
}

hipError_t launch_gemm_tiled(const uint16_t* x, const uint8_t* q, const float* s,
                             uint16_t* y, int64_t m, int64_t n, int64_t k,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  const TiledPlan p = plan_tiled(m, n, k);
  const int gk = (int)((k + kBlock - 1) / kBlock);
  const int tiles_m = (int)((m + p.bm - 1) / p.bm);
  const int tiles_n = (int)((n + p.bn - 1) / p.bn);
  float* part = nullptr;
  if (p.splits > 1) {
    if (ws == nullptr || ws_bytes < tiled_workspace_bytes(m, n, k)) return hipErrorInvalidValue;
    part = static_cast<float*>(ws);
  }
  const dim3 grid((uint32_t)(tiles_m * tiles_n), (uint32_t)p.splits);
  if (p.cfg == 0)
    hipLaunchKernelGGL((gemm_tiled_kernel<128, 256, 2, 8>), grid, dim3(512), 0, stream,
                       x, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                       p.kt_per_split);
  else if (p.cfg == 3)
    hipLaunchKernelGGL((gemm_tiled_kernel<256, 256, 1, 8>), grid, dim3(512), 0, stream,
                       x, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                       p.kt_per_split);
  else if (p.cfg == 1)
    hipLaunchKernelGGL((gemm_tiled_kernel<256, 128, 2, 4>), grid, dim3(kThreads), 0, stream,
                       x, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                       p.kt_per_split);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<128, 128, 2, 4>), grid, dim3(kThreads), 0, stream,
                       x, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                       p.kt_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_reduce_partials(part, y, p.splits, m, n, stream);
}

// Gate/up pair, never split (the SwiGLU needs whole sums). Two kernels:
//  - from 2048 rows, 128x128 tiles of four waves that each run both weights
//    (two accumulator sets fed by one X fragment read), two workgroups per
//    CU: X is staged once for both weights;
//  - below that, a paired tile of eight waves, the first four running gate
//    rows and the other four the matching up rows of the same 128 output
//    columns, one accumulator set per wave; the up half hands its bf16
//    products to the gate half through LDS for the SwiGLU. Its 256-row
//    (one workgroup per CU) or 128-row (two) form is picked by the tiled
//    planner's kind of cost model, with per-CU rates fitted to measurements
//    on MI355X (steps of 128x128x64 per microsecond).
// Same-box A/B (bit-identical outputs): the paired tile is 5% faster on
// 512x25600x5120, up to 11% on shapes of a few hundred rows and 1-4% at
// 1024-1536 rows (one shape within 1% the other way); the two-weight tile
// is 2-6% faster from 2048 rows. An eight-wave 128x256
// tile with both weights in every wave measured slower than both.
namespace {

// The gate/up planner's choice: 0 = two-weight tile, 1 = 256-row paired tile,
// 2 = 128-row paired tile; its time estimate (planner units) in *cost.
int plan_mlp(int64_t m, int64_t n, int64_t k, double* cost) {
  const int64_t nkt = (k + 63) / 64;
  const int64_t tiles_n = (n + 127) / 128;
  if (m >= 2048) {
    const int64_t per_cu = ((m + 127) / 128 * tiles_n + 511) / 512;
    *cost = (double)(per_cu * nkt) * 4 / 2.0;
    return 0;
  }
  const int64_t per_cu256 = ((m + 255) / 256 * tiles_n + 255) / 256;
  const int64_t per_cu128 = ((m + 127) / 128 * tiles_n + 255) / 256;
  const double cost256 = (double)per_cu256 * 4 / 2.2;
  const double cost128 = (double)per_cu128 * 2 / (per_cu128 <= 1 ? 1.51 : 2.09);
  *cost = (double)nkt * (cost256 < cost128 ? cost256 : cost128);
  return cost256 < cost128 ? 1 : 2;
}

}  // namespace

double mlp_tiled_cost(int64_t m, int64_t n, int64_t k) {
  double c = 0;
  plan_mlp(m, n, k, &c);
  return c;
}

hipError_t launch_mlp_gate_up(const uint16_t* x, const uint8_t* qg, const float* sg,
                              const uint8_t* qu, const float* su, uint16_t* h,
                              int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const int gk = (int)((k + kBlock - 1) / kBlock);
  const int tiles_n = (int)((n + 127) / 128);
  double cost = 0;
  const int kind = plan_mlp(m, n, k, &cost);
  if (kind == 0) {
    const int tiles_m = (int)((m + 127) / 128);
    hipLaunchKernelGGL((gemm_gated_kernel<128, 128, 2>), dim3((uint32_t)(tiles_m * tiles_n), 1),
                       dim3(kThreads), 0, stream, x, qg, sg, qu, su, h, (int)m, (int)n, (int)k,
                       gk, tiles_m, tiles_n);
    return hipGetLastError();
  }
  const int tm256 = (int)((m + 255) / 256), tm128 = (int)((m + 127) / 128);
  if (kind == 1)
    hipLaunchKernelGGL((gemm_gated_paired_kernel<256, 256, 1>),
                       dim3((uint32_t)(tm256 * tiles_n), 1), dim3(512), 0, stream, x, qg, sg, qu,
                       su, h, (int)m, (int)n, (int)k, gk, tm256, tiles_n);
  else
    hipLaunchKernelGGL((gemm_gated_paired_kernel<128, 256, 2>),
                       dim3((uint32_t)(tm128 * tiles_n), 1), dim3(512), 0, stream, x, qg, sg, qu,
                       su, h, (int)m, (int)n, (int)k, gk, tm128, tiles_n);
  return hipGetLastError();
}

}  // namespace fp8bl
