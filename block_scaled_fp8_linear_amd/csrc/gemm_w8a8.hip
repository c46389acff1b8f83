// W8A8 block-scaled GEMM on the gfx950 FP8 matrix cores:
//   Y[m,n] = bf16( sum_kb xs[kb,m] * S[n/128,kb] * sum_{k in kb} e4m3(XQ[m,k]) e4m3(Q[n,k]) )
// with the weight in the converter's format (E4M3 + fp32 weight_scale_inv
// per 128x128 block, FastVideo PR #1829 "Changes", converter bullet) and the
// activation quantized per token in 1x128 K groups (the quantizer the
// Blackwell route of the same PR, "Changes" first bullet, pairs with its
// groupwise GEMM; x_scale stored K-block-major [GK, M]).
//
// Every 128-wide K step is one scale block on both sides. A wave's 16x16
// output block takes one v_mfma_scale_f32_16x16x128_f8f6f4 per step with a
// zero accumulator (the instruction's own E8M0 block scales are held at 1.0,
// since the scales here are arbitrary fp32), giving the exact-product block
// sum P in fp32; the fp32 accumulator then takes P * (x_scale * w_scale) in
// one FMA. Scales are applied once per 128 products, on fp32 partials.
//
// Workgroup tile 128x128, 4 waves in a 2x2 grid, 64x64 per wave (4x4 MFMA
// blocks). X and W tiles (128 rows x 128 bytes each per step) and the tile's
// 128 activation scales are staged through LDS, double-buffered with one
// barrier per step; 16-byte chunks are XOR-swizzled per row (see tile_off)
// so the MFMA operand reads and the row-wise staging writes are both free of
// bank conflicts. The weight scale is uniform per workgroup and step (the
// N tile is one 128-row scale block).
//
// MFMA operand layout: lane l supplies 32 bytes (32 codes) of row l % 16 of
// its block for A and of column l % 16 for B; l / 16 picks the 32-wide K
// quarter. A and B use the same lane -> k assignment, so the sum over the
// 128 k of the step is the same whatever order the instruction takes them
// in. Result: lane l holds column l % 16, rows 4 (l / 16) .. +3.
//
// Each step's MFMA phase is ordered by hand (scheduling barriers between
// groups): the 16 blocks go in 2x2 zig-zag order, each operand fragment is
// read from LDS two MFMAs before its first use, and the four scale FMAs of a
// block run two MFMAs after it, so neither the reads nor the MFMA results
// are waited on in full. Left to itself the compiler issued all 20 operand
// reads, waited for every one, and followed each MFMA with its own FMAs
// (3-6% slower on the DiT and text-encoder shapes). The weight scale for
// the next step is a scalar load issued after the MFMA phase, so no scalar
// load is in flight while operand reads are (either would force the reads'
// waits to drain completely).
//
// Split-K over K blocks (gridDim.y > 1) writes fp32 partial tiles that the
// ordered reduce kernel sums, as in the bf16 path.
//
// Measured on MI355X (16384x3072x3072): no single resource bounds the
// step. At the full MFMA rate its LDS traffic (16 KB of A and B fragments
// per wave and 32 KB of staging writes per workgroup and step) would keep
// the LDS as busy as the matrix core; the counters show the matrix core
// busy about a third of the time. The same kernel without its global loads
// runs within 20% of the full one, without its MFMAs within 18%, while the
// global -> LDS staging alone takes 14% of the time: a chain of latencies
// per step rather than one bound. Tried and slower or no faster: B fragments
// loaded from memory straight into registers (1.6x slower: 16-row x 64-byte
// loads), 256x128 tiles with 8 waves and a three-stage direct-to-LDS ring,
// the staging loads issued two steps ahead through a second register set
// (2-7% slower), operand reads three MFMAs ahead instead of two (no
// different). Larger per-wave tiles (fewer LDS bytes per
// MFMA) would shorten the chain, at a register cost that leaves one
// workgroup per CU.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 128;                 // BM = BN = BK
constexpr uint32_t kOob = 0x80000000u;
constexpr int kFmtE4M3 = 0;                // f8f6f4 operand format code of E4M3
constexpr int kE8M0One = 127;              // E8M0 exponent of 1.0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` (128 bytes).
// The operand read has lanes 16g..16g+15 on 16 consecutive rows at chunk
// 2g (+1). Measured with SQ_LDS_BANK_CONFLICT on gfx950: XOR with
// (row >> 1) & 7 (the bf16 path's swizzle, conflict-free for its 32-row
// reads) costs 4 extra cycles per ds_read_b128 here; XOR with row & 7 and
// row bit 3 has none, for these reads and for the 8-lanes-per-row writes.
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * kTile + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

__global__ __launch_bounds__(kThreads, 2)
void gemm_w8a8_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                      const uint8_t* __restrict__ q, const float* __restrict__ s,
                      uint16_t* __restrict__ y, float* __restrict__ part, int M, int N, int K,
                      int gk, int tiles_m, int tiles_n, int kb_per_split) {
  __shared__ __attribute__((aligned(16))) uint8_t at[2][kTile * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t bt[2][kTile * kTile];
  __shared__ __attribute__((aligned(16))) float sx[2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order, as in the bf16 path.
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
  const int m0 = tm * kTile;
  const int n0 = tn * kTile;

  const int kb0 = blockIdx.y * kb_per_split;
  const int kb1 = min(kb0 + kb_per_split, gk);

  // ---- staging: thread moves chunk (tid & 7) of tile rows (tid >> 3) + 32 i
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xq + (size_t)m0 * K, (uint32_t)(min(M - m0, kTile) * K));
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(q + (size_t)n0 * K, (uint32_t)(min(N - n0, kTile) * K));
  const int ch = tid & 7;
  const int sr = tid >> 3;
  const uint32_t off0 = (uint32_t)(sr * K + ch * 16);
  const uint32_t row32 = (uint32_t)(32 * K);
  // activation scales: thread moves row (tid & 127) of the tile; the two
  // halves of the workgroup load and store identical values (no branch)
  const int srow = m0 + (tid & 127);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(xs, (uint32_t)((size_t)gk * M * 4));
  const float* __restrict__ wsc = s + (size_t)tn * gk;

  u32x4 xr[4], wr[4];
  float sv;
  auto load = [&](int kb) {
    const bool kin = kb < kb1 && kb * kTile + ch * 16 < K;
    const uint32_t base = (uint32_t)(kb * kTile);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xr[i] = buf_load16(xrs, kin ? off0 + i * row32 + base : kOob);
      wr[i] = buf_load16(wrs, kin ? off0 + i * row32 + base : kOob);
    }
    // rows past M and steps past the split read zero
    const bool sin = kb < kb1 && srow < M;
    sv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
             srs, sin ? (uint32_t)((kb * M + srow) * 4) : kOob, 0, 0));
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&at[buf][tile_off(sr + 32 * i, ch)]) = xr[i];
      *reinterpret_cast<u32x4*>(&bt[buf][tile_off(sr + 32 * i, ch)]) = wr[i];
    }
    sx[buf][tid & 127] = sv;
  };

  f32x4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4;          // K quarter of this lane's operands, row group of its results
  const int r16 = lane & 15;
  const f32x4v zero = {0.f, 0.f, 0.f, 0.f};

  if (kb0 < kb1) {
    load(kb0);
    store(0);
  }
  __syncthreads();
  // MFMA order: 2x2 blocks of (i, j), each operand read when first needed
  constexpr int kOrd[16][2] = {{0, 0}, {0, 1}, {1, 0}, {1, 1}, {0, 2}, {1, 2}, {0, 3}, {1, 3},
                               {2, 0}, {2, 1}, {3, 0}, {3, 1}, {2, 2}, {2, 3}, {3, 2}, {3, 3}};
  float wscale = kb0 < kb1 ? wsc[kb0] : 0.0f;
  for (int kb = kb0; kb < kb1; ++kb) {
    const int cur = (kb - kb0) & 1;
    load(kb + 1);                     // past the last step: zeros, staged but unused
    __builtin_amdgcn_sched_barrier(0);
    i32x8 a[4], b[4];
    f32x4v scl[4];
    auto read_a = [&](int i) {
      const int row = wm * 64 + i * 16 + r16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&at[cur][tile_off(row, 2 * g)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&at[cur][tile_off(row, 2 * g + 1)]);
      a[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      const f32x4v v = *reinterpret_cast<const f32x4v*>(&sx[cur][wm * 64 + i * 16 + g * 4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) scl[i][r] = __fmul_rn(v[r], wscale);
    };
    auto read_b = [&](int j) {
      const int row = wn * 64 + j * 16 + r16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&bt[cur][tile_off(row, 2 * g)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&bt[cur][tile_off(row, 2 * g + 1)]);
      b[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // operands first used by MFMA q of the order
    auto read_for = [&](int q) {
      const int i = kOrd[q][0], j = kOrd[q][1];
      bool need_a = true, need_b = true;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (e < q && kOrd[e][0] == i) need_a = false;
        if (e < q && kOrd[e][1] == j) need_b = false;
      }
      if (need_a) read_a(i);
      if (need_b) read_b(j);
    };
    f32x4v pr[16];
    auto fma_for = [&](int q) {
      const int i = kOrd[q][0], j = kOrd[q][1];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[q][r], scl[i][r], acc[i][j][r]);
    };
    __builtin_amdgcn_s_setprio(1);
    read_for(0);
    read_for(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q + 2 < 16) read_for(q + 2);
      pr[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          a[kOrd[q][0]], b[kOrd[q][1]], zero, kFmtE4M3, kFmtE4M3, 0, kE8M0One, 0, kE8M0One);
      if (q >= 2) fma_for(q - 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    fma_for(14);
    fma_for(15);
    __builtin_amdgcn_s_setprio(0);
    // Keep the staging writes behind the MFMAs: they wait for this step's
    // global loads, which then have the whole MFMA phase to arrive. The next
    // step's weight scale is a scalar load issued here, so no scalar load is
    // in flight while the operand reads are (their waits stay partial).
    __builtin_amdgcn_sched_barrier(0);
    wscale = wsc[min(kb + 1, kb1 - 1)];
    store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column r16 and rows 4g..4g+3 of each block
  if (gridDim.y == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + r16;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 64 + i * 16 + g * 4 + r;
          if (row < M) {
            const __bf16 v = (__bf16)acc[i][j][r];
            y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, v);
          }
        }
      }
  } else {
    float* __restrict__ p = part + blockIdx.y * partial_slab((size_t)M, (size_t)N);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + r16;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 64 + i * 16 + g * 4 + r;
          if (row < M) p[(size_t)row * N + col] = acc[i][j][r];
        }
      }
  }
}

struct W8a8Plan {
  int splits, kb_per_split;
  double cost;      // time estimate, microseconds
};

// Split K (in 128-wide blocks) only when there are fewer tiles than CUs,
// choosing the count that minimises the busiest CU's load plus the fp32
// partials' round trip (the same model as the bf16 path).
W8a8Plan plan_w8a8(int64_t m, int64_t n, int64_t k) {
  const int gk = (int)((k + kTile - 1) / kTile);
  const int64_t tiles = ((m + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
  // one 128x128x128 step of a workgroup, two workgroups per CU: 0.73 us
  // each (measured on 16384x3072x3072, 16384x12288x3072 and 4096^3)
  constexpr double kStepUs = 0.73;
  auto cost_of = [&](int sp) {
    const int steps = (gk + sp - 1) / sp;
    const int64_t w = tiles * sp;
    const double load = w <= 256 ? 1.67 : (double)((w + 255) / 256);
    double cost = load * steps * kStepUs;
    if (sp > 1) cost += (double)(6 * sp + 2) * (double)(m * n) / 5.0e6;
    return cost;
  };
  int splits = 1;
  double best = cost_of(1);
  if (tiles < 256) {
    for (int sp = 2; sp <= 8; ++sp) {
      if ((gk + sp - 1) / sp < 4) break;
      const double cost = cost_of(sp);
      if (cost < best) { best = cost; splits = sp; }
    }
  }
  W8a8Plan p;
  p.kb_per_split = (gk + splits - 1) / splits;
  p.splits = (gk + p.kb_per_split - 1) / p.kb_per_split;
  p.cost = best;
  return p;
}

}  // namespace

size_t w8a8_partials_bytes(int64_t m, int64_t n, int64_t k) {
  const W8a8Plan p = plan_w8a8(m, n, k);
  const size_t own = p.splits <= 1 ? 0
                   : round_up((size_t)p.splits * partial_slab(m, n) * sizeof(float), kWorkspaceAlign);
  const size_t large = (n % 8 == 0) ? w8a8_large_partials_bytes(m, n, k) : 0;
  return own > large ? own : large;
}

// The large-tile kernel (192 or 128 X rows x 256 weight rows) where it takes
// the shape (N % 8 == 0) and its time estimate is the lower. Measured on
// MI355X it is faster on the DiT shapes, 4096^3, 2048 x 8192 x 2048,
// 1536 x 8192 x 2048 and 512 x 25600 x 5120, and level with the 128 x 128
// kernel on 512 x 5120 x 5120; the estimates rank these the same way.
int w8a8_choose(int64_t m, int64_t n, int64_t k) {
  if (n % 8 != 0) return 0;
  return plan_w8a8_large(m, n, k).cost < plan_w8a8(m, n, k).cost ? 1 : 0;
}

hipError_t launch_gemm_w8a8(const uint8_t* xq, const float* xs, const uint8_t* q, const float* s,
                            uint16_t* y, int64_t m, int64_t n, int64_t k, void* ws,
                            size_t ws_bytes, hipStream_t stream, int kind) {
  if (kind < 0) kind = w8a8_choose(m, n, k);
  if (kind == 1) return launch_gemm_w8a8_large(xq, xs, q, s, y, m, n, k, ws, ws_bytes, stream);
  const W8a8Plan p = plan_w8a8(m, n, k);
  const int gk = (int)((k + kTile - 1) / kTile);
  const int tiles_m = (int)((m + kTile - 1) / kTile);
  const int tiles_n = (int)((n + kTile - 1) / kTile);
  float* part = nullptr;
  if (p.splits > 1) {
    if (ws == nullptr || ws_bytes < w8a8_partials_bytes(m, n, k)) return hipErrorInvalidValue;
    part = static_cast<float*>(ws);
  }
  hipLaunchKernelGGL(gemm_w8a8_kernel, dim3((uint32_t)(tiles_m * tiles_n), (uint32_t)p.splits),
                     dim3(kThreads), 0, stream, xq, xs, q, s, y, part, (int)m, (int)n, (int)k, gk,
                     tiles_m, tiles_n, p.kb_per_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_reduce_partials(part, y, p.splits, m, n, stream);
}

}  // namespace fp8bl
