// Fused block-FP8 linear for large M: Y[M,N] = X[M,K] * W_hat[N,K]^T, with
// W_hat = bf16(fl32(e4m3(Q) * S)) formed in registers only (FastVideo PR
// #1829, "Purpose": block-scaled weight to BF16, then an ordinary matmul;
// LightX2V PR #1657, "Walkthrough": FP32 accumulation).
//
// Tile 256 (X rows) x 256 (weight rows), one workgroup of four waves per CU.
// Wave w owns weight rows [64w, 64w + 64) of the tile against all 256 X
// rows: 2 x 8 blocks of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per
// lane. The decoded weight is the MFMA A operand and X the B operand, so a
// lane's accumulators hold four consecutive output columns of one output
// row (the epilogue regroups them through LDS into whole-line stores). Per 64-wide K step a wave reads 32 X fragments from
// LDS, and each fragment feeds both of its weight blocks: half the LDS
// traffic per MFMA of a one-block-per-wave layout. Every code is decoded
// once per workgroup, by the wave that owns its row.
//
// Data movement per step, through a ring of three LDS stages:
//  - X: 32 KB per stage, moved global -> LDS by 16-byte buffer loads that
//    write LDS directly (no registers). The 16-byte chunks of a 128-byte LDS
//    row are XOR-permuted by (row / 2) % 8, chosen on the global side, so
//    that the MFMA operand reads (16 lanes on 16 consecutive rows, one
//    chunk) hit 16 distinct bank groups.
//  - codes: 16 KB per stage, moved the same way (each wave loads only the 64
//    rows it decodes, 16 rows x 64 bytes per instruction), the 16-byte
//    chunks of a row XOR-permuted by (row / 4) % 4 so the decoding reads are
//    conflict-free.
//  - weight scale: one word per wave and step, moved into the stage the
//    same way, so that no global load in the main loop writes a register and
//    the compiler adds no waits of its own on them.
//  - the 13 loads of a wave's share of a stage go out two steps ahead,
//    spread over the first three quarters of a step (one per four MFMAs).
//    Issued in one burst after the barrier, as four waves at once, they
//    filled the CU's load queue and held the MFMA stream behind it.
//
// Register pipeline inside a step (four sub-steps of k16, 64 MFMAs): X
// fragments are read from LDS four ahead of their MFMAs into a ring of
// eight registers; sub-step t+1's weight operands are decoded during
// sub-step t (E4M3 -> fp32 convert, one fp32 multiply by the scale, RNE to
// bf16), the next step's first ones during the last two quarter-sub-steps.
// The step runs as 16 regions of 4 MFMAs, each with its own share of the
// reads, the decode and the loads, in a fixed order (a scheduling barrier
// between regions keeps the compiler from pairing an MFMA with a read it
// has just issued). One barrier per step, 8 MFMAs before its end.
//
// The K order inside a step is a permutation (A and B only have to agree):
// lane half h holds, for sub-step t, k = 16h + 32(t/2) + 8(t%2) .. +8, so a
// lane's codes for the step are two contiguous 16-byte runs of its row.
//
// Rows past M or N and K past the end read as zero through buffer
// descriptors that cover only valid rows and through per-lane out-of-range
// offsets; no branch in the main loop depends on data.
//
// Persistent: one workgroup per CU walks its (tile, K split) units; the
// loads of the next unit's first two steps go out during the last two steps
// of the current one, so the ring never drains between units.
//
// Split-K (units with a K split): every split writes its fp32 partial tile to
// the workspace and the ordered reduce kernel adds the splits and rounds once.
//
// Gated (the MLP gate/up pair with the SwiGLU epilogue): the tile covers 128
// output columns; waves 0 and 1 run its gate weight rows and waves 2 and 3
// the same rows of the up weight, everything else as above. Wave w and wave
// w + 2 then hold the two products of one 256 x 64 output slice, element for
// element, and finish half of it each after trading the other half through
// LDS.
#include <atomic>

#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

constexpr int kBK = 64;                     // K per step
constexpr int kBM = 256;                    // X rows per tile
constexpr int kBN = 256;                    // weight rows per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 3;
constexpr int kXElems = kBM * kBK;          // bf16 elements of one stage's X tile (32 KB)
constexpr int kWBytes = kBN * kBK;          // bytes of one stage's codes (16 KB)
constexpr int kSElems = kWaves * 64 * 4 / 2;  // the waves' block-scale slots (256 B each)
constexpr int kStageElems = kXElems + kWBytes / 2 + kSElems;   // stage size in bf16 elements (49 KB)
constexpr int kXLoads = kXElems * 2 / 16 / kThreads;   // 16-byte X loads per lane per step
constexpr int kWLoads = kWBytes / 16 / kThreads;       // 16-byte code loads per lane per step
constexpr int kLoadsPerStep = kXLoads + kWLoads + 1;   // + the scale
constexpr uint32_t kOob = 0x80000000u;      // buffer offset past every valid range

static_assert(kXLoads == 8, "one wave's X loads cover 64 rows of a stage");
static_assert(kWLoads == 4, "one wave's code loads cover its 64 rows of a stage");
static_assert(kBK == 64, "the X chunk permutation assumes 128-byte LDS rows");
static_assert(kLoadsPerStep == 13, "the load slots of the step schedule assume 13 loads");
static_assert((kStageElems * 2) % 256 == 0, "stages keep the LDS bank phase of their rows");

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt_hi[15:14],
// expcnt[6:4], lgkmcnt[11:8]). vm_wait(n): at most n vector-memory
// operations of this wave still outstanding, no wait on the others.
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kLgkmWait0 = 0xC07F;         // lgkmcnt(0) only

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: raw (untyped) buffer, 32-bit format, the gfx9
  // family layout; offsets at or past `bytes` read as zero. The size is made
  // wave-uniform so the descriptor lives in scalar registers.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Cache policy of the finished tile's bf16 stores: non-temporal (bit 1 of
// the buffer instruction's cache field on gfx950). Nothing in the kernel
// reads them back, and streaming them past the caches keeps more of X and
// the codes, which other tiles re-read, in L2 and the MALL: 1-3% on
// 16384 x 12288 x 3072 and 16384 x 3072 x 3072 (same box, A/B, identical
// outputs). Split-K partials keep the default policy: the reduce reads them.
constexpr int kNonTemporal = 2;

// (q, s) is the weight; for GATED it is the gate weight and (q2, s2) the up
// weight, and y receives the SwiGLU.
template <bool SPLIT, bool GATED>
__global__ __launch_bounds__(kThreads, 1)
void gemm_large_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                       const float* __restrict__ s, const uint8_t* __restrict__ q2,
                       const float* __restrict__ s2, uint16_t* __restrict__ y,
                       float* __restrict__ part, int M, int N, int K, int gk,
                       int tiles_m, int tiles_n, int kt_per_split, int splits, int steps_per_unit) {
  static_assert(!(SPLIT && GATED), "the SwiGLU needs whole sums: no K split");
  __shared__ __attribute__((aligned(1024))) uint16_t xs[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Output columns of a tile, and the first row of this wave's weight rows
  // within the tile's rows of its weight.
  constexpr int kTileN = GATED ? kBN / 2 : kBN;
  const int wrow = GATED ? 64 * (wave & 1) : 64 * wave;
  const uint8_t* const wq = (GATED && wave >= 2) ? q2 : q;
  const float* const wsc = (GATED && wave >= 2) ? s2 : s;

  // ---- Work units: (tile, K split) pairs, dealt to the persistent
  // workgroups round-robin (unit blockIdx.x + i * gridDim.x). Consecutive
  // workgroups sit on consecutive XCDs; the renumbering gives each XCD a
  // contiguous run of units, walked in groups of 8 M-tiles, so the tiles
  // running at once on an XCD share X and W rows in its L2.
  const int ntiles = tiles_m * tiles_n;
  const int units = ntiles * splits;
  const int my_units = (units - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int nkt = (K + kBK - 1) / kBK;
  struct Unit {
    int m0, n0, kt0, nreal, split;
  };
  auto unit_of = [&](int i) -> Unit {
    Unit U{0, 0, 0, 0, 0};              // past the last unit: no live step
    if (i >= my_units) return U;
    const int u = (int)blockIdx.x + i * (int)gridDim.x;
    const int r = (units & 7) == 0 ? (u & 7) * (units >> 3) + (u >> 3) : u;
    U.split = r / ntiles;
    const int id = r - U.split * ntiles;
    constexpr int GM = 8;
    const int group = id / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int in_group = id - group * GM * tiles_n;
    U.m0 = (first_m + in_group % gsize) * kBM;
    U.n0 = (in_group / gsize) * kTileN;
    U.kt0 = U.split * kt_per_split;
    U.nreal = min(kt_per_split, nkt - U.kt0);
    return U;
  };

  // ---- X staging: load i of wave w fills LDS rows 64w + 8i .. +8 of a
  // stage; lane l lands on row (l / 8) of those, physical chunk l % 8, and
  // fetches the logical chunk that the swizzle stores there: (l % 8) ^
  // ((4i + l/16) % 8), one of two chunks by the parity of i. The per-lane
  // offsets (row within the tile and chunk) are fixed for the whole kernel;
  // the tile goes in the descriptor and the step's K offset in the scalar
  // offset of the load. (The hardware checks only the per-lane part against
  // the descriptor's size, which is what guards the rows past M: the K
  // offset of a real chunk stays inside its row.)
  const int xc_even = (lane & 7) ^ (lane >> 4);
  const int xc_odd = (lane & 7) ^ (4 + (lane >> 4));
  uint32_t xvo[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i)
    xvo[i] = (uint32_t)((64 * wave + 8 * i + (lane >> 3)) * K * 2 + ((i & 1) ? xc_odd : xc_even) * 16);
  // codes: load i of wave w fills the stage's code rows 64w + 16i .. +16
  // (64 bytes each, the step's K range) from its weight rows wrow + 16i ..;
  // lane l lands on row (l / 4), physical 16-byte chunk l % 4, holding the
  // logical chunk (l % 4) ^ (l / 16) (the row's (row / 4) % 4), so the
  // decoding reads below are conflict-free. A wave loads, and later reads,
  // only its own rows.
  const int wc = (lane & 3) ^ (lane >> 4);
  uint32_t wvo[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) wvo[i] = (uint32_t)((wrow + 16 * i + (lane >> 2)) * K + 16 * wc);
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(wsc, (uint32_t)(((N + kBlock - 1) / kBlock) * gk * 4));

  // The unit whose steps are being loaded (two steps ahead of the one being
  // computed, so near the end of a unit it is the next one).
  Unit LU = unit_of(0);
  __amdgpu_buffer_rsrc_t xrs, wrs;
  bool lwave_live;
  int lsrow;
  auto set_load_unit = [&](const Unit& U) {
    LU = U;
    xrs = make_rsrc(x + (size_t)U.m0 * K, (uint32_t)(U.nreal > 0 ? min(M - U.m0, kBM) * K * 2 : 0));
    wrs = make_rsrc(wq + (size_t)U.n0 * K, (uint32_t)(U.nreal > 0 ? max(min(N - U.n0, kTileN), 0) * K : 0));
    lwave_live = U.n0 + wrow < N;
    lsrow = lwave_live ? (U.n0 + wrow) / kBlock : 0;
  };
  set_load_unit(LU);

  // Stage loads. `sb` is the stage's first element in xs (wave-uniform).
  // X load i (of 8) and code load i (of 4) as above; each sends a 1 KB
  // wave-wide piece straight into LDS.
  auto issue_x = [&](int sb, int kt, int i) {
    const int kbase = (LU.kt0 + kt) * kBK;
    // K left in this step (0 past the unit's range): a chunk is read iff it
    // starts below it
    const int klim = kt < LU.nreal ? K - kbase : 0;
    const bool in = ((i & 1) ? xc_odd : xc_even) * 8 < klim;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr_t)&xs[sb + (64 * wave + 8 * i) * kBK], 16,
                                             in ? xvo[i] : kOob, (uint32_t)(kbase * 2), 0, 0);
  };
  auto issue_w = [&](int sb, int kt, int i) {
    const int kbase = (LU.kt0 + kt) * kBK;
    const int klim = kt < LU.nreal ? K - kbase : 0;
    const bool kin = 16 * wc < klim;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wrs, (lds_ptr_t)&xs[sb + kXElems + (64 * wave + 16 * i) * kBK / 2], 16,
        kin ? wvo[i] : kOob, (uint32_t)kbase, 0, 0);
  };
  // Weight scale: one per wave and step (the wave's 64 rows lie in one
  // 128-row scale block, the 64-wide step in one 128-wide block), moved into
  // the stage like the codes: every lane fetches the same word, so the
  // wave's 256-byte slot holds 64 copies. No load in the main loop writes a
  // register, so the only waits on global loads are the explicit ones below.
  // Waves past N and dead steps read zero. (The address is always formed,
  // block clamped, and pushed out of range when dead.)
  auto issue_s = [&](int sb, int kt) {
    const int kb = min(((LU.kt0 + kt) * kBK) / kBlock, gk - 1);
    const bool live = lwave_live & (kt < LU.nreal);
    const uint32_t off = (uint32_t)((lsrow * gk + kb) * 4) + (live ? 0u : kOob);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        srs, (lds_ptr_t)&xs[sb + kXElems + kWBytes / 2 + wave * 128], 4, off, 0, 0, 0);
  };
  auto issue_all = [&](int sb, int kt) {
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) issue_x(sb, kt, i);
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) issue_w(sb, kt, i);
    issue_s(sb, kt);
  };
  auto read_s = [&](int sb) -> float {
    return *reinterpret_cast<const float*>(&xs[sb + kXElems + kWBytes / 2 + wave * 128]);
  };

  // Codes of weight block nb, K half j of a stage (the 16 codes of sub-steps
  // 2j and 2j+1): lane l reads row 64w + 32nb + l%32, logical chunk
  // l/32 + 2j, stored at chunk (l/32 + 2j) ^ ((l%32 / 4) % 4).
  const int crow = (64 * wave + (lane & 31)) * kBK;     // byte offset of the lane's row
  const int cswz = ((lane & 31) >> 2) & 3;
  const int crd0 = crow + ((((lane >> 5) + 0) ^ cswz) << 4);
  const int crd1 = crow + ((((lane >> 5) + 2) ^ cswz) << 4);
  auto read_w = [&](u32x4 (&c)[2], int sb, int j) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(&xs[sb + kXElems]) + (j ? crd1 : crd0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) c[nb] = *reinterpret_cast<const u32x4*>(base + nb * 32 * kBK);
  };
  // X fragment f of a stage (sub-step t = f / 8, row block mb = f % 8): the
  // MFMA B operand of the 32 X rows 32mb.. and the 16 K of sub-step t.
  const int arow = lane & 31;
  const int ahalf = lane >> 5;
  const int aswz = (arow >> 1) & 7;
  auto read_xf = [&](int sb, int f) -> bf16x8 {
    const int t = f >> 3, mb = f & 7;
    const int c = 2 * ahalf + 4 * (t >> 1) + (t & 1);
    return *reinterpret_cast<const bf16x8*>(&xs[sb + arow * kBK + ((c ^ aswz) << 3) + mb * 32 * kBK]);
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

  // Workgroup barrier; the empty asm statements keep the compiler from
  // moving any memory access (LDS reads included) across it.
  auto wg_barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- Register pipeline of a step (32 fragments f = 8t + mb; sub-step t
  // runs the 16 MFMAs of its 8 X fragments against its two decoded weight
  // operands):
  //  - X fragments are read four ahead of their MFMAs into a ring of eight;
  //    the last four of a step read the next stage, after the barrier;
  //  - sub-step t+1's weight operands are decoded during sub-step t (the
  //    next step's first ones during sub-step 3), codes read a K half ahead;
  //  - the 13 loads of the step two ahead are spread over fragments 0..24;
  //  - at fragment 24 the wave waits for its loads of the next step (the
  //    ones issued during the previous step) and reads its codes and scale;
  //  - at fragment 28 the barrier: every wave is done with this stage (its
  //    last reads returned), and the next stage is complete.
  // fragments f..f+5 are live in the region of f, f+1; 8 slots keep the
  // slot of a fragment the same in every step (32 fragments a step)
  constexpr int kRing = 8;
  constexpr int kAhead = 4;
  bf16x8 xr[kRing];
  u32x4 wdh[2][2];          // decoded weight operands (bf16 pairs), by sub-step parity
  u32x4 cA[2], cB[2];       // codes of K halves 0 and 1
  float sc;                 // this step's scale

  // Prologue: steps 0 and 1 of the first unit in flight (every unit has at
  // least three steps); wait for step 0, then prepare its first operands.
  issue_all(0, 0);
  issue_all(kStageElems, 1);
  __builtin_amdgcn_s_waitcnt(vm_wait(kLoadsPerStep));
  wg_barrier();
  read_w(cA, 0, 0);
  sc = read_s(0);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) wdh[0][nb] = __builtin_bit_cast(u32x4, dequant8(cA[nb][0], cA[nb][1], sc));
#pragma unroll
  for (int f = 0; f < kAhead; ++f) xr[f] = read_xf(0, f);

  const int col_lane = 64 * wave + 4 * ahalf;
  int S = 0;                 // stage of the step being computed
  int lkt = 1;               // step (of LU) most recently loaded
  for (int ci = 0; ci < my_units; ++ci) {
  for (int kt = 0; kt < steps_per_unit; ++kt) {
    // the step two ahead: next step of LU, or step 0 of the next unit
    if (++lkt == steps_per_unit) {
      set_load_unit(unit_of(ci + 1));
      lkt = 0;
    }
    const int Sn = S == kStages - 1 ? 0 : S + 1;
    const int L = Sn == kStages - 1 ? 0 : Sn + 1;
    const int sb = S * kStageElems, sbn = Sn * kStageElems, sbl = L * kStageElems;

#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t == 0) read_w(cB, sb, 1);
#pragma unroll
      for (int mb = 0; mb < 8; mb += 2) {
        // one region: the MFMAs of fragments f, f+1 with their share of the
        // other work, in a fixed order relative to the other regions
        const int f = 8 * t + mb;
        if (f == 24) {
          // this wave's loads of the next step (issued during the previous
          // step) have landed, with 12 of this step's still in flight: read
          // its codes of K half 0 and its scale
          __builtin_amdgcn_s_waitcnt(vm_wait(kLoadsPerStep - 1));
          read_w(cA, sbn, 0);
          sc = read_s(sbn);
        }
        if (f == 28) {
          // every wave is done with this stage (its last reads returned)
          // and has put its part of the next stage in place
          __builtin_amdgcn_s_waitcnt(kLgkmWait0);
          wg_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        // read ahead (the last four from the next stage, after the barrier)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int fa = f + j + kAhead;
          xr[fa % kRing] = fa < 32 ? read_xf(sb, fa) : read_xf(sbn, fa - 32);
        }
        // the loads of the step two ahead, into the stage freed by the last barrier
        if (f <= 14) issue_x(sbl, lkt, (f >> 1) + 0);
        if (f >= 16 && f <= 22) issue_w(sbl, lkt, (f - 16) >> 1);
        if (f == 24) issue_s(sbl, lkt);
        // the next sub-step's weight operands, a quarter (one block's half
        // K of the sub-step: four codes to bf16) per region: sub-steps 1..3
        // from this step's codes, the next step's sub-step 0 from its codes
        // read at fragment 24, in the two regions after the barrier
        auto piece = [&](int q4) {
          const int nb = q4 >> 1, half = q4 & 1;
          const int tn = (t + 1) & 3;          // sub-step being prepared
          const u32x4 (&c)[2] = tn <= 1 ? cA : cB;
          const u32x2 v = dequant4(c[nb][2 * (tn & 1) + half], sc);
          wdh[tn & 1][nb][2 * half] = v[0];
          wdh[tn & 1][nb][2 * half + 1] = v[1];
        };
        if (t < 3) {
          piece(mb >> 1);
        } else if (f >= 28) {
          piece(f - 28);
          piece(f - 28 + 1);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[nb][mb + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, wdh[t & 1][nb]), xr[(f + j) % kRing], acc[nb][mb + j], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    S = Sn;
  }

    // ---- Epilogue of unit ci (the next unit's first loads are already in
    // flight). acc[nb][mb][4g + e] is output row m0 + 32mb + l%32, column
    // n0 + 64w + 32nb + 8g + 4(l/32) + e. Stores go through a buffer
    // descriptor over the tile's valid rows, so rows past M are dropped by
    // the hardware; columns past N get an out-of-range offset. (The host
    // keeps 256 rows of the output within 2^31 bytes.)
    const Unit CU = unit_of(ci);
    const int rows = min(M - CU.m0, kBM);
    const int col_base = CU.n0 + col_lane;
    if constexpr (GATED) {
      // Gate wave w < 2 finishes row blocks 0..3 of the slice and up wave
      // w + 2 row blocks 4..7; each sends its partner the other four, rounded
      // to bf16 (the SwiGLU rounds both products to bf16 first, so nothing
      // is lost). Two rounds of two row blocks go through the sender's own
      // 8 KB of X rows in the stage the last step used, 16 bytes per lane,
      // lane-contiguous; a barrier after the writes hands them over, one
      // after the partner's reads gives the rows back. Each finished row
      // block then leaves as whole 128-byte lines through the same rows, as
      // in the plain epilogue below. (Only N % 8 == 0 comes here.)
      const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + (size_t)CU.m0 * N, (uint32_t)(rows * N * 2));
      const int stage0 = (S == 0 ? 2 : S - 1) * kStageElems;
      int le;
      asm volatile("" : "=v"(le) : "0"(lane));
      uint8_t* const own = reinterpret_cast<uint8_t*>(&xs[stage0 + wave * 64 * kBK]);
      const uint8_t* const peer = reinterpret_cast<const uint8_t*>(&xs[stage0 + (wave ^ 2) * 64 * kBK]);
      const bool up = wave >= 2;
      const int er = le & 31, eh = le >> 5;
      const int rr = le >> 3;
      const int col8 = CU.n0 + wrow + 8 * (le & 7);
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const f32x16 a = up ? acc[nb][2 * r2 + i] : acc[nb][4 + 2 * r2 + i];
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
              u32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(a[8 * gp + 2 * e], a[8 * gp + 2 * e + 1]);
              *reinterpret_cast<u32x4*>(own + ((2 * i + nb) * 2 + gp) * 1024 + le * 16) = v;
            }
          }
        __builtin_amdgcn_s_waitcnt(kLgkmWait0);
        wg_barrier();
        u32x4 got[2][2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp)
              got[i][nb][gp] = *reinterpret_cast<const u32x4*>(peer + ((2 * i + nb) * 2 + gp) * 1024 + le * 16);
        __builtin_amdgcn_s_waitcnt(kLgkmWait0);
        wg_barrier();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint8_t* const buf = own + i * 4096;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const f32x16 a = up ? acc[nb][4 + 2 * r2 + i] : acc[nb][2 * r2 + i];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              u32x2 v;
#pragma unroll
              for (int w2 = 0; w2 < 2; ++w2) {
                const uint32_t mine = pack_bf16x2(a[4 * g + 2 * w2], a[4 * g + 2 * w2 + 1]);
                const uint32_t theirs = got[i][nb][g >> 1][2 * (g & 1) + w2];
                v[w2] = swiglu_bf16x2(up ? theirs : mine, up ? mine : theirs);
              }
              const int chunk = (4 * nb + g) ^ ((er >> 1) & 7);
              *reinterpret_cast<u32x2*>(buf + er * 128 + chunk * 16 + 8 * eh) = v;
            }
          }
          const int mb = (up ? 4 : 0) + 2 * r2 + i;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 8 * j + rr;
            const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * 128 + (((le & 7) ^ ((r >> 1) & 7)) * 16));
            const uint32_t off = col8 < N ? (uint32_t)(((32 * mb + r) * N + col8) * 2) : kOob;
            __builtin_amdgcn_raw_buffer_store_b128(v, yrs, off, 0, kNonTemporal);
          }
        }
      }
    } else if constexpr (!SPLIT) {
      const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + (size_t)CU.m0 * N, (uint32_t)(rows * N * 2));
      if ((N & 3) == 0) {
        if ((N & 7) == 0) {
          // Through LDS, so that every store writes whole 128-byte lines:
          // lane l holds four consecutive columns of row l % 32 of each
          // 32x32 block, so direct stores write 16 bytes into each of 32
          // rows, and eight of them fill a line; written to memory that way
          // a tile takes about three times as long. Each 32-row block of
          // this wave's 256 x 64 slice goes row-major into 4 KB of LDS (16-byte
          // chunk c of row r at chunk c ^ ((r / 2) % 8)), then comes back as
          // 16 bytes per lane, 8 lanes per 128-byte row, 8 rows per store.
          // The LDS is the wave's own 8 KB of X rows in the stage the last
          // step used: every wave finished reading that stage before the last
          // barrier, and only this wave refills those rows, with loads it
          // issues after these reads have returned.
          const int tb = (S == 0 ? 2 : S - 1) * kStageElems + wave * 64 * kBK;
          // (the lane index through an empty asm: the compiler would otherwise
          // compute every address below once, before the loops, and keep
          // them in registers the main loop needs)
          int le;
          asm volatile("" : "=v"(le) : "0"(lane));
          const int er = le & 31, eh = le >> 5;
          const int rr = le >> 3;                   // row within 8 for the read-back
          const int col8 = CU.n0 + 64 * wave + 8 * (le & 7);
#pragma unroll
          for (int mb = 0; mb < 8; ++mb) {
            uint16_t* buf = &xs[tb + (mb & 1) * 2048];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x16& a = acc[nb][mb];
                const u32x2 v = {pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
                const int chunk = (4 * nb + g) ^ ((er >> 1) & 7);
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(buf) + er * 128 + chunk * 16 + 8 * eh) = v;
              }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 8 * j + rr;
              const u32x4 v = *reinterpret_cast<const u32x4*>(
                  reinterpret_cast<const uint8_t*>(buf) + r * 128 + (((le & 7) ^ ((r >> 1) & 7)) * 16));
              const uint32_t off = col8 < N ? (uint32_t)(((32 * mb + r) * N + col8) * 2) : kOob;
              __builtin_amdgcn_raw_buffer_store_b128(v, yrs, off, 0, kNonTemporal);
            }
          }
        } else {
#pragma unroll
          for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int col = col_base + 32 * nb + 8 * g;
                const uint32_t off = col < N ? (uint32_t)(((arow + 32 * mb) * N + col) * 2) : kOob;
                const f32x16& a = acc[nb][mb];
                const u32x2 v = {pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
                __builtin_amdgcn_raw_buffer_store_b64(v, yrs, off, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
              }
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int col = col_base + 32 * nb + 8 * (r >> 2) + (r & 3);
              const uint32_t off = col < N ? (uint32_t)(((arow + 32 * mb) * N + col) * 2) : kOob;
              __builtin_amdgcn_raw_buffer_store_b16(
                  __builtin_bit_cast(uint16_t, (__bf16)acc[nb][mb][r]), yrs, off, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
      }
    } else {
      const __amdgpu_buffer_rsrc_t prs =
          make_rsrc(part + (size_t)CU.split * partial_slab(M, N) + (size_t)CU.m0 * N,
                    (uint32_t)(rows * N * 4));
      if ((N & 3) == 0) {
        // fp32 partials through the same LDS slice, as whole lines: each
        // 32-row block of this wave's 256 x 64 slice row-major in its 8 KB
        // (256-byte rows, 16-byte chunk c of row r at c ^ (r % 16)), back as
        // 16 bytes per lane, 16 lanes per row, 4 rows per store.
        const int tb = (S == 0 ? 2 : S - 1) * kStageElems + wave * 64 * kBK;
        int le;
        asm volatile("" : "=v"(le) : "0"(lane));
        const int er = le & 31, eh = le >> 5;
        const int cc = le & 15, rq = le >> 4;
        const int col4 = CU.n0 + 64 * wave + 4 * cc;
        uint8_t* buf = reinterpret_cast<uint8_t*>(&xs[tb]);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x16& a = acc[nb][mb];
              // (__builtin_bit_cast of a vector element read element 0 here:
              // the values go through __float_as_uint instead.)
              const u32x4 v = {__float_as_uint(a[4 * g]), __float_as_uint(a[4 * g + 1]),
                               __float_as_uint(a[4 * g + 2]), __float_as_uint(a[4 * g + 3])};
              const int c = 8 * nb + 2 * g + eh;
              *reinterpret_cast<u32x4*>(buf + er * 256 + ((c ^ (er & 15)) << 4)) = v;
            }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 4 * j + rq;
            const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * 256 + ((cc ^ (r & 15)) << 4));
            const uint32_t off = col4 < N ? (uint32_t)(((32 * mb + r) * N + col4) * 4) : kOob;
            __builtin_amdgcn_raw_buffer_store_b128(v, prs, off, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int col = col_base + 32 * nb + 8 * (r >> 2) + (r & 3);
              const uint32_t off = col < N ? (uint32_t)(((arow + 32 * mb) * N + col) * 4) : kOob;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[nb][mb][r]), prs, off, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;
  }
  // The loads issued for the unit after the last one target the ring;
  // drain them before exit.
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
}

}  // namespace

// Split count from the cost model of the tile-planned kernel's planner, in
// the same units (microseconds, work counted in 128x128x64 steps): a CU
// runs this kernel's 256x256x64 step (4 of those) at 2.42 of them per
// microsecond (measured on 16384 x 12288 x 3072), plus about 2 us per unit
// for its first loads and its epilogue; the busiest CU sets the time, ceil(units /
// 256) units. K splits add the fp32 partials' round trip (as in that
// planner). The split count that puts about one unit on every CU wins at
// 512 rows (e.g. 6 for 512 x 5120 x 25600).
LargePlan plan_large(int64_t m, int64_t n, int64_t k) {
  const int nkt = (int)((k + kBK - 1) / kBK);
  const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
  LargePlan p{1, nkt, 0.0};
  double best = 1e300;
  for (int sp = 1; sp <= 8; ++sp) {
    const int steps = (nkt + sp - 1) / sp;
    if (sp > 1 && steps < 8) break;
    const int64_t per_cu = (tiles * sp + 255) / 256;
    double cost = (double)per_cu * (steps * 4 / 2.42 + 2.0);
    if (sp > 1) cost += (double)(6 * sp + 2) * (double)(m * n) / 5.0e6;
    if (cost < best) {
      best = cost;
      p.splits = sp;
    }
  }
  p.kt_per_split = (nkt + p.splits - 1) / p.splits;
  p.splits = (nkt + p.kt_per_split - 1) / p.kt_per_split;
  p.cost = best;
  return p;
}

size_t large_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const LargePlan p = plan_large(m, n, k);
  if (p.splits <= 1) return 0;
  return round_up((size_t)p.splits * partial_slab(m, n) * sizeof(float), kWorkspaceAlign);
}

namespace {

// Compute units of the current device (persistent grid size), cached.
constexpr int kMaxDev = 64;
std::atomic<int> g_cus[kMaxDev];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    g_cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace

hipError_t launch_gemm_large(const uint16_t* x, const uint8_t* q, const float* s, uint16_t* y,
                             int64_t m, int64_t n, int64_t k, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  const LargePlan p = plan_large(m, n, k);
  const int gk = (int)((k + kBlock - 1) / kBlock);
  const int tiles_m = (int)((m + kBM - 1) / kBM);
  const int tiles_n = (int)((n + kBN - 1) / kBN);
  const int units = tiles_m * tiles_n * p.splits;
  // one persistent workgroup per CU; every unit has at least two steps (the
  // prologue loads two; a padded step reads zeros)
  const int grid = units < device_cus() ? units : device_cus();
  const int spu = p.kt_per_split > 2 ? p.kt_per_split : 2;
  if (p.splits == 1) {
    hipLaunchKernelGGL((gemm_large_kernel<false, false>), dim3((uint32_t)grid), dim3(kThreads), 0,
                       stream, x, q, s, nullptr, nullptr, y, nullptr, (int)m, (int)n, (int)k, gk,
                       tiles_m, tiles_n, p.kt_per_split, 1, spu);
    return hipGetLastError();
  }
  if (ws == nullptr || ws_bytes < large_workspace_bytes(m, n, k)) return hipErrorInvalidValue;
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL((gemm_large_kernel<true, false>), dim3((uint32_t)grid), dim3(kThreads), 0,
                     stream, x, q, s, nullptr, nullptr, y, part, (int)m, (int)n, (int)k, gk,
                     tiles_m, tiles_n, p.kt_per_split, p.splits, spu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce_partials(part, y, p.splits, m, n, stream);
}

// The gated form's tiles are 256 x 128 outputs, each the work of a plain
// 256 x 256 tile, never split: the plain model at one split, with the rate
// measured on the gate/up pair at 512 and 768 rows (2.7 steps per
// microsecond per CU; the 2.42 above is from 16384 rows, where the chip runs
// at lower clocks). Against the tiled gate/up planner it picked the faster
// kernel on all seven shapes measured (128 to 4096 rows).
double large_gated_cost(int64_t m, int64_t n, int64_t k) {
  const int nkt = (int)((k + kBK - 1) / kBK);
  const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN / 2 - 1) / (kBN / 2));
  return (double)((tiles + 255) / 256) * (nkt * 4 / 2.7 + 2.0);
}

hipError_t launch_gemm_large_gated(const uint16_t* x, const uint8_t* qg, const float* sg,
                                   const uint8_t* qu, const float* su, uint16_t* h, int64_t m,
                                   int64_t n, int64_t k, hipStream_t stream) {
  if ((n & 7) != 0) return hipErrorInvalidValue;
  const int nkt = (int)((k + kBK - 1) / kBK);
  const int gk = (int)((k + kBlock - 1) / kBlock);
  const int tiles_m = (int)((m + kBM - 1) / kBM);
  const int tiles_n = (int)((n + kBN / 2 - 1) / (kBN / 2));
  const int units = tiles_m * tiles_n;
  const int grid = units < device_cus() ? units : device_cus();
  const int spu = nkt > 2 ? nkt : 2;
  hipLaunchKernelGGL((gemm_large_kernel<false, true>), dim3((uint32_t)grid), dim3(kThreads), 0,
                     stream, x, qg, sg, qu, su, h, nullptr, (int)m, (int)n, (int)k, gk, tiles_m,
                     tiles_n, nkt, 1, spu);
  return hipGetLastError();
}

}  // namespace fp8bl
