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
// row (8-byte stores). Per 64-wide K step a wave reads 32 X fragments from
// LDS, and each fragment feeds both of its weight blocks: half the LDS
// traffic per MFMA of a one-block-per-wave layout. Every code is decoded
// once per workgroup, by the wave that owns its row.
//
// Data movement per step:
//  - X: 32 KB per stage, moved global -> LDS by 16-byte buffer loads that
//    write LDS directly (no registers), into a ring of three stages. The
//    loads of step k+3 go out right after the barrier of step k, about two
//    steps ahead of use. The 16-byte chunks of a 128-byte LDS row are
//    XOR-permuted by (row / 2) % 8, chosen on the global side, so that the
//    MFMA operand reads (16 lanes on 16 consecutive rows, one chunk) hit 16
//    distinct bank groups.
//  - codes: 16 KB per stage, moved global -> LDS the same way into the same
//    ring (each wave loads only the 64 rows it decodes, 16 rows x 64 bytes
//    per instruction), the 16-byte chunks of a row XOR-permuted by
//    (row / 4) % 4 so the decoding reads are conflict-free.
//  - weight scale: one per wave and step (the wave's 64 rows lie in one
//    128-row scale block, the 64-wide step in one 128-wide block).
//
// Software pipeline inside a step (four sub-steps of k16): while the 16
// MFMAs of sub-step t run, the wave decodes the codes of sub-step t+1 (32
// VALU: E4M3 -> fp32 convert, one fp32 multiply by the scale, RNE to bf16)
// and reads the X fragments of sub-step t+1 from LDS. The decode of the
// next step's first sub-step runs inside the current step's last one, so
// the matrix core is never left waiting for VALU work. One barrier per step
// (inside the last sub-step, after this stage's last operand reads and with
// the next stage's loads complete).
//
// The K order inside a step is a permutation (A and B only have to agree):
// lane half h holds, for sub-step t, k = 16h + 32(t/2) + 8(t%2) .. +8, so a
// lane's codes for the step are two contiguous 16-byte runs of its row.
//
// Rows past M or N and K past the end read as zero through buffer
// descriptors that cover only valid rows and through per-lane out-of-range
// offsets; no branch in the main loop depends on data.
//
// Split-K (gridDim.y > 1): every split writes its fp32 partial tile to the
// workspace and the ordered reduce kernel adds the splits and rounds once.
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
constexpr int kStageElems = kXElems + kWBytes / 2;   // stage size in bf16 elements (48 KB)
constexpr int kXLoads = kXElems * 2 / 16 / kThreads;   // 16-byte X loads per lane per step
constexpr int kWLoads = kWBytes / 16 / kThreads;       // 16-byte code loads per lane per step
constexpr int kLoadsPerStep = kXLoads + kWLoads + 1;   // + the scale
constexpr uint32_t kOob = 0x80000000u;      // buffer offset past every valid range

static_assert(kXLoads == 8, "one wave's X loads cover 64 rows of a stage");
static_assert(kWLoads == 4, "one wave's code loads cover its 64 rows of a stage");
static_assert(kBK == 64, "the X chunk permutation assumes 128-byte LDS rows");

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

template <bool SPLIT>
__global__ __launch_bounds__(kThreads, 1)
void gemm_large_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                       const float* __restrict__ s, uint16_t* __restrict__ y,
                       float* __restrict__ part, int M, int N, int K, int gk,
                       int tiles_m, int tiles_n, int kt_per_split, int splits, int steps_per_unit) {
  __shared__ __attribute__((aligned(1024))) uint16_t xs[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
    U.n0 = (in_group / gsize) * kBN;
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
  // (64 bytes each, the step's K range); lane l lands on row (l / 4), physical
  // 16-byte chunk l % 4, holding the logical chunk (l % 4) ^ (l / 16) (the
  // row's (row / 4) % 4), so the decoding reads below are conflict-free.
  // A wave loads, and later reads, only its own rows.
  const int wc = (lane & 3) ^ (lane >> 4);
  uint32_t wvo[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) wvo[i] = (uint32_t)((64 * wave + 16 * i + (lane >> 2)) * K + 16 * wc);
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(s, (uint32_t)(((N + kBlock - 1) / kBlock) * gk * 4));

  // The unit whose steps are being loaded (up to three steps ahead of the
  // one being computed, so at the end of a unit it is the next one).
  Unit LU = unit_of(0);
  __amdgpu_buffer_rsrc_t xrs, wrs;
  bool lwave_live;
  int lsrow;
  auto set_load_unit = [&](const Unit& U) {
    LU = U;
    xrs = make_rsrc(x + (size_t)U.m0 * K, (uint32_t)(U.nreal > 0 ? min(M - U.m0, kBM) * K * 2 : 0));
    wrs = make_rsrc(q + (size_t)U.n0 * K, (uint32_t)(U.nreal > 0 ? max(min(N - U.n0, kBN), 0) * K : 0));
    lwave_live = U.n0 + 64 * wave < N;
    lsrow = lwave_live ? (U.n0 + 64 * wave) / kBlock : 0;
  };
  set_load_unit(LU);

  auto issue_x = [&](int stage, int kt) {
    const int kbase = (LU.kt0 + kt) * kBK;
    // K left in this step (0 past the unit's range): a chunk is read iff it
    // starts below it
    const int klim = kt < LU.nreal ? K - kbase : 0;
    const uint32_t soff = (uint32_t)(kbase * 2);
    const bool in_even = xc_even * 8 < klim, in_odd = xc_odd * 8 < klim;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (lds_ptr_t)&xs[stage * kStageElems + (64 * wave + 8 * i) * kBK], 16,
          ((i & 1) ? in_odd : in_even) ? xvo[i] : kOob, soff, 0, 0);
  };
  auto issue_w = [&](int stage, int kt) {
    const int kbase = (LU.kt0 + kt) * kBK;
    const int klim = kt < LU.nreal ? K - kbase : 0;
    const bool kin = 16 * wc < klim;
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrs, (lds_ptr_t)&xs[stage * kStageElems + kXElems + (64 * wave + 16 * i) * kBK / 2], 16,
          kin ? wvo[i] : kOob, (uint32_t)kbase, 0, 0);
  };
  // Weight scale: one per wave and step, loaded with the step's codes as a
  // vector load (every lane the same address), so it rides the same counter
  // as the codes and no scalar load is ever in flight next to the operand
  // reads. Waves past N and dead steps read zero. (The address is always
  // formed, block clamped, and pushed out of range when dead: a select
  // between two computed offsets became a branch.)
  auto issue_s = [&](float& sc, int kt) {
    const int kb = min(((LU.kt0 + kt) * kBK) / kBlock, gk - 1);
    const bool live = lwave_live & (kt < LU.nreal);
    const uint32_t off = (uint32_t)((lsrow * gk + kb) * 4) + (live ? 0u : kOob);
    sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, off, 0, 0));
  };

  // Codes of weight block nb, K half j of a stage (the 16 codes of sub-steps
  // 2j and 2j+1): lane l reads row 64w + 32nb + l%32, logical chunk
  // l/32 + 2j, stored at chunk (l/32 + 2j) ^ ((l%32 / 4) % 4).
  const int crow = (64 * wave + (lane & 31)) * kBK;     // byte offset of the lane's row
  const int cswz = ((lane & 31) >> 2) & 3;
  const int crd0 = crow + ((((lane >> 5) + 0) ^ cswz) << 4);
  const int crd1 = crow + ((((lane >> 5) + 2) ^ cswz) << 4);
  auto read_w = [&](u32x4 (&c)[2], int stage, int j) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(&xs[stage * kStageElems + kXElems]) + (j ? crd1 : crd0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) c[nb] = *reinterpret_cast<const u32x4*>(base + nb * 32 * kBK);
  };
  // Sub-step t from the codes of its K half -> the two A operands.
  auto decode = [&](bf16x8 (&wd)[2], const u32x4 (&c)[2], float sc, int t) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) wd[nb] = dequant8(c[nb][(t & 1) * 2], c[nb][(t & 1) * 2 + 1], sc);
  };
  // Sub-step t of a stage -> the eight B operands (X row blocks 0..7).
  const int arow = lane & 31;
  const int ahalf = lane >> 5;
  const int aswz = (arow >> 1) & 7;
  auto read_x = [&](bf16x8 (&xf)[8], int stage, int t) {
    const int c = 2 * ahalf + 4 * (t >> 1) + (t & 1);
    const uint16_t* base = &xs[stage * kStageElems + arow * kBK + ((c ^ aswz) << 3)];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      xf[mb] = *reinterpret_cast<const bf16x8*>(base + mb * 32 * kBK);
  };

  f32x16 acc[2][8];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

  // MFMAs of blocks [mb_lo, mb_hi) for one sub-step.
  auto mfma_part = [&](const bf16x8 (&wd)[2], const bf16x8 (&xf)[8], int mb_lo, int mb_hi) {
#pragma unroll
    for (int mb = mb_lo; mb < mb_hi; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wd[nb], xf[mb], acc[nb][mb], 0, 0, 0);
  };

  float ss0, ss1, ss2;
  u32x4 cA[2], cB[2];      // codes of K halves 0 and 1 of a step
  bf16x8 wd0[2], wd1[2];
  bf16x8 xf0[8], xf1[8];

  // Prologue: steps 0, 1, 2 of the first unit in flight (every unit has a
  // multiple of three steps); wait for step 0, then prepare the first
  // sub-step's operands.
  issue_x(0, 0);
  issue_w(0, 0);
  issue_s(ss0, 0);
  issue_x(1, 1);
  issue_w(1, 1);
  issue_s(ss1, 1);
  issue_x(2, 2);
  issue_w(2, 2);
  issue_s(ss2, 2);
  __builtin_amdgcn_s_waitcnt(vm_wait(2 * kLoadsPerStep));
  __builtin_amdgcn_s_barrier();
  read_w(cA, 0, 0);
  decode(wd0, cA, ss0, 0);
  read_x(xf0, 0, 0);

  // One sub-step's MFMAs with the next sub-step's decode and operand reads
  // spread between them.
  auto interleave16 = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // One step: scale of this step in sc, of the next in scn; X and codes in
  // stage S; `lkt` is the step of the load unit to fetch into the stage this
  // step frees and into sc. On entry wd0/xf0 hold sub-step 0's operands and
  // cA the codes of K half 0; on exit, the same for the next step.
  auto step = [&](int S, int lkt, float& sc, float& scn) {
    const int Sn = S == kStages - 1 ? 0 : S + 1;
    // sub-step 0: MFMAs on (wd0, xf0); prepare sub-step 1 into (wd1, xf1)
    // and read the codes of K half 1
    decode(wd1, cA, sc, 1);
    read_x(xf1, S, 1);
    read_w(cB, S, 1);
    mfma_part(wd0, xf0, 0, 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      if (i < 10) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1
    decode(wd0, cB, sc, 2);
    read_x(xf0, S, 2);
    mfma_part(wd1, xf1, 0, 8);
    interleave16();
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 2
    decode(wd1, cB, sc, 3);
    read_x(xf1, S, 3);
    mfma_part(wd0, xf0, 0, 8);
    interleave16();
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 3, first half: its operands are in registers once this
    // wave's reads of stage S have returned.
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    mfma_part(wd1, xf1, 0, 4);
    __builtin_amdgcn_sched_barrier(0);
    // The next step's loads have landed (only the step after it may still be
    // in flight), and every wave is done reading stage S: refill it three
    // steps ahead and reuse this step's scale register for that step. The
    // loads, the next step's first code reads, decode and operand reads run
    // between the second half's MFMAs.
    __builtin_amdgcn_s_waitcnt(vm_wait(kLoadsPerStep));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_x(S, lkt);
    issue_w(S, lkt);
    issue_s(sc, lkt);
    read_w(cA, Sn, 0);
    decode(wd0, cA, scn, 0);
    read_x(xf0, Sn, 0);
    mfma_part(wd1, xf1, 4, 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int col_lane = 64 * wave + 4 * ahalf;
  for (int ci = 0; ci < my_units; ++ci) {
    for (int kt = 0; kt < steps_per_unit; kt += 3) {
      // The loads of this triple are steps kt+3..kt+5 of this unit, or,
      // for its last triple, steps 0..2 of the next.
      int lkt = kt + 3;
      if (lkt == steps_per_unit) {
        set_load_unit(unit_of(ci + 1));
        lkt = 0;
      }
      step(0, lkt, ss0, ss1);
      step(1, lkt + 1, ss1, ss2);
      step(2, lkt + 2, ss2, ss0);
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
    if constexpr (!SPLIT) {
      const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + (size_t)CU.m0 * N, (uint32_t)(rows * N * 2));
      if ((N & 3) == 0) {
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
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = col_base + 32 * nb + 8 * g;
              const uint32_t off = col < N ? (uint32_t)(((arow + 32 * mb) * N + col) * 4) : kOob;
              const f32x16& a = acc[nb][mb];
              // (__builtin_bit_cast of a vector element read element 0 here:
              // the values go through __float_as_uint instead.)
              const u32x4 v = {__float_as_uint(a[4 * g]), __float_as_uint(a[4 * g + 1]),
                               __float_as_uint(a[4 * g + 2]), __float_as_uint(a[4 * g + 3])};
              __builtin_amdgcn_raw_buffer_store_b128(v, prs, off, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
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

LargePlan plan_large(int64_t m, int64_t n, int64_t k) {
  const int nkt = (int)((k + kBK - 1) / kBK);
  const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
  int splits = 1;
  // Split K only while the tiles leave most CUs idle and each split keeps
  // at least 8 steps.
  while (tiles * splits * 2 <= 256 && (nkt + 2 * splits - 1) / (2 * splits) >= 8) splits *= 2;
  LargePlan p;
  p.kt_per_split = (nkt + splits - 1) / splits;
  p.splits = (nkt + p.kt_per_split - 1) / p.kt_per_split;
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
  // one persistent workgroup per CU; every unit padded to a multiple of
  // three steps (the register ring's period; padded steps read zeros)
  const int grid = units < device_cus() ? units : device_cus();
  const int spu = (p.kt_per_split + 2) / 3 * 3;
  if (p.splits == 1) {
    hipLaunchKernelGGL(gemm_large_kernel<false>, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                       x, q, s, y, nullptr, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                       p.kt_per_split, 1, spu);
    return hipGetLastError();
  }
  if (ws == nullptr || ws_bytes < large_workspace_bytes(m, n, k)) return hipErrorInvalidValue;
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(gemm_large_kernel<true>, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                     x, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                     p.kt_per_split, p.splits, spu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce_partials(part, y, p.splits, m, n, stream);
}

}  // namespace fp8bl
