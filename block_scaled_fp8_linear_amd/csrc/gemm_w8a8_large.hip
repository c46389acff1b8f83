// W8A8 block-scaled GEMM for large M, N (same arithmetic as gemm_w8a8.hip):
//   Y[m,n] = bf16( sum_kb fl32(xs[kb,m] * S[n/128,kb]) * P_kb[m,n] ),
//   P_kb = the fp32 sum of the exact E4M3 x E4M3 products of K block kb,
// accumulated in fp32 with one FMA per K block (FastVideo PR #1829,
// "Changes": the converter's 128x128 weight blocks and the Blackwell route's
// per-token activation quantizer feeding a groupwise GEMM).
//
// Tile BM (X rows: 192 or 128, picked per shape) x 256 (weight rows), one
// workgroup of four waves per CU, persistent over (tile, K split) units like
// the bf16 large-M kernel. Wave w owns weight rows [64w, 64w + 64) of the
// tile against all BM X rows: 4 x (BM / 16) blocks of
// v_mfma_scale_f32_16x16x128_f8f6f4 (E8M0 block scales held at 1.0: the
// scales here are arbitrary fp32), BM fp32 accumulators per lane. (With 256
// X rows the accumulators take all 256 VGPRs a lane can address, every block
// sum lands in AGPRs and has to be copied out before its FMA: twice the VALU
// work, more than the MFMA time.)
// The weight block is the A operand and X the B operand, so a lane's four
// results of a block are four consecutive output columns of one output row:
// the block's combined scale is one number per lane (its X row's scale times
// the wave's weight scale, the wave's 64 rows lying in one 128-row block).
// Per K block a wave reads BM / 16 X fragments from LDS, each feeding 4
// MFMAs, half the LDS bytes per MFMA of the 64 x 64 per-wave tile.
//
// One step = one 128-wide K block. A stage holds the step's X codes (BM rows
// x 128 B), weight codes (256 rows x 128 B), the tile's activation scales and
// one weight scale per wave (58 KB at 192 rows, 50 KB at 128), all moved
// global -> LDS by direct-to-LDS buffer loads (no registers), the 16-byte
// chunks of a row XOR-permuted by (row & 7) ^ ((row >> 3) & 1) so the operand
// reads (16 lanes on 16 consecutive rows, one chunk) are conflict-free. Three
// stages fit at 128 rows (loads two steps ahead), two at 192 (one step ahead).
// A wave loads only its own BM / 4 X rows and 64 weight rows (16 or 14 loads
// per step), spread over the first part of the step; the barrier at the end
// of each step hands the stages over.
//
// MFMA operand layout (16x16x128, 8-bit operands): lane l supplies the 32
// codes of row l % 16 of its block at K quarter l / 16 (chunks 2(l/16) and
// 2(l/16) + 1 of the 128-byte row); A and B use the same lane -> k map.
// Result: lane l holds column l % 16 (the X row) and rows 4(l/16) .. +3 (the
// weight rows) of the 16 x 16 block.
//
// Rows past M or N and K past the end read as zero through buffer
// descriptors that cover only valid rows and per-lane out-of-range offsets;
// an activation scale past M and the weight scale of a wave past N read as
// zero too. The output needs N % 8 == 0 (whole 16-byte stores).
#include <atomic>

#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;                     // K per step: one scale block
constexpr int kBN = 256;                     // weight rows per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kWBytes = kBN * kBK;           // weight codes of a stage
constexpr int kWLoads = kBN / kWaves / 8;    // 16-byte loads per lane per step: weight rows (8 of 128 B each)
constexpr uint32_t kOob = 0x80000000u;
constexpr int kFmtE4M3 = 0;                  // f8f6f4 operand format code of E4M3
constexpr int kE8M0One = 127;                // E8M0 exponent of 1.0

// Stage layout for a tile of BM X rows (192 or 128): X codes, weight codes,
// 256 activation-scale slots, one 256-byte weight-scale slot per wave; as
// many stages (two or three) as fit the CU's 160 KB of LDS. Loads run
// kStages - 1 steps ahead.
template <int BM>
struct Stage {
  static constexpr int kMB = BM / 16;                  // 16-row X blocks
  static constexpr int kXBytes = BM * kBK;
  static constexpr int kSxOff = kXBytes + kWBytes;
  static constexpr int kSwOff = kSxOff + 256 * 4;
  static constexpr int kBytes = kSwOff + kWaves * 256;
  static constexpr int kXLoads = BM / kWaves / 8;      // X row loads per lane per step
  static constexpr int kLoads = kXLoads + kWLoads + 2; // loads per wave and step
  static constexpr int kStages = 3 * kBytes <= 160 * 1024 ? 3 : 2;
  static_assert(kBytes % 256 == 0, "stages keep the LDS bank phase of their rows");
  static_assert(kStages * kBytes <= 160 * 1024, "the stages fit the CU's LDS");
  static_assert(((BM / kWaves) & 15) == 0, "a wave's X rows start at a multiple of 16 (swizzle phase)");
  static_assert(kMB % 4 == 0 && kXLoads <= kWLoads, "row blocks in fours; X loads fit the load regions");
};

constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kLgkmWait0 = 0xC07F;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer, offsets at or past `bytes` read as zero; the size made
  // wave-uniform so the descriptor stays in scalar registers
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Physical 16-byte chunk of logical chunk c in tile row r (128-byte rows).
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

template <int BM, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1)
void gemm_w8a8_large_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                            const uint8_t* __restrict__ q, const float* __restrict__ s,
                            uint16_t* __restrict__ y, float* __restrict__ part, int M, int N,
                            int K, int gk, int tiles_m, int tiles_n, int kb_per_split, int splits,
                            int steps_per_unit) {
  using St = Stage<BM>;
  constexpr int kBM = BM, kMB = St::kMB, kXBytes = St::kXBytes, kSxOff = St::kSxOff,
                kSwOff = St::kSwOff, kStageBytes = St::kBytes, kXLoads = St::kXLoads,
                kStages = St::kStages, kAhead = kStages - 1;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- Work units (tile, K split), dealt to the persistent workgroups
  // round-robin; each XCD gets a contiguous run, split-major, walked in
  // groups of 8 M-tiles (as in the bf16 large-M kernel).
  const int ntiles = tiles_m * tiles_n;
  const int units = ntiles * splits;
  const int my_units = (units - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  struct Unit {
    int m0, n0, kb0, nreal, split;
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
    U.kb0 = U.split * kb_per_split;
    U.nreal = min(kb_per_split, gk - U.kb0);
    return U;
  };

  // ---- Staging. Load j of wave w fills X rows 48w + 8j .. +8 (weight rows
  // 64w + 8j .. +8): lane l lands on row (l / 8) of those, physical chunk
  // l % 8, and fetches the logical chunk swz puts there, (l % 8) ^ (l / 8) ^
  // (j & 1) (both first rows are multiples of 16). The step's K offset goes
  // in the scalar offset.
  const int c_even = (lane & 7) ^ (lane >> 3);
  uint32_t xvo[kXLoads], wvo[kWLoads];
#pragma unroll
  for (int j = 0; j < kXLoads; ++j)
    xvo[j] = (uint32_t)(((kBM / kWaves) * wave + 8 * j + (lane >> 3)) * K + (c_even ^ (j & 1)) * 16);
#pragma unroll
  for (int j = 0; j < kWLoads; ++j)
    wvo[j] = (uint32_t)(((kBN / kWaves) * wave + 8 * j + (lane >> 3)) * K + (c_even ^ (j & 1)) * 16);
  // Activation scales: slot 16 * c + b (b < 12) of the stage's 256 holds
  // the scale of tile row 16 * b + c, so a lane reads its 12 rows' scales
  // (rows l % 16 + 16 b) as 48 contiguous bytes. Wave w fills slots 64w ..
  // +64; slots with b >= 12 are loaded out of range (zero) and never read.
  const int sx_row = 16 * (lane & 15) + 4 * wave + (lane >> 4);
  const bool sx_slot = (lane & 15) < kMB;
  const __amdgpu_buffer_rsrc_t sxrs = make_rsrc(xs, (uint32_t)((size_t)gk * M * 4));
  const __amdgpu_buffer_rsrc_t swrs = make_rsrc(s, (uint32_t)(((N + kBlock - 1) / kBlock) * gk * 4));

  Unit LU = unit_of(0);
  __amdgpu_buffer_rsrc_t xrs, wrs;
  bool lwave_live, lsx_live;
  int lsrow;
  auto set_load_unit = [&](const Unit& U) {
    LU = U;
    xrs = make_rsrc(xq + (size_t)U.m0 * K, (uint32_t)(U.nreal > 0 ? min(M - U.m0, kBM) * K : 0));
    wrs = make_rsrc(q + (size_t)U.n0 * K, (uint32_t)(U.nreal > 0 ? max(min(N - U.n0, kBN), 0) * K : 0));
    lwave_live = U.n0 + 64 * wave < N;
    lsrow = lwave_live ? (U.n0 + 64 * wave) / kBlock : 0;
    lsx_live = sx_slot && U.m0 + sx_row < M;
  };
  set_load_unit(LU);

  // `sb` is the stage's first byte (wave-uniform), `kt` the step of LU.
  auto issue_row = [&](__amdgpu_buffer_rsrc_t rs, int region, int first_row, uint32_t vo, int sb,
                       int kt, int j) {
    const int kbase = (LU.kb0 + kt) * kBK;
    const int klim = kt < LU.nreal ? K - kbase : 0;
    const bool in = (c_even ^ (j & 1)) * 16 < klim;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&lds[sb + region + (first_row + 8 * j) * kBK], 16,
                                             in ? vo : kOob, (uint32_t)kbase, 0, 0);
  };
  auto issue_sx = [&](int sb, int kt) {
    const int kb = min(LU.kb0 + kt, gk - 1);
    const bool live = lsx_live & (kt < LU.nreal);
    const uint32_t off = (uint32_t)(((size_t)kb * M + LU.m0 + sx_row) * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sxrs, (lds_ptr_t)&lds[sb + kSxOff + 64 * wave * 4], 4,
                                             live ? off : kOob, 0, 0, 0);
  };
  // the wave's weight scale, every lane fetching the same word (64 copies)
  auto issue_sw = [&](int sb, int kt) {
    const int kb = min(LU.kb0 + kt, gk - 1);
    const bool live = lwave_live & (kt < LU.nreal);
    const uint32_t off = (uint32_t)((lsrow * gk + kb) * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(swrs, (lds_ptr_t)&lds[sb + kSwOff + wave * 256], 4,
                                             live ? off : kOob, 0, 0, 0);
  };
  // the loads of region r (0..7) of a step: X row load r (r < 6), weight
  // row load r, and the two scales in regions 0 and 1
  auto issue_region = [&](int sb, int kt, int r) {
    if (r < kXLoads) issue_row(xrs, 0, (kBM / kWaves) * wave, xvo[r], sb, kt, r);
    issue_row(wrs, kXBytes, (kBN / kWaves) * wave, wvo[r], sb, kt, r);
    if (r == 0) issue_sx(sb, kt);
    if (r == 1) issue_sw(sb, kt);
  };

  // ---- Operand reads.
  const int r16 = lane & 15;
  const int g = lane >> 4;
  auto read_frag = [&](int base, int row) -> i32x8 {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(&lds[base + row * kBK + (swz(row, 2 * g) << 4)]);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(&lds[base + row * kBK + (swz(row, 2 * g + 1) << 4)]);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto read_w = [&](int sb, int nb) { return read_frag(sb + kXBytes, 64 * wave + 16 * nb + r16); };
  auto read_x = [&](int sb, int mb) { return read_frag(sb, 16 * mb + r16); };

  f32x4v acc[4][kMB];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) acc[nb][mb] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const f32x4v zero = {0.f, 0.f, 0.f, 0.f};

  auto wg_barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Prologue: the first unit's first kAhead steps (every unit has at least
  // that many; a padded step reads zeros); wait for the first.
#pragma unroll
  for (int a = 0; a < kAhead; ++a)
#pragma unroll
    for (int r = 0; r < kWLoads; ++r) issue_region(a * kStageBytes, a, r);
  __builtin_amdgcn_s_waitcnt(vm_wait((kAhead - 1) * St::kLoads));
  wg_barrier();

  int S = 0;                 // stage of the step being computed
  int lkt = kAhead - 1;      // step (of LU) most recently loaded
  for (int ci = 0; ci < my_units; ++ci) {
    for (int kt = 0; kt < steps_per_unit; ++kt) {
      // the step kAhead ahead: of LU, or an early step of the next unit
      if (++lkt == steps_per_unit) {
        set_load_unit(unit_of(ci + 1));
        lkt = 0;
      }
      const int sb = S * kStageBytes;
      const int sbn = (S + kAhead < kStages ? S + kAhead : S + kAhead - kStages) * kStageBytes;

      i32x8 wf[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) wf[nb] = read_w(sb, nb);
      const float sw = *reinterpret_cast<const float*>(&lds[sb + kSwOff + wave * 256 + lane * 4]);
      f32x4v sxv[kMB / 4];
#pragma unroll
      for (int i = 0; i < kMB / 4; ++i)
        sxv[i] = *reinterpret_cast<const f32x4v*>(&lds[sb + kSxOff + r16 * 64 + 16 * i]);
      i32x8 xf[3];
      xf[0] = read_x(sb, 0);
      xf[1] = read_x(sb, 1);
      f32x4v pr[2][4];
      float sc[2];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        if (mb + 2 < kMB) xf[(mb + 2) % 3] = read_x(sb, mb + 2);
        if constexpr (kMB > kWLoads) {
          if (mb < kWLoads) issue_region(sbn, lkt, mb);
        } else if (mb < kWLoads / 2) {
          // as many regions as loads: two per region over the first half, so
          // the last ones are not issued just before the step's wait
          issue_region(sbn, lkt, 2 * mb);
          issue_region(sbn, lkt, 2 * mb + 1);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          pr[mb & 1][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[nb], xf[mb % 3], zero, kFmtE4M3, kFmtE4M3, 0, kE8M0One, 0, kE8M0One);
        sc[mb & 1] = __fmul_rn(sxv[mb >> 2][mb & 3], sw);
        if (mb >= 1) {
          const int pm = mb - 1;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[nb][pm][r] = __builtin_fmaf(pr[pm & 1][nb][r], sc[pm & 1], acc[nb][pm][r]);
        }
        // Region order: each MFMA of this block, then four FMAs of the
        // previous block (whose sums were issued four MFMAs earlier), with
        // the operand reads and loads between. Left to itself the compiler
        // put the previous block's 16 FMAs first, where they waited for the
        // last MFMAs and held this block's MFMAs behind them.
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (load to LDS)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[nb][kMB - 1][r] = __builtin_fmaf(pr[(kMB - 1) & 1][nb][r], sc[(kMB - 1) & 1], acc[nb][kMB - 1][r]);
      // this wave's part of the next stage has landed (only this step's own
      // loads may still be in flight) and its reads of this stage have
      // returned; after the barrier every wave's have
      __builtin_amdgcn_s_waitcnt(vm_wait((kAhead - 1) * St::kLoads));
      __builtin_amdgcn_s_waitcnt(kLgkmWait0);
      wg_barrier();
      S = S + 1 == kStages ? 0 : S + 1;
    }

    // ---- Epilogue of unit ci (the next unit's first steps are loaded or in
    // flight, from stage S on). acc[nb][mb][r] is output row m0 + 16mb +
    // l % 16, column n0 + 64w + 16nb + 4(l / 16) + r. The wave's 64 weight
    // rows (8 KB) of the stage the last step used are its own: every wave finished
    // reading that stage before the last barrier, and only this wave refills
    // those rows, with loads it issues after these reads have returned. Each
    // 16-row block goes there row-major and comes back as whole 128-byte
    // (bf16) or 256-byte (fp32) rows, 16 bytes per lane.
    const Unit CU = unit_of(ci);
    const int rows = min(M - CU.m0, kBM);
    const int tb = (S == 0 ? kStages - 1 : S - 1) * kStageBytes + kXBytes + (kBN / kWaves) * wave * kBK;
    int le;
    asm volatile("" : "=v"(le) : "0"(lane));   // keeps the addresses below out of the main loop's registers
    const int er = le & 15, eg = le >> 4;
    if constexpr (!SPLIT) {
      const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + (size_t)CU.m0 * N, (uint32_t)(rows * N * 2));
      const int cc = le & 7, rr = le >> 3;
      const int col8 = CU.n0 + 64 * wave + 8 * cc;
#pragma unroll
      for (int mb4 = 0; mb4 < kMB / 4; ++mb4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint8_t* buf = &lds[tb + i * 2048];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const f32x4v& a = acc[nb][4 * mb4 + i];
            const u32x2 v = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
            const int c = 2 * nb + (eg >> 1);
            *reinterpret_cast<u32x2*>(buf + er * 128 + ((c ^ (er & 7)) << 4) + 8 * (eg & 1)) = v;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint8_t* buf = &lds[tb + i * 2048];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int r = 8 * j + rr;
            const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * 128 + ((cc ^ (r & 7)) << 4));
            const uint32_t off = col8 < N ? (uint32_t)(((16 * (4 * mb4 + i) + r) * N + col8) * 2) : kOob;
            __builtin_amdgcn_raw_buffer_store_b128(v, yrs, off, 0, 0);
          }
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t prs =
          make_rsrc(part + (size_t)CU.split * partial_slab(M, N) + (size_t)CU.m0 * N,
                    (uint32_t)(rows * N * 4));
      const int cc = le & 15, rq = le >> 4;
      const int col4 = CU.n0 + 64 * wave + 4 * cc;
#pragma unroll
      for (int mb2 = 0; mb2 < kMB / 2; ++mb2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint8_t* buf = &lds[tb + i * 4096];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const f32x4v& a = acc[nb][2 * mb2 + i];
            const u32x4 v = {__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                             __float_as_uint(a[3])};
            const int c = 4 * nb + eg;
            *reinterpret_cast<u32x4*>(buf + er * 256 + ((c ^ er) << 4)) = v;
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint8_t* buf = &lds[tb + i * 4096];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + rq;
            const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * 256 + ((cc ^ r) << 4));
            const uint32_t off = col4 < N ? (uint32_t)(((16 * (2 * mb2 + i) + r) * N + col4) * 4) : kOob;
            __builtin_amdgcn_raw_buffer_store_b128(v, prs, off, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) acc[nb][mb] = f32x4v{0.f, 0.f, 0.f, 0.f};
  }
  // The loads issued for the step after the last one target the ring; drain
  // them before exit.
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
}

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

// Tile height, split count and time estimate (microseconds): the busiest
// CU runs ceil(units / 256) units of `steps` steps each, plus about 4 us per
// unit (its first loads and its epilogue); K splits add the fp32 partials'
// round trip. Per 256-wide weight slab and 128-wide K block, a step of 192 X
// rows takes 1.45 us on a CU and one of 128 rows 1.16 us (measured on
// 16384 x 3072 x 3072, 4096^3 and 512 x 25600 x 5120; the smaller tile
// issues 14 loads per wave for 32 MFMAs against 16 for 48). The lower tile
// wins where it fills the last round better: 16384 x 3072 x 3072 187 against
// 201 us (1536 tiles of 128 rows, 6 full rounds, against 1032 of 192 rows,
// 4.03 rounds), 4096^3 83 against 103; 192 rows win at 16384 x 12288 x 3072
// (630 against 771) and 1536 x 8192 x 2048 (35 against 45). The estimates
// rank all eight shapes measured the same way.
W8a8LargePlan plan_w8a8_large(int64_t m, int64_t n, int64_t k) {
  const int gk = (int)((k + kBK - 1) / kBK);
  W8a8LargePlan p{192, 1, gk, 1e300};
  for (const int bm : {192, 128}) {
    const double step_us = bm == 192 ? 1.45 : 1.16;
    const int64_t tiles = ((m + bm - 1) / bm) * ((n + kBN - 1) / kBN);
    for (int sp = 1; sp <= 8; ++sp) {
      const int steps = (gk + sp - 1) / sp;
      if (sp > 1 && steps < 4) break;
      const int64_t per_cu = (tiles * sp + 255) / 256;
      double cost = (double)per_cu * (steps * step_us + 4.0);
      if (sp > 1) cost += (double)(6 * sp + 2) * (double)(m * n) / 5.0e6;
      if (cost < p.cost) {
        p.cost = cost;
        p.bm = bm;
        p.splits = sp;
      }
    }
  }
  p.kb_per_split = (gk + p.splits - 1) / p.splits;
  p.splits = (gk + p.kb_per_split - 1) / p.kb_per_split;
  return p;
}

size_t w8a8_large_partials_bytes(int64_t m, int64_t n, int64_t k) {
  const W8a8LargePlan p = plan_w8a8_large(m, n, k);
  if (p.splits <= 1) return 0;
  return round_up((size_t)p.splits * partial_slab(m, n) * sizeof(float), kWorkspaceAlign);
}

namespace {

template <int BM>
hipError_t launch_bm(const uint8_t* xq, const float* xs, const uint8_t* q, const float* s,
                     uint16_t* y, int64_t m, int64_t n, int64_t k, void* ws, size_t ws_bytes,
                     const W8a8LargePlan& p, hipStream_t stream) {
  const int gk = (int)((k + kBK - 1) / kBK);
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)((n + kBN - 1) / kBN);
  const int units = tiles_m * tiles_n * p.splits;
  const int grid = units < device_cus() ? units : device_cus();
  // every unit runs at least the prologue's kStages - 1 steps (padded ones read zeros)
  const int spu = p.kb_per_split > Stage<BM>::kStages - 1 ? p.kb_per_split : Stage<BM>::kStages - 1;
  if (p.splits == 1) {
    hipLaunchKernelGGL((gemm_w8a8_large_kernel<BM, false>), dim3((uint32_t)grid), dim3(kThreads), 0,
                       stream, xq, xs, q, s, y, nullptr, (int)m, (int)n, (int)k, gk, tiles_m,
                       tiles_n, p.kb_per_split, 1, spu);
    return hipGetLastError();
  }
  if (ws == nullptr || ws_bytes < w8a8_large_partials_bytes(m, n, k)) return hipErrorInvalidValue;
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL((gemm_w8a8_large_kernel<BM, true>), dim3((uint32_t)grid), dim3(kThreads), 0,
                     stream, xq, xs, q, s, y, part, (int)m, (int)n, (int)k, gk, tiles_m, tiles_n,
                     p.kb_per_split, p.splits, spu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce_partials(part, y, p.splits, m, n, stream);
}

}  // namespace

hipError_t launch_gemm_w8a8_large(const uint8_t* xq, const float* xs, const uint8_t* q,
                                  const float* s, uint16_t* y, int64_t m, int64_t n, int64_t k,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if ((n & 7) != 0) return hipErrorInvalidValue;
  const W8a8LargePlan p = plan_w8a8_large(m, n, k);
  return p.bm == 192 ? launch_bm<192>(xq, xs, q, s, y, m, n, k, ws, ws_bytes, p, stream)
                     : launch_bm<128>(xq, xs, q, s, y, m, n, k, ws, ws_bytes, p, stream);
}

}  // namespace fp8bl
