// Skinny-M block-FP8 linear (M <= 32 per pass): the run is bound by the HBM
// bytes of the E4M3 weight, so the kernel is organised around streaming W
// once, at full bandwidth.
//
// Same arithmetic as the tiled path (FastVideo PR #1829, "Purpose": the
// weight goes to BF16, then an ordinary matmul; fp32 accumulation, one bf16
// rounding per output).
//
// Work unit: a workgroup of W waves owns 32 weight rows (two 16-row tiles)
// and one K range (its split; normally all of K). The range is cut into
// 256-wide super-steps dealt round-robin to the waves.
//
// Load shape. HBM streams well when each load instruction reads a few long
// runs: 4 rows x 256 contiguous bytes per 64-lane instruction reaches ~95%
// of a plain sequential read on MI355X, while the MFMA operand shape (16
// rows x 64 bytes) reaches ~60%. So codes are loaded 4 rows x 256 bytes at a
// time straight into a per-wave LDS slab (16-byte buffer loads that write
// LDS: lane i lands at byte 16*i of the instruction's 1 KB, and fetches the
// 16-byte chunk that puts each row's chunks XOR-permuted by the row index,
// so the MFMA-layout reads back are bank-conflict-free). No barrier is
// needed because each wave only reads what it loaded. Rows past N and the K
// tail read as zero through the buffer descriptors.
//
// The k order inside a super-step is permuted (the MFMA sums over k, so A
// and B only have to agree): MFMA 2h+e gives lane group g the codes
// k = 16*(g + 4h) + 8e .. +8, and X is loaded into registers with the same
// k. X (rows past M read as zero) is tiny and stays in L2; the two tiles of
// a wave share each X fragment. At the end the waves' partial sums meet in
// LDS and are added in wave order; with one split the result is rounded to
// bf16 directly, otherwise fp32 partials go to the workspace and are summed
// in split order by the reduce kernel (no atomics anywhere).
//
// v_mfma_f32_16x16x32_bf16: lane l gives 8 consecutive-k values of row
// (l % 16) of A and of column (l % 16) of B; lane group l / 16 picks the
// k chunk. Output: lane l holds rows (l/16)*4 + r, r = 0..3, column l % 16.
#include "fp8bl_device.h"
#include "fp8bl_internal.h"

namespace fp8bl {

namespace {

constexpr int kSuper = 256;               // K per super-step (16 chunks of 16 codes per row)
constexpr unsigned kXcds = 8;              // XCDs of an MI355X; workgroups are dealt to them in turn
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate (gfx9 encoding: vmcnt[3:0] + vmcnt_hi[15:14],
// expcnt[6:4], lgkmcnt[11:8]): at most n vector-memory operations of this
// wave outstanding, no wait on the others.
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// The codes go global -> LDS directly into a ring of D slots per wave, X
// into D register sets, and each super-step's X loads are issued ahead of
// its code loads. Loads return in issue order, so X, which comes from L2,
// does not wait behind the codes coming from HBM. On MI355X (8000 x 8192,
// rotated weight copies, same box) against the kernel this one replaced,
// which staged the codes through registers into LDS with one super-step in
// flight (outputs bit-identical with the same start order): 16.2 against
// 16.8 us at M = 16, 13.7 against 14.8 at M = 8, 13.0 against 13.7 at
// M = 1. Two slots (one
// super-step in flight behind the one computed) are fastest: three and four
// were 2-14% slower, so the bytes in flight per CU are not what holds the
// rate.
//
// Every super-step issues the same number of loads (steps past the range
// read zero through the buffer descriptors), so one wait for at most
// (D - 1) * kLoads outstanding loads covers the codes and X of the
// super-step about to be computed.
template <int MT, int NT, int WAVES, int D>
__global__ __launch_bounds__(WAVES * 64)
void gemm_skinny_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                        const float* __restrict__ s, uint16_t* __restrict__ y,
                        float* __restrict__ part, int M, int N, int K, int gk,
                        int ss_per_split) {
  constexpr int kSlot = NT * 16 * kSuper;         // one super-step's codes of the wave's tiles
  constexpr int kLoads = NT * 4 + MT * 8;         // code and X loads per super-step
  static_assert((D - 1) * kLoads <= 63, "outstanding loads fit the vmcnt counter");
  static_assert(NT == 1 || NT == 2, "one or two 16-row tiles per workgroup");
  static_assert(kBlock % (16 * NT) == 0, "a workgroup's rows share one scale row");
  __shared__ __attribute__((aligned(16))) uint8_t ring[WAVES][D][kSlot];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * (16 * NT);
  const int nss = (K + kSuper - 1) / kSuper;
  const int ss0 = blockIdx.y * ss_per_split;
  const int ss1 = min(ss0 + ss_per_split, nss);
  // No lambda below captures an array whose size is a template parameter
  // (the ring, the accumulators, the load offsets): hipcc then leaves the
  // host launch stub undefined, without a diagnostic.
  uint8_t* const wring = &ring[wave][0][0];

  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(q + (size_t)n0 * K, (uint32_t)(min(N - n0, 16 * NT) * K));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)(M * K * 2));
  // The workgroup's rows lie in one 128-row scale block (16 * NT divides 128).
  const float* const srow = s + (size_t)(n0 / kBlock) * gk;
  const bool live1 = n0 + 16 < N;    // tile 1 (NT = 2) has rows

  // Code loads: instruction r of tile j brings rows 4r..4r+3, 256 bytes
  // each; lane i lands at byte 16*i of the instruction's 1 KB of the slot
  // and fetches logical chunk (i & 15) ^ row.
  const int lrow4 = lane >> 4;
  const int lchk = lane & 15;
  uint32_t woff[4];       // tile 0's; tile j adds j * 16 rows
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * r + lrow4;
    woff[r] = (uint32_t)(row * K + (lchk ^ row) * 16);
  }
  const uint32_t tile_stride = (uint32_t)(16 * K);
  const int bn = lane & 15;
  const int bg = lane >> 4;
  const uint32_t xoff = (uint32_t)((bn * K + bg * 16) * 2);
  const uint32_t xtile_stride = (uint32_t)(16 * K * 2);

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int count = ss1 - ss0;
  // Every workgroup walks its K range from its own starting super-step, so
  // that at any moment the GPU reads many K offsets at once rather than all
  // rows at one offset (rows 8 KB apart then pile onto a few HBM channels:
  // 30% slower at 8000 x 8192). Workgroups are dealt to the 8 XCDs in turn,
  // so starting workgroup w at w / 8 gives the workgroups on each XCD every
  // start; w itself gave each XCD only four (4% slower at M = 16, 1% at
  // M = 1). The order is fixed per workgroup: results are run-to-run
  // identical.
  const int rot = count > 0 ? (int)((blockIdx.x / kXcds) % (unsigned)count) : 0;
  auto ss_of = [&](int i) {            // i-th super-step of the range, rotated
    if (i >= count) return ss1;        // past the end: loads read nothing
    const int r = i + rot;
    return ss0 + (r >= count ? r - count : r);
  };

  u32x4 xv[D][MT][4][2];
  auto issue = [&](int ss, int slot, u32x4 (&xa)[MT][4][2]) {
    const bool live = ss < ss1;
    const uint32_t kb = (uint32_t)(ss * kSuper);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const bool kin = live && (int)kb + (bg + 4 * h) * 16 < K;
        const uint32_t o = xoff + i * xtile_stride + (kb + (uint32_t)(64 * h)) * 2;
        xa[i][h][0] = buf_load16(xrs, kin ? o : kOob);
        xa[i][h][1] = buf_load16(xrs, kin ? o + 16 : kOob);
      }
    uint8_t* base = wring + slot * kSlot;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * r + lrow4;
      const bool kin = live && (int)kb + ((lchk ^ row) * 16) < K;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr_t)(base + j * 16 * kSuper + r * 1024), 16,
                                                 kin ? woff[r] + j * tile_stride + kb : kOob, 0, 0, kNonTemporal);
    }
  };
  auto compute = [&](int ss, int slot, const u32x4 (&xa)[MT][4][2], f32x4 (&ac)[MT][NT]) {
    // A super-step spans two 128-column scale blocks: logical chunks 0..7
    // (h = 0, 1) take the first, chunks 8..15 (h = 2, 3) the second. A K
    // tail never reads the second block's scale unless it exists.
    const int kb = 2 * ss;
    const float s0 = kb < gk ? srow[kb] : 0.0f;
    const float s1 = kb + 1 < gk ? srow[kb + 1] : 0.0f;
    const uint8_t* base = wring + slot * kSlot;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const bool tl = j == 0 || live1;
      const uint8_t* slab = base + j * 16 * kSuper;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float sc = tl ? (h < 2 ? s0 : s1) : 0.0f;
        const u32x4 c = *reinterpret_cast<const u32x4*>(slab + bn * kSuper + (((bg + 4 * h) ^ bn) << 4));
        const bf16x8 b0 = dequant8(c[0], c[1], sc);
        const bf16x8 b1 = dequant8(c[2], c[3], sc);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          ac[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][h][0]), b0, ac[i][j], 0, 0, 0);
          ac[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][h][1]), b1, ac[i][j], 0, 0, 0);
        }
      }
    }
  };

  // Iteration i computes the wave's super-step ss_of(wave + i * WAVES) from
  // slot i % D, after issuing iteration i + D - 1's loads into the slot that
  // iteration i - 1 has finished reading. The main loop runs whole rounds of
  // D iterations with no branch inside, so the compiler sees which register
  // set each load wrote and adds no wait of its own beyond the one below;
  // the last iters % D iterations run after it. Every register load issued
  // in the main loop is used (by the next round or the tail), so none is
  // dropped and the fixed count holds.
  constexpr int kAhead = D - 1;
#pragma unroll
  for (int p = 0; p < kAhead; ++p) issue(ss_of(wave + p * WAVES), p, xv[p]);
  const int iters = count > wave ? (count - wave + WAVES - 1) / WAVES : 0;
  int i0 = 0;
  for (; i0 + D <= iters; i0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int nslot = (u + kAhead) % D;
      issue(ss_of(wave + (i0 + u + kAhead) * WAVES), nslot, xv[nslot]);
      __builtin_amdgcn_s_waitcnt(vm_wait(kAhead * kLoads));
      compute(ss_of(wave + (i0 + u) * WAVES), u, xv[u], acc);
    }
  }
  // The last iterations' super-steps are already in flight; they issue
  // nothing more and wait for everything. (A load issued here would have
  // no use, and the compiler drops unused register loads, which would
  // leave a fixed wait count short.)
#pragma unroll
  for (int u = 0; u < D - 1; ++u) {
    if (i0 + u < iters) {
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
      compute(ss_of(wave + (i0 + u) * WAVES), u, xv[u], acc);
    }
  }
  // Loads past the range still write (zeros) into the ring: let them land
  // before the ring is reused for the cross-wave sum.
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  __syncthreads();

  f32x4* red = reinterpret_cast<f32x4*>(&ring[0][0][0]);   // [WAVES][MT * NT][64]
  static_assert(WAVES * MT * NT * 64 * 16 <= WAVES * D * kSlot, "the cross-wave sum fits the ring");
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[(wave * MT * NT + i * NT + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  // Each of the first MT*NT waves finishes one (m-tile, n-tile) pair.
  const int pair = wave;
  if (pair >= MT * NT) return;
  const int i = pair / NT, j = pair % NT;
  f32x4 t = red[pair * 64 + lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    const f32x4 o = red[(w * MT * NT + pair) * 64 + lane];
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
constexpr int kRing = 2;   // ring slots per wave: one super-step in flight behind the one computed

struct SkinnyPlan {
  int mt, nt, splits, ss_per_split;
};

// From measurements on MI355X (N=8000, K=8192): 4 waves per workgroup and
// 32 weight rows per workgroup (two 16-row tiles sharing each X fragment)
// for every M; 16 rows per workgroup, twice the workgroups, were 6% slower
// even at M = 1.
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k) {
  SkinnyPlan p;
  p.mt = m > 16 ? 2 : 1;
  p.nt = 2;
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
    if (p.mt == 1)
      hipLaunchKernelGGL((gemm_skinny_kernel<1, 2, kWaves, kRing>), grid, block, 0, stream, xp, q,
                         s, yp, part, (int)rows, (int)n, (int)k, gk, p.ss_per_split);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<2, 2, kWaves, kRing>), grid, block, 0, stream, xp, q,
                         s, yp, part, (int)rows, (int)n, (int)k, gk, p.ss_per_split);
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
