/*
 * fp8bl.h — C ABI of the block-scaled FP8 linear library for MI355X (gfx950).
 *
 * Format (FastVideo PR #1829, "[feat] MiniMax H3: block-FP8 text encoder on
 * Hopper, its converter, and a 4xH100 FastH3 profile", section "Changes",
 * converter bullet): a weight W[N,K] (nn.Linear out x in) is held as
 *   - Q[N,K]   one OCP E4M3FN byte per element, row-major, K contiguous;
 *   - S[GN,GK] one fp32 weight_scale_inv per 128x128 block, row-major,
 *              GN = ceil(N/128), GK = ceil(K/128); the last row/column block
 *              may be partial.
 * The block value is W ~ e4m3(Q) * S. Dequantization (same page, "Purpose")
 * turns each element into bf16( fl32( e4m3(Q[n,k]) * S[n/128][k/128] ) ):
 * an IEEE fp32 multiply, then round-to-nearest-even to bf16.
 *
 * Conventions shared by every call:
 *   - All data pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller. The library never allocates, frees or synchronises; work
 *     is enqueued on `stream` (NULL = the default stream) and the call returns.
 *   - bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *   - Row-major, contiguous. Dimensions are int64_t; zero rows or columns is a
 *     no-op that returns FP8BL_OK. K must be a positive multiple of 16; each
 *     dimension is below 2^31 and each matrix has fewer than 2^35 elements.
 *   - Data pointers must be 16-byte aligned (scale grids 4-byte aligned,
 *     workspaces 256-byte aligned). Outputs must not overlap inputs.
 *   - Every argument error is reported by the return code BEFORE anything is
 *     launched; no exception or abort crosses this interface. A fault inside a
 *     kernel surfaces, as in HIP, at the caller's next synchronisation.
 *   - The library keeps no state besides a per-device cached architecture
 *     check and the scratch of fp8_block_linear_noalloc; calls on different
 *     streams may run concurrently (fp8_block_linear_noalloc excepted).
 *   - Scales are expected finite; other scales still follow the dequant
 *     formula (NaN products become the canonical bf16 NaN 0x7FC0).
 */
#ifndef FP8BL_H
#define FP8BL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BL_ABI_VERSION 1
#define FP8BL_BLOCK 128

/* Return codes of every int-returning call. */
enum fp8bl_status {
  FP8BL_OK = 0,
  FP8BL_INVALID_ARG = 1,        /* null pointer, negative or unsupported size, K % 16 != 0, overlap */
  FP8BL_ALIGNMENT = 2,          /* a pointer is not aligned as required */
  FP8BL_WORKSPACE = 3,          /* workspace missing or smaller than the queried size */
  FP8BL_UNSUPPORTED_DEVICE = 4, /* the current device is not gfx950 */
  FP8BL_HIP_ERROR = 5           /* a HIP runtime call failed (device query or launch) */
};

/* Kernel choice for fp8_block_linear_ex. AUTO picks SKINNY for M <= 32 and
 * otherwise whichever of TILED and LARGE the library's cost model expects to
 * be faster for the shape (LARGE only for N < 2^21); the other values force
 * a kernel (for tests and measurements). TILED is the tile-planned kernel
 * (128- and 256-row tiles), LARGE the persistent 256x256 four-wave kernel,
 * which takes shapes with N < 2^21 (FP8BL_INVALID_ARG otherwise). Every
 * kernel computes the same function to the same error bound; results may
 * differ in the last bits between kernels (different K split counts). */
enum fp8bl_path {
  FP8BL_PATH_AUTO = 0,
  FP8BL_PATH_TILED = 1,
  FP8BL_PATH_SKINNY = 2,
  FP8BL_PATH_LARGE = 3
};

/* Version of this interface (FP8BL_ABI_VERSION). */
int fp8_block_abi_version(void);

/* Static string naming a return code; never NULL. */
const char* fp8_block_status_string(int status);

/* The runtime gate (the page's validate_runtime / get_min_capability pair,
 * FastVideo PR #1829 "Changes", first bullet): 1 if HIP device `device` is a
 * gfx950, else 0 (also 0 when the device cannot be queried). Host only. */
int fp8_block_device_supported(int device);

/* Standalone dequant (FastVideo PR #1829, "Purpose": the Hopper route turns
 * the block-scaled weight into BF16 ahead of the matmul; "Changes", tests
 * bullet: the result must equal, bit for bit, the decoded codes times the
 * scale grid expanded over its blocks).
 *   q          [n,k] E4M3 bytes          (in, 16-B aligned)
 *   scale_inv  [ceil(n/128),ceil(k/128)] fp32 (in, 4-B aligned)
 *   w_bf16     [n,k] bf16 bits           (out, 16-B aligned, may not overlap)
 * Output is bit-exact: bf16_rne(fl32(e4m3(q) * s)), NaN -> 0x7FC0. */
int fp8_block_dequant(const uint8_t* q, const float* scale_inv, uint16_t* w_bf16,
                      int64_t n, int64_t k, hipStream_t stream);

/* Bytes of device workspace fp8_block_linear / fp8_block_linear_ex need for
 * this shape with ANY path (0 when none). Host only; never fails. */
size_t fp8_block_linear_workspace_size(int64_t m, int64_t n, int64_t k);

/* The linear layer (FastVideo PR #1829, "Purpose": the weight goes to BF16,
 * then an ordinary matmul; LightX2V PR #1657, "Walkthrough": FP32 accumulation):
 *   y[m,n] = bf16_rne( sum_k x[m,k] * What[n,k] ),  What as in fp8_block_dequant,
 * with fp32 accumulation and one bf16 rounding per output. What is formed in
 * registers only. No bias. K may be at most 2^20.
 *   x          [m,k] bf16 bits  (in, 16-B aligned)
 *   q, scale_inv                (in, as above)
 *   y          [m,n] bf16 bits  (out, 16-B aligned, may not overlap)
 *   workspace  device scratch of at least fp8_block_linear_workspace_size
 *              bytes (256-B aligned), or NULL when that size is 0 (it holds
 *              fp32 split-K partials). Its contents need no initialisation
 *              and are not preserved. Calls that share a workspace must be
 *              ordered (same stream); calls that overlap on one workspace race. */
int fp8_block_linear(const uint16_t* x, const uint8_t* q, const float* scale_inv,
                     uint16_t* y, int64_t m, int64_t n, int64_t k,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fp8_block_linear with an explicit path (enum fp8bl_path). Same contract;
 * every path accepts every shape, except LARGE, which needs N < 2^21. */
int fp8_block_linear_ex(const uint16_t* x, const uint8_t* q, const float* scale_inv,
                        uint16_t* y, int64_t m, int64_t n, int64_t k,
                        void* workspace, size_t workspace_bytes, int path,
                        hipStream_t stream);

/* Size of the scratch array fp8_block_linear_noalloc keeps on each device. */
#define FP8BL_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/* fp8_block_linear for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same operation, arguments and error codes as fp8_block_linear
 * (AUTO path), except that the split-K partials go to a scratch array inside
 * the library instead of a caller workspace:
 *   - the scratch is FP8BL_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory
 *     per device, part of the library's code object, held until the process
 *     ends; the call allocates nothing (no hipMalloc, no hipFree);
 *   - a shape whose partials need more than that returns FP8BL_WORKSPACE
 *     before anything is launched (every shape with
 *     fp8_block_linear_workspace_size <= 64 MiB fits);
 *   - the first call on a device looks up the scratch's device address once
 *     (hipGetSymbolAddress), with that device current;
 *   - every call on a device shares that device's scratch, which keeps the
 *     last call's partials (nothing in it needs clearing): calls that overlap
 *     on one device (other streams, other host threads) race. Order them on
 *     one stream. */
int fp8_block_linear_noalloc(const uint16_t* x, const uint8_t* q, const float* scale_inv,
                             uint16_t* y, int64_t m, int64_t n, int64_t k, hipStream_t stream);

/* The MLP gate/up pair in one launch, with the SwiGLU epilogue (the step
 * after the gate and up linears; FastVideo fasth3_omniref_b200 README, "What
 * --lossless-accel turns on": SwiGLU rounds to bf16 where the eager ops do):
 *   g = bf16_rne(x Wg_hat^T),  u = bf16_rne(x Wu_hat^T)   (as fp8_block_linear)
 *   h = bf16_rne( bf16_rne(fl32(silu(g))) * u ),  silu(g) = g / (1 + e^-g)
 * Both weights share the shape [n,k] and the input x; g and u never reach
 * memory. silu is evaluated in fp32 with the hardware exp2 and reciprocal
 * (relative error at most (|g| + 4) 2^-23; below about g = -87 the
 * exponential overflows and silu gives -0), so h is graded against the exact
 * silu(G*) U* with a bound, not bit for bit: it can differ from the SwiGLU
 * of the exact-silu rounding where silu(g) lies that close to a bf16
 * rounding boundary.
 *   x                   [m,k] bf16 bits (in, 16-B aligned)
 *   q_gate, q_up        [n,k] E4M3 bytes (in, 16-B aligned)
 *   scale_inv_gate, scale_inv_up  [ceil(n/128),ceil(k/128)] fp32 (in, 4-B aligned)
 *   h                   [m,n] bf16 bits (out, 16-B aligned, may not overlap)
 * No workspace. K may be at most 2^20. */
int fp8_block_mlp_gate_up(const uint16_t* x, const uint8_t* q_gate, const float* scale_inv_gate,
                          const uint8_t* q_up, const float* scale_inv_up, uint16_t* h,
                          int64_t m, int64_t n, int64_t k, hipStream_t stream);

/* fp8_block_mlp_gate_up with the kernel named: FP8BL_PATH_AUTO (what
 * fp8_block_mlp_gate_up does: the lower of two cost-model estimates),
 * FP8BL_PATH_TILED (the tile-planned gate/up kernels) or FP8BL_PATH_LARGE
 * (the large-M kernel's gated form: 256 x 128 output tiles, gate and up rows
 * in separate waves; needs n % 8 == 0 and n < 2^21). Any other path value,
 * or LARGE with another n, is FP8BL_INVALID_ARG. Both kernels meet the same
 * bound; their h may differ in the last bit where their fp32 sums do. */
int fp8_block_mlp_gate_up_ex(const uint16_t* x, const uint8_t* q_gate, const float* scale_inv_gate,
                             const uint8_t* q_up, const float* scale_inv_up, uint16_t* h,
                             int64_t m, int64_t n, int64_t k, int path, hipStream_t stream);

/* ---- W8A8 route -------------------------------------------------------
 * FastVideo PR #1829, "Changes", first bullet: the Blackwell route pairs a
 * groupwise FP8 GEMM with a (Triton) quantizer. Read here as: activations
 * quantized per token in 1x128 K groups with the weight's arithmetic, and a
 * GEMM multiplying E4M3 codes exactly, applying x_scale * weight_scale_inv
 * to each 128-wide K block's fp32 sum. Activation scales are K-block-major:
 * x_scale[kb * m + row], kb < ceil(k/128). */

/* Per-token activation quantization: for every row and 1x128 group along K
 * (the last group may be shorter),
 *   S = fl32(amax / 448)  (1.0 for an all-zero group),
 *   XQ = nearest finite E4M3 to fl32(x / S), ties to even, saturating.
 *   x        [m,k] bf16 bits, finite (in, 16-B aligned)
 *   xq       [m,k] E4M3 bytes (out, 16-B aligned)
 *   x_scale  [ceil(k/128), m] fp32 (out, 4-B aligned)
 * Bit-exact. k % 16 == 0. Non-finite x gives unspecified codes. */
int fp8_act_quantize(const uint16_t* x, uint8_t* xq, float* x_scale, int64_t m, int64_t k,
                     hipStream_t stream);

/* Bytes of workspace fp8_block_linear_w8a8_bf16 needs (the quantized
 * activation, its scales and split-K partials); it also suffices for
 * fp8_block_linear_w8a8. Host only; 0 for empty or invalid shapes. */
size_t fp8_block_linear_w8a8_workspace_size(int64_t m, int64_t n, int64_t k);

/* W8A8 GEMM on pre-quantized activations:
 *   y[m,n] = bf16_rne( sum_kb x_scale[kb,m] * S[n/128,kb] *
 *                      sum_{k in block kb} e4m3(xq[m,k]) * e4m3(q[n,k]) )
 * with fp32 block sums and fp32 accumulation across blocks.
 *   xq, x_scale  as written by fp8_act_quantize (in; 16-B / 4-B aligned)
 *   q, scale_inv the block-FP8 weight, as for fp8_block_linear (in)
 *   y            [m,n] bf16 bits (out, 16-B aligned, may not overlap)
 *   workspace    as for fp8_block_linear (fp32 split-K partials), at least
 *                fp8_block_linear_w8a8_workspace_size bytes or NULL when the
 *                shape needs none; calls sharing it must be ordered.
 * K may be at most 2^20, and the activation scales (4 * m * ceil(k/128)
 * bytes) must stay below 2^32 bytes (FP8BL_INVALID_ARG otherwise; reached
 * only with very small k and m near 2^31). */
int fp8_block_linear_w8a8(const uint8_t* xq, const float* x_scale, const uint8_t* q,
                          const float* scale_inv, uint16_t* y, int64_t m, int64_t n, int64_t k,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fp8_block_linear_w8a8 with the kernel named: FP8BL_PATH_AUTO (what
 * fp8_block_linear_w8a8 does), FP8BL_PATH_TILED (128 x 128 tiles) or
 * FP8BL_PATH_LARGE (192 or 128 X rows x 256 weight rows per tile, by its
 * planner, one persistent workgroup per compute unit; needs n % 8 == 0 and
 * n < 2^21). Any other path, or LARGE with another n, is
 * FP8BL_INVALID_ARG. The workspace rule is the same for every path. Both
 * kernels meet the same bound; their outputs may differ in the last bit
 * where their fp32 sums do. */
int fp8_block_linear_w8a8_ex(const uint8_t* xq, const float* x_scale, const uint8_t* q,
                             const float* scale_inv, uint16_t* y, int64_t m, int64_t n, int64_t k,
                             void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

/* The whole W8A8 route from a bf16 activation: fp8_act_quantize into the
 * workspace, then fp8_block_linear_w8a8. Same result as those two calls.
 *   x          [m,k] bf16 bits, finite (in, 16-B aligned)
 *   workspace  at least fp8_block_linear_w8a8_workspace_size bytes,
 *              256-B aligned (required for every non-empty shape). */
int fp8_block_linear_w8a8_bf16(const uint16_t* x, const uint8_t* q, const float* scale_inv,
                               uint16_t* y, int64_t m, int64_t n, int64_t k, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* The converter's quantization (FastVideo PR #1829, "Changes", converter
 * bullet: E4M3 weight plus per-128x128 weight_scale_inv). For each block:
 *   amax = max |w| over the elements present in the block,
 *   S    = fl32(amax / 448)  (IEEE division; 1.0 when amax == 0),
 *   Q    = nearest finite E4M3 to fl32(w / S), ties to even code, saturating
 *          at +-448, sign kept (-0 and negative underflow give 0x80).
 *   w          [n,k] fp32, finite (in, 16-B aligned)
 *   q          [n,k] E4M3 bytes (out, 16-B aligned)
 *   scale_inv  [ceil(n/128),ceil(k/128)] fp32 (out, 4-B aligned)
 * Bit-exact. Non-finite w gives unspecified codes and scales. */
int fp8_block_quantize(const float* w, uint8_t* q, float* scale_inv,
                       int64_t n, int64_t k, hipStream_t stream);

/* fp8_block_quantize for a bf16 weight (the converter reading a bf16
 * checkpoint): each element is widened exactly to fp32, then quantized as
 * above. Same outputs, contract and bit-exactness.
 *   w_bf16     [n,k] bf16 bits, finite (in, 16-B aligned) */
int fp8_block_quantize_bf16(const uint16_t* w_bf16, uint8_t* q, float* scale_inv,
                            int64_t n, int64_t k, hipStream_t stream);

/* Measurement aid, not part of the layer: a plain streaming read of `bytes`
 * of device memory (16-byte non-temporal loads, grid-stride, `blocks`
 * workgroups of 256 threads), the practical HBM ceiling for the
 * bandwidth-bound kernels. Each thread writes the XOR of the 32-bit words it
 * read to sink[block * 256 + thread], so the XOR over the whole sink equals
 * the XOR of every word of the buffer.
 *   buf     device memory (in, 16-B aligned), bytes % 16 == 0
 *   sink    [blocks * 256] uint32 (out, 4-B aligned, not overlapping buf)
 *   blocks  1 .. 65536
 * bytes == 0 is a no-op. */
int fp8_block_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BL_H */
