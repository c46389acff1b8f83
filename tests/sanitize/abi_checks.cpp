// Host-side argument checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitize_cpu.py).
// Every call here returns from validation before any device work: null,
// misaligned and overlapping pointers, negative, zero, oversized and extreme
// sizes, so that the size arithmetic of the validators runs under the
// sanitizers. No pointer passed here is ever dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime.h>

#include "fp8bl.h"

namespace {

int g_fail = 0;

void expect(const char* what, long long got, long long want) {
  if (got != want) {
    std::printf("FAIL %s: got %lld want %lld\n", what, got, want);
    ++g_fail;
  }
}

template <typename T>
T* at(uintptr_t a) { return reinterpret_cast<T*>(a); }

}  // namespace

int main() {
  // Many calls below carry valid sizes with made-up pointers: they stop at
  // the device gate only because there is no GPU. With a device present,
  // run nothing.
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    std::printf("SKIP: a HIP device is present\n");
    return 0;
  }
  const uintptr_t F = (uintptr_t)1 << 20;   // 16-byte aligned, never dereferenced
  const int64_t big = INT64_MAX;
  const int64_t sizes[] = {-1, 0, 1, 15, 16, 17, 127, 128, 129, (int64_t)1 << 20, ((int64_t)1 << 20) + 16,
                           ((int64_t)1 << 31) - 1, (int64_t)1 << 31, (int64_t)1 << 35, big, INT64_MIN};

  expect("abi_version", fp8_block_abi_version(), FP8BL_ABI_VERSION);
  for (int st = -3; st < 10; ++st) expect("status_string non-null", fp8_block_status_string(st) != nullptr, 1);
  expect("status 99", std::strcmp(fp8_block_status_string(99), "FP8BL_UNKNOWN_STATUS"), 0);

  // workspace queries never fail, whatever the sizes
  for (int64_t m : sizes)
    for (int64_t n : sizes)
      for (int64_t k : sizes) {
        (void)fp8_block_linear_workspace_size(m, n, k);
        (void)fp8_block_linear_w8a8_workspace_size(m, n, k);
      }
  expect("ws of empty M", (long long)fp8_block_linear_workspace_size(0, 8, 16), 0);
  expect("ws of bad K", (long long)fp8_block_linear_workspace_size(4, 8, 15), 0);

  uint16_t* x = at<uint16_t>(F);
  uint8_t* q = at<uint8_t>(8 * F);
  float* s = at<float>(16 * F);
  uint16_t* y = at<uint16_t>(24 * F);

  // the linear: every extreme size combination either is an error or an empty no-op
  for (int64_t m : sizes)
    for (int64_t n : sizes)
      for (int64_t k : sizes)
        for (int path = -1; path < 6; ++path) {
          const int st = fp8_block_linear_ex(x, q, s, y, m, n, k, nullptr, 0, path, nullptr);
          const bool ok_empty = st == FP8BL_OK && (m == 0 || n == 0);
          const bool err = st == FP8BL_INVALID_ARG || st == FP8BL_WORKSPACE || st == FP8BL_ALIGNMENT ||
                           st == FP8BL_UNSUPPORTED_DEVICE || st == FP8BL_HIP_ERROR;
          if (!(ok_empty || err)) {
            std::printf("FAIL linear_ex m=%lld n=%lld k=%lld path=%d -> %d\n", (long long)m, (long long)n,
                        (long long)k, path, st);
            ++g_fail;
          }
        }
  expect("linear K%16", fp8_block_linear(x, q, s, y, 4, 8, 15, nullptr, 0, nullptr), FP8BL_INVALID_ARG);
  expect("linear null x", fp8_block_linear(nullptr, q, s, y, 4, 8, 16, nullptr, 0, nullptr), FP8BL_INVALID_ARG);
  expect("linear x misaligned", fp8_block_linear(at<uint16_t>(F + 2), q, s, y, 4, 8, 16, nullptr, 0, nullptr),
         FP8BL_ALIGNMENT);
  expect("linear y over x", fp8_block_linear(x, q, s, x, 4, 8, 16, nullptr, 0, nullptr), FP8BL_INVALID_ARG);
  expect("linear M*K 2^35", fp8_block_linear(x, q, s, y, (int64_t)1 << 19, 1 << 16, 1 << 16, nullptr, 0, nullptr),
         FP8BL_INVALID_ARG);
  expect("linear K too big", fp8_block_linear(x, q, s, y, 1, 8, ((int64_t)1 << 20) + 16, nullptr, 0, nullptr),
         FP8BL_INVALID_ARG);
  expect("linear empty", fp8_block_linear(nullptr, nullptr, nullptr, nullptr, 0, 0, 16, nullptr, 0, nullptr),
         FP8BL_OK);
  for (int64_t m : sizes)
    for (int64_t n : sizes)
      for (int64_t k : sizes) {
        const int st = fp8_block_linear_noalloc(x, q, s, y, m, n, k, nullptr);
        if (st == FP8BL_OK && m != 0 && n != 0) {
          std::printf("FAIL noalloc accepted m=%lld n=%lld k=%lld\n", (long long)m, (long long)n, (long long)k);
          ++g_fail;
        }
      }
  expect("noalloc over scratch",
         fp8_block_linear_noalloc(at<uint16_t>(F << 20), at<uint8_t>(F << 21), at<float>(F << 22),
                                  at<uint16_t>(F << 23), 768, 8192, 65536, nullptr),
         FP8BL_WORKSPACE);

  // dequant / quantize / activation quantizer / stream read
  for (int64_t n : sizes)
    for (int64_t k : sizes) {
      const int a = fp8_block_dequant(q, s, y, n, k, nullptr);
      const int b = fp8_block_quantize(at<float>(32 * F), q, s, n, k, nullptr);
      const int c = fp8_block_quantize_bf16(x, q, s, n, k, nullptr);
      const int d = fp8_act_quantize(x, q, s, n, k, nullptr);
      for (int st : {a, b, c, d})
        if (st == FP8BL_OK && n != 0) {
          std::printf("FAIL elementwise accepted n=%lld k=%lld\n", (long long)n, (long long)k);
          ++g_fail;
        }
    }
  expect("dequant overlap", fp8_block_dequant(q, s, at<uint16_t>(8 * F), 8, 16, nullptr), FP8BL_INVALID_ARG);
  expect("stream null", fp8_block_stream_read(nullptr, 1 << 20, at<uint32_t>(64 * F), 2048, nullptr),
         FP8BL_INVALID_ARG);
  expect("stream blocks", fp8_block_stream_read(x, 1 << 20, at<uint32_t>(64 * F), 65537, nullptr),
         FP8BL_INVALID_ARG);
  expect("stream huge", fp8_block_stream_read(x, SIZE_MAX - 15, at<uint32_t>(64 * F), 2048, nullptr) != FP8BL_OK,
         1);

  // gated pair and W8A8
  for (int64_t m : sizes)
    for (int64_t n : sizes)
      for (int64_t k : sizes) {
        const int a = fp8_block_mlp_gate_up(x, q, s, at<uint8_t>(40 * F), at<float>(48 * F), y, m, n, k, nullptr);
        const int b = fp8_block_linear_w8a8(q, s, at<uint8_t>(40 * F), at<float>(48 * F), y, m, n, k,
                                            nullptr, 0, nullptr);
        const int c = fp8_block_linear_w8a8_bf16(x, q, s, y, m, n, k, nullptr, 0, nullptr);
        const int c2 = fp8_block_linear_w8a8_ex(q, s, at<uint8_t>(40 * F), at<float>(48 * F), y, m, n, k,
                                                nullptr, 0, FP8BL_PATH_LARGE, nullptr);
        const int d = fp8_block_mlp_gate_up_ex(x, q, s, at<uint8_t>(40 * F), at<float>(48 * F), y, m, n, k,
                                               FP8BL_PATH_LARGE, nullptr);
        const int e = fp8_block_mlp_gate_up_ex(x, q, s, at<uint8_t>(40 * F), at<float>(48 * F), y, m, n, k,
                                               7, nullptr);
        if (e != FP8BL_INVALID_ARG) {
          std::printf("FAIL gated path 7 accepted\n");
          ++g_fail;
        }
        for (int st : {a, b, c, c2, d})
          if (st == FP8BL_OK && m != 0 && n != 0) {
            std::printf("FAIL gated/w8a8 accepted m=%lld n=%lld k=%lld\n", (long long)m, (long long)n,
                        (long long)k);
            ++g_fail;
          }
      }

  std::printf("%s: %d failures\n", g_fail ? "FAILED" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
