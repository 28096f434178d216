// Host-side driver for the C ABI's argument validation, built with the host
// address and undefined-behaviour sanitizers (tests/test_host_sanitizers.py).
// Every call either fails validation before touching memory or a device, or
// is a documented no-op; the fake device addresses below are never
// dereferenced. With the argument --no-device (given only where the host has
// no GPU driver at all) one fully valid call is made too, which must report
// I8MM_ENODEVICE. Prints "ALL OK" and exits 0 when every status matches.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "i8mm.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d (%s), want %d\n", what, got, i8mm_status_string(got), want);
    ++failures;
  }
}

template <class T>
static T* fake(uintptr_t a) { return reinterpret_cast<T*>(a); }

int main(int argc, char** argv) {
  const int64_t big = std::numeric_limits<int64_t>::max();
  const float nan = std::nanf("");
  auto* A16 = fake<uint16_t>(0x10000);
  auto* M16 = fake<uint16_t>(0x10008);   // not 16-byte aligned
  auto* A8 = fake<int8_t>(0x20000);
  auto* F = fake<float>(0x30000);
  auto* U32 = fake<uint32_t>(0x40000);
  auto* I32 = fake<int32_t>(0x50000);
  void* WS = fake<void>(0x100000);
  const int64_t kmax16 = I8MM_MAX_K / 16 * 16;

  // weight quantization
  expect(int8_quantize_colwise_weight(nullptr, 4, 16, A8, F, nullptr), I8MM_EINVAL, "colwise null W");
  expect(int8_quantize_colwise_weight(A16, -1, 16, A8, F, nullptr), I8MM_EINVAL, "colwise N<0");
  expect(int8_quantize_colwise_weight(A16, 4, 24, A8, F, nullptr), I8MM_EALIGN, "colwise K%16");
  expect(int8_quantize_colwise_weight(M16, 4, 16, A8, F, nullptr), I8MM_EALIGN, "colwise misaligned");
  expect(int8_quantize_colwise_weight(A16, 4, kmax16 + 16, A8, F, nullptr), I8MM_ERANGE, "colwise K>max");
  expect(int8_quantize_colwise_weight(A16, big, 16, A8, F, nullptr), I8MM_EINVAL, "colwise N huge");
  expect(int8_quantize_colwise_weight(A16, 4, big / 16 * 16, A8, F, nullptr), I8MM_ERANGE, "colwise K huge");
  expect(int8_quantize_colwise_weight(A16, 0, 16, A8, F, nullptr), I8MM_OK, "colwise empty");

  // row quantization
  expect(int8_quantize_rowwise(nullptr, 4, 16, nullptr, A8, F, nullptr), I8MM_EINVAL, "rowwise null X");
  expect(int8_quantize_rowwise(A16, 4, 16, fake<uint32_t>(0x40008), A8, F, nullptr), I8MM_EALIGN, "rowwise bitmap");
  expect(int8_quantize_rowwise(A16, 4, 8, nullptr, A8, F, nullptr), I8MM_EALIGN, "rowwise K%16");
  expect(int8_quantize_rowwise(A16, big, 16, nullptr, A8, F, nullptr), I8MM_EINVAL, "rowwise M huge");
  expect(int8_quantize_rowwise(A16, 0, 16, nullptr, A8, F, nullptr), I8MM_OK, "rowwise empty");

  // detection
  expect(outlier_detect_gather(A16, 4, 16, nan, U32, I32, I32, nullptr, nullptr), I8MM_EINVAL, "detect NaN");
  expect(outlier_detect_gather(A16, 4, 16, 6.f, nullptr, I32, I32, nullptr, nullptr), I8MM_EINVAL, "detect bitmap");
  expect(outlier_detect_gather(A16, 4, 16, 6.f, U32, nullptr, I32, nullptr, nullptr), I8MM_EINVAL, "detect cols");
  expect(outlier_detect_gather(A16, 4, 16, 6.f, U32, I32, nullptr, nullptr, nullptr), I8MM_EINVAL, "detect n");
  expect(outlier_detect_gather(A16, 4, 16, 6.f, U32, I32, I32, M16, nullptr), I8MM_EALIGN, "detect Xo");
  expect(outlier_detect_gather(A16, 4, 40, 6.f, U32, I32, I32, nullptr, nullptr), I8MM_EALIGN, "detect K%16");
  expect(outlier_detect_gather(A16, -3, 16, 6.f, U32, I32, I32, nullptr, nullptr), I8MM_EINVAL, "detect M<0");

  // the GEMM step
  expect(int8_mm_dequant(nullptr, A8, F, F, 4, 4, 16, nullptr, nullptr, nullptr, nullptr, A16, nullptr, nullptr), I8MM_EINVAL, "mm null Xq");
  expect(int8_mm_dequant(A8, A8, F, F, 4, 4, 16, A16, nullptr, nullptr, nullptr, A16, nullptr, nullptr), I8MM_EINVAL, "mm Xo alone");
  expect(int8_mm_dequant(A8, A8, F, F, 4, 4, 16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), I8MM_EINVAL, "mm no output");
  expect(int8_mm_dequant(A8, A8, F, F, 4, 4, 16, nullptr, nullptr, nullptr, M16, A16, nullptr, nullptr), I8MM_EALIGN, "mm bias");
  expect(int8_mm_dequant(A8, A8, F, F, 4, 4, 17, nullptr, nullptr, nullptr, nullptr, A16, nullptr, nullptr), I8MM_EALIGN, "mm K%16");
  expect(int8_mm_dequant(A8, A8, F, F, 4, -2, 16, nullptr, nullptr, nullptr, nullptr, A16, nullptr, nullptr), I8MM_EINVAL, "mm N<0");
  expect(int8_mm_dequant(A8, A8, F, F, big, big, 16, nullptr, nullptr, nullptr, nullptr, A16, nullptr, nullptr), I8MM_EINVAL, "mm M,N huge");
  expect(int8_mm_dequant(A8, A8, F, F, 0, 4, 16, nullptr, nullptr, nullptr, nullptr, A16, nullptr, nullptr), I8MM_OK, "mm empty");

  // workspace sizes and layout: invalid sizes give 0 / EINVAL, no overflow
  expect((int)(linear_int8_mixed_workspace_bytes(4, 20) == 0), 1, "ws K%16");
  expect((int)(linear_int8_mixed_workspace_bytes(-1, 16) == 0), 1, "ws M<0");
  expect((int)(linear_int8_mixed_workspace_bytes(big, 16) == 0), 1, "ws M huge");
  expect((int)(linear_int8_mixed_workspace_bytes(16, big / 16 * 16) == 0), 1, "ws K huge");
  expect((int)(linear_int8_mixed_workspace_bytes_many_outliers(16, 4096, -1) == 0), 1, "ws N<0");
  expect((int)(linear_int8_mixed_workspace_bytes_many_outliers(16, 4096, big) == 0), 1, "ws N huge");
  int64_t off[7];
  expect(i8mm_workspace_layout(4, 16, nullptr), I8MM_EINVAL, "layout null");
  expect(i8mm_workspace_layout(big, 16, off), I8MM_EINVAL, "layout M huge");
  expect(i8mm_workspace_layout(2048, 4096, off), I8MM_OK, "layout ok");
  expect((int)(off[6] == (int64_t)linear_int8_mixed_workspace_bytes(2048, 4096)), 1, "layout total");

  // the layer calls
  const int64_t M = 8, K = 64, N = 32;
  const size_t need = linear_int8_mixed_workspace_bytes(M, K);
  expect(linear_int8_mixed(A16, M, K, A8, F, N, nullptr, 6.f, A16, WS, need - 1, nullptr), I8MM_EWORKSPACE, "layer ws small");
  expect(linear_int8_mixed(A16, M, K, A8, F, N, nullptr, 6.f, A16, nullptr, need, nullptr), I8MM_EWORKSPACE, "layer ws null");
  expect(linear_int8_mixed(A16, M, K, A8, F, N, nullptr, 6.f, A16, fake<void>(0x100010), need, nullptr), I8MM_EALIGN, "layer ws align");
  expect(linear_int8_mixed(A16, M, K, A8, F, N, nullptr, nan, A16, WS, need, nullptr), I8MM_EINVAL, "layer NaN");
  expect(linear_int8_mixed(A16, M, K, A8, F, N, nullptr, 6.f, nullptr, WS, need, nullptr), I8MM_EINVAL, "layer Y");
  expect(linear_int8_mixed(A16, M, 72, A8, F, N, nullptr, 6.f, A16, WS, need, nullptr), I8MM_EALIGN, "layer K%16");
  expect(linear_int8_mixed(A16, M, K, A8, F, big, nullptr, 6.f, A16, WS, need, nullptr), I8MM_EINVAL, "layer N huge");
  expect(linear_int8_mixed(A16, 0, K, A8, F, N, nullptr, 6.f, A16, WS, linear_int8_mixed_workspace_bytes(0, K), nullptr), I8MM_OK, "layer empty");
  expect(linear_int8_mixed_noalloc(A16, 8192, 8192, A8, F, N, nullptr, 6.f, A16, nullptr), I8MM_EWORKSPACE, "noalloc too big");
  expect(linear_int8_mixed_noalloc(A16, M, K, A8, F, N, nullptr, nan, A16, nullptr), I8MM_EINVAL, "noalloc NaN");
  expect(linear_int8_mixed_noalloc(A16, M, K, A8, F, N, nullptr, 6.f, nullptr, nullptr), I8MM_EINVAL, "noalloc Y");
  expect(linear_int8_mixed_noalloc(A16, 0, K, A8, F, N, nullptr, 6.f, A16, nullptr), I8MM_OK, "noalloc empty");
  expect(linear_int8_mixed_fp16_weights(A16, M, K, nullptr, N, A8, F, 1, nullptr, 6.f, A16, WS, need, nullptr), I8MM_EINVAL, "fp16w W");
  expect(linear_int8_mixed_fp16_weights(A16, M, K, M16, N, A8, F, 1, nullptr, 6.f, A16, WS, need, nullptr), I8MM_EALIGN, "fp16w align");
  expect(outlier_detect_quantize(A16, M, K, nan, WS, need, nullptr), I8MM_EINVAL, "x side NaN");
  expect(outlier_detect_quantize(A16, M, K, 6.f, WS, need - 1, nullptr), I8MM_EWORKSPACE, "x side ws");

  // GELU
  expect(i8mm_gelu_f16(A16, -1, A16, nullptr), I8MM_EINVAL, "gelu count");
  expect(i8mm_gelu_f16(M16, 4, A16, nullptr), I8MM_EALIGN, "gelu align");
  expect(i8mm_gelu_f16(A16, 0, A16, nullptr), I8MM_OK, "gelu empty");

  // messages
  for (int st = -7; st <= 0; ++st)
    if (!i8mm_status_string(st)) { std::printf("FAIL status string %d\n", st); ++failures; }
  if (!i8mm_last_error()) { std::printf("FAIL last error\n"); ++failures; }

  // a valid call with no GPU: no device, nothing launched (never made where a
  // GPU could take the fake addresses)
  if (argc > 1 && std::strcmp(argv[1], "--no-device") == 0)
    expect(int8_quantize_colwise_weight(A16, 4, 16, A8, F, nullptr), I8MM_ENODEVICE, "no device");

  if (failures) return 1;
  std::printf("ALL OK\n");
  return 0;
}
