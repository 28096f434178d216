// C-ABI of the i8mm library: argument validation, workspace layout and the
// launch sequence of each entry point. Declarations and the contract of each
// call are in include/i8mm.h.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime.h>

#include "i8mm.h"
#include "launchers.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return I8MM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(I8MM_ENODEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) {
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 1) return I8MM_OK;
    if (st == 2) return fail(I8MM_ENODEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess)
    return fail(I8MM_ENODEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < kMaxDevices) g_dev_state[dev].store(good ? 1 : 2, std::memory_order_release);
  if (!good) return fail(I8MM_ENODEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return I8MM_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(I8MM_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return I8MM_OK;
}

#define I8MM_TRY(expr)        \
  do {                        \
    int _st = (expr);         \
    if (_st != I8MM_OK) return _st; \
  } while (0)

// Common shape checks: sizes non-negative and within int32 row/column counts,
// K a multiple of 16 and within the int32 accumulation bound.
int check_dims(const char* fn, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(I8MM_EINVAL, "%s: negative size", fn);
  if (M > INT32_MAX || N > INT32_MAX) return fail(I8MM_EINVAL, "%s: size beyond int32", fn);
  if (K % 16 != 0) return fail(I8MM_EALIGN, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (K > I8MM_MAX_K) return fail(I8MM_ERANGE, "%s: K=%lld exceeds %d", fn, (long long)K, I8MM_MAX_K);
  return I8MM_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, bool required) {
  if (!p) return required ? fail(I8MM_EINVAL, "%s: %s is NULL", fn, name) : I8MM_OK;
  if (!aligned16(p)) return fail(I8MM_EALIGN, "%s: %s is not 16-byte aligned", fn, name);
  return I8MM_OK;
}

constexpr int64_t kAlign = 256;
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Workspace of linear_int8_mixed: bitmap | cols | n | sx | Xq | Xo |
// partial flag words (kMaxFlagBands x ceil(K/32), at *part when given) |
// the GEMM's k-block list (1 + ceil(K/64) ints, at *kbl when given).
bool layout(int64_t M, int64_t K, int64_t* off, int64_t* part = nullptr,
            int64_t* kbl = nullptr) {
  if (M < 0 || K < 0 || K % 16 != 0 || K > I8MM_MAX_K || M > INT32_MAX) return false;
  int64_t p = 0;
  off[0] = p; p = round_up(p + (K + 31) / 32 * 4, kAlign);
  off[1] = p; p = round_up(p + K * 4, kAlign);
  off[2] = p; p = round_up(p + 4, kAlign);
  off[3] = p; p = round_up(p + M * 4, kAlign);
  off[4] = p; p = round_up(p + M * K, kAlign);
  off[5] = p; p = round_up(p + M * I8MM_OUTLIER_LD(K) * 2, kAlign);
  if (part) *part = p;
  p = round_up(p + i8mm::kMaxFlagBands * ((K + 31) / 32) * 4, kAlign);
  if (kbl) *kbl = p;
  p = round_up(p + (1 + (K + 63) / 64) * 4, kAlign);
  off[6] = p;
  return true;
}

// Bytes of the region of linear_int8_mixed_workspace_bytes_many_outliers
// after the minimal workspace: the recovered fp16 outlier weight columns
// for up to I8MM_OUTLIER_REGION_COLS outlier columns.
int64_t wo_region_bytes(int64_t N, int64_t K) {
  return round_up(N * I8MM_OUTLIER_LD(std::min<int64_t>(K, I8MM_OUTLIER_REGION_COLS)) * 2, kAlign);
}

}  // namespace

extern "C" {

const char* i8mm_last_error(void) { return g_err; }

const char* i8mm_status_string(int status) {
  switch (status) {
    case I8MM_OK: return "I8MM_OK";
    case I8MM_EINVAL: return "I8MM_EINVAL";
    case I8MM_EALIGN: return "I8MM_EALIGN";
    case I8MM_EWORKSPACE: return "I8MM_EWORKSPACE";
    case I8MM_ENODEVICE: return "I8MM_ENODEVICE";
    case I8MM_ELAUNCH: return "I8MM_ELAUNCH";
    case I8MM_ERANGE: return "I8MM_ERANGE";
    default: return "I8MM_UNKNOWN";
  }
}

size_t linear_int8_mixed_workspace_bytes(int64_t M, int64_t K) {
  int64_t off[7];
  return layout(M, K, off) ? (size_t)off[6] : 0;
}

size_t linear_int8_mixed_workspace_bytes_many_outliers(int64_t M, int64_t K, int64_t N) {
  int64_t off[7];
  if (N < 0 || N > INT32_MAX || !layout(M, K, off)) return 0;
  return (size_t)(off[6] + wo_region_bytes(N, K));
}

int i8mm_workspace_layout(int64_t M, int64_t K, int64_t* offsets) {
  if (!offsets) return fail(I8MM_EINVAL, "i8mm_workspace_layout: offsets is NULL");
  if (!layout(M, K, offsets)) return fail(I8MM_EINVAL, "i8mm_workspace_layout: invalid sizes");
  return ok();
}

int int8_quantize_colwise_weight(const uint16_t* W, int64_t N, int64_t K, int8_t* Wq, float* sw,
                                 i8mm_stream_t stream) {
  const char* fn = "int8_quantize_colwise_weight";
  I8MM_TRY(check_dims(fn, N, 0, K));
  I8MM_TRY(check_ptr(fn, "W", W, N * K > 0));
  I8MM_TRY(check_ptr(fn, "Wq", Wq, N * K > 0));
  I8MM_TRY(check_ptr(fn, "sw", sw, N > 0));
  if (N == 0) return ok();
  I8MM_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  I8MM_TRY(launched(i8mm::launch_rows(W, N, K, nullptr, Wq, sw, nullptr, nullptr, nullptr, s), fn));
  return ok();
}

int int8_quantize_rowwise(const uint16_t* X, int64_t M, int64_t K, const uint32_t* outlier_bitmap,
                          int8_t* Xq, float* sx, i8mm_stream_t stream) {
  const char* fn = "int8_quantize_rowwise";
  I8MM_TRY(check_dims(fn, M, 0, K));
  I8MM_TRY(check_ptr(fn, "X", X, M * K > 0));
  I8MM_TRY(check_ptr(fn, "outlier_bitmap", outlier_bitmap, false));
  I8MM_TRY(check_ptr(fn, "Xq", Xq, M * K > 0));
  I8MM_TRY(check_ptr(fn, "sx", sx, M > 0));
  if (M == 0) return ok();
  I8MM_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  I8MM_TRY(launched(
      i8mm::launch_rows(X, M, K, outlier_bitmap, Xq, sx, nullptr, nullptr, nullptr, s), fn));
  return ok();
}

int outlier_detect_gather(const uint16_t* X, int64_t M, int64_t K, float threshold,
                          uint32_t* bitmap, int32_t* cols, int32_t* n_outliers, uint16_t* Xo,
                          i8mm_stream_t stream) {
  const char* fn = "outlier_detect_gather";
  I8MM_TRY(check_dims(fn, M, 0, K));
  if (std::isnan(threshold)) return fail(I8MM_EINVAL, "%s: threshold is NaN", fn);
  I8MM_TRY(check_ptr(fn, "X", X, M * K > 0));
  I8MM_TRY(check_ptr(fn, "bitmap", bitmap, K > 0));
  I8MM_TRY(check_ptr(fn, "cols", cols, K > 0));
  I8MM_TRY(check_ptr(fn, "n_outliers", n_outliers, true));
  I8MM_TRY(check_ptr(fn, "Xo", Xo, false));
  I8MM_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  const int64_t nwords = (K + 31) / 32;
  I8MM_TRY(launched(i8mm::launch_fill_u32(bitmap, nwords, 0u, s), fn));
  if (M > 0) I8MM_TRY(launched(i8mm::launch_outlier_flags(X, M, K, i8mm::fp16_threshold_pattern(threshold), bitmap, s), fn));
  I8MM_TRY(launched(i8mm::launch_cols_from_bitmap(bitmap, K, cols, n_outliers, s), fn));
  if (Xo && M > 0)
    I8MM_TRY(launched(
        i8mm::launch_rows(X, M, K, bitmap, nullptr, nullptr, Xo, nullptr, nullptr, s), fn));
  return ok();
}

int int8_mm_dequant(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                    int64_t M, int64_t N, int64_t K, const uint16_t* Xo, const int32_t* cols,
                    const int32_t* n_outliers, const uint16_t* bias, uint16_t* Y, int32_t* C,
                    i8mm_stream_t stream) {
  const char* fn = "int8_mm_dequant";
  I8MM_TRY(check_dims(fn, M, N, K));
  I8MM_TRY(check_ptr(fn, "Xq", Xq, M * K > 0));
  I8MM_TRY(check_ptr(fn, "Wq", Wq, N * K > 0));
  I8MM_TRY(check_ptr(fn, "sx", sx, M > 0));
  I8MM_TRY(check_ptr(fn, "sw", sw, N > 0));
  const bool any_o = Xo || cols || n_outliers;
  const bool all_o = Xo && cols && n_outliers;
  if (any_o && !all_o)
    return fail(I8MM_EINVAL, "%s: Xo, cols and n_outliers must be given together", fn);
  I8MM_TRY(check_ptr(fn, "Xo", Xo, false));
  I8MM_TRY(check_ptr(fn, "cols", cols, false));
  I8MM_TRY(check_ptr(fn, "n_outliers", n_outliers, false));
  I8MM_TRY(check_ptr(fn, "bias", bias, false));
  I8MM_TRY(check_ptr(fn, "Y", Y, false));
  I8MM_TRY(check_ptr(fn, "C", C, false));
  if (!Y && !C) return fail(I8MM_EINVAL, "%s: neither Y nor C given", fn);
  if (M == 0 || N == 0) return ok();
  I8MM_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  I8MM_TRY(launched(
      i8mm::launch_gemm(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_outliers, bias, Y, C, nullptr, 0,
                        nullptr, nullptr, nullptr, nullptr, s),
      fn));
  return ok();
}

}  // extern "C"

namespace {

// The activation side of the layer (steps a1-a3) into the workspace:
// detection as per-band partial flags (no clearing launch), then the row
// pass, which ORs them, writes the bitmap, cols, n and the GEMM's k-block
// list, gathers the outlier columns into Xo and quantizes the normal part
// into Xq, sx.
int x_side(const char* fn, const uint16_t* X, int64_t M, int64_t K, uint32_t tau16, char* ws,
           const int64_t* off, int64_t off_part, int64_t off_kbl, hipStream_t s) {
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws + off[0]);
  int32_t* cols = reinterpret_cast<int32_t*>(ws + off[1]);
  int32_t* n_o = reinterpret_cast<int32_t*>(ws + off[2]);
  float* sx = reinterpret_cast<float*>(ws + off[3]);
  int8_t* Xq = reinterpret_cast<int8_t*>(ws + off[4]);
  uint16_t* Xo = reinterpret_cast<uint16_t*>(ws + off[5]);
  uint32_t* part = reinterpret_cast<uint32_t*>(ws + off_part);
  int32_t* kbl = reinterpret_cast<int32_t*>(ws + off_kbl);
  const int bands = i8mm::flag_bands(M, K);
  I8MM_TRY(launched(i8mm::launch_outlier_flag_bands(X, M, K, tau16, bands, part, s), fn));
  I8MM_TRY(launched(
      i8mm::launch_rows_banded(X, M, K, part, bands, bitmap, Xq, sx, Xo, cols, n_o, kbl, s),
      fn));
  return I8MM_OK;
}

// Workspace pointer and size checks shared by the calls that take one.
int check_workspace(const char* fn, const void* workspace, size_t workspace_bytes,
                    const int64_t* off) {
  if (!workspace) return fail(I8MM_EWORKSPACE, "%s: workspace is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(I8MM_EALIGN, "%s: workspace is not 256-byte aligned", fn);
  if ((int64_t)workspace_bytes < off[6])
    return fail(I8MM_EWORKSPACE, "%s: workspace has %zu bytes, needs %lld", fn, workspace_bytes,
                (long long)off[6]);
  return I8MM_OK;
}

// Argument checks of the layer calls (all before any device work).
int check_layer_args(const char* fn, const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
                     const float* sw, int64_t N, const uint16_t* bias, float threshold,
                     const uint16_t* Y) {
  I8MM_TRY(check_dims(fn, M, N, K));
  if (std::isnan(threshold)) return fail(I8MM_EINVAL, "%s: threshold is NaN", fn);
  I8MM_TRY(check_ptr(fn, "X", X, M * K > 0));
  I8MM_TRY(check_ptr(fn, "Wq", Wq, N * K > 0));
  I8MM_TRY(check_ptr(fn, "sw", sw, N > 0));
  I8MM_TRY(check_ptr(fn, "bias", bias, false));
  I8MM_TRY(check_ptr(fn, "Y", Y, M * N > 0));
  return I8MM_OK;
}

// The whole layer after argument checks common to both weight modes. Wf: the
// fp16 weight when the layer keeps one (its outlier columns feed the outlier
// product), else nullptr (they are recovered from Wq, sw). quantize_w: write
// Wf's codes into Wq, sw first.
int run_layer(const char* fn, const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
              const float* sw, int64_t N, const uint16_t* bias, float threshold, uint16_t* Y,
              void* workspace, size_t workspace_bytes, hipStream_t s, const uint16_t* Wf,
              bool quantize_w) {
  I8MM_TRY(check_layer_args(fn, X, M, K, Wq, sw, N, bias, threshold, Y));
  int64_t off[7], off_part = 0, off_kbl = 0;
  layout(M, K, off, &off_part, &off_kbl);
  I8MM_TRY(check_workspace(fn, workspace, workspace_bytes, off));
  if (M == 0 || N == 0) return ok();
  I8MM_TRY(check_device());
  char* ws = static_cast<char*>(workspace);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws + off[0]);
  int32_t* cols = reinterpret_cast<int32_t*>(ws + off[1]);
  int32_t* n_o = reinterpret_cast<int32_t*>(ws + off[2]);
  float* sx = reinterpret_cast<float*>(ws + off[3]);
  int8_t* Xq = reinterpret_cast<int8_t*>(ws + off[4]);
  uint16_t* Xo = reinterpret_cast<uint16_t*>(ws + off[5]);
  const uint32_t tau16 = i8mm::fp16_threshold_pattern(threshold);
  if (quantize_w)
    I8MM_TRY(launched(i8mm::launch_rows(Wf, N, K, nullptr, const_cast<int8_t*>(Wq),
                                        const_cast<float*>(sw), nullptr, nullptr, nullptr, s),
                      fn));
  if (i8mm::decode_applies(M, K)) {
    // few tokens: the whole layer in one launch
    I8MM_TRY(launched(i8mm::launch_decode(X, Wq, sw, M, N, K, tau16, bias, Y, Wf, bitmap, cols,
                                          n_o, sx, Xq, Xo, s),
                      fn));
    return ok();
  }
  I8MM_TRY(x_side(fn, X, M, K, tau16, ws, off, off_part, off_kbl, s));
  // The workspace beyond the minimal layout holds the recovered fp16 outlier
  // weight columns for the tiled GEMM, N rows of LD(n) halfs, for n up to the
  // columns it has room for (the kernels do nothing for 16 or fewer columns,
  // or for more than that room; the GEMM's dense loop takes those).
  uint16_t* Wo = nullptr;
  int wo_cols = 0;
  if (!i8mm::gemv_applies(M)) {
    const int64_t room = ((int64_t)workspace_bytes - off[6]) / (2 * N) / 32 * 32;
    if (room >= 32) {
      wo_cols = (int)std::min<int64_t>(room, I8MM_OUTLIER_LD(K));
      Wo = reinterpret_cast<uint16_t*>(ws + off[6]);
      if (Wf)
        I8MM_TRY(launched(i8mm::launch_gather_w_cols(Wf, N, K, cols, n_o, wo_cols, Wo, s), fn));
      else
        I8MM_TRY(launched(
            i8mm::launch_recover_outlier_w(Wq, sw, N, K, cols, n_o, wo_cols, Wo, s), fn));
    }
  }
  I8MM_TRY(launched(i8mm::launch_gemm(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_o, bias, Y, nullptr,
                                      Wo, wo_cols, Wf, X, bitmap,
                                      reinterpret_cast<const int32_t*>(ws + off_kbl), s),
                    fn));
  return ok();
}

}  // namespace

extern "C" {

int linear_int8_mixed(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* sw,
                      int64_t N, const uint16_t* bias, float threshold, uint16_t* Y,
                      void* workspace, size_t workspace_bytes, i8mm_stream_t stream) {
  return run_layer("linear_int8_mixed", X, M, K, Wq, sw, N, bias, threshold, Y, workspace,
                   workspace_bytes, (hipStream_t)stream, nullptr, false);
}

int linear_int8_mixed_fp16_weights(const uint16_t* X, int64_t M, int64_t K, const uint16_t* W,
                                   int64_t N, int8_t* Wq, float* sw, int quantize_weight,
                                   const uint16_t* bias, float threshold, uint16_t* Y,
                                   void* workspace, size_t workspace_bytes,
                                   i8mm_stream_t stream) {
  const char* fn = "linear_int8_mixed_fp16_weights";
  I8MM_TRY(check_ptr(fn, "W", W, N * K > 0));
  return run_layer(fn, X, M, K, Wq, sw, N, bias, threshold, Y, workspace, workspace_bytes,
                   (hipStream_t)stream, W, quantize_weight != 0);
}

int outlier_detect_quantize(const uint16_t* X, int64_t M, int64_t K, float threshold,
                            void* workspace, size_t workspace_bytes, i8mm_stream_t stream) {
  const char* fn = "outlier_detect_quantize";
  I8MM_TRY(check_dims(fn, M, 0, K));
  if (std::isnan(threshold)) return fail(I8MM_EINVAL, "%s: threshold is NaN", fn);
  I8MM_TRY(check_ptr(fn, "X", X, M * K > 0));
  int64_t off[7], off_part = 0, off_kbl = 0;
  layout(M, K, off, &off_part, &off_kbl);
  I8MM_TRY(check_workspace(fn, workspace, workspace_bytes, off));
  if (M == 0) return ok();
  I8MM_TRY(check_device());
  I8MM_TRY(x_side(fn, X, M, K, i8mm::fp16_threshold_pattern(threshold),
                  static_cast<char*>(workspace), off, off_part, off_kbl, (hipStream_t)stream));
  return ok();
}

}  // extern "C"

namespace {

// Workspace of linear_int8_mixed_noalloc, for callers that cannot allocate:
// one copy per GPU the library runs on, held until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[I8MM_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call there (concurrent first calls look up the same address).
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(I8MM_ENODEVICE, "%s: no HIP device: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(I8MM_ENODEVICE, "%s: device %d beyond the %d the library tracks", fn, dev,
                kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(I8MM_ELAUNCH, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return I8MM_OK;
}

}  // namespace

extern "C" {

int linear_int8_mixed_noalloc(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
                              const float* sw, int64_t N, const uint16_t* bias, float threshold,
                              uint16_t* Y, i8mm_stream_t stream) {
  const char* fn = "linear_int8_mixed_noalloc";
  I8MM_TRY(check_layer_args(fn, X, M, K, Wq, sw, N, bias, threshold, Y));
  int64_t off[7];
  layout(M, K, off);
  if (off[6] > (int64_t)I8MM_NOALLOC_SCRATCH_BYTES)
    return fail(I8MM_EWORKSPACE,
                "%s: M=%lld, K=%lld need %lld bytes of workspace, more than the %lld of the "
                "library's scratch; use linear_int8_mixed with a workspace",
                fn, (long long)M, (long long)K, (long long)off[6],
                (long long)I8MM_NOALLOC_SCRATCH_BYTES);
  if (M == 0 || N == 0) return ok();
  I8MM_TRY(check_device());
  void* ws = nullptr;
  I8MM_TRY(scratch_address(fn, &ws));
  return run_layer(fn, X, M, K, Wq, sw, N, bias, threshold, Y, ws,
                   (size_t)I8MM_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream, nullptr, false);
}

int i8mm_gelu_f16(const uint16_t* X, int64_t count, uint16_t* Y, i8mm_stream_t stream) {
  const char* fn = "i8mm_gelu_f16";
  if (count < 0) return fail(I8MM_EINVAL, "%s: negative count", fn);
  I8MM_TRY(check_ptr(fn, "X", X, count > 0));
  I8MM_TRY(check_ptr(fn, "Y", Y, count > 0));
  if (count == 0) return ok();
  I8MM_TRY(check_device());
  I8MM_TRY(launched(i8mm::launch_gelu(X, count, Y, (hipStream_t)stream), fn));
  return ok();
}

}  // extern "C"
