// Internal launch wrappers of the i8mm kernels. Arguments are validated by
// the C-ABI layer before these are called; each returns the hipError_t of its
// launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i8mm.h"

namespace i8mm {

hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, hipStream_t s);

// tau16: smallest fp16 magnitude bit pattern (sign cleared) whose value is
// >= the threshold (0 for a threshold <= 0, 0x7c00 above the largest finite
// fp16); see fp16_threshold_pattern.
hipError_t launch_outlier_flags(const uint16_t* X, int64_t M, int64_t K, uint32_t tau16,
                                uint32_t* bitmap, hipStream_t s);

uint32_t fp16_threshold_pattern(float threshold);

hipError_t launch_cols_from_bitmap(const uint32_t* bitmap, int64_t K, int32_t* cols,
                                   int32_t* n_out, hipStream_t s);

// The layer's detection without a cleared bitmap: part[b][w] (bands x
// ceil(K/32) words, every word written) holds the flags of row band b, rows
// [b * ceil(M/bands), ...); the bitmap is their OR. flag_bands(M, K) is the
// band count the layer uses (1 .. kMaxFlagBands, no band empty).
constexpr int kMaxFlagBands = 16;
int flag_bands(int64_t M, int64_t K);
hipError_t launch_outlier_flag_bands(const uint16_t* X, int64_t M, int64_t K, uint32_t tau16,
                                     int bands, uint32_t* part, hipStream_t s);

// Row pass over X (or W): optional absmax quantization (Xq, sx), optional
// gather of outlier columns (Xo), optional cols/n output from the first row's
// block. bitmap == nullptr means no outlier columns.
hipError_t launch_rows(const uint16_t* X, int64_t M, int64_t K, const uint32_t* bitmap,
                       int8_t* Xq, float* sx, uint16_t* Xo, int32_t* cols, int32_t* n_out,
                       hipStream_t s);
// The same with the flags given as `bands` partial bitmaps (bands x
// ceil(K/32) words, see launch_outlier_flag_bands); the first block also
// writes their OR to bitmap_out when it is given, and, when kbl is given,
// the list of 64-column k-blocks that hold a normal column (kbl[0] = count,
// then the blocks ascending; 1 + ceil(K/64) ints).
hipError_t launch_rows_banded(const uint16_t* X, int64_t M, int64_t K, const uint32_t* flags,
                              int bands, uint32_t* bitmap_out, int8_t* Xq, float* sx,
                              uint16_t* Xo, int32_t* cols, int32_t* n_out, int32_t* kbl,
                              hipStream_t s);

// Wo: the fp16 outlier weight columns [N, LD(n)] written by
// launch_recover_outlier_w (or launch_gather_w_cols) with room for wo_cols
// columns, or nullptr; with 16 < n <= wo_cols and Wo given, the outlier
// product runs as a second main-loop segment over them. Xd, bmp: the
// layer's X [M, K] and its outlier bitmap, or nullptr; given, more than 16
// outlier columns that Wo does not take run as the dense second segment over
// all K columns. Otherwise the outlier product runs in the epilogue. Wf: the
// fp16 weight [N, K] when the layer keeps one (its columns are the outlier
// weights), or nullptr (they are recovered from Wq and sw).
// kbl: the k-block list of launch_rows_banded, or nullptr; given, the
// int8 loop of the segment modes visits only those k-blocks.
hipError_t launch_gemm(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                       int64_t M, int64_t N, int64_t K, const uint16_t* Xo,
                       const int32_t* cols, const int32_t* n_out, const uint16_t* bias,
                       uint16_t* Y, int32_t* C, const uint16_t* Wo, int wo_cols,
                       const uint16_t* Wf, const uint16_t* Xd, const uint32_t* bmp,
                       const int32_t* kbl, hipStream_t s);

// Wo[j, t] = fp16(fl32(fl32(Wq[j, cols[t]] * sw[j]) / 127)) for t < n, +0.0 up
// to LD(n); nothing when n <= 16 or n > wo_cols (n read on the device).
hipError_t launch_recover_outlier_w(const int8_t* Wq, const float* sw, int64_t N, int64_t K,
                                    const int32_t* cols, const int32_t* n_out, int wo_cols,
                                    uint16_t* Wo, hipStream_t s);

// Wo[j, t] = Wf[j, cols[t]] (the fp16 weight's own columns) for t < n, +0.0
// up to LD(n); nothing when n <= 16 or n > wo_cols (n read on the device).
hipError_t launch_gather_w_cols(const uint16_t* Wf, int64_t N, int64_t K, const int32_t* cols,
                                const int32_t* n_out, int wo_cols, uint16_t* Wo, hipStream_t s);

// The whole layer in one launch for 1 <= M <= 16 tokens whose codes fit in
// LDS (decode_applies): detection, row quantization and the few-token
// matmul with its epilogue. Writes the same intermediates as the separate
// kernels (bitmap, cols, n, sx, Xq, Xo with leading dimension LD(n)) and Y.
// Wf: the fp16 weight when the layer keeps one, else nullptr.
bool decode_applies(int64_t M, int64_t K);
hipError_t launch_decode(const uint16_t* X, const int8_t* Wq, const float* sw, int64_t M,
                         int64_t N, int64_t K, uint32_t tau16, const uint16_t* bias, uint16_t* Y,
                         const uint16_t* Wf, uint32_t* bitmap, int32_t* cols, int32_t* n_out,
                         float* sx, int8_t* Xq, uint16_t* Xo, hipStream_t s);

// Few-token form of launch_gemm (same arguments and results), used for
// 1 <= M <= 64.
bool gemv_applies(int64_t M);
hipError_t launch_gemv(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                       int64_t M, int64_t N, int64_t K, const uint16_t* Xo,
                       const int32_t* cols, const int32_t* n_out, const uint16_t* bias,
                       uint16_t* Y, int32_t* C, const uint16_t* Wf, hipStream_t s);

hipError_t launch_gelu(const uint16_t* X, int64_t count, uint16_t* Y, hipStream_t s);

}  // namespace i8mm
