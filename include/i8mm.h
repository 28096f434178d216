/*
 * i8mm: LLM.int8() mixed-precision int8 linear layer for AMD Instinct MI355X
 * (gfx950). C ABI.
 *
 * Pages cited (title and section):
 *   [HF-blog]  Hugging Face blog "A Gentle Introduction to 8-bit Matrix
 *              Multiplication for transformers at scale using Hugging Face
 *              Transformers, Accelerate and bitsandbytes".
 *   [Summary]  Paper summary page "LLM.int8(): 8-Bit Matrix Multiplication for
 *              Transformers at Scale".
 *
 * The layer computes Y = X . W^T for fp16 activations X [M, K] (M tokens,
 * K hidden features) and a weight W [N, K] (nn.Linear layout, N output
 * features) in three parts ([HF-blog] "A gentle summary of LLM.int8()";
 * [Summary] "The full picture"):
 *   - hidden columns of X holding any value with abs(x) >= threshold are the
 *     outlier columns; they are multiplied in fp16 against the matching
 *     weight columns;
 *   - the other columns are absmax-quantized to int8 with one scale per row
 *     of X and one per output row of W, multiplied in int8 with int32
 *     accumulation, and dequantized by the outer product of the two absmax
 *     vectors divided by 127^2;
 *   - the two results are added and returned in fp16.
 *
 * Conventions shared by every call:
 *   - Every pointer is a DEVICE pointer (memory on the GPU the call runs on)
 *     unless marked "host". Matrices are row-major with dense rows.
 *   - fp16 values are IEEE binary16 bit patterns passed as uint16_t.
 *   - The caller allocates and owns every buffer. The library allocates no
 *     device memory and keeps no state other than a per-device architecture
 *     check made on first use.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream). Nothing is synchronized with the host; device-side results
 *     (such as the outlier count) stay in device memory.
 *   - Calls return a status code and never throw. Invalid arguments are
 *     rejected on the host before anything is launched. A call that fails
 *     leaves its outputs unspecified.
 *   - K must be a multiple of 16 and every base pointer 16-byte aligned.
 *   - K <= I8MM_MAX_K, the largest K for which sum_k q_x q_w cannot overflow
 *     int32 (127 * 127 * K < 2^31).
 *   - M == 0 or N == 0 is valid and does nothing (except where stated).
 *   - K == 0 is valid: the products are empty sums (a layer returns Y = bias,
 *     or 0), every row's absmax is 0 and no column is an outlier column.
 *   - A pointer to an array with no elements (one of its sizes is 0) may be
 *     NULL.
 *   - Calls are thread-safe; calls on one stream are ordered; calls that write
 *     the same buffers from different streams race.
 */
#ifndef I8MM_H
#define I8MM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define I8MM_API __attribute__((visibility("default")))
#else
#define I8MM_API
#endif

/* hipStream_t, kept opaque so this header does not need the HIP headers. */
typedef void* i8mm_stream_t;

#define I8MM_OK          0
#define I8MM_EINVAL     -1  /* NULL pointer, negative size, NaN threshold     */
#define I8MM_EALIGN     -2  /* K % 16 != 0 or a pointer not 16-byte aligned   */
#define I8MM_EWORKSPACE -3  /* workspace missing or smaller than required     */
#define I8MM_ENODEVICE  -4  /* the current HIP device is not a gfx950 GPU     */
#define I8MM_ELAUNCH    -5  /* a kernel launch failed (HIP error)             */
#define I8MM_ERANGE     -6  /* K > I8MM_MAX_K (int32 accumulation could wrap) */

#define I8MM_MAX_K 133144

/* Outlier columns gathered from X are stored with a row stride of
 * I8MM_OUTLIER_LD(n) halfs: n rounded up to a multiple of 32; the pad
 * columns hold +0.0. */
#define I8MM_OUTLIER_LD(n) ((((int64_t)(n)) + 31) / 32 * 32)

/*
 * int8_quantize_colwise_weight  (step: weight quantization, once per weight)
 *
 * [HF-blog] "Introduction to model quantization": vector-wise quantization
 * takes the absmax of each column of B in A*B; for Y = X . W^T, B = W^T, so
 * each column of B is an output row of W ("Inside the MatMul": weights are
 * quantized column-wise). [HF-blog] "Usage": this runs once, when the weight
 * is placed on the device; the int8 weight and the per-row absmax are the
 * CB and SCB pair.
 *
 *   W   fp16 [N, K], read only.
 *   Wq  int8 [N, K], written: Wq[j,k] = rne(fl32(W[j,k] * fl32(127 / sw[j]))),
 *       in [-127, 127]; a row whose absmax is 0 gets all-zero codes.
 *   sw  fp32 [N], written: sw[j] = max_k abs(W[j,k]) (exact fp16 value).
 *
 * The input type is fp16, so an int8 weight cannot be quantized a second time
 * through this call. Errors: EINVAL, EALIGN, ERANGE, ENODEVICE, ELAUNCH.
 */
I8MM_API int int8_quantize_colwise_weight(const uint16_t* W, int64_t N, int64_t K,
                                 int8_t* Wq, float* sw, i8mm_stream_t stream);

/*
 * int8_quantize_rowwise  (step: row-wise absmax quantization of X)
 *
 * [HF-blog] "Inside the MatMul": hidden states are quantized row-wise;
 * [Summary] "Second innovation" / "The full picture" step 3: only the normal
 * (non-outlier) part is quantized to int8.
 *
 *   X               fp16 [M, K], read only.
 *   outlier_bitmap  uint32 [ceil(K/32)] or NULL; bit (k % 32) of word k / 32
 *                   set marks column k as an outlier column. NULL = none.
 *   Xq              int8 [M, K], written: codes of the non-outlier columns,
 *                   0 in outlier columns.
 *   sx              fp32 [M], written: absmax of row i over non-outlier
 *                   columns (0 for a row with no nonzero normal entry, whose
 *                   codes are then all 0).
 *
 * Codes: rne(fl32(x * fl32(127 / sx[i]))), in [-127, 127].
 * Errors: EINVAL, EALIGN, ERANGE, ENODEVICE, ELAUNCH.
 */
I8MM_API int int8_quantize_rowwise(const uint16_t* X, int64_t M, int64_t K,
                          const uint32_t* outlier_bitmap,
                          int8_t* Xq, float* sx, i8mm_stream_t stream);

/*
 * outlier_detect_gather  (steps: outlier-column detection; X-side split)
 *
 * [HF-blog] "A gentle summary of LLM.int8()" step 1 and "Inside the MatMul":
 * outliers are taken column-wise from the hidden states, magnitude 6 or more;
 * [Summary] "The full picture" steps 1-2: a feature dimension is an outlier
 * when at least one of its values reaches the threshold; X is split along
 * those dimensions. The set is the union over all M rows of this call.
 *
 *   X          fp16 [M, K], read only.
 *   threshold  host float; column k is an outlier iff some abs(X[i,k]) >=
 *              threshold (exact comparison of the fp16 value) or some X[i,k]
 *              is NaN; a threshold <= 0 flags every column; +inf flags the
 *              columns holding +-inf or NaN. NaN threshold -> EINVAL.
 *   bitmap     uint32 [ceil(K/32)], written (bit layout as above).
 *   cols       int32 [K] capacity, written: the outlier columns ascending in
 *              cols[0 .. n-1].
 *   n_outliers int32 [1] (device), written: n, the number of outlier columns.
 *   Xo         fp16 [M, I8MM_OUTLIER_LD(n)] capacity M * I8MM_OUTLIER_LD(K),
 *              or NULL; written: Xo[i, t] = X[i, cols[t]] for t < n, +0.0 in
 *              the pad columns.
 *
 * M == 0 writes an all-zero bitmap and n = 0.
 * Errors: EINVAL, EALIGN, ERANGE, ENODEVICE, ELAUNCH.
 */
I8MM_API int outlier_detect_gather(const uint16_t* X, int64_t M, int64_t K, float threshold,
                          uint32_t* bitmap, int32_t* cols, int32_t* n_outliers,
                          uint16_t* Xo, i8mm_stream_t stream);

/*
 * int8_mm_dequant  (steps: int8 matmul with int32 accumulation, fp16 outlier
 * product, dequantize and merge)
 *
 * [Summary] "The full picture" steps 3-4: Int8 matmul with an Int32 result,
 * dequantized by the outer product of the scale vectors, plus the 16-bit
 * outlier product. [HF-blog] "Introduction to model quantization": the outer
 * product of the absmax vectors denormalizes the result. [HF-blog] "Usage":
 * the fp16 weight columns of the outlier matmul are recovered from the int8
 * weight as CB * SCB / 127, per output row.
 *
 *   Xq, sx     int8 [M, K], fp32 [M]: quantized activations (outlier columns
 *              hold code 0).
 *   Wq, sw     int8 [N, K], fp32 [N]: quantized weight and its row absmax.
 *   Xo, cols, n_outliers
 *              the outputs of outlier_detect_gather (all three NULL = no
 *              outlier part). The outlier weight columns are
 *              Wo[j, t] = fp16(fl32(fl32(Wq[j, cols[t]] * sw[j]) / 127)).
 *   bias       fp16 [N] or NULL.
 *   Y          fp16 [M, N] or NULL, written:
 *              Y = fp16( C * sx[i] * sw[j] / 127^2 + sum_t Xo[i,t] Wo[j,t]
 *                        + bias[j] ), sums in fp32.
 *   C          int32 [M, N] or NULL, written: C[i,j] = sum_k Xq[i,k] Wq[j,k]
 *              (exact). At least one of Y and C must be given.
 *
 * Errors: EINVAL, EALIGN, ERANGE, ENODEVICE, ELAUNCH.
 */
I8MM_API int int8_mm_dequant(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                    int64_t M, int64_t N, int64_t K,
                    const uint16_t* Xo, const int32_t* cols, const int32_t* n_outliers,
                    const uint16_t* bias, uint16_t* Y, int32_t* C, i8mm_stream_t stream);

/*
 * outlier_detect_quantize  (steps: outlier-column detection, X-side split and
 * row-wise quantization of the normal part, fused as the layer runs them)
 *
 * [Summary] "The full picture" steps 1-3 on the activation side: find the
 * outlier feature dimensions, split X along them, quantize the normal part
 * row-wise ([HF-blog] "Inside the MatMul"). It performs exactly the
 * activation side of linear_int8_mixed (the same two kernel launches, one
 * read of X for detection and one for the row pass) and leaves its results
 * in the workspace, where int8_mm_dequant can take them: a caller that runs
 * the matmul itself, or times the two sides apart.
 *
 *   X          fp16 [M, K], read only.
 *   threshold  host float, as in outlier_detect_gather.
 *   workspace  as in linear_int8_mixed (at least
 *              linear_int8_mixed_workspace_bytes(M, K) bytes, 256-byte
 *              aligned). Written, at the offsets i8mm_workspace_layout
 *              reports: the bitmap, cols and n as outlier_detect_gather
 *              writes them; sx and Xq as int8_quantize_rowwise writes them
 *              given that bitmap; Xo [M, I8MM_OUTLIER_LD(n)] with zero pads.
 *
 * M == 0 does nothing. Errors: EINVAL, EALIGN, EWORKSPACE, ERANGE,
 * ENODEVICE, ELAUNCH.
 */
I8MM_API int outlier_detect_quantize(const uint16_t* X, int64_t M, int64_t K, float threshold,
                                     void* workspace, size_t workspace_bytes,
                                     i8mm_stream_t stream);

/*
 * linear_int8_mixed  (the whole layer for an already-quantized weight)
 *
 * [HF-blog] "A gentle summary of LLM.int8()" steps 1-3 and "Inside the
 * MatMul"; [Summary] "The full picture" steps 1-4: detect outlier columns,
 * split, fp16 outlier matmul and int8 matmul of the row-quantized normal
 * part, dequantize, add. The weight comes from int8_quantize_colwise_weight.
 *
 *   X          fp16 [M, K], read only.
 *   Wq, sw     int8 [N, K], fp32 [N].
 *   bias       fp16 [N] or NULL.
 *   threshold  host float (6.0 in the pages), as in outlier_detect_gather.
 *   Y          fp16 [M, N], written.
 *   workspace  device buffer of at least linear_int8_mixed_workspace_bytes(M,K)
 *              bytes, 256-byte aligned; it receives the intermediates (outlier
 *              bitmap, cols, n, sx, Xq, Xo) at the offsets that
 *              i8mm_workspace_layout reports. Bytes beyond
 *              linear_int8_mixed_workspace_bytes(M, K) are a region for the
 *              recovered outlier weight columns, with room for
 *              floor(extra / (2 N) / 32) * 32 columns (see
 *              linear_int8_mixed_workspace_bytes_many_outliers).
 *
 * All kernels run in order on `stream` with no host synchronization; the
 * outlier count stays on the device. Errors: EINVAL, EALIGN, EWORKSPACE,
 * ERANGE, ENODEVICE, ELAUNCH.
 */
I8MM_API int linear_int8_mixed(const uint16_t* X, int64_t M, int64_t K,
                      const int8_t* Wq, const float* sw, int64_t N,
                      const uint16_t* bias, float threshold, uint16_t* Y,
                      void* workspace, size_t workspace_bytes, i8mm_stream_t stream);

/*
 * linear_int8_mixed_noalloc  (linear_int8_mixed without a workspace argument)
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The same
 * layer as linear_int8_mixed, with the same kernels and results; its
 * workspace is the library's own scratch, a static device array of
 * I8MM_NOALLOC_SCRATCH_BYTES bytes per GPU, held until the process ends. The
 * call allocates nothing (no hipMalloc, no hipFree); on its first call on a
 * device it looks up that device's scratch address.
 *
 *   X, Wq, sw, N, bias, threshold, Y  as in linear_int8_mixed.
 *
 * The sizes must satisfy linear_int8_mixed_workspace_bytes(M, K) <=
 * I8MM_NOALLOC_SCRATCH_BYTES (for example M * K <= about 11 million:
 * 2048 x 4096 fits), else EWORKSPACE and nothing is launched. Every call on
 * one GPU shares that GPU's scratch: calls that overlap on one GPU (other
 * streams, other host threads) race; calls ordered on one stream do not. The
 * scratch keeps the last call's intermediates; no part of it needs to be
 * zero on entry. Errors: EINVAL, EALIGN, EWORKSPACE, ERANGE, ENODEVICE,
 * ELAUNCH.
 */
#define I8MM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
I8MM_API int linear_int8_mixed_noalloc(const uint16_t* X, int64_t M, int64_t K,
                                       const int8_t* Wq, const float* sw, int64_t N,
                                       const uint16_t* bias, float threshold, uint16_t* Y,
                                       i8mm_stream_t stream);

/*
 * linear_int8_mixed_fp16_weights  (the whole layer for a weight kept in fp16)
 *
 * [HF-blog] "Usage": with has_fp16_weights=True (the module's default, meant
 * for mixed Int8/FP16 training) the layer keeps W in fp16. The steps are
 * those of linear_int8_mixed, with two differences: the int8 codes of W are
 * those of this call's W, and the outlier matmul takes the weight columns
 * from W itself ([HF-blog] "Inside the MatMul": an fp16 matmul of the outlier
 * columns of X and the matching weight columns), not from CB * SCB / 127.
 *
 *   X          fp16 [M, K], read only.
 *   W          fp16 [N, K] (nn.Linear layout), read only.
 *   Wq, sw     int8 [N, K], fp32 [N], caller-owned. With quantize_weight != 0
 *              this call first writes W's per-output-row absmax codes and
 *              absmaxes into them (as int8_quantize_colwise_weight does);
 *              with quantize_weight == 0 they must already hold exactly those
 *              of this W (a caller whose W has not changed since it last
 *              quantized it skips that pass).
 *   bias, threshold, Y, workspace
 *              as in linear_int8_mixed. Given the larger workspace of
 *              linear_int8_mixed_workspace_bytes_many_outliers(M, K, N), the
 *              region after the minimal workspace receives the fp16 weight
 *              columns of the outlier columns, Wo[j, t] = W[j, cols[t]].
 *
 *   Y = fp16( C * sx[i] * sw[j] / 127^2 + sum_t X[i, cols[t]] W[j, cols[t]]
 *             + bias[j] ), sums in fp32.
 *
 * M == 0 or N == 0: no work (Wq, sw untouched). All kernels run in order on
 * `stream` with no host synchronization. Errors: EINVAL, EALIGN, EWORKSPACE,
 * ERANGE, ENODEVICE, ELAUNCH.
 */
I8MM_API int linear_int8_mixed_fp16_weights(const uint16_t* X, int64_t M, int64_t K,
                      const uint16_t* W, int64_t N, int8_t* Wq, float* sw,
                      int quantize_weight, const uint16_t* bias, float threshold,
                      uint16_t* Y, void* workspace, size_t workspace_bytes,
                      i8mm_stream_t stream);

/* Bytes of workspace linear_int8_mixed needs for M tokens and K features
 * (0 if the sizes are invalid). Host-only, pure. */
I8MM_API size_t linear_int8_mixed_workspace_bytes(int64_t M, int64_t K);

/* Outlier columns the region of
 * linear_int8_mixed_workspace_bytes_many_outliers has room for. */
#define I8MM_OUTLIER_REGION_COLS 512

/* Bytes of workspace with a region for the recovered fp16 weight columns of
 * up to I8MM_OUTLIER_REGION_COLS outlier columns (0 if the sizes are
 * invalid). Host-only, pure. It is linear_int8_mixed_workspace_bytes(M, K)
 * plus N rows of I8MM_OUTLIER_LD(min(K, I8MM_OUTLIER_REGION_COLS)) halfs.
 *
 * The region starts at linear_int8_mixed_workspace_bytes(M, K) and holds the
 * recovered weights ([HF-blog] "Usage": CB * SCB / 127 per output row),
 * Wo[j, t] = fp16(fl32(fl32(Wq[j, cols[t]] * sw[j]) / 127)), N rows of
 * I8MM_OUTLIER_LD(n) halfs. Any workspace larger than the minimal one has
 * such a region: its room is floor(extra bytes / (2 N) / 32) * 32 columns
 * (at most I8MM_OUTLIER_LD(K)), so a caller with memory to spare may pass
 * more than this size (N * I8MM_OUTLIER_LD(K) * 2 extra bytes give room for
 * every count). With more than 16 outlier columns, room for them and more
 * than 64 tokens, the layer fills the region and runs the outlier product
 * as a second main loop of its GEMM over those columns. Otherwise (more than
 * 16 columns) the GEMM runs the outlier product as a second loop over all K
 * columns, converting the int8 weight tile to fp16 itself (the recovered
 * weights' factor sw[j] / 127 applied to the sum): every outlier count runs
 * without a region, and the region speeds up the counts it has room for.
 * The two loops sum in different orders, so Y may differ in the last bits
 * between them (both within the tolerance of the method). */
I8MM_API size_t linear_int8_mixed_workspace_bytes_many_outliers(int64_t M, int64_t K, int64_t N);

/* Byte offsets inside the workspace, host-only and pure. Writes, in order:
 * offsets[0] bitmap (uint32 [ceil(K/32)]), [1] cols (int32 [K]),
 * [2] n (int32 [1]), [3] sx (fp32 [M]), [4] Xq (int8 [M, K]),
 * [5] Xo (fp16 [M, I8MM_OUTLIER_LD(K)] capacity), [6] total bytes. Between
 * the end of Xo and the total lies scratch of the layer (per-row-band
 * partial flag words of the detection, 16 x ceil(K/32) uint32 at most, and
 * the GEMM's list of the 64-column k-blocks that hold a normal column,
 * 1 + ceil(K/64) int32), whose contents on entry do not matter.
 * `offsets` is a host array of 7 int64. Errors: EINVAL. */
I8MM_API int i8mm_workspace_layout(int64_t M, int64_t K, int64_t* offsets);

/*
 * i8mm_gelu_f16: exact-erf GELU, y = fp16(x * erfc(-x / sqrt 2) / 2) (equal to
 * x * (1 + erf(x / sqrt 2)) / 2) computed in fp32. Not a step of the method: the activation between the two
 * linear layers of an MLP block built from linear_int8_mixed.
 *   X, Y  fp16 [count] (Y may equal X).  Errors: EINVAL, EALIGN, ENODEVICE,
 *   ELAUNCH.
 */
I8MM_API int i8mm_gelu_f16(const uint16_t* X, int64_t count, uint16_t* Y, i8mm_stream_t stream);

/* Text of the last error raised on the calling host thread ("" if none). */
I8MM_API const char* i8mm_last_error(void);

/* Static name of a status code. */
I8MM_API const char* i8mm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* I8MM_H */
