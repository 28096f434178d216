// Bandwidth-bound kernels of the LLM.int8() layer on gfx950:
//   - outlier-column detection (column OR-reduce of abs(x) >= threshold):
//     atomically into a cleared bitmap for the step call, or as per-row-band
//     partial words with plain stores for the layer,
//   - bitmap -> ascending outlier-column list,
//   - per-row absmax int8 quantization (of X rows over the non-outlier
//     columns, or of W rows over the full row) fused with the gather of the
//     outlier columns of X,
//   - the fp16 outlier weight columns Wo for the GEMM's second segment
//     (recovered from the int8 weight, or the fp16 weight's own columns),
//   - exact-erf GELU for MLP blocks built from the layer.
//
// Pages cited: [HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit
// Matrix Multiplication for transformers at scale using Hugging Face
// Transformers, Accelerate and bitsandbytes"; [Summary] paper summary page
// "LLM.int8(): 8-Bit Matrix Multiplication for Transformers at Scale".
//
// Every kernel reads its rows as 16-byte chunks (8 fp16), one chunk per lane,
// so a wavefront touches 1 KiB of contiguous memory per load.

#include <cmath>

#include <algorithm>

#include <atomic>

#include "device_common.h"
#include "i8mm.h"
#include "launchers.h"

namespace i8mm {

namespace {

constexpr int kRowThreads = 256;

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t count, uint32_t value) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = value;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));

// Per-column maximum of the fp16 magnitude patterns of a 16-byte chunk (8
// columns), folded into mx[4] (element 2i in the low half of mx[i], 2i+1 in
// the high half).
__device__ __forceinline__ void fold_abs8(u16x2 mx[4], const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    mx[i] = __builtin_elementwise_max(mx[i], __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
}

// Bit e set when column e of the chunk has a maximum pattern >= tau16.
__device__ __forceinline__ uint32_t flag_mask8(const u16x2 mx[4], uint32_t tau16) {
  uint32_t mask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mask |= ((uint32_t)mx[i][0] >= tau16 ? 1u : 0u) << (2 * i);
    mask |= ((uint32_t)mx[i][1] >= tau16 ? 1u : 0u) << (2 * i + 1);
  }
  return mask;
}

// Column OR-reduce. Block = 4 waves over one 512-column group; lane owns an
// 8-column chunk; wave w scans rows r0+w, r0+w+4, ... of the block's row
// range, keeping the per-column maximum of the fp16 magnitude bit patterns
// (sign cleared) with packed 16-bit max. For non-NaN values that order is
// the order of magnitudes, so column k holds some abs(x) >= tau exactly when
// its maximum pattern is >= tau16, the smallest fp16 pattern whose value is
// >= tau ([HF-blog] "Inside the MatMul": magnitude 6 or greater; [Summary]
// "The full picture" step 1). NaN patterns exceed every threshold pattern, so
// a column holding NaN is flagged too and NaN never enters the int8 path.
// Flag bits are merged into the (pre-zeroed) bitmap with atomicOr: the four
// lanes of a 32-column word and the four waves of the block are OR-ed first,
// and the atomic is issued only when it sets a bit the word does not have yet
// (with many outlier columns most words fill early, and every block would
// otherwise hit the same few words). OR is order-free.
__global__ __launch_bounds__(256) void k_outlier_flags(const uint16_t* __restrict__ X, int64_t M,
                                                       int64_t K, uint32_t tau16, int rows_per_block,
                                                       uint32_t* __restrict__ bitmap) {
  __shared__ uint32_t s_word[4][16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = ((int64_t)blockIdx.x * 64 + lane) * 8;
  const bool col_ok = col0 < K;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = col_ok ? min(M, r0 + (int64_t)rows_per_block) : r0;
  const uint16_t* base = X + (col_ok ? col0 : 0);
  u16x2 mx[4] = {u16x2{0, 0}, u16x2{0, 0}, u16x2{0, 0}, u16x2{0, 0}};
  int64_t r = r0 + wave;
  for (; r + 12 < r1; r += 16) {
    const uint4 v0 = ld16(base + r * K);
    const uint4 v1 = ld16(base + (r + 4) * K);
    const uint4 v2 = ld16(base + (r + 8) * K);
    const uint4 v3 = ld16(base + (r + 12) * K);
    fold_abs8(mx, v0); fold_abs8(mx, v1); fold_abs8(mx, v2); fold_abs8(mx, v3);
  }
  if (r < r1) {
    // the last rows in one round trip: slots past the end read the block's
    // last row again (a duplicate leaves the maximum as it is)
    uint4 v[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] = ld16(base + min(r + 4 * i, r1 - 1) * K);
#pragma unroll
    for (int i = 0; i < 3; ++i) fold_abs8(mx, v[i]);
  }
  uint32_t mask = flag_mask8(mx, tau16);
  if (!col_ok) mask = 0;   // (with threshold 0 an empty max would pass)
  uint32_t word = mask << (col0 & 31);
  word |= (uint32_t)__shfl_xor((int)word, 1, kWave);
  word |= (uint32_t)__shfl_xor((int)word, 2, kWave);
  if ((lane & 3) == 0) s_word[wave][lane >> 2] = word;
  __syncthreads();
  if (threadIdx.x < 16) {
    const uint32_t w = s_word[0][threadIdx.x] | s_word[1][threadIdx.x] | s_word[2][threadIdx.x] |
                       s_word[3][threadIdx.x];
    const int64_t widx = (int64_t)blockIdx.x * 16 + threadIdx.x;
    if (w && widx * 32 < K) {
      const uint32_t cur = __atomic_load_n(&bitmap[widx], __ATOMIC_RELAXED);
      if ((cur & w) != w) atomicOr(&bitmap[widx], w);
    }
  }
}

// The layer's detection, without atomics: the rows are split into `bands`
// row bands, and block (g, b) writes the 4 flag words of 128-column group g
// over band b's rows to part[b][4g .. 4g+3] with plain stores, zero words
// included, so the partial words need no clearing beforehand; the row pass
// ORs the bands of each word. Lane (row slot, 16-lane column slot): 16 lanes
// cover a group's 256 bytes of one row, a wavefront 4 rows and the block 16
// rows per pass, 8 passes in flight per lane. The flag test is the one above.
constexpr int kFlagGroupCols = 128;
__global__ __launch_bounds__(256) void k_outlier_flag_bands(const uint16_t* __restrict__ X,
                                                            int64_t M, int64_t K, uint32_t tau16,
                                                            int64_t rows_per_band, int64_t nwords,
                                                            uint32_t* __restrict__ part) {
  __shared__ uint32_t s_word[4][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15;
  const int64_t col0 = (int64_t)blockIdx.x * kFlagGroupCols + sub * 8;
  const bool col_ok = col0 < K;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_band;
  const int64_t r1 = col_ok ? min(M, r0 + rows_per_band) : r0;
  const uint16_t* base = X + (col_ok ? col0 : 0);
  u16x2 mx[4] = {u16x2{0, 0}, u16x2{0, 0}, u16x2{0, 0}, u16x2{0, 0}};
  int64_t r = r0 + wave * 4 + (lane >> 4);
  for (; r + 112 < r1; r += 128) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ld16(base + (r + 16 * i) * K);
#pragma unroll
    for (int i = 0; i < 8; ++i) fold_abs8(mx, v[i]);
  }
  if (r < r1) {
    // the band's last partial batch, in one round trip as well: its rows past
    // the band's end read the band's last row again (a row of the band read
    // twice leaves the maximum as it is). One load at a time, these took a
    // memory round trip each.
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ld16(base + min(r + 16 * i, r1 - 1) * K);
#pragma unroll
    for (int i = 0; i < 8; ++i) fold_abs8(mx, v[i]);
  }
  uint32_t mask = flag_mask8(mx, tau16);
  if (!col_ok || r0 >= M) mask = 0;   // (with threshold 0 an empty max would pass)
  // the four rows of a wavefront at one column slot, then the 4 slots of a word
  mask |= (uint32_t)__shfl_xor((int)mask, 16, kWave);
  mask |= (uint32_t)__shfl_xor((int)mask, 32, kWave);
  uint32_t word = mask << ((sub & 3) * 8);
  word |= (uint32_t)__shfl_xor((int)word, 1, kWave);
  word |= (uint32_t)__shfl_xor((int)word, 2, kWave);
  if (lane < 16 && (lane & 3) == 0) s_word[wave][lane >> 2] = word;
  __syncthreads();
  if (tid < 4) {
    const int64_t widx = (int64_t)blockIdx.x * 4 + tid;
    if (widx < nwords)
      part[(int64_t)blockIdx.y * nwords + widx] =
          s_word[0][tid] | s_word[1][tid] | s_word[2][tid] | s_word[3][tid];
  }
}

__global__ __launch_bounds__(256) void k_cols_from_bitmap(const uint32_t* __restrict__ bitmap,
                                                          int64_t K, int32_t* __restrict__ cols,
                                                          int32_t* __restrict__ n_out) {
  extern __shared__ uint32_t smem[];
  __shared__ int sred[kRowThreads / kWave];
  const int nwords = (int)((K + 31) / 32);
  uint32_t* sbm = smem;
  uint32_t* spre = smem + nwords;
  for (int w = threadIdx.x; w < nwords; w += kRowThreads) sbm[w] = bitmap[w];
  __syncthreads();
  int n = bitmap_prefix(sbm, spre, nwords, sred);
  write_cols(sbm, spre, nwords, n, cols, n_out);
}

// Row pass. Block = 4 wavefronts; each wavefront owns whole rows (rows
// row0 + wave, row0 + wave + 4, ... of the block's range), so the per-row
// absmax is a wavefront reduction and the row loop has no block barrier. The
// outlier bitmap and its popcount prefix are built once per block in LDS.
// CPT = 16-byte chunks per lane kept in registers (K <= CPT * 8 * 64); CPT ==
// 0 streams the row twice (any K).
//
// Quantization ([HF-blog] "Introduction to model quantization", worked
// absmax example; "Inside the MatMul": rows of the hidden states, columns of
// B = output rows of W): a = absmax over the row's non-outlier entries,
// s = fl32(127 / a) (correctly rounded divide), code = rne(fl32(x * s))
// clamped to [-127, 127]; a == 0 gives s = 0 and all-zero codes. Outlier
// columns get code 0 ([Summary] "The full picture" step 2: they leave the
// int8 part). Their fp16 values are gathered into Xo [M, ld], ld = n rounded
// up to 32, in ascending column order.
//
// The absmax is taken on the fp16 bit patterns with the sign cleared: for
// non-NaN values the unsigned order of those patterns is the order of the
// magnitudes, and the maximum is exact.
// Flag source of the row pass: none (weight rows), one bitmap, or the
// layer's per-band partial words.
enum RowFlags { kNoFlags = 0, kBitmap = 1, kBands = 2 };
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int CPT, int FMODE>
__global__ __launch_bounds__(256) void k_rows(const uint16_t* __restrict__ X, int64_t M,
                                              int64_t K, int rows_per_block,
                                              const uint32_t* __restrict__ flags, int bands,
                                              uint32_t* __restrict__ bitmap_out,
                                              int8_t* __restrict__ Xq, float* __restrict__ sx,
                                              uint16_t* __restrict__ Xo, int32_t* __restrict__ cols,
                                              int32_t* __restrict__ n_out,
                                              int32_t* __restrict__ kbl) {
  constexpr bool kFlags = FMODE != kNoFlags;
  extern __shared__ uint32_t smem[];
  __shared__ int sred[kRowThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwords = (int)((K + 31) / 32);
  const int64_t nchunks = K / 8;
  uint32_t* sbm = smem;
  uint32_t* spre = smem + nwords;
  const int64_t row_lo = (int64_t)blockIdx.x * rows_per_block;
  const int64_t row_hi = min(M, row_lo + rows_per_block);
  const int64_t row0 = row_lo + wave;

  if (nchunks == 0) {   // K == 0: empty rows (absmax 0), no outlier columns
    if (sx && lane == 0)
      for (int64_t row = row0; row < row_hi; row += kRowThreads / kWave) sx[row] = 0.0f;
    if (blockIdx.x == 0 && tid == 0 && n_out) *n_out = 0;
    return;
  }

  // The flag words are loaded first, then the first row, and the flags are
  // only combined after that, so waiting for them leaves the row's loads in
  // flight. Every load is unconditional, indices clamped into range (a
  // clamped chunk is masked out below; a wave without a row in the last block
  // reads that block's last row again): loads under a branch would leave the
  // compiler unsure how many are outstanding, and it would wait for all.
  constexpr int NFL = FMODE == kBands ? kMaxFlagBands : 1;
  const int wi = tid < nwords ? tid : nwords - 1;
  uint32_t fl[NFL];
  if constexpr (kFlags) {
#pragma unroll
    for (int b = 0; b < NFL; ++b) fl[b] = flags[(int64_t)(b < bands ? b : 0) * nwords + wi];
  }
  asm volatile("" ::: "memory");   // the flag loads go out before the row's
  uint4 v[CPT > 0 ? CPT : 1];
  auto load_row = [&](int64_t row) {
    if constexpr (CPT > 0) {
      const uint16_t* xr = X + row * K;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int64_t c = min(lane + (int64_t)j * kWave, nchunks - 1);
        if constexpr (!kFlags) {
          // the weight is read once: a streaming (nontemporal) load
          const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + c * 8));
          v[j] = make_uint4(t[0], t[1], t[2], t[3]);
        } else {
          v[j] = ld16(xr + c * 8);
        }
      }
    }
  };
  load_row(row0 < row_hi ? row0 : row_hi - 1);

  int n = 0;
  if constexpr (kFlags) {
    uint32_t fw = 0;
#pragma unroll
    for (int b = 0; b < NFL; ++b) fw |= fl[b];
    // unconditional (threads past the last word store that word's own value
    // again), so the loads above cannot be moved into a branch
    sbm[wi] = fw;
    for (int w = tid + kRowThreads; w < nwords; w += kRowThreads) {
      uint32_t o = 0;
      for (int b = 0; b < bands; ++b) o |= flags[(int64_t)b * nwords + w];
      sbm[w] = o;
    }
    // LDS-only barriers: the first row's loads stay in flight meanwhile
    lds_only_barrier();
    if (Xo || cols || n_out) n = bitmap_prefix<true>(sbm, spre, nwords, sred);
  }
  if (blockIdx.x == 0) {
    if constexpr (kFlags) {
      write_cols(sbm, spre, nwords, n, cols, n_out);
      write_kblocks(sbm, K, kbl);
      if (bitmap_out)
        for (int w = tid; w < nwords; w += kRowThreads) bitmap_out[w] = sbm[w];
    } else {
      if (n_out && tid == 0) *n_out = 0;
    }
  }
  auto outl8 = [&](int64_t c) -> uint32_t {
    if constexpr (!kFlags) return 0u;
    const int64_t k = c * 8;
    return (sbm[k >> 5] >> (k & 31)) & 0xffu;
  };
  const int64_t ld = ((int64_t)n + 31) / 32 * 32;

  // Position in Xo of chunk c's first outlier column (its rank among them).
  auto rank8 = [&](int64_t c) -> int {
    const int64_t k0 = c * 8;
    return (int)spre[k0 >> 5] + __popc(sbm[k0 >> 5] & ((1u << (k0 & 31)) - 1u));
  };
  // With the row in registers (CPT > 0) the chunks a lane holds are the same
  // for every row, so their outlier masks and Xo positions are taken from
  // LDS once, while the first row is still in flight: meta[j] = rank << 8 |
  // mask (0 for a clamped chunk).
  uint32_t meta[CPT > 0 ? CPT : 1];
  if constexpr (CPT > 0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = lane + (int64_t)j * kWave;
      const uint32_t om = c < nchunks ? outl8(c) : 0u;
      meta[j] = om ? ((Xo ? (uint32_t)rank8(c) << 8 : 0u) | om) : 0u;
    }
  }

  // Element e of a chunk (e = 0..7): v_perm_b32 picks bytes 2(e%4), 2(e%4)+1
  // of words (x, y) and of (z, w) (selector byte 0x0c gives 0), then e/4
  // chooses. Selecting among the words themselves would make the compiler
  // address the row array in memory (scratch) instead of registers.
  auto pick_half = [](const uint4& t, int e) -> uint32_t {
    const uint32_t h = (uint32_t)(e & 3) * 2u;
    const uint32_t sel = 0x0c0c0000u | ((h + 1u) << 8) | h;
    const uint32_t p01 = __builtin_amdgcn_perm(t.y, t.x, sel);
    const uint32_t p23 = __builtin_amdgcn_perm(t.w, t.z, sel);
    return (e & 4) ? p23 : p01;
  };
  // Outlier elements of a chunk: gather them to Xo (rare path), then zero
  // them in the register copy, so the absmax and the codes below need no
  // per-element test (a zero element has magnitude 0 and code 0).
  // m = rank << 8 | mask, as in meta.
  auto strip = [&](int64_t row, uint32_t m, uint4& t) {
    const uint32_t om = m & 0xffu;
    if (om) {
      if (Xo) {
        int pos = (int)(m >> 8);
        uint16_t* dst = Xo + row * ld;
        if (om == 0xffu && (pos & 7) == 0) {
          // 8 outlier columns in a row land at 8 consecutive aligned positions
          st16(dst + pos, t);
        } else {
          for (uint32_t bits = om; bits; bits &= bits - 1u)
            dst[pos++] = (uint16_t)pick_half(t, __builtin_ctz(bits));
        }
      }
      uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t keep = ((om >> (2 * i)) & 1u ? 0u : 0xffffu) |
                              ((om >> (2 * i + 1)) & 1u ? 0u : 0xffff0000u);
        w[i] &= keep;
      }
      t = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  auto absmax_fold = [&](u16x2 m, const uint4& t) -> u16x2 {
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
    return m;
  };
  auto codes8 = [](const uint4& t, float s) -> uint2 { return codes8_rne(t, s); };

  for (int64_t row = row0; row < row_hi; row += kRowThreads / kWave) {
    const uint16_t* xr = X + row * K;
    u16x2 m2 = u16x2{0, 0};
    if constexpr (CPT > 0) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const bool ok = lane + (int64_t)j * kWave < nchunks;
        strip(row, meta[j], v[j]);
        m2 = absmax_fold(m2, ok ? v[j] : make_uint4(0, 0, 0, 0));
      }
    } else {
      for (int64_t c = lane; c < nchunks; c += kWave) {
        uint4 t = ld16(xr + c * 8);
        const uint32_t om = outl8(c);
        if (om) strip(row, (Xo ? (uint32_t)rank8(c) << 8 : 0u) | om, t);
        m2 = absmax_fold(m2, t);
      }
    }
    uint32_t mx = m2[0] > m2[1] ? m2[0] : m2[1];
    mx = wave_max_u32_dpp(mx);
    const float a = h2f(mx);
    const float s = a != 0.0f ? 127.0f / a : 0.0f;
    if (Xq) {
      if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const int64_t c = lane + (int64_t)j * kWave;
          if (c < nchunks) {
            const uint2 q = codes8(v[j], s);
            if constexpr (!kFlags) {
              // the weight codes are not read again by this call: streaming
              // stores (with the loads above, 5.05 -> 5.22 TB/s on the
              // 49152 x 12288 weight)
              __builtin_nontemporal_store(v2u32{q.x, q.y}, reinterpret_cast<v2u32*>(Xq + row * K + c * 8));
            } else {
              *reinterpret_cast<uint2*>(Xq + row * K + c * 8) = q;
            }
          }
        }
      } else {
        for (int64_t c = lane; c < nchunks; c += kWave) {
          uint4 t = ld16(xr + c * 8);
          const uint32_t om = outl8(c);
          if (om) {
            uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] &= ((om >> (2 * i)) & 1u ? 0u : 0xffffu) |
                      ((om >> (2 * i + 1)) & 1u ? 0u : 0xffff0000u);
            t = make_uint4(w[0], w[1], w[2], w[3]);
          }
          *reinterpret_cast<uint2*>(Xq + row * K + c * 8) = codes8(t, s);
        }
      }
      if (lane == 0) sx[row] = a;
    }
    if (Xo)
      for (int64_t t = n + lane; t < ld; t += kWave) Xo[row * ld + t] = 0;
    if (row + kRowThreads / kWave < row_hi) load_row(row + kRowThreads / kWave);
  }
}

// Row pass of the layer (and of int8_quantize_rowwise with a bitmap) for
// K <= 2048 * CPB. A block takes one row at a time, persistent over rows
// blockIdx.x, blockIdx.x + gridDim.x, ...: thread t holds the 16-byte chunks
// t, t + 256, ... (CPB of them), so a row costs a few registers per thread
// and many waves stay resident. The next row's loads are issued before the
// current row is worked on (two register sets). The outlier masks of a
// thread's chunks are the same for every row and are taken once per block.
// Per row: the outlier elements are gathered into Xo (rare), masked out, the
// row absmax is a wave maximum (DPP) and one LDS exchange between the four
// waves (one barrier per row; the exchange slots alternate between rows),
// the codes are stored chunk by chunk. Loads and stores are buffer
// operations over the row (the chunk offset in the scalar operand), so a
// chunk past the row reads 0 and its store is dropped. Arithmetic as k_rows.
// STG: the row's Xo is assembled in LDS (a buffer of ld_max elements per row
// parity, after the bitmap words) and written after the row's barrier as
// aligned 16-byte stores, zeros past n included. Written straight to memory,
// a chunk's outlier elements land at positions that are multiples of 8 only
// by chance when most columns are outlier columns, and then go out as 2-byte
// stores, one per element.
template <int CPB, int FMODE, bool STG>
__global__ __launch_bounds__(256) void k_rows_flagged(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ flags,
    int bands, uint32_t* __restrict__ bitmap_out, int8_t* __restrict__ Xq,
    float* __restrict__ sx, uint16_t* __restrict__ Xo, int32_t* __restrict__ cols,
    int32_t* __restrict__ n_out, int32_t* __restrict__ kbl) {
  static_assert(CPB > 0 && CPB <= 8 && FMODE != kNoFlags, "flagged rows, K <= 16384");
  extern __shared__ uint32_t smem[];
  __shared__ int sred[kRowThreads / kWave];
  __shared__ uint32_t s_max[2][kRowThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwords = (int)((K + 31) / 32);
  const int64_t nchunks = K / 8;
  uint32_t* sbm = smem;
  uint32_t* spre = smem + nwords;
  // STG only: 16-byte aligned, after the bitmap words and their prefix
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem + (2 * nwords + 3) / 4 * 4);
  const int64_t ld_max = (K + 31) / 32 * 32;
  const int64_t row0 = blockIdx.x, rstep = gridDim.x;

  // flag words first, then the first row: waiting for the flags leaves the
  // row's loads in flight
  constexpr int NFL = FMODE == kBands ? kMaxFlagBands : 1;
  const int wi = tid < nwords ? tid : nwords - 1;
  uint32_t fl[NFL];
#pragma unroll
  for (int b = 0; b < NFL; ++b) fl[b] = flags[(int64_t)(b < bands ? b : 0) * nwords + wi];
  asm volatile("" ::: "memory");
  const int voff_x = tid * 16;   // chunk t + 256 j: byte offset tid * 16 + j * 4096
  // X is not read again by the layer after this pass: streaming loads
  // (cache policy 2, nontemporal), 14.0 -> 13.3 us at 2048 x 4096
  auto load_row = [&](int64_t row, uint4 (&v)[CPB]) {
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(X + row * K, (uint32_t)(2 * K));
#pragma unroll
    for (int j = 0; j < CPB; ++j)
      v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x, j * 4096, 2));
  };
  uint4 va[CPB], vb[CPB];
  load_row(row0, va);   // row0 < M: the grid has at most M blocks

  uint32_t fw = 0;
#pragma unroll
  for (int b = 0; b < NFL; ++b) fw |= fl[b];
  sbm[wi] = fw;
  for (int w = tid + kRowThreads; w < nwords; w += kRowThreads) {
    uint32_t o = 0;
    for (int b = 0; b < bands; ++b) o |= flags[(int64_t)b * nwords + w];
    sbm[w] = o;
  }
  lds_only_barrier();   // LDS only: the first row's loads stay in flight
  int n = 0;
  if (Xo || cols || n_out) n = bitmap_prefix<true>(sbm, spre, nwords, sred);
  if (blockIdx.x == 0) {
    write_cols(sbm, spre, nwords, n, cols, n_out);
    write_kblocks(sbm, K, kbl);
    if (bitmap_out)
      for (int w = tid; w < nwords; w += kRowThreads) bitmap_out[w] = sbm[w];
  }
  const int64_t ld = ((int64_t)n + 31) / 32 * 32;

  // outlier masks of the thread's chunks, four to a register (0 past the row)
  constexpr int NPK = (CPB + 3) / 4;
  uint32_t pk[NPK];
#pragma unroll
  for (int i = 0; i < NPK; ++i) pk[i] = 0;
#pragma unroll
  for (int j = 0; j < CPB; ++j) {
    const int64_t c = tid + (int64_t)j * kRowThreads;
    const int64_t k = c * 8;
    const uint32_t om = c < nchunks ? (sbm[k >> 5] >> (k & 31)) & 0xffu : 0u;
    pk[j / 4] |= om << (8 * (j % 4));
  }
  uint32_t any = 0;
#pragma unroll
  for (int i = 0; i < NPK; ++i) any |= pk[i];
  auto om_of = [&](int j) -> uint32_t { return (pk[j / 4] >> (8 * (j % 4))) & 0xffu; };
  auto pick_half = [](const uint4& t, int e) -> uint32_t {
    const uint32_t h = (uint32_t)(e & 3) * 2u;
    const uint32_t sel = 0x0c0c0000u | ((h + 1u) << 8) | h;
    const uint32_t p01 = __builtin_amdgcn_perm(t.y, t.x, sel);
    const uint32_t p23 = __builtin_amdgcn_perm(t.w, t.z, sel);
    return (e & 4) ? p23 : p01;
  };
  const int voff_q = tid * 8;

  auto process = [&](int64_t row, uint4 (&v)[CPB], int parity) {
    // outlier elements: gathered into Xo from the unmodified chunk, then
    // zeroed in it (a zero has magnitude 0 and code 0)
    if (any) {
#pragma unroll
      for (int j = 0; j < CPB; ++j) {
        const uint32_t om = om_of(j);
        if (om) {
          if (Xo) {
            const int64_t k0 = (tid + (int64_t)j * kRowThreads) * 8;
            int pos = (int)spre[k0 >> 5] + __popc(sbm[k0 >> 5] & ((1u << (k0 & 31)) - 1u));
            uint16_t* dst = STG ? stage + parity * ld_max : Xo + row * ld;
            if (om == 0xffu && (pos & 7) == 0) {
              st16(dst + pos, v[j]);   // 8 outlier columns at 8 aligned positions
            } else {
              for (uint32_t bits = om; bits; bits &= bits - 1u)
                dst[pos++] = (uint16_t)pick_half(v[j], __builtin_ctz(bits));
            }
          }
          uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] &= ((om >> (2 * i)) & 1u ? 0u : 0xffffu) |
                    ((om >> (2 * i + 1)) & 1u ? 0u : 0xffff0000u);
          v[j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
    // row absmax: thread, wave (DPP), then the four waves through LDS
    u16x2 m2 = u16x2{0, 0};
#pragma unroll
    for (int j = 0; j < CPB; ++j) {
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
    }
    const uint32_t mw = wave_max_u32_dpp(m2[0] > m2[1] ? m2[0] : m2[1]);
    if (lane == 0) s_max[parity][wave] = mw;
    lds_only_barrier();
    uint32_t mx = s_max[parity][0];
#pragma unroll
    for (int w = 1; w < kRowThreads / kWave; ++w) mx = mx > s_max[parity][w] ? mx : s_max[parity][w];
    const float a = h2f(mx);
    const float sc = a != 0.0f ? 127.0f / a : 0.0f;
    if (Xq) {
      const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Xq + row * K, (uint32_t)K);
#pragma unroll
      for (int j = 0; j < CPB; ++j) {
        const uint2 q = codes8_rne(v[j], sc);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32, q), rq, voff_q, j * 2048, 0);
      }
      if (tid == 0) sx[row] = a;
    }
    if (Xo) {
      if constexpr (STG) {
        // the row's Xo from LDS, 8 elements a thread, zeros past n
        const uint16_t* st = stage + parity * ld_max;
        for (int64_t t = (int64_t)tid * 8; t < ld; t += kRowThreads * 8) {
          uint4 w = make_uint4(0u, 0u, 0u, 0u);
          if (t < n) {
            w = *reinterpret_cast<const uint4*>(st + t);
            const int64_t valid = n - t;   // elements of the chunk below n
            if (valid < 8) {
              uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
              for (int i = 0; i < 4; ++i)
                ww[i] &= (2 * i < valid ? 0xffffu : 0u) | (2 * i + 1 < valid ? 0xffff0000u : 0u);
              w = make_uint4(ww[0], ww[1], ww[2], ww[3]);
            }
          }
          st16(Xo + row * ld + t, w);
        }
      } else {
        for (int64_t t = n + tid; t < ld; t += kRowThreads) Xo[row * ld + t] = 0;
      }
    }
  };

  // two rows per iteration, alternating register sets (static indices)
  for (int64_t row = row0; row < M; row += 2 * rstep) {
    const int64_t r1 = row + rstep;
    if (r1 < M) load_row(r1, vb);
    process(row, va, 0);
    if (r1 >= M) break;
    const int64_t r2 = r1 + rstep;
    if (r2 < M) load_row(r2, va);
    process(r1, vb, 1);
  }
}

// Flagged row pass with the rows held across the block (K <= 2048 * CPB).
template <int CPB>
hipError_t launch_rows_flagged_t(const uint16_t* X, int64_t M, int64_t K, const uint32_t* flags,
                                 int bands, uint32_t* bitmap_out, int8_t* Xq, float* sx,
                                 uint16_t* Xo, int32_t* cols, int32_t* n_out, int32_t* kbl,
                                 hipStream_t s) {
  const int nwords = (int)((K + 31) / 32);
  size_t shm = (size_t)nwords * 2 * sizeof(uint32_t);
  // four resident blocks per CU on 256 CUs; each block walks its rows
  const int64_t blocks = std::min<int64_t>(M, 1024);
  // Xo assembled in LDS for the widest rows only (the shapes whose many
  // outlier columns made the direct stores the bound); one row buffer per
  // register set in use (a block with one row uses one)
  constexpr bool kStage = CPB == 8;
  if (kStage && Xo) {
    shm = (size_t)((2 * nwords + 3) / 4 * 4) * sizeof(uint32_t) +
          (size_t)(M > blocks ? 2 : 1) * (size_t)((K + 31) / 32 * 32) * 2;
    // up to 68 KB at K = 16384 (two row buffers), above the default limit
    // of dynamic LDS: allowed once per device for both instantiations (the
    // value is the same for every caller, so concurrent first calls are
    // benign)
    constexpr int kMaxDev = 64;
    static std::atomic<bool> lds_set[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int slot = dev >= 0 && dev < kMaxDev ? dev : 0;
    if (!lds_set[slot].load(std::memory_order_acquire)) {
      const int max_words = (2 * ((2048 * CPB + 31) / 32) + 3) / 4 * 4;
      const int max_bytes = max_words * (int)sizeof(uint32_t) + 2 * (2048 * CPB) * 2;
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rows_flagged<CPB, kBitmap, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_bytes);
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rows_flagged<CPB, kBands, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, max_bytes);
      if (e != hipSuccess) return e;
      lds_set[slot].store(true, std::memory_order_release);
    }
  }
  auto kern = kStage && Xo ? (bands == 1 ? k_rows_flagged<CPB, kBitmap, kStage>
                                         : k_rows_flagged<CPB, kBands, kStage>)
                           : (bands == 1 ? k_rows_flagged<CPB, kBitmap, false>
                                         : k_rows_flagged<CPB, kBands, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kRowThreads), shm, s, X, M, K, flags,
                     bands, bitmap_out, Xq, sx, Xo, cols, n_out, kbl);
  return hipGetLastError();
}

template <int CPT>
hipError_t launch_rows_t(const uint16_t* X, int64_t M, int64_t K, const uint32_t* flags,
                         int bands, uint32_t* bitmap_out, int8_t* Xq, float* sx, uint16_t* Xo,
                         int32_t* cols, int32_t* n_out, int32_t* kbl, hipStream_t s) {
  const int nwords = (int)((K + 31) / 32);
  const size_t shm = flags ? (size_t)nwords * 2 * sizeof(uint32_t) : 0;
  // 4 rows per block (one per wavefront) while that keeps >= 1024 blocks;
  // more rows per block beyond that amortize the bitmap prefix.
  int64_t rpb = 4;
  while (rpb < 64 && (M + rpb * 2 - 1) / (rpb * 2) >= 1024) rpb *= 2;
  const int64_t blocks = (M + rpb - 1) / rpb;
  auto kern = !flags ? k_rows<CPT, kNoFlags> : bands == 1 ? k_rows<CPT, kBitmap>
                                                           : k_rows<CPT, kBands>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kRowThreads), shm, s, X, M, K, (int)rpb,
                     flags, bands, bitmap_out, Xq, sx, Xo, cols, n_out, kbl);
  return hipGetLastError();
}

// Wo [N, LD(n)] is built one 16-byte piece (8 columns of a row) per thread,
// the threads laid flat over the N * LD(n) / 8 (row, piece) items so that
// consecutive threads fill consecutive pieces: with a few dozen outlier
// columns a row is only a handful of pieces, and a block per row would
// leave almost all of its threads idle and walk its rows one after another.
// f(j, t0): row j, columns t0 .. t0+7.
constexpr int kWoThreads = 256;
template <class F>
__device__ __forceinline__ void for_each_wo_piece(int64_t N, int64_t ld, F&& f) {
  const int64_t per_row = ld / 8;
  const int64_t items = N * per_row;
  const int64_t stride = (int64_t)gridDim.x * kWoThreads;
  for (int64_t it = (int64_t)blockIdx.x * kWoThreads + threadIdx.x; it < items; it += stride) {
    const int64_t j = it / per_row;
    f(j, (it - j * per_row) * 8);
  }
}

// cols[t0 .. t0+7], -1 from n on (the zero pad).
__device__ __forceinline__ void load_cols8(const int32_t* __restrict__ cols, int64_t t0, int n,
                                           int c[8]) {
  if (t0 + 8 <= n) {
    const uint4 c0 = ld16(cols + t0), c1 = ld16(cols + t0 + 4);
    c[0] = (int)c0.x; c[1] = (int)c0.y; c[2] = (int)c0.z; c[3] = (int)c0.w;
    c[4] = (int)c1.x; c[5] = (int)c1.y; c[6] = (int)c1.z; c[7] = (int)c1.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = t0 + e < n ? cols[t0 + e] : -1;
  }
}

// Recovered fp16 weight columns of the outlier columns, for the GEMM's
// outlier segment ([HF-blog] "Usage": the fp16 weights of the outlier matmul
// come back from CB * SCB / 127, per output row):
//   Wo[j, t] = fp16(fl32(fl32(Wq[j, cols[t]] * sw[j]) / 127))  for t < n,
//   +0.0 for n <= t < LD(n), rows LD(n) halfs apart.
// n is read on the device; with 16 or fewer outlier columns the GEMM stages
// them itself and this does nothing. Up to 96 columns (LD(n) <= 96) each
// thread computes its 8 values directly over the flat pieces. Beyond that a
// row has enough columns for a table to pay: the value depends only on the
// code q and the row and is odd in q (each of the three roundings is
// symmetric), so a block takes one row (up to 2048 columns) at a time, builds
// the values of q = 0..128 with the same arithmetic in LDS, and each thread
// looks up its 8 (sign bit from the code). Both give the same bits.
constexpr int kRecoverCols = 2048;   // columns per block and row: 256 threads x 8
__global__ __launch_bounds__(kWoThreads) void k_recover_outlier_w(
    const int8_t* __restrict__ Wq, const float* __restrict__ sw, int64_t N, int64_t K,
    const int32_t* __restrict__ cols, const int32_t* __restrict__ n_out, int wo_cols,
    uint16_t* __restrict__ Wo) {
  __shared__ uint16_t s_lut[130];   // q = 0..128 (-128 is a valid int8)
  const int n = *n_out;
  if (n <= 16 || n > wo_cols) return;   // the GEMM's other paths take those
  const int64_t ld = ((int64_t)n + 31) / 32 * 32;
  auto codes = [&](int64_t j, int64_t t0, int c[8], int q[8]) {
    load_cols8(cols, t0, n, c);
    const int8_t* row = Wq + j * K;
    if (c[0] >= 0 && c[7] == c[0] + 7 && (c[0] & 7) == 0) {
      // 8 consecutive columns (they ascend) from a multiple of 8: one load
      const uint2 v = *reinterpret_cast<const uint2*>(row + c[0]);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = (int)(int8_t)((e < 4 ? v.x : v.y) >> (8 * (e & 3)));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = c[e] >= 0 ? (int)row[c[e]] : 0;
    }
  };
  auto store = [&](int64_t j, int64_t t0, const uint32_t h[8]) {
    st16(Wo + j * ld + t0, make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                      h[4] | (h[5] << 16), h[6] | (h[7] << 16)));
  };
  if (ld <= 96) {
    for_each_wo_piece(N, ld, [&](int64_t j, int64_t t0) {
      int c[8], q[8];
      codes(j, t0, c, q);
      const float s = sw[j];
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = c[e] >= 0 ? f2h(((float)q[e] * s) / 127.0f) : 0u;
      store(j, t0, h);
    });
    return;
  }
  const int64_t chunks = (ld + kRecoverCols - 1) / kRecoverCols;
  const int tid = threadIdx.x;
  for (int64_t task = blockIdx.x; task < N * chunks; task += gridDim.x) {
    const int64_t j = task / chunks;
    const int64_t t0 = (task - j * chunks) * kRecoverCols + (int64_t)tid * 8;
    // the codes are fetched before the table is built, so their latency
    // overlaps it
    int c[8], q[8];
    if (t0 < ld) codes(j, t0, c, q);
    __syncthreads();   // the previous task's lookups are done
    if (tid <= 128) s_lut[tid] = f2h(((float)tid * sw[j]) / 127.0f);
    __syncthreads();
    if (t0 < ld) {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t mag = s_lut[q[e] < 0 ? -q[e] : q[e]];
        h[e] = c[e] >= 0 ? (mag | (q[e] < 0 ? 0x8000u : 0u)) : 0u;
      }
      store(j, t0, h);
    }
  }
}

// Outlier weight columns of a layer that keeps its weight in fp16 ([HF-blog]
// "Usage", has_fp16_weights=True): Wo[j, t] = W[j, cols[t]] as they are, for
// t < n, +0.0 up to LD(n), with the same pieces as the recovery above.
// Nothing when n <= 16 (the GEMM stages those itself) or n > wo_cols (the
// region has no room: the GEMM's dense segment reads W itself).
__global__ __launch_bounds__(kWoThreads) void k_gather_w_cols(
    const uint16_t* __restrict__ W, int64_t N, int64_t K, const int32_t* __restrict__ cols,
    const int32_t* __restrict__ n_out, int wo_cols, uint16_t* __restrict__ Wo) {
  const int n = *n_out;
  if (n <= 16 || n > wo_cols) return;   // the GEMM's other paths take those
  const int64_t ld = ((int64_t)n + 31) / 32 * 32;
  for_each_wo_piece(N, ld, [&](int64_t j, int64_t t0) {
    int c[8];
    load_cols8(cols, t0, n, c);
    const uint16_t* row = W + j * K;
    if (c[0] >= 0 && c[7] == c[0] + 7 && (c[0] & 7) == 0) {
      st16(Wo + j * ld + t0, ld16(row + c[0]));   // 8 consecutive columns: one load
      return;
    }
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = c[e] >= 0 ? (uint32_t)row[c[e]] : 0u;
    st16(Wo + j * ld + t0, make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                      h[4] | (h[5] << 16), h[6] | (h[7] << 16)));
  });
}

// Exact-erf GELU in fp32 (activation between the two layers of an MLP block).
// Eight elements per thread: one 16-byte load and store each (the pointers
// are 16-byte aligned), the last partial group element by element.
constexpr int kGeluPer = 8;
__device__ __forceinline__ uint32_t gelu_h(uint32_t h) {
  const float x = h2f(h);
  // x * Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2: no cancellation for
  // large negative x (1 + erf would lose every digit there).
  return f2h(0.5f * x * erfcf(-x * 0.70710678118654752f));
}
__global__ void k_gelu(const uint16_t* __restrict__ X, int64_t count, uint16_t* __restrict__ Y) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * kGeluPer;
  if (i0 >= count) return;
  if (i0 + kGeluPer <= count) {
    const uint4 v = ld16(X + i0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = gelu_h(w[i] & 0xffffu) | (gelu_h(w[i] >> 16) << 16);
    st16(Y + i0, make_uint4(o[0], o[1], o[2], o[3]));
  } else {
    for (int64_t i = i0; i < count; ++i) Y[i] = (uint16_t)gelu_h(X[i]);
  }
}


}  // namespace

// Value of a non-negative fp16 bit pattern (p <= 0x7c00).
static double fp16_pattern_value(uint32_t p) {
  const uint32_t e = (p >> 10) & 0x1f, m = p & 0x3ff;
  if (e == 0x1f) return HUGE_VAL;
  if (e == 0) return std::ldexp((double)m, -24);
  return std::ldexp((double)(1024 + m), (int)e - 25);
}

uint32_t fp16_threshold_pattern(float threshold) {
  if (!(threshold > 0.0f)) return 0;          // every magnitude is >= threshold
  uint32_t lo = 0, hi = 0x7c00;               // value(0x7c00) = inf >= any threshold
  while (lo < hi) {
    const uint32_t mid = (lo + hi) / 2;
    if (fp16_pattern_value(mid) >= (double)threshold) hi = mid; else lo = mid + 1;
  }
  return lo;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((count + threads - 1) / threads)), dim3(threads),
                     0, s, p, count, value);
  return hipGetLastError();
}

hipError_t launch_outlier_flags(const uint16_t* X, int64_t M, int64_t K, uint32_t tau16,
                                uint32_t* bitmap, hipStream_t s) {
  if (M <= 0 || K <= 0) return hipSuccess;
  const int64_t col_groups = (K / 8 + 63) / 64;
  // Row blocks of 32 rows (8 per wave): enough 16-byte loads in flight per
  // lane while keeping the grid well above the CU count at prefill sizes.
  const int rows_per_block = 32;
  const int64_t row_blocks = (M + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(k_outlier_flags, dim3((unsigned)col_groups, (unsigned)row_blocks), dim3(256),
                     0, s, X, M, K, tau16, rows_per_block, bitmap);
  return hipGetLastError();
}

hipError_t launch_cols_from_bitmap(const uint32_t* bitmap, int64_t K, int32_t* cols,
                                   int32_t* n_out, hipStream_t s) {
  const int nwords = (int)((K + 31) / 32);
  size_t shm = (size_t)nwords * 2 * sizeof(uint32_t);
  hipLaunchKernelGGL(k_cols_from_bitmap, dim3(1), dim3(kRowThreads), shm, s, bitmap, K, cols,
                     n_out);
  return hipGetLastError();
}

hipError_t launch_rows_banded(const uint16_t* X, int64_t M, int64_t K, const uint32_t* flags,
                              int bands, uint32_t* bitmap_out, int8_t* Xq, float* sx,
                              uint16_t* Xo, int32_t* cols, int32_t* n_out, int32_t* kbl,
                              hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (flags && K > 0) {
    // the block-per-row pass (chunks per thread: ceil(K / 2048))
    const int64_t cpb = (K / 8 + kRowThreads - 1) / kRowThreads;
#define I8MM_ROWSF(CPB) \
  launch_rows_flagged_t<CPB>(X, M, K, flags, bands, bitmap_out, Xq, sx, Xo, cols, n_out, kbl, s)
    if (cpb <= 1) return I8MM_ROWSF(1);
    if (cpb <= 2) return I8MM_ROWSF(2);
    if (cpb <= 4) return I8MM_ROWSF(4);
    if (cpb <= 6) return I8MM_ROWSF(6);
    if (cpb <= 8) return I8MM_ROWSF(8);
#undef I8MM_ROWSF
  }
  const int64_t per_lane = (K / 8 + kWave - 1) / kWave;
#define I8MM_ROWS(CPT) \
  launch_rows_t<CPT>(X, M, K, flags, bands, bitmap_out, Xq, sx, Xo, cols, n_out, kbl, s)
  if (per_lane <= 1) return I8MM_ROWS(1);
  if (per_lane <= 2) return I8MM_ROWS(2);
  if (per_lane <= 4) return I8MM_ROWS(4);
  if (per_lane <= 8) return I8MM_ROWS(8);
  if (per_lane <= 16) return I8MM_ROWS(16);
  if (per_lane <= 24) return I8MM_ROWS(24);
  if (per_lane <= 32) return I8MM_ROWS(32);
  return I8MM_ROWS(0);
#undef I8MM_ROWS
}

hipError_t launch_rows(const uint16_t* X, int64_t M, int64_t K, const uint32_t* bitmap,
                       int8_t* Xq, float* sx, uint16_t* Xo, int32_t* cols, int32_t* n_out,
                       hipStream_t s) {
  return launch_rows_banded(X, M, K, bitmap, 1, nullptr, Xq, sx, Xo, cols, n_out, nullptr, s);
}

int flag_bands(int64_t M, int64_t K) {
  const int64_t nwords = (K + 31) / 32;
  if (M <= 0 || nwords == 0) return 1;
  // about 2048 partial words in all: few loads per word in the row pass
  int64_t b = std::min<int64_t>(kMaxFlagBands, std::max<int64_t>(1, 2048 / nwords));
  // at least one pass of 16 rows per band
  b = std::min<int64_t>(b, std::max<int64_t>(1, M / 16));
  // no empty band: ceil(M / ceil(M / b)) bands of ceil(M / b) rows
  const int64_t rpb = (M + b - 1) / b;
  return (int)((M + rpb - 1) / rpb);
}

hipError_t launch_outlier_flag_bands(const uint16_t* X, int64_t M, int64_t K, uint32_t tau16,
                                     int bands, uint32_t* part, hipStream_t s) {
  if (M <= 0 || K <= 0) return hipSuccess;
  const int64_t rows_per_band = (M + bands - 1) / bands;
  const int64_t groups = (K + kFlagGroupCols - 1) / kFlagGroupCols;
  hipLaunchKernelGGL(k_outlier_flag_bands, dim3((unsigned)groups, (unsigned)bands), dim3(256), 0,
                     s, X, M, K, tau16, rows_per_band, (K + 31) / 32, part);
  return hipGetLastError();
}

// Blocks for the Wo builders: n is only known on the device, so the grid is
// sized for the largest n that runs (K columns, or the region's room), at
// most 2048 blocks (a grid-stride
// loop covers the rest); blocks past the last piece exit at once.
static unsigned wo_blocks(int64_t N, int64_t K) {
  const int64_t pieces = N * (I8MM_OUTLIER_LD(K) / 8);
  return (unsigned)std::min<int64_t>((pieces + kWoThreads - 1) / kWoThreads, 2048);
}

hipError_t launch_recover_outlier_w(const int8_t* Wq, const float* sw, int64_t N, int64_t K,
                                    const int32_t* cols, const int32_t* n_out, int wo_cols,
                                    uint16_t* Wo, hipStream_t s) {
  if (N <= 0 || K <= 0 || wo_cols <= 16) return hipSuccess;
  hipLaunchKernelGGL(k_recover_outlier_w, dim3(wo_blocks(N, std::min<int64_t>(K, wo_cols))),
                     dim3(kWoThreads), 0, s, Wq, sw, N, K, cols, n_out, wo_cols, Wo);
  return hipGetLastError();
}

hipError_t launch_gather_w_cols(const uint16_t* Wf, int64_t N, int64_t K, const int32_t* cols,
                                const int32_t* n_out, int wo_cols, uint16_t* Wo, hipStream_t s) {
  if (N <= 0 || K <= 0 || wo_cols <= 16) return hipSuccess;
  hipLaunchKernelGGL(k_gather_w_cols, dim3(wo_blocks(N, std::min<int64_t>(K, wo_cols))),
                     dim3(kWoThreads), 0, s, Wf, N, K, cols, n_out, wo_cols, Wo);
  return hipGetLastError();
}

hipError_t launch_gelu(const uint16_t* X, int64_t count, uint16_t* Y, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int threads = 256;
  const int64_t groups = (count + kGeluPer - 1) / kGeluPer;
  hipLaunchKernelGGL(k_gelu, dim3((unsigned)((groups + threads - 1) / threads)), dim3(threads), 0,
                     s, X, count, Y);
  return hipGetLastError();
}

}  // namespace i8mm
