// Bandwidth-bound kernels of the LLM.int8() layer on gfx950:
//   - outlier-column detection (column OR-reduce of abs(x) >= threshold),
//   - bitmap -> ascending outlier-column list,
//   - per-row absmax int8 quantization (of X rows over the non-outlier
//     columns, or of W rows over the full row) fused with the gather of the
//     outlier columns of X,
//   - exact-erf GELU for MLP blocks built from the layer.
//
// Pages cited: [HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit
// Matrix Multiplication for transformers at scale using Hugging Face
// Transformers, Accelerate and bitsandbytes"; [Summary] paper summary page
// "LLM.int8(): 8-Bit Matrix Multiplication for Transformers at Scale".
//
// Every kernel reads its rows as 16-byte chunks (8 fp16), one chunk per lane,
// so a wavefront touches 1 KiB of contiguous memory per load.

#include "device_common.h"
#include "launchers.h"

namespace i8mm {

namespace {

constexpr int kRowThreads = 256;

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t count, uint32_t value) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = value;
}

// 8 flags, bit e set when abs(element e) >= tau. [HF-blog] "Inside the MatMul"
// (magnitude 6 or greater) and [Summary] "The full picture" step 1. The fp16
// value is widened exactly and compared in fp32; NaN never compares true.
__device__ __forceinline__ uint32_t threshold_flags8(const uint4& v, float tau) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) m |= (fabsf(h2f(half_of(v, e))) >= tau ? 1u : 0u) << e;
  return m;
}

// Column OR-reduce. Block = 4 waves over one 512-column group; lane owns an
// 8-column chunk; wave w scans rows r0+w, r0+w+4, ... of the block's row
// range. Flag bits are merged into the (pre-zeroed) bitmap with atomicOr,
// which is issued only for chunks that hold an outlier; OR is order-free, so
// the result does not depend on scheduling.
__global__ __launch_bounds__(256) void k_outlier_flags(const uint16_t* __restrict__ X, int64_t M,
                                                       int64_t K, float tau, int rows_per_block,
                                                       uint32_t* __restrict__ bitmap) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = ((int64_t)blockIdx.x * 64 + lane) * 8;
  if (col0 >= K) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(M, r0 + (int64_t)rows_per_block);
  const uint16_t* base = X + col0;
  uint32_t mask = 0;
  int64_t r = r0 + wave;
  for (; r + 12 < r1; r += 16) {
    uint4 v0 = ld16(base + r * K);
    uint4 v1 = ld16(base + (r + 4) * K);
    uint4 v2 = ld16(base + (r + 8) * K);
    uint4 v3 = ld16(base + (r + 12) * K);
    mask |= threshold_flags8(v0, tau) | threshold_flags8(v1, tau) | threshold_flags8(v2, tau) |
            threshold_flags8(v3, tau);
  }
  for (; r < r1; r += 4) mask |= threshold_flags8(ld16(base + r * K), tau);
  if (mask) atomicOr(&bitmap[col0 >> 5], mask << (col0 & 31));
}

// Exclusive prefix of popcount over the bitmap words, in LDS. Returns the
// total (the outlier count n). All threads of the block must call it.
__device__ int bitmap_prefix(const uint32_t* sbm, uint32_t* spre, int nwords, int* sred) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (nwords + kRowThreads - 1) / kRowThreads;
  const int w0 = tid * per;
  const int w1 = min(nwords, w0 + per);
  int local = 0;
  for (int w = w0; w < w1; ++w) local += __popc(sbm[w]);
  int incl = wave_inclusive_scan(local, lane);
  if (lane == 63) sred[wave] = incl;
  __syncthreads();
  int wave_off = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kRowThreads / kWave; ++i) {
    wave_off += i < wave ? sred[i] : 0;
    total += sred[i];
  }
  int run = wave_off + incl - local;
  for (int w = w0; w < w1; ++w) {
    spre[w] = (uint32_t)run;
    run += __popc(sbm[w]);
  }
  __syncthreads();
  return total;
}

// Writes cols[p] = k for the p-th set bit k (ascending) and *n_out.
__device__ void write_cols(const uint32_t* sbm, const uint32_t* spre, int nwords, int n,
                           int32_t* __restrict__ cols, int32_t* __restrict__ n_out) {
  if (cols) {
    for (int w = threadIdx.x; w < nwords; w += kRowThreads) {
      uint32_t bits = sbm[w];
      int p = (int)spre[w];
      while (bits) {
        int b = __builtin_ctz(bits);
        cols[p++] = w * 32 + b;
        bits &= bits - 1;
      }
    }
  }
  if (n_out && threadIdx.x == 0) *n_out = n;
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

// One block per row. CPT = 16-byte chunks per thread kept in registers
// (K <= CPT * 8 * 256); CPT == 0 streams the row twice (any K).
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
template <int CPT>
__global__ __launch_bounds__(256) void k_rows(const uint16_t* __restrict__ X, int64_t M,
                                              int64_t K, const uint32_t* __restrict__ bitmap,
                                              int8_t* __restrict__ Xq, float* __restrict__ sx,
                                              uint16_t* __restrict__ Xo, int32_t* __restrict__ cols,
                                              int32_t* __restrict__ n_out) {
  extern __shared__ uint32_t smem[];
  __shared__ int sred[kRowThreads / kWave];
  __shared__ uint32_t smax[kRowThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nwords = (int)((K + 31) / 32);
  const int64_t nchunks = K / 8;
  uint32_t* sbm = smem;
  uint32_t* spre = smem + nwords;
  const uint16_t* xr = X + row * K;

  int n = 0;
  if (bitmap) {
    for (int w = tid; w < nwords; w += kRowThreads) sbm[w] = bitmap[w];
    __syncthreads();
    if (Xo || cols || n_out) n = bitmap_prefix(sbm, spre, nwords, sred);
  }
  auto outl8 = [&](int64_t c) -> uint32_t {
    if (!bitmap) return 0u;
    int64_t k = c * 8;
    return (sbm[k >> 5] >> (k & 31)) & 0xffu;
  };

  // ---- pass 1: absmax of the normal entries
  uint4 v[CPT > 0 ? CPT : 1];
  uint32_t mx = 0;
  if constexpr (CPT > 0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      int64_t c = tid + (int64_t)j * kRowThreads;
      v[j] = c < nchunks ? ld16(xr + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      int64_t c = tid + (int64_t)j * kRowThreads;
      uint32_t om = c < nchunks ? outl8(c) : 0xffu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t m = (om >> e) & 1u ? 0u : (half_of(v[j], e) & 0x7fffu);
        mx = mx > m ? mx : m;
      }
    }
  } else {
    for (int64_t c = tid; c < nchunks; c += kRowThreads) {
      uint4 t = ld16(xr + c * 8);
      uint32_t om = outl8(c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t m = (om >> e) & 1u ? 0u : (half_of(t, e) & 0x7fffu);
        mx = mx > m ? mx : m;
      }
    }
  }
  mx = wave_max_u32(mx);
  if (lane == 0) smax[wave] = mx;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kRowThreads / kWave; ++i) mx = mx > smax[i] ? mx : smax[i];

  const float a = h2f(mx);
  const float s = a != 0.0f ? 127.0f / a : 0.0f;

  // ---- pass 2: codes, stores, gather
  auto emit = [&](int64_t c, const uint4& t) {
    uint32_t om = outl8(c);
    if (Xq) {
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float q = __builtin_rintf(h2f(half_of(t, e)) * s);
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        int qi = (om >> e) & 1u ? 0 : (int)q;
        packed[e >> 2] |= ((uint32_t)qi & 0xffu) << ((e & 3) * 8);
      }
      *reinterpret_cast<uint2*>(Xq + row * K + c * 8) = make_uint2(packed[0], packed[1]);
    }
    if (Xo && om) {
      const int64_t ld = ((int64_t)n + 31) / 32 * 32;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((om >> e) & 1u) {
          int64_t k = c * 8 + e;
          uint32_t w = sbm[k >> 5];
          int pos = (int)spre[k >> 5] + __popc(w & ((1u << (k & 31)) - 1u));
          Xo[row * ld + pos] = (uint16_t)half_of(t, e);
        }
      }
    }
  };
  if constexpr (CPT > 0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      int64_t c = tid + (int64_t)j * kRowThreads;
      if (c < nchunks) emit(c, v[j]);
    }
  } else {
    for (int64_t c = tid; c < nchunks; c += kRowThreads) emit(c, ld16(xr + c * 8));
  }
  if (Xq && tid == 0) sx[row] = a;
  if (Xo) {
    const int64_t ld = ((int64_t)n + 31) / 32 * 32;
    for (int64_t t = n + tid; t < ld; t += kRowThreads) Xo[row * ld + t] = 0;
  }
  if (row == 0 && bitmap) write_cols(sbm, spre, nwords, n, cols, n_out);
  else if (row == 0 && n_out && tid == 0) *n_out = 0;
}

// Exact-erf GELU in fp32 (activation between the two layers of an MLP block).
__global__ void k_gelu(const uint16_t* __restrict__ X, int64_t count, uint16_t* __restrict__ Y) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float x = h2f(X[i]);
  // x * Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2: no cancellation for
  // large negative x (1 + erf would lose every digit there).
  float y = 0.5f * x * erfcf(-x * 0.70710678118654752f);
  Y[i] = f2h(y);
}

template <int CPT>
hipError_t launch_rows_t(const uint16_t* X, int64_t M, int64_t K, const uint32_t* bitmap,
                         int8_t* Xq, float* sx, uint16_t* Xo, int32_t* cols, int32_t* n_out,
                         hipStream_t s) {
  const int nwords = (int)((K + 31) / 32);
  size_t shm = bitmap ? (size_t)nwords * 2 * sizeof(uint32_t) : 0;
  hipLaunchKernelGGL(k_rows<CPT>, dim3((unsigned)M), dim3(kRowThreads), shm, s, X, M, K, bitmap,
                     Xq, sx, Xo, cols, n_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((count + threads - 1) / threads)), dim3(threads),
                     0, s, p, count, value);
  return hipGetLastError();
}

hipError_t launch_outlier_flags(const uint16_t* X, int64_t M, int64_t K, float tau,
                                uint32_t* bitmap, hipStream_t s) {
  if (M <= 0 || K <= 0) return hipSuccess;
  const int64_t col_groups = (K / 8 + 63) / 64;
  // Row blocks of 32 rows (8 per wave): enough 16-byte loads in flight per
  // lane while keeping the grid well above the CU count at prefill sizes.
  const int rows_per_block = 32;
  const int64_t row_blocks = (M + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(k_outlier_flags, dim3((unsigned)col_groups, (unsigned)row_blocks), dim3(256),
                     0, s, X, M, K, tau, rows_per_block, bitmap);
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

hipError_t launch_rows(const uint16_t* X, int64_t M, int64_t K, const uint32_t* bitmap,
                       int8_t* Xq, float* sx, uint16_t* Xo, int32_t* cols, int32_t* n_out,
                       hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int64_t per_thread = (K / 8 + kRowThreads - 1) / kRowThreads;
  if (per_thread <= 1) return launch_rows_t<1>(X, M, K, bitmap, Xq, sx, Xo, cols, n_out, s);
  if (per_thread <= 2) return launch_rows_t<2>(X, M, K, bitmap, Xq, sx, Xo, cols, n_out, s);
  if (per_thread <= 4) return launch_rows_t<4>(X, M, K, bitmap, Xq, sx, Xo, cols, n_out, s);
  if (per_thread <= 6) return launch_rows_t<6>(X, M, K, bitmap, Xq, sx, Xo, cols, n_out, s);
  if (per_thread <= 8) return launch_rows_t<8>(X, M, K, bitmap, Xq, sx, Xo, cols, n_out, s);
  if (per_thread <= 16) return launch_rows_t<16>(X, M, K, bitmap, Xq, sx, Xo, cols, n_out, s);
  return launch_rows_t<0>(X, M, K, bitmap, Xq, sx, Xo, cols, n_out, s);
}

hipError_t launch_gelu(const uint16_t* X, int64_t count, uint16_t* Y, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(k_gelu, dim3((unsigned)((count + threads - 1) / threads)), dim3(threads), 0,
                     s, X, count, Y);
  return hipGetLastError();
}

}  // namespace i8mm
