// The whole few-token layer in one launch: outlier-column detection, row
// quantization of X, int8 matmul with int32 accumulation, dequantization,
// fp16 outlier product and bias, for 1 <= M <= 8 tokens. At these sizes the
// layer is bound by streaming the int8 weight from HBM once; run as separate
// kernels, the steps on X cost more in launches than the weight stream.
//
// Pages cited: [HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit
// Matrix Multiplication for transformers at scale using Hugging Face
// Transformers, Accelerate and bitsandbytes"; [Summary] paper summary page
// "LLM.int8(): 8-Bit Matrix Multiplication for Transformers at Scale".
//
// Same arithmetic as the separate kernels, step for step:
//   outlier columns  O = {k : some abs(X[i, k]) >= threshold}, NaN included
//                    ([HF-blog] "Inside the MatMul"; [Summary] "The full
//                    picture" step 1), compared on fp16 magnitude patterns;
//   row codes        a = absmax of row i over k not in O, s = fl32(127 / a),
//                    Xq = rne(fl32(x * s)), 0 on O ([HF-blog] "Introduction
//                    to model quantization"; [Summary] step 3);
//   output           Y = fp16(C * (a / 127) * (sw / 127) + sum_t X[i, O_t] *
//                    Wo[j, t] + bias), C exact in int32, Wo the recovered
//                    (CB * SCB / 127) or fp16 weight columns ([HF-blog]
//                    "Usage"; [Summary] steps 3-4).
//
// Block = 4 wavefronts. Every block does the X side itself (X is at most
// 8 x 16384 fp16, read from L2 by all blocks). Thread t holds the 16-byte
// chunks t, t + 256, ... of every token row in registers, so each 8-column
// flag mask is its own maximum over the rows (no exchange beyond the four
// lanes of a bitmap word), the outlier elements are masked out from its own
// bits, and the row maxima need one block reduction for all rows at once.
// The X loads are issued before the first weight tile's loads and waited for
// alone, so the X side runs while the weight is in flight. The codes go to
// LDS; block 0 also writes the intermediates (bitmap, cols, n, sx, Xq, Xo)
// to the workspace. Then blocks walk 16-feature weight tiles (persistent
// grid) like the few-token GEMV: waves split K in 256-byte chunks, weight
// rows straight from HBM into registers in the operand layout of
// v_mfma_i32_16x16x64_i8, token fragments from the LDS codes (rows padded so
// the 16 token rows of one read hit distinct banks), partial tiles summed
// through LDS.

#include <algorithm>

#include "device_common.h"
#include "launchers.h"

namespace i8mm {

namespace {

constexpr int kDcThreads = kBlockThreads;   // 4 wavefronts
constexpr int kDcWaves = kDcThreads / kWave;
constexpr int kDcFeat = 16;                 // output features per tile
constexpr int kDcChunk = 256;               // K bytes per MFMA chunk
constexpr int kDcBatch = 4;                 // chunks per wave held in registers at once
constexpr int kDcMaxTok = 8;
constexpr int kDcMaxOut = 32;               // outlier columns staged in LDS
constexpr int kDcXRegs = 32;                // 16-byte X chunks a thread holds
constexpr int kDcPad = 16;                  // LDS row padding of the codes

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dc_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

__host__ __device__ constexpr int dc_round16(int v) { return (v + 15) / 16 * 16; }

// LDS row pitch of the int8 codes: K rounded up to 256 bytes, plus 16, so
// the 16 token rows of one fragment read hit distinct banks.
__host__ __device__ constexpr int dc_pitch(int K) { return (K + 255) / 256 * 256 + kDcPad; }

// Dynamic LDS: [codes M x pitch][bitmap][prefix].
__host__ __device__ constexpr int dc_lds_bytes(int M, int K) {
  return dc_round16(M * dc_pitch(K)) + 8 * ((K + 31) / 32);
}

// Thread t holds the 16-byte chunks t, t + 256, ... (JC of them, K <= JC *
// 2048) of each of the first MR token rows (M <= MR, MR * JC <= kDcXRegs).
template <int MR, int JC>
__global__ __launch_bounds__(kDcThreads) void k_decode_i8(
    const uint16_t* __restrict__ X, const int8_t* __restrict__ Wq, const float* __restrict__ sw,
    int M, int N, int K, uint32_t tau16, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ Y, const uint16_t* __restrict__ Wf, uint32_t* __restrict__ bitmap_g,
    int32_t* __restrict__ cols_g, int32_t* __restrict__ n_g, float* __restrict__ sx_g,
    int8_t* __restrict__ Xq_g, uint16_t* __restrict__ Xo_g) {
  static_assert(MR * JC <= kDcXRegs, "X chunks held per thread");
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  __shared__ int32_t red[kDcWaves][16 * 16];
  __shared__ float s_wo[kDcMaxOut][16];             // outlier weights, [t][j]
  __shared__ uint16_t s_xo[kDcMaxTok][kDcMaxOut];   // outlier activations, [m][t]
  __shared__ float s_sx[kDcMaxTok];
  __shared__ int s_cols[kDcMaxOut];
  __shared__ int sred[kDcWaves];
  __shared__ uint32_t s_rmax[kDcWaves][kDcMaxTok];   // per-wave row maxima

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nchunks = K / 8;            // 16-byte chunks of a row
  const int nwords = (K + 31) / 32;
  const int ldx = dc_pitch(K);          // LDS row pitch of the codes (bytes)
  int8_t* s_xq = reinterpret_cast<int8_t*>(dsm);
  uint32_t* sbm = reinterpret_cast<uint32_t*>(dsm + dc_round16(M * ldx));
  uint32_t* spre = sbm + nwords;
  const bool first = blockIdx.x == 0;

  // ---- X into registers (issued first: waited for alone below)
  uint4 xr[MR][JC];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int j = 0; j < JC; ++j) {
      const int c = tid + kDcThreads * j;
      xr[m][j] = (m < M && c < nchunks) ? ld16(X + (int64_t)m * K + c * 8) : make_uint4(0, 0, 0, 0);
    }
  }

  // ---- the first weight tile's loads
  const int nkc = (K + kDcChunk - 1) / kDcChunk;
  const int r16 = lane & 15;                 // weight row / token of the MFMA operands
  const int seg = (lane >> 4) * 16;          // this lane's 16 bytes of each 64-byte k-slice
  constexpr int kOob = 0x7ffffff0;
  v4i32 wf[kDcBatch][4];
  __amdgpu_buffer_rsrc_t rw;
  auto load_w = [&](int c0) {
#pragma unroll
    for (int b = 0; b < kDcBatch; ++b) {
      const int c = c0 + b * kDcWaves;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = c * kDcChunk + 64 * j + seg;
        wf[b][j] = __builtin_bit_cast(
            v4i32, __builtin_amdgcn_raw_buffer_load_b128(
                       rw, (c < nkc && k < K) ? r16 * K + k : kOob, 0, 0));
      }
    }
  };
  auto tile_rsrc = [&](int64_t f0) {
    const int rows_w = (int)min<int64_t>(kDcFeat, N - f0);
    rw = dc_rsrc(Wq + f0 * K, (uint32_t)rows_w * (uint32_t)K);
  };
  tile_rsrc((int64_t)blockIdx.x * kDcFeat);
  load_w(wave);
  __builtin_amdgcn_sched_barrier(0);

  // ---- column flags: a thread holds whole columns, so each 8-column mask
  // is its own maximum over the rows; the four masks of a 32-column word are
  // OR-ed by shuffles (consecutive threads hold consecutive chunks)
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  uint32_t om[JC];   // outlier bits of chunk j (bit e: element e)
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    const int c = tid + kDcThreads * j;
    u16x2 mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = u16x2{0, 0};
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
        const uint32_t w[4] = {xr[m][j].x, xr[m][j].y, xr[m][j].z, xr[m][j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mx[i] = __builtin_elementwise_max(mx[i], __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
      }
    }
    uint32_t mask = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mask |= ((uint32_t)mx[i][0] >= tau16 ? 1u : 0u) << (2 * i);
      mask |= ((uint32_t)mx[i][1] >= tau16 ? 1u : 0u) << (2 * i + 1);
    }
    om[j] = c < nchunks ? mask : 0u;
    uint32_t word = om[j] << (8 * (c & 3));
    word |= (uint32_t)__shfl_xor((int)word, 1, kWave);
    word |= (uint32_t)__shfl_xor((int)word, 2, kWave);
    if ((c & 3) == 0 && c < nchunks) sbm[c >> 2] = word;
  }
  __syncthreads();
  const int n = bitmap_prefix(sbm, spre, nwords, sred);
  const int64_t ld = ((int64_t)n + 31) / 32 * 32;
#pragma unroll 1
  for (int w = tid; w < nwords; w += kDcThreads) {
    uint32_t bits = sbm[w];
    int p = (int)spre[w];
    while (bits && p < kDcMaxOut) {
      s_cols[p++] = w * 32 + __builtin_ctz(bits);
      bits &= bits - 1;
    }
  }
  if (first) {
#pragma unroll 1
    for (int w = tid; w < nwords; w += kDcThreads) bitmap_g[w] = sbm[w];
    write_cols(sbm, spre, nwords, n, cols_g, n_g);
#pragma unroll 1
    for (int64_t i = tid; i < (int64_t)M * (ld - n); i += kDcThreads) {
      const int64_t m = i / (ld - n);
      Xo_g[m * ld + n + (i - m * (ld - n))] = 0;
    }
  }

  // ---- row absmax over the block, outlier elements masked out (branch-free,
  // from the thread's own flag bits): per thread, per wave (DPP), then the
  // four waves through LDS
  auto strip = [&](uint32_t bits, const uint4& t) -> uint4 {
    uint32_t h[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t b = bits >> (2 * q);
      h[q] &= ((b & 1u) ? 0u : 0x0000ffffu) | ((b & 2u) ? 0u : 0xffff0000u);
    }
    return make_uint4(h[0], h[1], h[2], h[3]);
  };
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < M) {
      u16x2 m2 = u16x2{0, 0};
#pragma unroll
      for (int j = 0; j < JC; ++j) {
        const uint4 t = strip(om[j], xr[m][j]);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
      }
      const uint32_t mx = wave_max_u32_dpp(m2[0] > m2[1] ? m2[0] : m2[1]);
      if (lane == 0) s_rmax[wave][m] = mx;
    }
  }
  __syncthreads();

  // ---- codes into LDS (block 0: also the workspace)
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < M) {
      uint32_t mx = s_rmax[0][m];
#pragma unroll
      for (int w = 1; w < kDcWaves; ++w) mx = mx > s_rmax[w][m] ? mx : s_rmax[w][m];
      const float a = h2f(mx);
      const float s = a != 0.0f ? 127.0f / a : 0.0f;
#pragma unroll
      for (int j = 0; j < JC; ++j) {
        const int c = tid + kDcThreads * j;
        if (c < nchunks) {
          const uint2 q = codes8_rne(strip(om[j], xr[m][j]), s);
          *reinterpret_cast<uint2*>(s_xq + m * ldx + c * 8) = q;
          if (first) *reinterpret_cast<uint2*>(Xq_g + (int64_t)m * K + c * 8) = q;
        }
      }
      if (tid == 0) {
        s_sx[m] = a;
        if (first) sx_g[m] = a;
      }
    }
  }

  // ---- outlier activations (a chunk with a set bit; rare), last: its loop
  // may wait for the weight loads, which the tiles wait for anyway
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    if (om[j]) {
      const int c = tid + kDcThreads * j;
      const int w = c >> 2, sh = 8 * (c & 3);
      const int pos0 = (int)spre[w] + __popc(sbm[w] & ((1u << sh) - 1u));
#pragma unroll 1
      for (int e = 0; e < 8; ++e) {
        if ((om[j] >> e) & 1u) {
          const int pos = pos0 + __popc(om[j] & ((1u << e) - 1u));
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            if (m < M) {
              // select from a copy: no dynamic index into the register array
              const uint4 t = xr[m][j];
              const uint32_t wd = (e >> 1) == 0 ? t.x : (e >> 1) == 1 ? t.y : (e >> 1) == 2 ? t.z : t.w;
              const uint16_t v = (uint16_t)((e & 1) ? (wd >> 16) : (wd & 0xffffu));
              if (pos < kDcMaxOut) s_xo[m][pos] = v;
              if (first) Xo_g[m * ld + pos] = v;
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- weight tiles
  const bool staged = n <= kDcMaxOut;
  const int jf = tid & 15, mt = tid >> 4;   // epilogue: feature jf, token mt
  bool first_tile = true;
  for (int64_t tile = blockIdx.x; tile * kDcFeat < N; tile += gridDim.x) {
    const int64_t f0 = tile * kDcFeat;
    const int rows_w = (int)min<int64_t>(kDcFeat, N - f0);
    if (!first_tile) {
      tile_rsrc(f0);
      load_w(wave);
    }
    first_tile = false;
    const int64_t f = f0 + jf;
    const bool f_ok = jf < rows_w;
    const float sw_f = f_ok ? sw[f] : 0.0f;
    const float bias_f = (bias && f_ok) ? h2f(bias[f]) : 0.0f;
    int qv[2] = {0, 0};
    if (staged && n > 0) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int t = (tid >> 4) + 16 * s2, j = tid & 15;
        if (t < n && j < rows_w) {
          const int64_t off = (f0 + j) * K + s_cols[t];
          qv[s2] = Wf ? (int)Wf[off] : (int)Wq[off];
        }
      }
    }

    v4i32 acc = v4i32{0, 0, 0, 0};
    const int8_t* xrow = s_xq + (r16 < M ? r16 : 0) * ldx;
    for (int c0 = wave; c0 < nkc; c0 += kDcWaves * kDcBatch) {
      if (c0 != wave) load_w(c0);
      v4i32 xf[kDcBatch][4];
#pragma unroll
      for (int b = 0; b < kDcBatch; ++b) {
        const int c = c0 + b * kDcWaves;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = c * kDcChunk + 64 * j + seg;
          const bool ok = r16 < M && c < nkc && k < K;
          const v4i32 v = *reinterpret_cast<const v4i32*>(xrow + (ok ? k : 0));
          xf[b][j] = ok ? v : v4i32{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int b = 0; b < kDcBatch; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[b][j], xf[b][j], acc, 0, 0, 0);
    }
    // D layout of the 16x16 MFMA: lane l, register r -> token l%16 (B
    // column), feature 4*(l/16) + r (A row).
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][(4 * (lane >> 4) + r) * 16 + r16] = acc[r];
    if (staged && n > 0) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int t = (tid >> 4) + 16 * s2, j = tid & 15;
        if (t < n && j < rows_w)
          s_wo[t][j] = Wf ? h2f((uint32_t)qv[s2]) : h2f(f2h(((float)qv[s2] * sw[f0 + j]) / 127.0f));
      }
    }
    __syncthreads();

    if (f_ok && mt < M) {
      int32_t acc_s = 0;
#pragma unroll
      for (int w = 0; w < kDcWaves; ++w) acc_s += red[w][jf * 16 + mt];
      const float fw = sw_f / 127.0f;
      const float y = (float)acc_s * (s_sx[mt] / 127.0f) * fw;
      float yo = 0.0f;
      if (staged) {
        for (int t = 0; t < n; ++t) yo += h2f(s_xo[mt][t]) * s_wo[t][jf];
      } else {
        // ascending outlier columns straight from the bitmap, X and W
        for (int w = 0; w < nwords; ++w) {
          uint32_t bits = sbm[w];
          while (bits) {
            const int k = w * 32 + __builtin_ctz(bits);
            bits &= bits - 1;
            const float wo = Wf ? h2f(Wf[f * K + k])
                                : h2f(f2h(((float)Wq[f * K + k] * sw_f) / 127.0f));
            yo += h2f(X[(int64_t)mt * K + k]) * wo;
          }
        }
      }
      Y[(int64_t)mt * N + f] = f2h(y + yo + bias_f);
    }
    __syncthreads();   // red and s_wo are rewritten by the next tile
  }
}

int g_cus = 0;

template <int MR, int JC>
hipError_t launch_decode_t(const uint16_t* X, const int8_t* Wq, const float* sw, int64_t M,
                           int64_t N, int64_t K, uint32_t tau16, const uint16_t* bias,
                           uint16_t* Y, const uint16_t* Wf, uint32_t* bitmap, int32_t* cols,
                           int32_t* n_out, float* sx, int8_t* Xq, uint16_t* Xo, hipStream_t s) {
  const int lds = dc_lds_bytes((int)M, (int)K);
  static bool lds_set = false;   // per instantiation: allow the largest dynamic LDS once
  if (!lds_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode_i8<MR, JC>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             dc_lds_bytes(MR, JC * kDcThreads * 8));
    if (e != hipSuccess) return e;
    lds_set = true;
  }
  if (g_cus == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    g_cus = cus;
  }
  // two blocks per CU while both fit in LDS (static part about 7.5 KiB)
  const int64_t per_cu = lds + 8 * 1024 <= 80 * 1024 ? 2 : 1;
  const int64_t tiles = (N + kDcFeat - 1) / kDcFeat;
  const int64_t blocks = std::min<int64_t>(tiles, per_cu * g_cus);
  hipLaunchKernelGGL((k_decode_i8<MR, JC>), dim3((unsigned)blocks), dim3(kDcThreads), (size_t)lds, s, X,
                     Wq, sw, (int)M, (int)N, (int)K, tau16, bias, Y, Wf, bitmap, cols, n_out, sx,
                     Xq, Xo);
  return hipGetLastError();
}

}  // namespace

bool decode_applies(int64_t M, int64_t K) {
  // a thread holds ceil(K / 2048) chunks of each of MR rows, MR * chunks <=
  // kDcXRegs: K <= 16384 for M <= 4, 8192 for M <= 8. Beyond 8 tokens the X
  // side, repeated by every block, costs more than the launches it saves.
  if (M < 1 || M > kDcMaxTok || K < 16) return false;
  const int64_t jc = (K + kDcThreads * 8 - 1) / (kDcThreads * 8);
  return jc <= (M <= 4 ? 8 : 4);
}

hipError_t launch_decode(const uint16_t* X, const int8_t* Wq, const float* sw, int64_t M,
                         int64_t N, int64_t K, uint32_t tau16, const uint16_t* bias, uint16_t* Y,
                         const uint16_t* Wf, uint32_t* bitmap, int32_t* cols, int32_t* n_out,
                         float* sx, int8_t* Xq, uint16_t* Xo, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int64_t jc = (K + kDcThreads * 8 - 1) / (kDcThreads * 8);   // chunks per row per thread
#define I8MM_DECODE(MR_, JC_)                                                                   \
  return launch_decode_t<MR_, JC_>(X, Wq, sw, M, N, K, tau16, bias, Y, Wf, bitmap, cols, n_out, \
                                   sx, Xq, Xo, s)
  if (M == 1) {
    if (jc <= 2) I8MM_DECODE(1, 2);
    if (jc <= 4) I8MM_DECODE(1, 4);
    I8MM_DECODE(1, 8);
  }
  if (M <= 4) {
    if (jc <= 2) I8MM_DECODE(4, 2);
    if (jc <= 4) I8MM_DECODE(4, 4);
    I8MM_DECODE(4, 8);
  }
  if (jc <= 2) I8MM_DECODE(8, 2);
  I8MM_DECODE(8, 4);
#undef I8MM_DECODE
}

}  // namespace i8mm
