// int8 GEMM with int32 accumulation on CDNA4 i8 MFMA, with the dequantize,
// fp16 outlier product and bias fused into the epilogue.
//
// Pages cited: [HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit
// Matrix Multiplication for transformers at scale using Hugging Face
// Transformers, Accelerate and bitsandbytes"; [Summary] paper summary page
// "LLM.int8(): 8-Bit Matrix Multiplication for Transformers at Scale".
//
// Y[i, j] = fp16( C[i, j] * (sx[i] / 127) * (sw[j] / 127)
//                 + sum_t Xo[i, t] * Wo[j, t] + bias[j] ),
// C[i, j] = sum_k Xq[i, k] * Wq[j, k]                     (exact int32)
// Wo[j, t] = fp16(fl32(fl32(Wq[j, cols[t]] * sw[j]) / 127))
//
// [Summary] "The full picture" step 3 (Int8 matmul, Int32 result,
// dequantized by the outer product of the scale vectors) and step 4 (add the
// 16-bit outlier product); [HF-blog] "Usage" (fp16 weight columns for the
// outlier matmul recovered as CB * SCB / 127, per output row).
//
// Mapping onto the matrix cores. Both operands are K-contiguous (Xq [M, K],
// Wq [N, K]). v_mfma_i32_32x32x32_i8 takes a 32 x 32-byte slice of each: the
// "A" operand is a 32-row slice of Wq (output features), the "B" operand a
// 32-row slice of Xq (tokens). A lane's 16 accumulators then hold 4 runs of 4
// consecutive output features of one token, so the fp16 result leaves as
// 8-byte stores along a row of Y. A and B fragments use the same lane -> k
// assignment, so the sum over k is the same whatever order the instruction
// uses inside its 32-byte slice (integer sums are exact).
//
// Block = 4 wavefronts in a 2 x 2 grid over a BN x BM (features x tokens)
// tile; K advances in 128-byte stages, double-buffered in LDS. Each LDS row
// is 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored at
// position c ^ (r & 7), so the 16-byte fragment reads of consecutive rows
// fall on different banks.

#include "device_common.h"
#include "launchers.h"

namespace i8mm {

namespace {

constexpr int kBK = 128;  // bytes of K per pipeline stage

template <int BM, int BN>
struct GemmCfg {
  static constexpr int WM = BM / 2;              // tokens per wave
  static constexpr int WN = BN / 2;              // features per wave
  static constexpr int TM = WM / 32;             // MFMA tiles per wave, token dim
  static constexpr int TN = WN / 32;             // MFMA tiles per wave, feature dim
  static constexpr int ROWS = BM + BN;           // LDS rows per stage (W rows first)
  static constexpr int CHUNKS = ROWS * (kBK / 16) / 256;  // 16-byte loads per thread
  static constexpr int STAGE_BYTES = ROWS * kBK;
  static_assert(TM >= 1 && TN >= 1, "tile too small");
  static_assert(ROWS * (kBK / 16) % 256 == 0, "loads must divide evenly");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

template <int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_i8(
    const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, const float* __restrict__ sx,
    const float* __restrict__ sw, int M, int N, int K, const uint16_t* __restrict__ Xo,
    const int32_t* __restrict__ cols, const int32_t* __restrict__ n_out,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C) {
  using Cfg = GemmCfg<BM, BN>;
  constexpr int WM = Cfg::WM, WN = Cfg::WN, TM = Cfg::TM, TN = Cfg::TN;
  __shared__ __attribute__((aligned(16))) int8_t lds[2 * Cfg::STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int l32 = lane & 31, lhi = lane >> 5;

  // ---- global -> register staging of one K stage
  uint4 stage[Cfg::CHUNKS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < Cfg::CHUNKS; ++i) {
      const int idx = tid + i * 256;
      const int r = idx >> 3, c = idx & 7;
      const int kk = k0 + c * 16;
      const int8_t* src;
      bool ok;
      if (r < BN) {
        const int64_t g = n0 + r;
        ok = g < N && kk < K;
        src = Wq + g * K + kk;
      } else {
        const int64_t g = m0 + (r - BN);
        ok = g < M && kk < K;
        src = Xq + g * K + kk;
      }
      stage[i] = ok ? ld16(src) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    int8_t* base = lds + buf * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Cfg::CHUNKS; ++i) {
      const int idx = tid + i * 256;
      const int r = idx >> 3, c = idx & 7;
      st16(base + swz(r, c), stage[i]);
    }
  };

  v16i32 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

  const int nk = (K + kBK - 1) / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const int8_t* base = lds + buf * Cfg::STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int chunk = ks * 2 + lhi;
      v4i32 fa[TN], fb[TM];
#pragma unroll
      for (int a = 0; a < TN; ++a)
        fa[a] = *reinterpret_cast<const v4i32*>(base + swz(wn * WN + a * 32 + l32, chunk));
#pragma unroll
      for (int b = 0; b < TM; ++b)
        fb[b] = *reinterpret_cast<const v4i32*>(base + swz(BN + wm * WM + b * 32 + l32, chunk));
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  // Lane (l32, lhi), accumulator r of tile (a, b):
  //   token   = m0 + wm*WM + b*32 + l32
  //   feature = n0 + wn*WN + a*32 + 8*(r/4) + 4*lhi + (r%4)
  const bool n4 = (N & 3) == 0;
  int64_t tok[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b) tok[b] = m0 + wm * WM + b * 32 + l32;

  if (C) {
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        if (tok[b] >= M) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t f = n0 + wn * WN + a * 32 + 8 * g + 4 * lhi;
          int32_t* dst = C + tok[b] * N + f;
          if (n4 && f + 3 < N) {
            *reinterpret_cast<int4*>(dst) =
                make_int4(acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                          acc[a][b][4 * g + 3]);
          } else {
            for (int e = 0; e < 4; ++e)
              if (f + e < N) dst[e] = acc[a][b][4 * g + e];
          }
        }
      }
  }
  if (!Y) return;

  float ax[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b) ax[b] = tok[b] < M ? sx[tok[b]] / 127.0f : 0.0f;

  v16f32 yf[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    float fw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t f = n0 + wn * WN + a * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
      fw[r] = f < N ? sw[f] / 127.0f : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) yf[a][b][r] = (float)acc[a][b][r] * ax[b] * fw[r];
  }

  // fp16 outlier product on v_mfma_f32_32x32x16_f16, 16 outlier columns per
  // step; A = recovered fp16 weight columns (32 features), B = gathered fp16
  // activations (32 tokens), same lane -> t assignment on both sides.
  const int n_o = (Xo && cols && n_out) ? *n_out : 0;
  if (n_o > 0) {
    const int64_t ldo = ((int64_t)n_o + 31) / 32 * 32;
    for (int t0 = 0; t0 < n_o; t0 += 16) {
      v8f16 wa[TN], xb[TM];
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int64_t f = n0 + wn * WN + a * 32 + l32;
        const float swf = f < N ? sw[f] : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = t0 + lhi * 8 + e;
          float w = 0.0f;
          if (t < n_o && f < N) {
            const float q = (float)Wq[f * K + cols[t]];
            w = (q * swf) / 127.0f;
          }
          wa[a][e] = (_Float16)w;
        }
      }
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        if (tok[b] < M) {
          uint4 raw = ld16(Xo + tok[b] * ldo + t0 + lhi * 8);
          xb[b] = __builtin_bit_cast(v8f16, raw);
        } else {
          xb[b] = v8f16{};
        }
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
          yf[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa[a], xb[b], yf[a][b], 0, 0, 0);
    }
  }

#pragma unroll
  for (int a = 0; a < TN; ++a) {
    float bv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t f = n0 + wn * WN + a * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
      bv[r] = (bias && f < N) ? h2f(bias[f]) : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      if (tok[b] >= M) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t f = n0 + wn * WN + a * 32 + 8 * g + 4 * lhi;
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = f2h(yf[a][b][4 * g + e] + bv[4 * g + e]);
        uint16_t* dst = Y + tok[b] * N + f;
        if (n4 && f + 3 < N) {
          *reinterpret_cast<uint2*>(dst) =
              make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        } else {
          for (int e = 0; e < 4; ++e)
            if (f + e < N) dst[e] = h[e];
        }
      }
    }
  }
}

template <int BM, int BN>
hipError_t launch_gemm_t(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                         int64_t M, int64_t N, int64_t K, const uint16_t* Xo, const int32_t* cols,
                         const int32_t* n_out, const uint16_t* bias, uint16_t* Y, int32_t* C,
                         hipStream_t s) {
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL((k_gemm_i8<BM, BN>), grid, dim3(256), 0, s, Xq, Wq, sx, sw, (int)M, (int)N,
                     (int)K, Xo, cols, n_out, bias, Y, C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                       int64_t M, int64_t N, int64_t K, const uint16_t* Xo, const int32_t* cols,
                       const int32_t* n_out, const uint16_t* bias, uint16_t* Y, int32_t* C,
                       hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  return launch_gemm_t<128, 128>(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_out, bias, Y, C, s);
}

}  // namespace i8mm
