// Few-token (decode) form of the int8 matmul with the fused dequantize,
// outlier product and bias: the same result as the tiled GEMM, shaped for
// M <= 64 tokens, where the layer is bound by streaming the int8 weight
// from HBM once.
//
// Pages cited: [HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit
// Matrix Multiplication for transformers at scale using Hugging Face
// Transformers, Accelerate and bitsandbytes"; [Summary] paper summary page
// "LLM.int8(): 8-Bit Matrix Multiplication for Transformers at Scale".
//
// Y[i, j] = fp16( C[i, j] * (sx[i] / 127) * (sw[j] / 127)
//                 + sum_t Xo[i, t] * Wo[j, t] + bias[j] ),
// C[i, j] = sum_k Xq[i, k] * Wq[j, k]                     (exact int32)
// Wo[j, t] = fp16(fl32(fl32(Wq[j, cols[t]] * sw[j]) / 127)), or Wf[j, cols[t]]
// when the fp16 weight Wf is given
// ([Summary] "The full picture" steps 3-4; [HF-blog] "Usage": outlier weight
// columns recovered from CB * SCB / 127, per output row, when the module holds
// only the int8 weight; the fp16 weight's own columns when it keeps one.)
//
// One block of 4 wavefronts per 16 output features; the waves split K in
// 256-byte chunks (chunk c goes to wave c % 4). A chunk is four 64-byte
// k-slices; for slice j, lane l loads k = chunk*256 + 64j + 16*(l/16) + 0..15
// of weight row l%16 and of token row l%16 straight into registers (buffer
// loads; each instruction reads 64 contiguous bytes of 16 rows, the next one
// the other half of those lines), which is the operand layout of
// v_mfma_i32_16x16x64_i8, so slice j feeds MFMA j directly and exactly. All
// of a wave's weight loads are issued before its first MFMA, so the whole
// weight is in flight at once across the chip. Tokens go in groups of 16 (the
// MFMA's B width); the weight fragments stay in registers across groups.
// The four waves' int32 partial tiles are summed through LDS, then each
// thread finishes (token, feature) outputs: dequantize, outlier product in
// fp32 from the gathered int8 weight columns (fetched at kernel start and
// staged in LDS for up to 32 outlier columns), bias, fp16 store.

#include "device_common.h"
#include "launchers.h"

namespace i8mm {

namespace {

constexpr int kGvThreads = 256;
constexpr int kGvWaves = kGvThreads / 64;
constexpr int kGvFeat = 16;            // output features per block
constexpr int kGvChunk = 256;          // K bytes per chunk
constexpr int kGvBatch = 4;            // chunks per wave held in registers at once
constexpr int kGvMaxTok = 64;          // largest M this kernel takes
constexpr int kGvGroups = kGvMaxTok / 16;
constexpr int kGvMaxOut = 32;          // outlier columns staged in LDS

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gv_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

__device__ __forceinline__ v4i32 gv_load(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(v4i32, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <bool WITH_C>
__global__ __launch_bounds__(kGvThreads) void k_gemv_i8(
    const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, const float* __restrict__ sx,
    const float* __restrict__ sw, int M, int N, int K, const uint16_t* __restrict__ Xo,
    const int32_t* __restrict__ cols, const int32_t* __restrict__ n_out,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C,
    const uint16_t* __restrict__ Wf) {
  __shared__ int32_t red[kGvWaves][kGvGroups][16 * 16];
  __shared__ float s_wo[kGvMaxOut][16];          // outlier weights, [t][j]
  __shared__ uint16_t s_xo[kGvMaxTok][kGvMaxOut]; // gathered activations, [m][t]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t f0 = (int64_t)blockIdx.x * kGvFeat;
  const int rows_w = (int)min<int64_t>(kGvFeat, N - f0);
  const int groups = (M + 15) / 16;

  // Buffer descriptors: reads past the valid rows return 0.
  const __amdgpu_buffer_rsrc_t rw = gv_rsrc(Wq + f0 * K, (uint32_t)rows_w * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rx = gv_rsrc(Xq, (uint32_t)M * (uint32_t)K);
  const int r16 = lane & 15;           // weight row / token within the group
  const int seg = (lane >> 4) * 16;    // this lane's 16 bytes of each 64-byte k-slice
  constexpr int kOob = 0x7ffffff0;     // an offset past every descriptor's range

  // Phase 1, small loads with no dependence on anything: the first outlier
  // column indices of this thread's two outlier slots, this thread's output
  // factors (feature tid % 16, tokens tid / 16 + 16 i), the outlier count.
  // They are issued before the weight stream, so waiting for them later does
  // not wait for the stream (vector loads complete in issue order).
  // (Branch-free buffer loads: a disabled or out-of-range element reads 0.)
  const bool has_o = Xo && cols && n_out && Y;
  const __amdgpu_buffer_rsrc_t rc =
      gv_rsrc(has_o ? (const void*)cols : (const void*)Wq, has_o ? (uint32_t)min(K, 32) * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rsw = gv_rsrc(sw + f0, (uint32_t)rows_w * 4u);
  const __amdgpu_buffer_rsrc_t rb =
      gv_rsrc(bias ? (const void*)(bias + f0) : (const void*)Wq, (bias && Y) ? (uint32_t)rows_w * 2u : 0u);
  const __amdgpu_buffer_rsrc_t rsx = gv_rsrc(sx, Y ? (uint32_t)M * 4u : 0u);
  int cidx[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    cidx[s2] = __builtin_amdgcn_raw_buffer_load_b32(rc, ((tid >> 4) + 16 * s2) * 4, 0, 0);
  const int jf = tid & 15;
  const int64_t f = f0 + jf;
  const bool f_ok = f < N;
  const float sw_f = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsw, jf * 4, 0, 0));
  const float bias_f = h2f(__builtin_amdgcn_raw_buffer_load_b16(rb, jf * 2, 0, 0));
  float sx_m[kGvMaxTok / 16];
#pragma unroll
  for (int i = 0; i < kGvMaxTok / 16; ++i)
    sx_m[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            rsx, ((tid >> 4) + 16 * i) * 4, 0, 0));
  const int n_o = has_o ? __builtin_amdgcn_readfirstlane(*n_out) : 0;
  const int64_t ldo = ((int64_t)n_o + 31) / 32 * 32;
  const bool staged = n_o <= kGvMaxOut;

  // Phase 2, the weight stream of this wave's first batch of chunks.
  const int nchunks = (K + kGvChunk - 1) / kGvChunk;
  v4i32 wf[kGvBatch][4];
  auto load_w = [&](int c0) {
#pragma unroll
    for (int b = 0; b < kGvBatch; ++b) {
      const int c = c0 + b * kGvWaves;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = c * kGvChunk + 64 * j + seg;
        wf[b][j] = gv_load(rw, (c < nchunks && k < K) ? r16 * K + k : kOob);
      }
    }
  };
  load_w(wave);
  __builtin_amdgcn_sched_barrier(0);

  // Phase 3, outlier part for up to kGvMaxOut columns: the weight bytes
  // Wq[f0 + j, cols[t]] (or the fp16 weights Wf[f0 + j, cols[t]] when the
  // layer keeps them) and the gathered activations Xo[m, t]; they reach LDS
  // after the main loop. More columns take the slow path in the epilogue.
  int qv[2] = {0, 0};
  uint4 xv = make_uint4(0, 0, 0, 0);
  if (staged && n_o > 0) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int t = (tid >> 4) + 16 * s2, j = tid & 15;
      if (t < n_o && j < rows_w)
        qv[s2] = Wf ? (int)Wf[(f0 + j) * K + cidx[s2]] : (int)Wq[(f0 + j) * K + cidx[s2]];
    }
    const int m = tid >> 2;
    if (m < M) xv = ld16(Xo + m * ldo + 8 * (tid & 3));
  }

  v4i32 acc[kGvGroups];
#pragma unroll
  for (int g = 0; g < kGvGroups; ++g) acc[g] = v4i32{0, 0, 0, 0};

  for (int c0 = wave; c0 < nchunks; c0 += kGvWaves * kGvBatch) {
    if (c0 != wave) load_w(c0);
#pragma unroll
    for (int g = 0; g < kGvGroups; ++g) {
      if (g >= groups) break;
      const int tok = g * 16 + r16;
      v4i32 xf[kGvBatch][4];
#pragma unroll
      for (int b = 0; b < kGvBatch; ++b) {
        const int c = c0 + b * kGvWaves;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = c * kGvChunk + 64 * j + seg;
          xf[b][j] = gv_load(rx, (c < nchunks && k < K && tok < M) ? tok * K + k : kOob);
        }
      }
      // every load of the batch is issued before the first MFMA waits on one
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < kGvBatch; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[b][j], xf[b][j], acc[g], 0, 0, 0);
    }
  }

  // D layout of the 16x16 MFMA: lane l, register r -> token l%16 (B column),
  // feature 4*(l/16) + r (A row).
#pragma unroll
  for (int g = 0; g < kGvGroups; ++g) {
    if (g >= groups) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][g][(4 * (lane >> 4) + r) * 16 + r16] = acc[g][r];
  }
  if (staged && n_o > 0) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int t = (tid >> 4) + 16 * s2, j = tid & 15;
      if (t < n_o && j < rows_w)
        s_wo[t][j] = Wf ? h2f((uint32_t)qv[s2]) : h2f(f2h(((float)qv[s2] * sw[f0 + j]) / 127.0f));
    }
    const int m = tid >> 2;
    if (m < M) st16(&s_xo[m][8 * (tid & 3)], xv);
  }
  __syncthreads();

  if (!f_ok) return;
  const float fw = sw_f / 127.0f;
  const float swf = sw_f;
  const float bv = bias_f;
#pragma unroll
  for (int i = 0; i < kGvMaxTok / 16; ++i) {
    const int m = (tid >> 4) + 16 * i;
    if (m >= M) break;
    const int g = m >> 4, t16 = m & 15;
    int32_t s = 0;
#pragma unroll
    for (int w = 0; w < kGvWaves; ++w) s += red[w][g][jf * 16 + t16];
    if (WITH_C) C[(int64_t)m * N + f] = s;
    if (!Y) continue;
    float y = (float)s * (sx_m[i] / 127.0f) * fw;
    float yo = 0.0f;
    if (staged) {
      for (int t = 0; t < n_o; ++t) yo += h2f(s_xo[m][t]) * s_wo[t][jf];
    } else {
      for (int t = 0; t < n_o; ++t) {
        const float wo = Wf ? h2f(Wf[f * K + cols[t]])
                            : h2f(f2h(((float)Wq[f * K + cols[t]] * swf) / 127.0f));
        yo += h2f(Xo[m * ldo + t]) * wo;
      }
    }
    Y[(int64_t)m * N + f] = f2h(y + yo + bv);
  }
}

}  // namespace

bool gemv_applies(int64_t M) { return M > 0 && M <= kGvMaxTok; }

hipError_t launch_gemv(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                       int64_t M, int64_t N, int64_t K, const uint16_t* Xo, const int32_t* cols,
                       const int32_t* n_out, const uint16_t* bias, uint16_t* Y, int32_t* C,
                       const uint16_t* Wf, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((N + kGvFeat - 1) / kGvFeat);
  if (C)
    hipLaunchKernelGGL(k_gemv_i8<true>, dim3(blocks), dim3(kGvThreads), 0, s, Xq, Wq, sx, sw,
                       (int)M, (int)N, (int)K, Xo, cols, n_out, bias, Y, C, Wf);
  else
    hipLaunchKernelGGL(k_gemv_i8<false>, dim3(blocks), dim3(kGvThreads), 0, s, Xq, Wq, sx, sw,
                       (int)M, (int)N, (int)K, Xo, cols, n_out, bias, Y, C, Wf);
  return hipGetLastError();
}

}  // namespace i8mm
