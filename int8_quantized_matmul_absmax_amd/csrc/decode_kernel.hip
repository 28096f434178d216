// The whole few-token layer in one launch: outlier-column detection, row
// quantization of X, int8 matmul with int32 accumulation, dequantization,
// fp16 outlier product and bias, for 1 <= M <= 16 tokens. At these sizes the
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
// Block = 12 wavefronts in two roles. Waves 0-3 stream the block's 16-feature
// weight tiles straight from HBM into registers (in the operand layout of
// v_mfma_i32_16x16x64_i8: waves split K in 256-byte chunks) and run the
// MFMAs. Waves 4-11 do the X side and the epilogue. Every block does the X
// side itself (X is at most 16 x 4096 or 4 x 16384 fp16 and comes from L2): a weight
// wave is held up issuing its loads until the memory system takes them,
// about as long as the weight takes to stream, so an X side that shared its
// waves started only when the weight had almost landed. Split, it runs while
// the weight streams. The X waves' loads go out first (a barrier orders them
// before the weight loads); all barriers are LDS-only, so none waits for
// loads in flight. Eight X waves, two per SIMD, cover each other's latencies
// (4096 -> 4096: M = 1 8.0 -> 7.6 us, M = 4 10.9 -> 10.3 us against four).
// While the weight loads are being issued, the memory pipeline is full: an X
// wave that issued a load or store then would be held with them, so the X
// side touches memory only for X itself until it has the codes (by then the
// weight is on its way).
//
// X side: X-wave thread t holds the 16-byte chunks t, t + 512, ... of every
// token row in registers, so each 8-column flag mask is its own maximum over
// the rows, the outlier elements are masked out from its own bits, and the
// row maxima and outlier counts need one exchange between the eight X waves
// (through an LDS counter only they wait on; after it every X thread knows
// the row scales and its chunks' positions in the ascending outlier column
// list). The codes go to LDS. After the barrier that hands them to the
// weight waves, the blocks write the intermediates (bitmap, cols, n, sx,
// Xq, Xo) to the workspace from LDS, the codes shared out between blocks.
// Per tile, the X waves gather the tile's outlier weights (the first tile's
// requested just before that barrier) while the weight waves run the MFMAs
// (token fragments from the LDS codes, rows padded so the 16 token rows of
// one read hit distinct banks), the partial tiles meet in LDS, and the X
// waves write Y.

#include <atomic>
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launchers.h"

namespace i8mm {

namespace {

constexpr int kDcThreads = 768;             // 12 wavefronts
constexpr int kDcWWaves = 4;                // waves 0-3: weight tiles and MFMAs
constexpr int kDcXThreads = 512;            // waves 4-11: X side and epilogue
constexpr int kDcFeat = 16;                 // output features per tile
constexpr int kDcChunk = 256;               // K bytes per MFMA chunk
constexpr int kDcBatch = 4;                 // chunks per wave held in registers at once
constexpr int kDcMaxTok = 16;
constexpr int kDcMaxOut = 32;               // outlier columns staged in LDS
constexpr int kDcXRegs = 32;                // 16-byte X chunks an X thread holds
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

// int8 codes of 8 fp16 elements with the scale s, as the row quantizer forms
// them: y = fl32(x * s), then y + 1.5 * 2^23 rounds to the nearest integer
// with ties to even and its low byte is the two's complement code. The
// product is taken as fma(x, s, +0), one mixed-precision instruction that
// reads the fp16 half directly: x * s is exact before its one rounding
// either way, and a -0 product becoming +0 does not change the code. The
// last two byte permutes take their selectors from the caller (0x05040100
// keeps all four codes of a word; a selector byte 0x0c writes a zero code).
__device__ __forceinline__ uint2 dc_codes8(const uint4& t, float s, uint32_t sel_x,
                                           uint32_t sel_y) {
  const float magic = 12582912.0f;
  const uint32_t w[4] = {t.x, t.y, t.z, t.w};
  uint32_t r[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(w[q] & 0xffffu));
    const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(w[q] >> 16));
    r[2 * q] = __builtin_bit_cast(uint32_t, __builtin_fmaf((float)lo, s, 0.0f) + magic);
    r[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_fmaf((float)hi, s, 0.0f) + magic);
  }
  const uint32_t lo01 = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);
  const uint32_t lo23 = __builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(r[5], r[4], 0x0c0c0400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(r[7], r[6], 0x0c0c0400u);
  return make_uint2(__builtin_amdgcn_perm(lo23, lo01, sel_x),
                    __builtin_amdgcn_perm(hi23, hi01, sel_y));
}

// Maxima over the 64 lanes of a wave of V values per lane, all V at once.
// Each step pairs every lane with a partner and, while more than one value
// is left, halves the values a lane holds: by one lane bit it keeps the
// lower or the upper half and takes its partner's copy of the same half
// (V - 1 exchanges in all, where V separate reductions take 6 V). The
// pairings: lanes i and i ^ 32 (v_permlane32_swap), i and i ^ 16
// (v_permlane16_swap), then within each 16-lane row i and 15 - i
// (row_mirror), i and 7 - i within each 8 (row_half_mirror), i and i ^ 2,
// i and i ^ 1 (quad_perm). The halving steps take lane bits 5, 4, 3, 2 in
// that order; each later pairing keeps those bits (the mirrors flip only
// lower ones), so partners always hold the same values, and the lanes each
// step adds are new. Once one value is left the steps are plain maxima.
// Afterwards lane (64 / V) * r (and the lanes up to the next such one)
// holds the maximum of value r.
template <int V>
__device__ __forceinline__ void wave_max_transposed(uint32_t (&v)[V], int lane) {
  static_assert(V == 1 || V == 2 || V == 4 || V == 8 || V == 16, "values per lane");
  auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  constexpr int H1 = V / 2, H2 = V / 4, H3 = V / 8, H4 = V / 16;   // halves per step (0: plain)
  // lanes i and i ^ 32: after the swap the first result holds (own, partner)
  // of the lower value at the lower lanes, the second (partner, own) of the
  // upper value at the upper lanes
  if constexpr (H1 > 0) {
#pragma unroll
    for (int k = 0; k < H1; ++k) {
      const auto p = __builtin_amdgcn_permlane32_swap(v[k], v[k + H1], false, false);
      v[k] = umax(p[0], p[1]);
    }
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(v[0], v[0], false, false);
    v[0] = umax(p[0], p[1]);
  }
  // lanes i and i ^ 16, the same way on 16-lane rows
  if constexpr (H2 > 0) {
#pragma unroll
    for (int k = 0; k < H2; ++k) {
      const auto p = __builtin_amdgcn_permlane16_swap(v[k], v[k + H2], false, false);
      v[k] = umax(p[0], p[1]);
    }
  } else {
    const auto p = __builtin_amdgcn_permlane16_swap(v[0], v[0], false, false);
    v[0] = umax(p[0], p[1]);
  }
  // within 16 lanes through DPP: a halving step keeps half h by lane bit g
  // and sends the other half to the partner
  auto dpp_step = [&](auto ctrl_c, int g, auto h_c) __attribute__((always_inline)) {
    constexpr int ctrl = decltype(ctrl_c)::value, h = decltype(h_c)::value;
    if constexpr (h > 0) {
      const bool up = (lane >> g) & 1;
#pragma unroll
      for (int k = 0; k < h; ++k) {
        const uint32_t keep = up ? v[k + h] : v[k];
        const uint32_t send = up ? v[k] : v[k + h];
        v[k] = umax(keep, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, ctrl, 0xf, 0xf, false));
      }
    } else {
      v[0] = umax(v[0], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[0], ctrl, 0xf, 0xf, false));
    }
  };
  using ic = std::integral_constant<int, 0>;
  dpp_step(std::integral_constant<int, 0x140>{}, 3, std::integral_constant<int, H3>{});   // row_mirror
  dpp_step(std::integral_constant<int, 0x141>{}, 2, std::integral_constant<int, H4>{});   // row_half_mirror
  dpp_step(std::integral_constant<int, 0x4e>{}, 0, ic{});   // quad_perm [2,3,0,1]
  dpp_step(std::integral_constant<int, 0xb1>{}, 0, ic{});   // quad_perm [1,0,3,2]
}

// LDS row pitch of the int8 codes: K rounded up to 256 bytes, plus 16, so
// the 16 token rows of one fragment read hit distinct banks.
__host__ __device__ constexpr int dc_pitch(int K) { return (K + 255) / 256 * 256 + kDcPad; }

// Dynamic LDS: [codes M x pitch][bitmap].
__host__ __device__ constexpr int dc_lds_bytes(int M, int K) {
  return dc_round16(M * dc_pitch(K)) + 4 * ((K + 31) / 32);
}

// X thread t holds the 16-byte chunks t, t + 512, ... (JC of them, K <= JC *
// 4096) of each of the first MR token rows (M <= MR, MR * JC <= kDcXRegs);
// FULL: M == MR, so no loop over the rows needs a bound.
template <int MR, int JC, bool FULL>
__global__ __launch_bounds__(kDcThreads) void k_decode_i8(
    const uint16_t* __restrict__ X, const int8_t* __restrict__ Wq, const float* __restrict__ sw,
    int M, int N, int K, uint32_t tau16, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ Y, const uint16_t* __restrict__ Wf, uint32_t* __restrict__ bitmap_g,
    int32_t* __restrict__ cols_g, int32_t* __restrict__ n_g, float* __restrict__ sx_g,
    int8_t* __restrict__ Xq_g, uint16_t* __restrict__ Xo_g) {
  static_assert(MR * JC <= kDcXRegs && MR <= kDcMaxTok, "X chunks held per thread");
  constexpr int XW = kDcXThreads / kWave;   // X waves
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  __shared__ int32_t red[kDcWWaves][16 * 16];
  __shared__ __attribute__((aligned(16))) float s_wo[16][kDcMaxOut + 4];   // outlier weights, [j][t]
  __shared__ __attribute__((aligned(16))) uint16_t s_xo[kDcMaxTok][kDcMaxOut];   // outlier activations, [m][t]
  __shared__ float s_sx[kDcMaxTok];
  __shared__ int s_cols[kDcMaxOut];
  __shared__ int s_cnt[XW][JC];                     // outlier columns per X wave and j
  __shared__ uint32_t s_rmax[XW][kDcMaxTok];        // row maxima per X wave
  __shared__ int s_xsync;                           // X waves past their flags

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool wrole = wave < kDcWWaves;      // uniform per wave
  const int xt = tid - kDcWWaves * kWave;   // X-side thread index (X waves)
  const int xw = wave - kDcWWaves;          // X wave index (X waves)
  const int nchunks = K / 8;                // 16-byte chunks of a row
  const int nwords = (K + 31) / 32;
  const int ldx = dc_pitch(K);              // LDS row pitch of the codes (bytes)
  int8_t* s_xq = reinterpret_cast<int8_t*>(dsm);
  uint32_t* sbm = reinterpret_cast<uint32_t*>(dsm + dc_round16(M * ldx));
  const bool first = blockIdx.x == 0;
  const int jf = xt & 15, mt = xt >> 4;     // epilogue (X waves): feature jf, token mt

  const int nkc = (K + kDcChunk - 1) / kDcChunk;
  const int r16 = lane & 15;                 // weight row / token of the MFMA operands
  const int seg = (lane >> 4) * 16;          // this lane's 16 bytes of each 64-byte k-slice

  // The two roles run separate code between the same sequence of barriers:
  // B0 (the X loads are out), B2 (codes, row factors and staged outlier
  // columns), then two per tile (partial tiles and outlier weights in LDS;
  // LDS free again). Between B0 and B2 the X waves exchange their flag
  // words, counts and row maxima through a counter in LDS that only they
  // wait on, so they do not wait for the weight waves, which are held up
  // issuing their loads until the memory system takes them.
  if (wrole) {
    // ---- weight waves
    constexpr int kOob = 0x7ffffff0;
    v4i32 wf[kDcBatch][4];
    __amdgpu_buffer_rsrc_t rw;
    auto load_w = [&](int c0) {
#pragma unroll
      for (int b = 0; b < kDcBatch; ++b) {
        const int c = c0 + b * kDcWWaves;
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
    lds_only_barrier();   // B0
    tile_rsrc((int64_t)blockIdx.x * kDcFeat);
    load_w(wave);
    lds_only_barrier();   // B2
    for (int64_t tile = blockIdx.x; tile * kDcFeat < N; tile += gridDim.x) {
      v4i32 acc = v4i32{0, 0, 0, 0};
      const int8_t* xrow = s_xq + (r16 < M ? r16 : 0) * ldx;
      for (int c0 = wave; c0 < nkc; c0 += kDcWWaves * kDcBatch) {
        if (c0 != wave) load_w(c0);
        v4i32 xf[kDcBatch][4];
#pragma unroll
        for (int b = 0; b < kDcBatch; ++b) {
          const int c = c0 + b * kDcWWaves;
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
      // the next tile's weight is in flight during this tile's epilogue
      const int64_t next = tile + gridDim.x;
      if (next * kDcFeat < N) {
        tile_rsrc(next * kDcFeat);
        load_w(wave);
      }
      lds_only_barrier();   // partial tiles in LDS
      lds_only_barrier();   // the epilogue has read them
    }
    return;
  }

  // ---- X waves: X into registers
  // The X loads are unconditional (rows and chunks past the end are
  // clamped; clamped chunks are masked out of every use below, rows m >= M
  // are not used). The tile's factors are loaded per tile, the first tile's
  // once the X side is done: no wait before then covers them, and the
  // epilogue that needs them waits for the tile's weight anyway.
  uint4 xr[MR][JC];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int j = 0; j < JC; ++j) {
      const int c = min(xt + kDcXThreads * j, nchunks - 1);
      xr[m][j] = ld16(X + (int64_t)min(m, M - 1) * K + c * 8);
    }
  }
  float sw_f = 0.0f;
  uint32_t bias_h = 0;
  auto load_factors = [&](int64_t f0) {
    const uint32_t nf = (uint32_t)min<int64_t>(kDcFeat, N - f0);
    const __amdgpu_buffer_rsrc_t rs = dc_rsrc(sw + f0, nf * 4u);
    const __amdgpu_buffer_rsrc_t rb = dc_rsrc(bias ? bias + f0 : nullptr, bias ? nf * 2u : 0u);
    sw_f = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, jf * 4, 0, 0));
    bias_h = __builtin_amdgcn_raw_buffer_load_b16(rb, jf * 2, 0, 0);
  };
  if (xt == 0) s_xsync = 0;
  lds_only_barrier();   // B0

  // column flags (a thread holds whole columns, so each 8-column mask is its
  // own maximum over the rows; the four masks of a 32-column word are OR-ed
  // by shuffles), each thread's place in the ascending outlier list within
  // its wave, and the row maxima over the normal columns (outlier elements
  // masked out from the thread's own bits)
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  uint32_t om[JC];   // outlier bits of chunk j (bit e: element e)
  int excl[JC];      // outlier columns before chunk j's within the wave
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    const int c = xt + kDcXThreads * j;
    u16x2 mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = u16x2{0, 0};
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (FULL || m < M) {
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
    word = quad_or_dpp(word);
    if ((c & 3) == 0 && c < nchunks) {
      sbm[c >> 2] = word;
    }
    const int cnt = __popc(om[j]);
    const int incl = wave_inclusive_scan_dpp(cnt);
    excl[j] = incl - cnt;
    if (lane == kWave - 1) s_cnt[xw][j] = incl;
  }
  // per chunk: the magnitude bits of its normal elements (outlier elements
  // and sign bits cleared), and the code-packing selectors that write zero
  // codes at the outlier elements
  uint32_t amk[JC][4], bsel[JC][2];
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    const bool cv = xt + kDcXThreads * j < nchunks;   // not a clamped chunk
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t b = om[j] >> (2 * q);
      amk[j][q] = cv ? ((b & 1u) ? 0u : 0x00007fffu) | ((b & 2u) ? 0u : 0x7fff0000u) : 0u;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t k = 0x05040100u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((om[j] >> (4 * h + e)) & 1u) k = (k & ~(0xffu << (8 * e))) | (0x0cu << (8 * e));
      bsel[j][h] = k;
    }
  }
  // the row maxima of all MR rows reduced over the wave together (rows past
  // M hold a copy of row M - 1, from the clamped loads, and are not read)
  {
    uint32_t rv[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      u16x2 m2 = u16x2{0, 0};
#pragma unroll
      for (int j = 0; j < JC; ++j) {
        const uint32_t w[4] = {xr[m][j].x, xr[m][j].y, xr[m][j].z, xr[m][j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & amk[j][i]));
      }
      rv[m] = m2[0] > m2[1] ? m2[0] : m2[1];
    }
    wave_max_transposed<MR>(rv, lane);
    constexpr int kStride = kWave / MR;   // lane kStride * r holds row r
    if ((lane & (kStride - 1)) == 0) s_rmax[xw][lane / kStride] = rv[0];
  }
  // the X waves' exchange: each arrives once its LDS writes are done, and
  // waits until all eight have (every X wave reaches each exchange; the
  // counter only grows, so exchange e waits for e * 8 arrivals)
  auto x_exchange = [&](int e) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (lane == 0) __hip_atomic_fetch_add(&s_xsync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (__hip_atomic_load(&s_xsync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < e * XW)
      __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
  };
  x_exchange(1);

  // positions (chunk order: j, then X wave, then lane), codes, outlier
  // columns and activations
  int pos0[JC];
  int n = 0;
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < XW; ++w) {
      const int v = s_cnt[w][j];
      before += w < xw ? v : 0;
      tot += v;
    }
    pos0[j] = n + before + excl[j];
    n += tot;
  }
  const int64_t ld = ((int64_t)n + 31) / 32 * 32;
  // row factors: lane m of every X wave combines the X waves' maxima of row
  // m; each row's scale then comes from lane m (readlane), one division per
  // lane instead of one per row
  float sc_l = 0.0f;
  if (lane < M) {
    uint32_t mx = s_rmax[0][lane];
#pragma unroll
    for (int w = 1; w < XW; ++w) mx = mx > s_rmax[w][lane] ? mx : s_rmax[w][lane];
    const float a = h2f(mx);
    sc_l = a != 0.0f ? 127.0f / a : 0.0f;
    if (xw == 0) s_sx[lane] = a;
  }
  float scm[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m)
    scm[m] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_l), m));
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    const int c = xt + kDcXThreads * j;
    if (c < nchunks) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (FULL || m < M)
          *reinterpret_cast<uint2*>(s_xq + m * ldx + c * 8) =
              dc_codes8(xr[m][j], scm[m], bsel[j][0], bsel[j][1]);
      }
    }
  }
  // Element e (0..7) of a 16-byte chunk: v_perm_b32 picks bytes 2(e%4),
  // 2(e%4)+1 of words (x, y) and of (z, w), then e/4 chooses; no dynamic
  // index into the registers of X.
  auto pick_half = [](const uint4& t, int e) -> uint32_t {
    const uint32_t h = (uint32_t)(e & 3) * 2u;
    const uint32_t sel = 0x0c0c0000u | ((h + 1u) << 8) | h;
    const uint32_t p01 = __builtin_amdgcn_perm(t.y, t.x, sel);
    const uint32_t p23 = __builtin_amdgcn_perm(t.w, t.z, sel);
    return (e & 4) ? p23 : p01;
  };
#pragma unroll
  for (int j = 0; j < JC; ++j) {
    if (om[j]) {   // (rare) the set bits only
      const int c = xt + kDcXThreads * j;
      int pos = pos0[j];
      for (uint32_t bits = om[j]; bits; bits &= bits - 1u) {
        const int e = __builtin_ctz(bits);
        const int col = c * 8 + e;
        if (pos < kDcMaxOut) {
          s_cols[pos] = col;
#pragma unroll
          for (int m = 0; m < MR; ++m)
            if (FULL || m < M) s_xo[m][pos] = (uint16_t)pick_half(xr[m][j], e);
        } else if (first) {   // (more than fit in LDS)
          cols_g[pos] = col;
#pragma unroll
          for (int m = 0; m < MR; ++m)
            if (FULL || m < M) Xo_g[m * ld + pos] = (uint16_t)pick_half(xr[m][j], e);
        }
        ++pos;
      }
    }
  }
  // The first tile's factors and outlier weights are requested now, once
  // every outlier column is in LDS (a second exchange): the loads wait in
  // the memory pipeline behind the weight loads, as the weight waves do
  // before B2, and each gathered byte arrives with its own line of the
  // weight stream rather than after all of it.
  const bool staged = n <= kDcMaxOut;
  uint32_t raw[2] = {0u, 0u};
  auto gather_issue = [&](int64_t f0) {
    if (staged && n > 0 && xt < 256) {   // 16 features x up to 32 columns
      // bounded buffer loads; a slot past n or a row past N reads 0 and is
      // not stored
      const int rows_w = (int)min<int64_t>(kDcFeat, N - f0);
      const __amdgpu_buffer_rsrc_t rwo =
          Wf ? dc_rsrc(Wf + f0 * K, (uint32_t)rows_w * (uint32_t)K * 2u)
             : dc_rsrc(Wq + f0 * K, (uint32_t)rows_w * (uint32_t)K);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int t = mt + 16 * s2;
        const bool ok = t < n && jf < rows_w;
        const int off = ok ? jf * K + s_cols[t] : 0x3ffffff0;
        raw[s2] = Wf ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rwo, off * 2, 0, 0)
                     : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rwo, off, 0, 0);
      }
    }
  };
  x_exchange(2);
  load_factors((int64_t)blockIdx.x * kDcFeat);
  gather_issue((int64_t)blockIdx.x * kDcFeat);
  lds_only_barrier();   // B2

  // The workspace intermediates go out only now, from LDS: until the weight
  // waves have issued their loads, the memory pipeline is full and a store
  // holds its wave until it is taken. Every block holds the same codes, so
  // block b writes the code chunks c = b, b + G, ... of every row; block 0
  // writes the rest (the outlier columns and activations past the first 32
  // went out above).
  {
    const int G = gridDim.x, b = blockIdx.x;
    const int per = b < nchunks ? (nchunks - b + G - 1) / G : 0;
#pragma unroll 1
    for (int i = xt; i < M * per; i += kDcXThreads) {
      const int m = i / per, c = b + G * (i - m * per);
      *reinterpret_cast<uint2*>(Xq_g + (int64_t)m * K + c * 8) =
          *reinterpret_cast<const uint2*>(s_xq + m * ldx + c * 8);
    }
    if (first) {
#pragma unroll 1
      for (int w = xt; w < nwords; w += kDcXThreads) bitmap_g[w] = sbm[w];
      if (xt < M) sx_g[xt] = s_sx[xt];
      if (xt == 0) *n_g = n;
      const int ns = min(n, kDcMaxOut);
#pragma unroll 1
      for (int i = xt; i < M * ns; i += kDcXThreads) {
        const int m = i / ns, t = i - m * ns;
        if (m == 0) cols_g[t] = s_cols[t];
        Xo_g[m * ld + t] = s_xo[m][t];
      }
#pragma unroll 1
      for (int64_t i = xt; i < (int64_t)M * (ld - n); i += kDcXThreads) {
        const int64_t m = i / (ld - n);
        Xo_g[m * ld + n + (i - m * (ld - n))] = 0;
      }
    }
  }

  // per tile: the tile's outlier weights while the weight waves run the
  // MFMAs, then Y
  bool first_tile = true;
  for (int64_t tile = blockIdx.x; tile * kDcFeat < N; tile += gridDim.x) {
    const int64_t f0 = tile * kDcFeat;
    const int rows_w = (int)min<int64_t>(kDcFeat, N - f0);
    if (!first_tile) {
      load_factors(f0);
      gather_issue(f0);
    }
    first_tile = false;
    if (staged && n > 0 && xt < 256) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int t = mt + 16 * s2;
        if (t < n && jf < rows_w)
          s_wo[jf][t] = Wf ? h2f(raw[s2])
                           : h2f(f2h(((float)(int8_t)(uint8_t)raw[s2] * sw_f) / 127.0f));
      }
    }
    lds_only_barrier();   // partial tiles and outlier weights in LDS
    if (jf < rows_w && mt < M) {
      const int64_t f = f0 + jf;
      int32_t acc_s = 0;
#pragma unroll
      for (int w = 0; w < kDcWWaves; ++w) acc_s += red[w][jf * 16 + mt];
      const float fw = sw_f / 127.0f;
      const float y = (float)acc_s * (s_sx[mt] / 127.0f) * fw;
      float yo = 0.0f;
      if (staged) {
        // four columns per step (one read of each side), summed in order
        for (int t = 0; t < n; t += 4) {
          const uint2 xo4 = *reinterpret_cast<const uint2*>(&s_xo[mt][t]);
          const float4 wo4 = *reinterpret_cast<const float4*>(&s_wo[jf][t]);
          yo += h2f(xo4.x & 0xffffu) * wo4.x;
          if (t + 1 < n) yo += h2f(xo4.x >> 16) * wo4.y;
          if (t + 2 < n) yo += h2f(xo4.y & 0xffffu) * wo4.z;
          if (t + 3 < n) yo += h2f(xo4.y >> 16) * wo4.w;
        }
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
      Y[(int64_t)mt * N + f] = f2h(y + yo + h2f(bias_h));
    }
    lds_only_barrier();   // the next tile rewrites red and s_wo
  }
}

// One-time per-device state of the launcher. Concurrent first calls from
// several host threads may both set it; the values are the same, and the
// atomics make that benign.
constexpr int kDcMaxDevices = 64;
std::atomic<int> g_cus[kDcMaxDevices];

template <int MR, int JC, bool FULL>
hipError_t launch_decode_t(const uint16_t* X, const int8_t* Wq, const float* sw, int64_t M,
                           int64_t N, int64_t K, uint32_t tau16, const uint16_t* bias,
                           uint16_t* Y, const uint16_t* Wf, uint32_t* bitmap, int32_t* cols,
                           int32_t* n_out, float* sx, int8_t* Xq, uint16_t* Xo, hipStream_t s) {
  const int lds = dc_lds_bytes((int)M, (int)K);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int slot = dev >= 0 && dev < kDcMaxDevices ? dev : 0;
  // per instantiation and device: allow the largest dynamic LDS once
  static std::atomic<bool> lds_set[kDcMaxDevices];
  if (!lds_set[slot].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode_i8<MR, JC, FULL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            dc_lds_bytes(MR, JC * kDcXThreads * 8));
    if (e != hipSuccess) return e;
    lds_set[slot].store(true, std::memory_order_release);
  }
  int cus = g_cus[slot].load(std::memory_order_acquire);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    g_cus[slot].store(cus, std::memory_order_release);
  }
  // one block of eight waves per CU (two waves per SIMD); blocks beyond the
  // first round take further tiles in turn
  const int64_t tiles = (N + kDcFeat - 1) / kDcFeat;
  const int64_t blocks = std::min<int64_t>(tiles, cus);
  hipLaunchKernelGGL((k_decode_i8<MR, JC, FULL>), dim3((unsigned)blocks), dim3(kDcThreads), (size_t)lds,
                     s, X, Wq, sw, (int)M, (int)N, (int)K, tau16, bias, Y, Wf, bitmap, cols,
                     n_out, sx, Xq, Xo);
  return hipGetLastError();
}

}  // namespace

bool decode_applies(int64_t M, int64_t K) {
  // an X thread holds ceil(K / 4096) chunks of each of MR rows: K <= 16384
  // for M <= 4, 8192 for M <= 8, 4096 for M <= 16. Every block repeats the
  // X side, so it grows with M; at 16 tokens (4096 -> 4096) one launch
  // takes 11.2 us against 14.9 us for the separate kernels (12 tokens: 10.4
  // against 14.3 us).
  if (M < 1 || M > kDcMaxTok || K < 16) return false;
  const int64_t jc = (K + kDcXThreads * 8 - 1) / (kDcXThreads * 8);
  return jc <= (M <= 4 ? 4 : M <= 8 ? 2 : 1);
}

hipError_t launch_decode(const uint16_t* X, const int8_t* Wq, const float* sw, int64_t M,
                         int64_t N, int64_t K, uint32_t tau16, const uint16_t* bias, uint16_t* Y,
                         const uint16_t* Wf, uint32_t* bitmap, int32_t* cols, int32_t* n_out,
                         float* sx, int8_t* Xq, uint16_t* Xo, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  // chunks per row per X thread
  const int64_t jc = (K + kDcXThreads * 8 - 1) / (kDcXThreads * 8);
#define I8MM_DECODE(MR_, JC_, FULL_)                                                        \
  return launch_decode_t<MR_, JC_, FULL_>(X, Wq, sw, M, N, K, tau16, bias, Y, Wf, bitmap, cols, \
                                          n_out, sx, Xq, Xo, s)
#define I8MM_DECODE_MR(MR_, JC_)            \
  do {                                      \
    if (M == MR_) I8MM_DECODE(MR_, JC_, true); \
    I8MM_DECODE(MR_, JC_, false);           \
  } while (0)
  if (M == 1) {
    if (jc <= 1) I8MM_DECODE(1, 1, true);
    if (jc <= 2) I8MM_DECODE(1, 2, true);
    I8MM_DECODE(1, 4, true);
  }
  if (M <= 4) {
    if (jc <= 1) I8MM_DECODE_MR(4, 1);
    if (jc <= 2) I8MM_DECODE_MR(4, 2);
    I8MM_DECODE_MR(4, 4);
  }
  if (M <= 8) {
    if (jc <= 1) I8MM_DECODE_MR(8, 1);
    I8MM_DECODE_MR(8, 2);
  }
  I8MM_DECODE_MR(16, 1);
#undef I8MM_DECODE_MR
#undef I8MM_DECODE
}

}  // namespace i8mm
