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
// Wo[j, t] = fp16(fl32(fl32(Wq[j, cols[t]] * sw[j]) / 127)),
//            or Wf[j, cols[t]] when the fp16 weight Wf is given
//
// [Summary] "The full picture" step 3 (Int8 matmul, Int32 result,
// dequantized by the outer product of the scale vectors) and step 4 (add the
// 16-bit outlier product); [HF-blog] "Usage" (fp16 weight columns for the
// outlier matmul recovered as CB * SCB / 127, per output row, when the module
// holds only the int8 weight; taken from the fp16 weight when it keeps one).
//
// Mapping onto the matrix cores. Both operands are K-contiguous (Xq [M, K],
// Wq [N, K]). v_mfma_i32_32x32x32_i8 takes a 32 x 32-byte slice of each: the
// "A" operand is a 32-row slice of Wq (output features), the "B" operand a
// 32-row slice of Xq (tokens). A lane's 16 accumulators then hold 4 runs of 4
// consecutive output features of one token. A and B fragments use the same
// lane -> k assignment, so the sum over k is the same whatever order the
// instruction uses inside its 32-byte slice (integer sums are exact).
//
// Block = 8 wavefronts, two per SIMD, in a 2 x 4 grid over a BN x BM
// (features x tokens) tile; each wave owns a (BN/2) x (BM/4) sub-tile (4 x 2
// MFMA tiles of 32 x 32 for 256 x 256, 128 accumulator registers), so while
// one wave of a SIMD waits on LDS or a barrier the other issues MFMAs. Small
// grids (fewer 256 x 256 tiles than CUs) use 128 x 128 tiles of 4 waves.
// K advances in BK = 64-byte stages through a ring of five LDS buffers (all
// of LDS) filled by direct-to-LDS buffer loads (no register staging). Rows
// past M / N and chunks past K are loaded through an out-of-range offset,
// which the buffer descriptor turns into zeros.
//
// Main loop, step k: wait until stage k+1 has landed, workgroup barrier (stage
// k+1 visible to every wave; every wave is done reading stage k), issue half
// of the loads of stages k+4 and k+5 (even k) or the other half (odd k), the
// same rows of both back to back so each operand row is fetched as a whole
// 128-byte line, then the fragment reads of stage k+1 into one register set
// interleaved with the MFMAs of stage k from the other set, so LDS traffic is
// spread over the MFMA phase instead of bursting after each barrier.
//
// LDS layout of one stage: rows of BK = 64 bytes (Wq rows first, then Xq
// rows); 16-byte chunk c of row r sits at position c ^ f(r), f(r) =
// (r >> 2) & 3. A fragment read (lane l < 32 at row l, lane l + 32 at the
// same row, next chunk) then completes in the minimum number of LDS cycles;
// the bank-conflict counter reads zero for it, as it does for 16-byte reads
// of consecutive addresses. Measured alternatives: with no swizzle such a
// read takes 3.9x the cycles; with f(r) = ((r >> 1) ^ (r >> 3)) & 3 it takes
// 1.95x. The layout only permutes which chunk each lane's DMA load fetches:
// every row is still read as one 64-byte segment and written to LDS in order.
//
// Epilogue: per-tile dequantization with the row / column factors staged in
// LDS; the fp16 outlier product (first 16 outlier columns: gathered in the
// prologue, held in registers through the main loop, then staged in LDS;
// further columns read per 16-column step) runs on v_mfma_f32_32x32x16_f16
// onto the dequantized tile; lane swaps
// (v_permlane32_swap) and a pass through LDS turn each pair of 32-feature
// slices into whole 128-byte row segments of Y per 8 lanes.
//
// Tile order: blocks are dealt to the 8 XCDs round-robin by block id; the id
// is remapped so each XCD owns a contiguous range of tiles, rastered in groups
// of 4 token-tiles per weight-tile column, so blocks running together on one
// XCD share their Wq and Xq panels in that XCD's L2. (Groups of 4 against 8:
// 3.5% faster at 2048 x 4096 -> 16384, 0.6% at 4096 x 12288 -> 49152, even
// on the 1024-token shapes; groups of 2 or 16 were slower.)

#include <type_traits>

#include "device_common.h"
#include "launchers.h"

namespace i8mm {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;


// WAVES_M x 2 wavefronts per block (WAVES_M = 2: one per SIMD, each wave
// 128 x 128 of a 256 x 256 tile; WAVES_M = 4: two per SIMD, 64 x 128 each).
template <int BM_, int BN_, int BK_, int STAGES_, int WAVES_M_ = 2>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = 2, WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WAVES_M;           // tokens per wave
  static constexpr int WN = BN / WAVES_N;           // features per wave
  static constexpr int TM = WM / 32;                // MFMA tiles per wave, token dim
  static constexpr int TN = WN / 32;                // MFMA tiles per wave, feature dim
  static constexpr int KS = BK / 32;                // MFMA k-steps per stage
  static constexpr int CPR = BK / 16;               // 16-byte chunks per LDS row
  static constexpr int ROWS = BM + BN;              // LDS rows per stage
  static constexpr int STAGE_BYTES = ROWS * BK;
  static constexpr int ROWS_PER_LOAD = 64 / CPR;    // rows one wave-wide load fills
  static constexpr int LOADS = ROWS / ROWS_PER_LOAD / WAVES;  // loads per wave per stage
  static constexpr int NREADS = KS * (TN + TM);     // fragment reads per stage
  static constexpr int NMFMA = KS * TN * TM;        // MFMAs per stage
  // LDS: STAGES stage buffers; after the main loop the same bytes hold the
  // epilogue's [scales][outlier tiles][output staging].
  static constexpr int STAGE0 = 0;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int SCALE_BYTES = (BM + 2 * BN) * 4;
  static constexpr int OUTL0 = SCALE_BYTES;
  static constexpr int OUTL_BYTES = (BN + BM) * 16 * 2;
  static constexpr int OUT_ROW = 64 * 2 + 16;
  static constexpr int OUT0 = (OUTL0 + OUTL_BYTES + 1023) / 1024 * 1024;
  static_assert(OUT0 + WAVES * WM * OUT_ROW <= LDS_BYTES, "epilogue views fit the stages");
  static_assert(CPR == 4, "swizzle is written for 4 chunks per row");
  static_assert(BN % (4 * ROWS_PER_LOAD) == 0 && BM % (4 * ROWS_PER_LOAD) == 0, "split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(NMFMA % LOADS == 0 && NREADS % LOADS == 0, "interleave");
};

__device__ __forceinline__ int swz_key(int r) { return (r >> 2) & 3; }

// Buffer descriptor over [base, base + bytes); reads past `bytes` return 0.
// The fields go through readfirstlane so the descriptor lives in SGPRs (the
// callers pass wave-uniform values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS: wait for this wave's LDS operations (an explicit
// lgkmcnt(0) the compiler accounts for), barrier, then an acquire fence on LDS
// so later LDS accesses stay after it. A release fence is not used: it would
// also wait for every in-flight LDS-DMA load, which the explicit vmcnt waits
// already order.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Token tile / feature tile of this block: XCD-contiguous id, then grouped
// raster (GROUP token-tiles per feature-tile column).
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int XCDS = 8, GROUP = 4;
  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int per = T / XCDS, rem = T % XCDS;
  const int xcd = b % XCDS, slot = b / XCDS;
  const int t = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int span = GROUP * tiles_n;
  const int g = t / span;
  const int first_m = g * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int in = t - g * span;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// Kernel modes, separate instantiations so that each carries only its code
// (register pressure):
//   kPlain   fp16 output; outlier product in the epilogue. Given Wo, it
//            returns at once when there are more than 16 outlier columns
//            (kOutlierSeg does those).
//   kInt32   kPlain that also writes the raw int32 accumulators (parity mode).
//   kOutlierSeg  only for more than 16 outlier columns with Wo given
//            (returns at once otherwise): the outlier product as a second
//            main-loop segment.
enum GemmMode { kPlain = 0, kInt32 = 1, kOutlierSeg = 2 };
template <class Cfg, int MODE>
__global__ __launch_bounds__(Cfg::THREADS) void k_gemm_i8(
    const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, const float* __restrict__ sx,
    const float* __restrict__ sw, int M, int N, int K, const uint16_t* __restrict__ Xo,
    const int32_t* __restrict__ cols, const int32_t* __restrict__ n_out,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C,
    const uint16_t* __restrict__ Wo, const uint16_t* __restrict__ Wf) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, STAGES = Cfg::STAGES;
  constexpr int WM = Cfg::WM, WN = Cfg::WN, TM = Cfg::TM, TN = Cfg::TN, KS = Cfg::KS;
  constexpr int LOADS = Cfg::LOADS, RPL = Cfg::ROWS_PER_LOAD;
  __shared__ __attribute__((aligned(1024))) int8_t lds[Cfg::LDS_BYTES];
  float* s_ax = reinterpret_cast<float*>(lds);          // sx[m] / 127
  float* s_fw = s_ax + BM;                               // sw[n] / 127
  float* s_bias = s_fw + BN;                             // bias[n]
  int8_t* stages = lds + Cfg::STAGE0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wn = wave % Cfg::WAVES_N, wm = wave / Cfg::WAVES_N;
  const int l32 = lane & 31, lhi = lane >> 5;

  int tile_m, tile_n;
  tile_of_block((M + BM - 1) / BM, (N + BN - 1) / BN, tile_m, tile_n);
  const int64_t m0 = (int64_t)tile_m * BM;
  const int64_t n0 = (int64_t)tile_n * BN;

  // ---- outlier columns, 16 at a time: the recovered fp16 weight columns of
  // this block's BN features and the gathered fp16 activations of its BM
  // tokens are staged in LDS for the epilogue. Chunk 0 is held in registers
  // until the main loop has freed LDS: its activations are read in the
  // prologue, between the stage loads; its int8 weight codes are picked out
  // of the stage buffers as the main loop streams Wq through LDS (the fp16
  // weight's own values, with Wf given, are read in the prologue). Further
  // chunks (more than 16 outlier columns) are read in the epilogue.
  const int n_o = (Xo && cols && n_out && Y) ? *n_out : 0;
  const int64_t ldo = ((int64_t)n_o + 31) / 32 * 32;
  // More than 16 outlier columns with the recovered weights materialized (Wo
  // [N, ldo] fp16): the outlier product runs as a second main-loop segment
  // over the outlier columns (fp16 MFMA on Wo and Xo through the same stage
  // pipeline) instead of in the epilogue.
  constexpr bool WITH_C = MODE == kInt32;
  const bool many = Wo != nullptr && n_o > 16;
  if (MODE == kOutlierSeg ? !many : many) return;   // the other mode's case
  constexpr bool seg2 = MODE == kOutlierSeg;
  uint16_t* s_wo = reinterpret_cast<uint16_t*>(lds + Cfg::OUTL0);   // [BN][16]
  uint16_t* s_xo = s_wo + BN * 16;                                  // [BM][16]
  // Values held in registers from the prologue to the end of the main loop
  // (the stage buffers fill all of LDS until then), split so that no thread
  // holds more than ten: thread tid < BM keeps token m0 + tid's gathered
  // outlier activations (keep[0..7]) and factor (keep[8]); thread BM + f
  // keeps feature n0 + f's outlier weights (keep[0..3]: int8 codes, four per
  // register; keep[0..7] with the weight kept in fp16, Wf given: the fp16
  // values themselves), factor (keep[8]) and bias (keep[9]).
  static_assert(BM + BN <= Cfg::THREADS, "one held row per thread");
  const bool tok_side = tid < BM;   // uniform per wave
  const int hr = tok_side ? tid : tid - BM;
  const bool h_ok = tok_side ? m0 + hr < M : (hr < BN && n0 + hr < N);
  uint32_t keep[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) keep[i] = 0;
  auto fetch_outliers = [&]() {
    if (!h_ok) return;
    if (tok_side) {
      const uint16_t* src = Xo + (m0 + hr) * ldo;
      const uint4 x0 = ld16(src), x1 = ld16(src + 8);
      keep[0] = x0.x; keep[1] = x0.y; keep[2] = x0.z; keep[3] = x0.w;
      keep[4] = x1.x; keep[5] = x1.y; keep[6] = x1.z; keep[7] = x1.w;
    } else if (Wf) {
      const uint16_t* row = Wf + (n0 + hr) * K;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        // cols[t] is the same for every lane (a scalar load)
        const int c = t < n_o ? __builtin_amdgcn_readfirstlane(cols[t]) : 0;
        const uint32_t h = t < n_o ? (uint32_t)row[c] : 0u;
        keep[t / 2] |= h << (16 * (t % 2));
      }
    }
  };
  // The int8 weight codes of chunk 0 come from the stage buffers: while the
  // stage holding k-block kb (Wq[n0 .. n0+BN), columns kb*BK ..) is resident,
  // thread BM + f reads its row's byte of every outlier column in it. A gather
  // from Wq in memory instead would fetch a separate line for every (row,
  // column) and hold up the prologue. The columns are ascending and the
  // k-blocks come in order, so two uniform values track them: pt, the number
  // picked so far, and pc, the next one's column (INT_MAX after the last),
  // read with a scalar load as soon as the previous one is picked. A step
  // without an outlier column costs one scalar compare.
  const bool pick_w = !seg2 && Wf == nullptr && n_o > 0;
  const int n_pick = pick_w ? min(n_o, 16) : 0;
  int pt = 0;
  int pc = n_pick > 0 ? cols[0] : INT_MAX;
  auto pick_stage = [&](int kb) __attribute__((always_inline)) {
    while (pc < (kb + 1) * BK) {
      if (!tok_side) {
        const int o = pc - kb * BK;   // byte in the row's k-block
        const int8_t* row = stages + (kb % STAGES) * Cfg::STAGE_BYTES + hr * BK;
        const uint32_t q = (uint8_t)row[(((o >> 4) ^ swz_key(hr)) << 4) + (o & 15)];
        const uint32_t qs = q << (8 * (pt & 3));
#pragma unroll
        for (int i = 0; i < 4; ++i) keep[i] |= (pt >> 2) == i ? qs : 0u;
      }
      ++pt;
      pc = pt < n_pick ? cols[min(pt, n_pick - 1)] : INT_MAX;
    }
  };
  auto store_outliers = [&]() {
    if (tok_side) {
      st16(s_xo + hr * 16, make_uint4(keep[0], keep[1], keep[2], keep[3]));
      st16(s_xo + hr * 16 + 8, make_uint4(keep[4], keep[5], keep[6], keep[7]));
    } else if (hr < BN && Wf) {
      st16(s_wo + hr * 16, make_uint4(keep[0], keep[1], keep[2], keep[3]));
      st16(s_wo + hr * 16 + 8, make_uint4(keep[4], keep[5], keep[6], keep[7]));
    } else if (hr < BN) {
      const float swf = __builtin_bit_cast(float, keep[8]);
      uint32_t wpk[8];
#pragma unroll
      for (int t = 0; t < 16; t += 2) {
        const float q0 = (float)(int8_t)(keep[t / 4] >> (8 * (t % 4)));
        const float q1 = (float)(int8_t)(keep[t / 4] >> (8 * (t % 4) + 8));
        wpk[t / 2] = f2h((q0 * swf) / 127.0f) | (f2h((q1 * swf) / 127.0f) << 16);
      }
      st16(s_wo + hr * 16, make_uint4(wpk[0], wpk[1], wpk[2], wpk[3]));
      st16(s_wo + hr * 16 + 8, make_uint4(wpk[4], wpk[5], wpk[6], wpk[7]));
    }
  };
  // ---- loader: the first half of the waves fill the Wq rows [0, BN), the
  // second half the Xq rows.
  // Wave-wide load j of wave w fills LDS rows R0 .. R0+RPL-1 of the stage,
  // lane l -> row R0 + l/4, physical chunk l%4, logical chunk (l%4)^f(row).
  const bool loads_w = wave < Cfg::WAVES / 2;
  const int op_rows_valid =
      loads_w ? (int)min<int64_t>(BN, N - n0) : (int)min<int64_t>(BM, M - m0);
  const int8_t* op_base = loads_w ? Wq + n0 * K : Xq + m0 * K;
  // Operand rows are `rstride` bytes apart and hold `rowbytes` bytes of K
  // (the int8 codes: K and K; the outlier segment: 2 * ldo and 2 * ldo).
  __amdgpu_buffer_rsrc_t rsrc = make_rsrc(op_base, (uint32_t)op_rows_valid * (uint32_t)K);
  int rstride = K, rowbytes = K;
  const int row_first = (loads_w ? 0 : BN) + (wave % (Cfg::WAVES / 2)) * (LOADS * RPL);
  // Lane offsets: load j covers rows row_first + 16j + lane/4; the swizzle
  // key of those rows depends on j only through its parity.
  // The row-group and k offsets go in the scalar operand, which the hardware
  // bounds check leaves out, so each lane tests its row and k chunk itself:
  // kleft[p] = rowbytes - its chunk's byte offset, rleft[p] = valid rows -
  // its row (both must stay positive).
  int voff[2], kleft[2], rleft[2];
  auto set_offsets = [&]() {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = row_first + p * RPL + (lane >> 2);
      const int c = (lane & 3) ^ swz_key(r);
      const int rl = r - (loads_w ? 0 : BN);
      voff[p] = rl * rstride + c * 16;
      kleft[p] = rowbytes - c * 16;
      rleft[p] = op_rows_valid - rl;
    }
  };
  set_offsets();
  // Wave-wide load j of stage kt (LOADS per wave per stage).
  auto issue_load = [&](int kt, int j) {
    const int k0 = kt * BK;
    int8_t* sbase = stages + (kt % STAGES) * Cfg::STAGE_BYTES + row_first * BK;
    const int soff = __builtin_amdgcn_readfirstlane((j & ~1) * RPL * rstride + k0);
    const bool ok = k0 < kleft[j & 1] && (j & ~1) * RPL < rleft[j & 1];
    const int vo = ok ? voff[j & 1] : 0x7ffffff0 - soff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(sbase + j * RPL * BK), 16, vo,
                                             soff, 0, 0);
  };
  auto issue_pair = [&](int kt) {   // stages kt, kt + 1, row block by row block
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      issue_load(kt, j);
      issue_load(kt + 1, j);
    }
  };

  // ---- fragment read offsets (bytes inside a stage)
  int aoff[KS][TN], boff[KS][TM];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = ks * 2 + lhi;
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int r = wn * WN + a * 32 + l32;
      aoff[ks][a] = r * BK + ((c ^ swz_key(r)) << 4);
    }
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int r = BN + wm * WM + b * 32 + l32;
      boff[ks][b] = r * BK + ((c ^ swz_key(r)) << 4);
    }
  }

  v16i32 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

  v4i32 fa[2][KS][TN], fb[2][KS][TM];
  // Fragment r of a stage, in the order the MFMAs of a step consume them:
  // per k-step ks, A tile 0, B tiles 0..TM-1, then A tiles 1..TN-1.
  auto read_one = [&](const int8_t* base, int r, int set) {
    const int ks = r / (TN + TM), i = r % (TN + TM);
    if (i == 0)
      fa[set][ks][0] = *reinterpret_cast<const v4i32*>(base + aoff[ks][0]);
    else if (i <= TM)
      fb[set][ks][i - 1] = *reinterpret_cast<const v4i32*>(base + boff[ks][i - 1]);
    else
      fa[set][ks][i - TM] = *reinterpret_cast<const v4i32*>(base + aoff[ks][i - TM]);
  };
  auto read_frags = [&](int kt, int set) {
    const int8_t* base = stages + (kt % STAGES) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int r = 0; r < Cfg::NREADS; ++r) read_one(base, r, set);
  };
  // MFMA m of a step: k-step ks, A tile a, B tile b. The outlier segment
  // reads the same 16-byte fragments as 8 fp16 values (16 k per MFMA instead
  // of 32) and keeps its fp32 sums in the same accumulator registers.
  auto mfma_one = [&](int m, int set, auto f16) {
    const int ks = m / (TN * TM), a = (m / TM) % TN, b = m % TM;
    if constexpr (decltype(f16)::value) {
      const v16f32 r = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          __builtin_bit_cast(v8f16, fa[set][ks][a]), __builtin_bit_cast(v8f16, fb[set][ks][b]),
          __builtin_bit_cast(v16f32, acc[a][b]), 0, 0, 0);
      acc[a][b] = __builtin_bit_cast(v16i32, r);
    } else {
      acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[set][ks][a], fb[set][ks][b],
                                                        acc[a][b], 0, 0, 0);
    }
  };
  // Step k: PRE MFMAs on stage k, wait until stage k+1 has landed, barrier
  // (stage k+1 visible to every wave; every wave is done reading stage k),
  // then LOADS groups in a fixed order, each of one stage load, a few
  // fragment reads of stage k+1 into the other register set, and an equal
  // share of the remaining MFMAs on stage k.
  // Loads go out two stages at a time: the steps k (even) and k+1 together
  // issue stages k+4 and k+5, each step half of the rows of both, alternating
  // between the two stages. Back-to-back loads of the same rows of two
  // consecutive k-blocks fill whole 128-byte lines of each operand row, which
  // the vector L1 merges, where a single stage fetches half lines. Stage k+5
  // takes stage k's buffer and stage k+4 that of k-1, both read by the time
  // of step k's barrier. The waits follow from the issue order: before an
  // even step the youngest 2*LOADS loads (the last two steps') may still be
  // in flight; before an odd step only the even step's LOADS and the last
  // load of the pair before it, the other stage of that pair.
  // The reads fill the first RGROUPS groups so they have landed by the next
  // barrier's LDS wait; the scheduling barriers keep the compiler from
  // regrouping them (which would force both register sets into one and
  // serialize the reads behind the MFMAs).
  static_assert(STAGES == 5, "the paired issue order is written for five stages");
  constexpr int RGROUPS = LOADS * 3 / 4;
  // The MFMAs of step k use fragments read during step k-1, so the first PRE
  // of them go out before the wait and barrier, and the MFMA pipe has work
  // while the waves synchronize. With two waves per SIMD this made the GEMM
  // 1-1.4% faster (same products, same order); with one wave per SIMD it
  // gained nothing.
  constexpr int PRE = Cfg::WAVES_M == 4 ? Cfg::NMFMA / 4 : 0;
  constexpr int NM = Cfg::NMFMA;
  auto step = [&](int k, int set, auto f16) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < PRE; ++m) mfma_one(m, set, f16);
    if constexpr (PRE > 0) __builtin_amdgcn_sched_barrier(0);
    if (set == 0) wait_vmcnt<2 * LOADS>(); else wait_vmcnt<LOADS + 1>();
    lds_barrier();
    if constexpr (!decltype(f16)::value)
      if (pick_w) pick_stage(k + 1);   // stage k+1 has landed and stays until step k+1
    const int8_t* rbase = stages + ((k + 1) % STAGES) * Cfg::STAGE_BYTES;
    const int pair0 = set == 0 ? k + 4 : k + 3;
    const int row_half = set == 0 ? 0 : LOADS / 2;
#pragma unroll
    for (int g = 0; g < LOADS; ++g) {
      issue_load(pair0 + (g & 1), row_half + g / 2);
#pragma unroll
      for (int r = 0; r < Cfg::NREADS; ++r)
        if (r * RGROUPS / Cfg::NREADS == g) read_one(rbase, r, set ^ 1);
#pragma unroll
      for (int m = PRE + g * (NM - PRE) / LOADS; m < PRE + (g + 1) * (NM - PRE) / LOADS; ++m)
        mfma_one(m, set, f16);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // sw/127 (and bias) of the 16 features lane (l32, lhi) holds in slice a.
  auto load_fw = [&](int a, float* fw, float* bv) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int fl = wn * WN + a * 32 + 8 * g + 4 * lhi;
      const float4 f4 = *reinterpret_cast<const float4*>(s_fw + fl);
      fw[4 * g] = f4.x; fw[4 * g + 1] = f4.y; fw[4 * g + 2] = f4.z; fw[4 * g + 3] = f4.w;
      if (bv) {
        const float4 b4 = *reinterpret_cast<const float4*>(s_bias + fl);
        bv[4 * g] = b4.x; bv[4 * g + 1] = b4.y; bv[4 * g + 2] = b4.z; bv[4 * g + 3] = b4.w;
      }
    }
  };

  // With every column an outlier column the int8 codes are all zero and the
  // int8 segment is skipped.
  const int nk = (seg2 && n_o == K) ? 0 : (K + BK - 1) / BK;
  const std::integral_constant<bool, false> kInt8{};
  const std::integral_constant<bool, true> kF16{};
  // Runs main-loop steps 0 .. steps-1 over the current operands, after
  // stages 0 .. 3 have been issued (issue_pair(0), then issue_pair(2)); the
  // first wait leaves in flight the second pair and at most one load before
  // it (stage 1's last, or the last outlier gather), so stage 0 has landed.
  auto run_steps = [&](int steps, auto f16) __attribute__((always_inline)) {
    wait_vmcnt<2 * LOADS + 1>();
    lds_barrier();
    read_frags(0, 0);
    if constexpr (!decltype(f16)::value)
      if (pick_w) pick_stage(0);
    step(0, 0, f16);
    int k = 1;
    for (; k + 1 < steps; k += 2) {
      step(k, 1, f16);
      step(k + 1, 0, f16);
    }
    if (k < steps) step(k, 1, f16);
    wait_vmcnt<0>();
  };
  // Prologue: the row / column factors are read into registers, then the
  // first four stages are issued with the chunk-0 outlier gathers between
  // stages 0-1 and 2-3; factors and gathers go to LDS after the main loop.
  if (Y && h_ok) {
    if (tok_side) {
      keep[8] = __builtin_bit_cast(uint32_t, sx[m0 + hr]);
    } else {
      keep[8] = __builtin_bit_cast(uint32_t, sw[n0 + hr]);
      if (bias) keep[9] = bias[n0 + hr];
    }
  }
  // The outlier gathers go after stages 0-1 and before stages 2-3: the first
  // wait (for stages 0-1) then covers them too, and no later wait counts them
  // as younger than a stage it needs.
  if (nk > 0) issue_pair(0);
  if (n_o > 0 && !seg2) fetch_outliers();
  if (nk > 0) issue_pair(2);
  auto store_scales = [&]() {
    if (Y) {
      if (tok_side) {
        s_ax[hr] = __builtin_bit_cast(float, keep[8]) / 127.0f;
      } else if (hr < BN) {
        s_fw[hr] = __builtin_bit_cast(float, keep[8]) / 127.0f;
        s_bias[hr] = h2f((uint16_t)keep[9]);
      }
    }
  };
  if (nk > 0) run_steps(nk, kInt8);
  lds_barrier();   // every wave is done with the stage buffers
  store_scales();
  if (n_o > 0 && !seg2) store_outliers();

  if (seg2) {
    lds_barrier();   // the factors are in LDS
    // Dequantize in place, C * (sx/127) * (sw/127) in fp32 (the same
    // expression as the epilogue's), then the outlier segment adds
    // sum_t Xo[i, t] * Wo[j, t] onto it.
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      float fw[16];
      load_fw(a, fw, nullptr);
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const float ax = s_ax[wm * WM + b * 32 + l32];
        v16f32 y;
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = (float)acc[a][b][r] * ax * fw[r];
        acc[a][b] = __builtin_bit_cast(v16i32, y);
      }
    }
    const uint16_t* seg_base = loads_w ? Wo + n0 * ldo : Xo + m0 * ldo;
    rstride = rowbytes = (int)(2 * ldo);
    rsrc = make_rsrc(seg_base, (uint32_t)op_rows_valid * (uint32_t)rowbytes);
    set_offsets();
    lds_barrier();   // every wave has read its factors
    issue_pair(0);
    issue_pair(2);
    run_steps(rowbytes / BK, kF16);
    lds_barrier();
    store_scales();
  }
  // every wave is done with the stage buffers before the epilogue reuses them
  if (Y) lds_barrier();

  // ---- epilogue
  // Lane (l32, lhi), accumulator r of tile (a, b):
  //   token   = m0 + wm*WM + b*32 + l32
  //   feature = n0 + wn*WN + a*32 + 8*(r/4) + 4*lhi + (r%4)
  if (WITH_C) {
    const bool n4 = (N & 3) == 0;
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const int64_t tok = m0 + wm * WM + b * 32 + l32;
        if (tok >= M) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t f = n0 + wn * WN + a * 32 + 8 * g + 4 * lhi;
          int32_t* dst = C + tok * N + f;
          if (n4 && f + 3 < N) {
            *reinterpret_cast<int4*>(dst) =
                make_int4(acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                          acc[a][b][4 * g + 3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (f + e < N) dst[e] = acc[a][b][4 * g + e];
          }
        }
      }
  }
  if (!Y) return;

  // ---- fp16 output
  // Two 32-feature slices at a time go through this wave's part of the (now
  // idle) stage buffers: after packing to fp16, lanes l and l+32 hold
  // features 8g + 0..3 and 8g + 4..7 of group g; v_permlane32_swap on groups
  // (g, g+1) gives lane l all 8 features of group g and lane l+32 all 8 of
  // group g+1, written to LDS as 16-byte pieces of [token][64 features] rows.
  // They are read back row-contiguous, so 8 consecutive lanes store one whole
  // 128-byte row segment of Y: write misses reach memory as full lines
  // rather than as 16-byte pieces of 32 different rows.
  constexpr int OUT_ROW = Cfg::OUT_ROW;
  static_assert(TN % 2 == 0, "slices are stored in pairs");
  int8_t* s_out = lds + Cfg::OUT0 + wave * (WM * OUT_ROW);
  const bool n8 = (N & 7) == 0;
  auto stage_tile = [&](int a, int b, const v16f32& y) {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = f2h(y[2 * i]) | (f2h(y[2 * i + 1]) << 16);
#pragma unroll
    for (int gp = 0; gp < 4; gp += 2) {
      // p[2gp], p[2gp+1]: group gp; p[2gp+2], p[2gp+3]: group gp+1
      const auto s0 = __builtin_amdgcn_permlane32_swap(p[2 * gp], p[2 * gp + 2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(p[2 * gp + 1], p[2 * gp + 3], false, false);
      const int row = b * 32 + l32;
      const int col = (a & 1) * 64 + 16 * (gp + lhi);   // byte offset in the row
      *reinterpret_cast<uint4*>(s_out + row * OUT_ROW + col) =
          make_uint4(s0[0], s1[0], s0[1], s1[1]);
    }
  };
  auto flush_pair = [&](int a0) {
    // a0 even: slices a0, a0+1 = features wn*WN + a0*32 + [0, 64)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t f = n0 + wn * WN + a0 * 32 + 8 * (lane & 7);
#pragma unroll 4
    for (int it = 0; it < WM / 8; ++it) {
      const int row = it * 8 + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4*>(s_out + row * OUT_ROW + 16 * (lane & 7));
      const int64_t tok = m0 + wm * WM + row;
      if (tok < M) {
        uint16_t* dst = Y + tok * N + f;
        if (n8 && f + 7 < N) {
          // streaming store: Y is written once and not read back by this
          // kernel, so it should not displace operand lines in the caches
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (f + e < N) dst[e] = (uint16_t)half_of(v, e);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // LDS outlier fragments: 8 fp16 (t = 8*lhi .. 8*lhi+7) of row l32 of a
  // 32-row slice; same lane -> t assignment on the weight and token side.
  auto wo_frag = [&](int a) -> v8f16 {
    return *reinterpret_cast<const v8f16*>(s_wo + (wn * WN + a * 32 + l32) * 16 + lhi * 8);
  };
  auto xo_frag = [&](int b) -> v8f16 {
    return *reinterpret_cast<const v8f16*>(s_xo + (wm * WM + b * 32 + l32) * 16 + lhi * 8);
  };

  // Fragments of outlier chunks beyond the first (more than 16 outlier
  // columns), built straight from global memory: the weight columns are read
  // from Wf when the weight is kept in fp16, else recovered from Wq as
  // fp16(fl32(fl32(q * sw) / 127)); the activations are read from Xo. Slow,
  // but it keeps the per-slice register footprint small.
  auto wo_frag_g = [&](int a, int t0) -> v8f16 {
    v8f16 w;
    const int64_t f = n0 + wn * WN + a * 32 + l32;
    const float swf = f < N ? sw[f] : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t0 + lhi * 8 + e;
      if (Wf) {
        w[e] = (t < n_o && f < N) ? __builtin_bit_cast(_Float16, Wf[f * K + cols[t]])
                                  : (_Float16)0.0f;
      } else {
        float v = 0.0f;
        if (t < n_o && f < N) v = ((float)Wq[f * K + cols[t]] * swf) / 127.0f;
        w[e] = (_Float16)v;
      }
    }
    return w;
  };
  auto xo_frag_g = [&](int b, int t0) -> v8f16 {
    const int64_t tok = m0 + wm * WM + b * 32 + l32;
    if (tok >= M) return v8f16{};
    return __builtin_bit_cast(v8f16, ld16(Xo + tok * ldo + t0 + lhi * 8));
  };

  // One 32-feature slice a at a time, its TM token tiles in VGPRs: dequantize
  // y = C * (sx/127) * (sw/127), add the fp16 outlier product on
  // v_mfma_f32_32x32x16_f16 (first 16 columns from the LDS-staged fragments,
  // further chunks from global memory), add the bias, store.
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    float fw[16], bv[16];
    load_fw(a, fw, bias ? bv : nullptr);
    v16f32 y[TM];
    if (seg2) {
      // already dequantized, with the outlier product added
#pragma unroll
      for (int b = 0; b < TM; ++b) y[b] = __builtin_bit_cast(v16f32, acc[a][b]);
    } else {
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const float ax = s_ax[wm * WM + b * 32 + l32];
#pragma unroll
        for (int r = 0; r < 16; ++r) y[b][r] = (float)acc[a][b][r] * ax * fw[r];
      }
    }
    if (n_o > 0 && !seg2) {
      const v8f16 wa = wo_frag(a);
#pragma unroll
      for (int b = 0; b < TM; ++b)
        y[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa, xo_frag(b), y[b], 0, 0, 0);
    }
    for (int t0 = 16; t0 < (seg2 ? 0 : n_o); t0 += 16) {
      const v8f16 wa = wo_frag_g(a, t0);
#pragma unroll
      for (int b = 0; b < TM; ++b)
        y[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa, xo_frag_g(b, t0), y[b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      if (bias) {
#pragma unroll
        for (int r = 0; r < 16; ++r) y[b][r] += bv[r];
      }
      stage_tile(a, b, y[b]);
    }
    if (a & 1) flush_pair(a - 1);
  }
}

template <class Cfg>
hipError_t launch_gemm_t(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                         int64_t M, int64_t N, int64_t K, const uint16_t* Xo, const int32_t* cols,
                         const int32_t* n_out, const uint16_t* bias, uint16_t* Y, int32_t* C,
                         const uint16_t* Wo, const uint16_t* Wf, hipStream_t s) {
  const int64_t tiles = ((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
  if (C) {
    // parity mode: the epilogue outlier path only
    hipLaunchKernelGGL((k_gemm_i8<Cfg, kInt32>), dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, s, Xq,
                       Wq, sx, sw, (int)M, (int)N, (int)K, Xo, cols, n_out, bias, Y, C, nullptr, Wf);
    return hipGetLastError();
  }
  // The outlier count is only known on the device: with Wo given both modes
  // are launched and the one whose case it is not returns at once.
  hipLaunchKernelGGL((k_gemm_i8<Cfg, kPlain>), dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, s, Xq,
                     Wq, sx, sw, (int)M, (int)N, (int)K, Xo, cols, n_out, bias, Y, C, Wo, Wf);
  if (Wo) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_i8<Cfg, kOutlierSeg>), dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, s,
                       Xq, Wq, sx, sw, (int)M, (int)N, (int)K, Xo, cols, n_out, bias, Y, C, Wo, Wf);
  }
  return hipGetLastError();
}

#ifndef I8MM_LARGE_WAVES_M
#define I8MM_LARGE_WAVES_M 4
#endif
using CfgLarge = GemmCfg<256, 256, 64, 5, I8MM_LARGE_WAVES_M>;
using CfgSmall = GemmCfg<128, 128, 64, 5>;
#ifndef I8MM_LARGE_TILE_MIN
#define I8MM_LARGE_TILE_MIN 256
#endif
constexpr int64_t kLargeTileMin = I8MM_LARGE_TILE_MIN;

}  // namespace

hipError_t launch_gemm(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                       int64_t M, int64_t N, int64_t K, const uint16_t* Xo, const int32_t* cols,
                       const int32_t* n_out, const uint16_t* bias, uint16_t* Y, int32_t* C,
                       const uint16_t* Wo, const uint16_t* Wf, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // (K == 0 goes to the tiled kernel, whose empty main loop leaves only the
  // epilogue: Y = bias, or 0)
  if (gemv_applies(M) && K > 0)
    return launch_gemv(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_out, bias, Y, C, Wf, s);
  // 256 x 256 tiles when they give every CU at least one; otherwise the
  // 128 x 128 tiles (four times as many, two blocks per CU).
  const int64_t tiles_large = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles_large >= kLargeTileMin)
    return launch_gemm_t<CfgLarge>(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_out, bias, Y, C, Wo, Wf, s);
  return launch_gemm_t<CfgSmall>(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_out, bias, Y, C, Wo, Wf, s);
}

}  // namespace i8mm
