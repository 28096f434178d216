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
// Wq [N, K]). v_mfma_i32_16x16x64_i8 takes a 16 x 64-byte slice of each (a
// whole stage of K): the "A" operand is a 16-row slice of Wq (output
// features), the "B" operand a 16-row slice of Xq (tokens); lane l holds 16
// bytes of row l % 16 at k group l / 16. A lane's 4 accumulators then hold 4
// consecutive output features of one token. A and B fragments use the same
// lane -> k assignment, so the sum over k is the same whatever order the
// instruction uses inside its slice (integer sums are exact). The same work
// as v_mfma_i32_32x32x32_i8 tiles ran 4-6% faster on these 16 x 16 tiles
// (175B shape 1952 -> 1867 us, OPT shape 119.5 -> 112 us, Y bit-identical).
//
// Block = 8 wavefronts, two per SIMD, in a 2 x 4 grid over a BN x BM
// (features x tokens) tile; each wave owns a (BN/2) x (BM/4) sub-tile (8 x 4
// MFMA tiles of 16 x 16 for 256 x 256, 128 accumulator registers), so while
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
// rows); 16-byte chunk c of row r sits at position c ^ f(r), f(r) = bit 0
// of r | bit 3 of r << 1. A probe timed the fragment read (lane l at row
// l % 16, logical chunk l / 16) under all 256 keys that XOR two parities of
// the row's low four bits into the chunk: the best ones, this among them,
// run 1.30x faster than the key (r >> 2) & 3 (which suited the 32 x 32
// tiles' read, lane l < 32 at row l and lane l + 32 at the next chunk) and
// 1.08x faster than reads of consecutive addresses. The key depends on the
// row's low four bits only, so it repeats every 16 rows. The layout only
// permutes which chunk each lane's DMA load fetches: every row is still
// read as one 64-byte segment and written to LDS in order.
//
// Epilogue: per-tile dequantization with the row / column factors staged in
// LDS; the fp16 outlier product (first 16 outlier columns: gathered in the
// prologue, held in registers through the main loop, then staged in LDS;
// further columns read per 16-column step) runs on v_mfma_f32_16x16x16_f16
// onto the dequantized tile; a pass through LDS turns each four 16-feature
// slices into whole 128-byte row segments of Y per 8 lanes. The outlier
// segments run v_mfma_f32_16x16x32_f16 on the same fragment layout.
//
// Tile order: blocks are dealt to the 8 XCDs round-robin by block id; the id
// is remapped so each XCD owns a contiguous range of tiles, rastered in groups
// of 4 token-tiles per weight-tile column, so blocks running together on one
// XCD share their Wq and Xq panels in that XCD's L2. (Groups of 4 against 8:
// 3.5% faster at 2048 x 4096 -> 16384, 0.6% at 4096 x 12288 -> 49152, even
// on the 1024-token shapes; groups of 2 or 16 were slower.)

#include <type_traits>

#include "device_common.h"
#include "i8mm.h"
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
  static constexpr int TM = WM / 16;                // MFMA tiles per wave, token dim
  static constexpr int TN = WN / 16;                // MFMA tiles per wave, feature dim
  static constexpr int KS = BK / 64;                // MFMA k-steps per stage
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

__device__ __forceinline__ int swz_key(int r) { return (r & 1) | ((r >> 2) & 2); }

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
//   kPlain   fp16 output; outlier product in the epilogue. Returns at once
//            when one of the two segment modes below takes the layer.
//   kInt32   kPlain that also writes the raw int32 accumulators (parity mode).
//   kOutlierSeg  only for more than 16 outlier columns with Wo given and
//            room for them in it, wo_cols (returns at once otherwise): the
//            outlier product as a second main-loop segment.
//   kDenseSeg  more than 16 outlier columns, X given, and Wo not given or
//            without room for them (returns at once otherwise): the
//            outlier product as a dense second segment over all K columns,
//            the weight columns recovered from Wq in the loop.
//   kDenseSegW  kDenseSeg with the weight kept in fp16 (Wf), launched
//            instead of it when Wf is given.
enum GemmMode { kPlain = 0, kInt32 = 1, kOutlierSeg = 2, kDenseSeg = 3, kDenseSegW = 4 };
template <class Cfg, int MODE>
__global__ __launch_bounds__(Cfg::THREADS) void k_gemm_i8(
    const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, const float* __restrict__ sx,
    const float* __restrict__ sw, int M, int N, int K, const uint16_t* __restrict__ Xo,
    const int32_t* __restrict__ cols, const int32_t* __restrict__ n_out,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C,
    const uint16_t* __restrict__ Wo, int wo_cols, const uint16_t* __restrict__ Wf,
    const uint16_t* __restrict__ Xd, const uint32_t* __restrict__ bmp,
    const int32_t* __restrict__ kbl) {
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
  const int l16 = lane & 15, lq = lane >> 4;   // MFMA operand row, 16-byte k group

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
  constexpr bool WITH_C = MODE == kInt32;
  // With more than 16 outlier columns the outlier product runs as a second
  // segment: over the materialized recovered weights Wo ([N, ldo] fp16) and
  // Xo when the columns fit Wo's region (compact), else over all K columns
  // with the weight tile converted in the kernel and X itself (dense, X
  // given). Either runs fp16 MFMA through the same stage pipeline.
  const bool compact = n_o > 16 && Wo != nullptr && n_o <= wo_cols;
  const bool dense_case = n_o > 16 && !compact && Xd != nullptr && bmp != nullptr;
  // each mode returns at once when the case is another mode's
  if (MODE == kOutlierSeg && !compact) return;
  if ((MODE == kDenseSeg || MODE == kDenseSegW) && !dense_case) return;
  if ((MODE == kPlain || MODE == kInt32) && (compact || dense_case)) return;
  constexpr bool seg2 = MODE == kOutlierSeg || MODE == kDenseSeg || MODE == kDenseSegW;
  constexpr bool dense = MODE == kDenseSeg || MODE == kDenseSegW;
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
  // The k-blocks the int8 loop visits. In the segment modes, given the list
  // the row pass writes (kbl[0] = count, then the k-blocks that hold at least
  // one normal column, ascending), only those: a k-block of outlier columns
  // has all-zero codes. Otherwise all of them (none with every column an
  // outlier column). Stage kt holds k-block kmap(kt); past the last visited
  // stage, kmap gives a k-block past K, whose loads read zeros.
  static_assert(BK == 64, "the k-block list is in 64-column blocks");
  const int nkb_all = (K + BK - 1) / BK;
  bool list_on = seg2 && kbl != nullptr;
  const int nk = list_on ? __builtin_amdgcn_readfirstlane(kbl[0])
                         : ((seg2 && n_o == K) ? 0 : nkb_all);
  auto kmap = [&](int kt) -> int {
    if constexpr (!seg2) {
      return kt;
    } else {
      if (!list_on) return kt;
      return kt < nk ? __builtin_amdgcn_readfirstlane(kbl[1 + kt]) : nkb_all;
    }
  };
  // Wave-wide load j of stage kt, k-block kb (LOADS per wave per stage).
  auto issue_load = [&](int kt, int kb, int j) {
    const int k0 = kb * BK;
    int8_t* sbase = stages + (kt % STAGES) * Cfg::STAGE_BYTES + row_first * BK;
    const int soff = __builtin_amdgcn_readfirstlane((j & ~1) * RPL * rstride + k0);
    const bool ok = k0 < kleft[j & 1] && (j & ~1) * RPL < rleft[j & 1];
    const int vo = ok ? voff[j & 1] : 0x7ffffff0 - soff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(sbase + j * RPL * BK), 16, vo,
                                             soff, 0, 0);
  };
  auto issue_pair = [&](int kt) {   // stages kt, kt + 1, row block by row block
    const int kb0 = kmap(kt), kb1 = kmap(kt + 1);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      issue_load(kt, kb0, j);
      issue_load(kt + 1, kb1, j);
    }
  };

  // ---- fragment read offsets (bytes inside a stage)
  int aoff[KS][TN], boff[KS][TM];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = ks * 4 + lq;
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int r = wn * WN + a * 16 + l16;
      aoff[ks][a] = r * BK + ((c ^ swz_key(r)) << 4);
    }
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int r = BN + wm * WM + b * 16 + l16;
      boff[ks][b] = r * BK + ((c ^ swz_key(r)) << 4);
    }
  }

  v4i32 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][b][r] = 0;

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
  // reads the same 16-byte fragments as 8 fp16 values (32 k per MFMA instead
  // of 64) and keeps its fp32 sums in the same accumulator registers.
  auto mfma_one = [&](int m, int set, auto f16) {
    const int ks = m / (TN * TM), a = (m / TM) % TN, b = m % TM;
    if constexpr (decltype(f16)::value) {
      const v4f32 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(v8f16, fa[set][ks][a]), __builtin_bit_cast(v8f16, fb[set][ks][b]),
          __builtin_bit_cast(v4f32, acc[a][b]), 0, 0, 0);
      acc[a][b] = __builtin_bit_cast(v4i32, r);
    } else {
      acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[set][ks][a], fb[set][ks][b],
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
  // k-blocks of the pair of stages the current two steps load (pkb) and of
  // the next pair (npkb, looked up one step ahead so the scalar loads of the
  // list have landed when the loads need them)
  int pkb0 = 0, pkb1 = 0, npkb0 = 0, npkb1 = 0;
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
    if constexpr (seg2) {
      if (set == 0) {
        pkb0 = npkb0;
        pkb1 = npkb1;
      } else {
        npkb0 = kmap(k + 5);
        npkb1 = kmap(k + 6);
      }
    }
#pragma unroll
    for (int g = 0; g < LOADS; ++g) {
      const int st = pair0 + (g & 1);
      issue_load(st, seg2 ? ((g & 1) ? pkb1 : pkb0) : st, row_half + g / 2);
#pragma unroll
      for (int r = 0; r < Cfg::NREADS; ++r)
        if (r * RGROUPS / Cfg::NREADS == g) read_one(rbase, r, set ^ 1);
#pragma unroll
      for (int m = PRE + g * (NM - PRE) / LOADS; m < PRE + (g + 1) * (NM - PRE) / LOADS; ++m)
        mfma_one(m, set, f16);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // sw/127 (and the bias) of the 4 features lane (l16, lq) holds in slice a.
  auto load_fw = [&](int a, float* fw, float* bv) {
    const int fl = wn * WN + a * 16 + 4 * lq;
    const float4 f4 = *reinterpret_cast<const float4*>(s_fw + fl);
    fw[0] = f4.x; fw[1] = f4.y; fw[2] = f4.z; fw[3] = f4.w;
    if (bv) {
      const float4 b4 = *reinterpret_cast<const float4*>(s_bias + fl);
      bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
    }
  };

  const std::integral_constant<bool, false> kInt8{};
  const std::integral_constant<bool, true> kF16{};
  // Runs main-loop steps 0 .. steps-1 over the current operands, after
  // stages 0 .. 3 have been issued (issue_pair(0), then issue_pair(2)); the
  // first wait leaves in flight the second pair and at most one load before
  // it (stage 1's last, or the last outlier gather), so stage 0 has landed.
  auto run_steps = [&](int steps, auto f16) __attribute__((always_inline)) {
    if constexpr (seg2) {
      npkb0 = kmap(4);
      npkb1 = kmap(5);
    }
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
  // Dense outlier segment: the outlier product over all K columns, 32 columns
  // per stage through the five stage buffers, in the main loop's LDS layout
  // (weight rows, then token rows, 64 bytes each, same swizzle), so the
  // fragment reads and fp16 MFMAs are those of the compact segment. The
  // weight tile comes through registers: thread t converts 16 columns of
  // weight row t / 2 exactly to fp16 (the int8 codes, or the fp16 weight Wf
  // itself) with the normal columns zeroed (bitmap word of the stage), and
  // writes them to LDS. The token rows are X itself, by DMA: X is finite on
  // the normal columns (a column holding inf or NaN is an outlier column),
  // so the zeroed weights remove them exactly. On the 256 x 256 tiles a stage
  // whose bitmap word is 0 issues no fragment reads and no MFMA; on the
  // 128 x 128 tiles every stage runs them (see the step below).
  // Step st: stage st+1's loads have landed; its weights go to LDS; barrier
  // (stage st+1 visible to every wave; every wave is done reading stage st);
  // the loads of stage st+4 (registers: set (st+4) % 4; DMA: the buffer of
  // stage st-1); the fragment reads of stage st+1 into one register set and
  // the MFMAs of stage st from the other. Loads past the last stage read
  // zeros, so every step issues the same loads and the waits are fixed.
  auto dense_segment = [&]() __attribute__((always_inline)) {
    constexpr int DNB = STAGES;                 // stage buffers
    constexpr int DLB = BM / 16 / Cfg::WAVES;   // token-row DMA loads per wave and stage
    static_assert(Cfg::THREADS == 2 * BN, "two threads per weight row");
    static_assert(DLB * 16 * Cfg::WAVES == BM && DLB == 2, "token rows per wave");
    static_assert(DNB == 5, "four stages in flight");
    const int S = (K + 31) / 32;
    // bitmap word of stage st (0 past the last stage): a scalar load
    auto word_of = [&](int st) -> uint32_t {
      const uint32_t w = __builtin_amdgcn_readfirstlane(bmp[st < S ? st : S - 1]);
      return st < S ? w : 0u;
    };
    // weight side: row ra, columns 16 * hf .. of each stage
    const int ra = tid >> 1, hf = tid & 1;
    const int rows_a = (int)min<int64_t>(BN, N - n0);
    constexpr bool wide = MODE == kDenseSegW;   // fp16 weight: 32 bytes a thread
    const __amdgpu_buffer_rsrc_t rsa = wide
        ? make_rsrc(Wf + n0 * K, (uint32_t)rows_a * (uint32_t)K * 2u)
        : make_rsrc(Wq + n0 * K, (uint32_t)rows_a * (uint32_t)K);
    const int key_a = swz_key(ra);
    uint4 areg[4][2];
    auto load_a = [&](int st, int set) {
      const int col = st * 32 + 16 * hf;
      const bool ok = col < K;
      // Both weight sources issue the same two loads (the int8 codes need
      // only the first; their second reads past the buffer and returns
      // zeros, with no memory access), so a register set is only ever
      // written by loads. Written by a load on one source and a constant on
      // the other, the second half made the compiler wait for every load in
      // flight before each step's constant, which left one stage of loads
      // in flight instead of four.
      const int off0 = wide ? (ok ? (ra * K + col) * 2 : 0x7fffffe0) : (ok ? ra * K + col : 0x7fffffe0);
      const int off1 = wide ? off0 + 16 : 0x7ffffff0;
      areg[set][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsa, off0, 0, 0));
      areg[set][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsa, off1, 0, 0));
    };
    // token side: wave w fills token rows w * 32 + 16 p + lane / 4
    const int rows_b = (int)min<int64_t>(BM, M - m0);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(Xd + m0 * K, (uint32_t)rows_b * (uint32_t)K * 2u);
    int vb[DLB];
    bool okb[DLB];
#pragma unroll
    for (int p = 0; p < DLB; ++p) {
      const int rb = wave * (16 * DLB) + 16 * p + (lane >> 2);
      const int c = (lane & 3) ^ swz_key(BN + rb);
      okb[p] = rb < rows_b;
      vb[p] = okb[p] ? rb * K * 2 + c * 16 : 0;
    }
    const int cb = ((lane & 3) ^ swz_key(BN + wave * (16 * DLB) + (lane >> 2))) * 16;
    auto load_b = [&](int st) {
      int8_t* sbase = stages + (st % DNB) * Cfg::STAGE_BYTES + (BN + wave * 16 * DLB) * BK;
      const int soff = __builtin_amdgcn_readfirstlane(st * 64);
#pragma unroll
      for (int p = 0; p < DLB; ++p) {
        const bool ok = okb[p] && st * 64 + cb < 2 * K;
        const int vo = ok ? vb[p] : 0x7ffffff0 - soff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(sbase + p * 16 * BK), 16, vo,
                                                 soff, 0, 0);
      }
    };
    // A 16-byte LDS store of the converted weights. Written as ds_write_b128
    // itself: as a plain store the compiler cannot tell it from the DMA
    // loads in flight into the same stage buffers and waits for every one
    // before it (vmcnt 0), which drains the prefetch at each stage. It never
    // overlaps them: it writes weight rows, the DMA token rows, and the loads
    // into its own buffer have been waited for (wait_next). The barrier that
    // follows waits for it (lgkmcnt 0) before any wave reads the stage.
    auto lds_store16 = [](int8_t* p, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
      typedef uint32_t u4v __attribute__((ext_vector_type(4)));
      const uint32_t addr = (uint32_t)(uintptr_t)(lds_ptr_t)p;
      const u4v d = {a0, a1, a2, a3};
      asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(d) : "memory");
    };
    // 4 int8 codes -> 4 fp16 (exact): bytes b + 128 under the exponent of
    // 1024 give 1024 + b + 128, minus 1152
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    auto cvt4 = [](uint32_t d) -> uint2 {
      const uint32_t u = d ^ 0x80808080u;
      const h2 k = h2{(_Float16)1152.0f, (_Float16)1152.0f};
      const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - k;
      const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - k;
      return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    };
    // The converted fp16 weights of one register set: 16 columns of the
    // thread's row, non-outlier columns zeroed (W: the weight is kept in
    // fp16). The byte mask (0xff where a column is an outlier column) comes
    // from a byte permute whose selector bytes are 0x0c (a zero byte) or 0x0d
    // (0xff): two full-rate operations instead of a quarter-rate multiply.
    auto convert_a = [&](int set, uint32_t word, uint32_t (&h)[8]) __attribute__((always_inline)) {
      const uint32_t bits = (word >> (16 * hf)) & 0xffffu;   // outlier columns of the 16
      if constexpr (wide) {
        const uint32_t w8[8] = {areg[set][0].x, areg[set][0].y, areg[set][0].z, areg[set][0].w,
                                areg[set][1].x, areg[set][1].y, areg[set][1].z, areg[set][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t b2 = (bits >> (2 * i)) & 3u;
          h[i] = w8[i] & (((b2 & 1u) | ((b2 & 2u) << 15)) * 0xffffu);
        }
      } else {
        const uint32_t w4[4] = {areg[set][0].x, areg[set][0].y, areg[set][0].z, areg[set][0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t b4 = (bits >> (4 * i)) & 15u;
          const uint32_t m1 = (b4 * 0x00204081u) & 0x01010101u;
          const uint32_t keep = __builtin_amdgcn_perm(0u, 0u, 0x0c0c0c0cu | m1);
          const uint2 c = cvt4(w4[i] & keep);
          h[2 * i] = c.x;
          h[2 * i + 1] = c.y;
        }
      }
    };
    auto store_a = [&](int st, const uint32_t (&h)[8]) __attribute__((always_inline)) {
      int8_t* row = stages + (st % DNB) * Cfg::STAGE_BYTES + ra * BK;
      lds_store16(row + (((2 * hf) ^ key_a) << 4), h[0], h[1], h[2], h[3]);
      lds_store16(row + (((2 * hf + 1) ^ key_a) << 4), h[4], h[5], h[6], h[7]);
    };
    auto write_a = [&](int st, int set, uint32_t word) {
      uint32_t h[8];
      convert_a(set, word, h);
      store_a(st, h);
    };
    const std::integral_constant<bool, true> f16{};
    auto read_stage = [&](int st, int fset) {
      const int8_t* base = stages + (st % DNB) * Cfg::STAGE_BYTES;
#pragma unroll
      for (int r = 0; r < Cfg::NREADS; ++r) read_one(base, r, fset);
    };
    // loads per step: the two weight register loads, the token DMA (DLB);
    // stage st+1's are followed by those of stages st+2 and st+3
    auto wait_next = [&]() { wait_vmcnt<2 * (2 + DLB)>(); };
    // With one wave per SIMD (the 128 x 128 tiles) the fragments of stage
    // st+1 are read while the MFMAs of stage st run (two register sets);
    // with two (the 256 x 256 tiles) the other wave covers the reads, and a
    // stage's fragments are read just before its MFMAs, which keeps the
    // registers within two waves' share.
    constexpr bool DBF = Cfg::WAVES_M != 4;
    // q: the register set of stage st+4 (= st mod 4); fragment set of stage
    // st: st mod 2
    uint32_t w_cur = 0, w_next = 0;   // bitmap words of stages st, st+1
    // With the double-buffered fragments (one wave per SIMD), every step runs
    // all of stage st's MFMAs, a stage without outlier columns included (its
    // converted weights are zeros and add nothing: an accumulator that is
    // +0 or nonzero is unchanged by zero products, and none is ever -0), so
    // the step is one branch-free block: the first half of the MFMAs is
    // interleaved with the weight conversion of stage st+1, one MFMA then a
    // few VALU operations, and the matrix pipe runs while the wave converts;
    // the rest go with the fragment reads of stage st+1 after the barrier.
    constexpr int PRE = Cfg::NMFMA / 2;
    auto dstep = [&](int st, auto Q) __attribute__((always_inline)) {
      constexpr int q = decltype(Q)::value;
      wait_next();
      if constexpr (DBF) {
#pragma unroll
        for (int m = 0; m < PRE; ++m) mfma_one(m, q & 1, f16);
        uint32_t h[8];
        convert_a((q + 1) & 3, w_next, h);
#pragma unroll
        for (int i = 0; i < PRE; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // then VALU
        }
        store_a(st + 1, h);
      } else {
        uint32_t h[8];
        convert_a((q + 1) & 3, w_next, h);
        store_a(st + 1, h);
      }
      lds_barrier();
      load_a(st + 4, q);
      load_b(st + 4);
      const uint32_t w_after = word_of(st + 2);
      if constexpr (DBF) {
        read_stage(st + 1, (q + 1) & 1);
#pragma unroll
        for (int m = PRE; m < Cfg::NMFMA; ++m) mfma_one(m, q & 1, f16);
      } else {
        if (w_cur) {
          read_stage(st, 0);
#pragma unroll
          for (int m = 0; m < Cfg::NMFMA; ++m) mfma_one(m, 0, f16);
        }
      }
      w_cur = w_next;
      w_next = w_after;
    };
    // prologue: stages 0-3 in flight, stage 0's weights to LDS, its fragments
    for (int st = 0; st < 4; ++st) {
      load_a(st, st);
      load_b(st);
    }
    w_cur = word_of(0);
    w_next = word_of(1);
    wait_vmcnt<3 * (2 + DLB)>();
    write_a(0, 0, w_cur);
    lds_barrier();
    if constexpr (DBF) read_stage(0, 0);
    const std::integral_constant<int, 0> q0{};
    const std::integral_constant<int, 1> q1{};
    const std::integral_constant<int, 2> q2{};
    const std::integral_constant<int, 3> q3{};
    // in fours (steps past the last stage find zeros and a bitmap word of
    // 0, so their MFMAs add nothing), so the register sets stay where they
    // are
    for (int st = 0; st < S; st += 4) {
      dstep(st, q0);
      dstep(st + 1, q1);
      dstep(st + 2, q2);
      dstep(st + 3, q3);
    }
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
    // expression as the epilogue's), then the compact segment adds
    // sum_t Xo[i, t] * Wo[j, t] onto it. The dense segment over the int8
    // weight adds sum_{k in O} X[i, k] * q[j, k] onto C * (sx/127) and the
    // epilogue multiplies by sw/127: the recovered weight q * sw / 127 per
    // output row ([HF-blog] "Usage"), its factor taken out of the sum. Over
    // the fp16 weight (Wf) it adds sum_{k in O} X[i, k] * Wf[j, k] onto the
    // whole dequantized value, as the compact segment does.
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      float fw[4];
      load_fw(a, fw, nullptr);
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const float ax = s_ax[wm * WM + b * 16 + l16];
        v4f32 y;
        if (dense && Wf == nullptr) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = (float)acc[a][b][r] * ax;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = (float)acc[a][b][r] * ax * fw[r];
        }
        acc[a][b] = __builtin_bit_cast(v4i32, y);
      }
    }
    if constexpr (!dense) {
      const uint16_t* seg_base = loads_w ? Wo + n0 * ldo : Xo + m0 * ldo;
      rstride = rowbytes = (int)(2 * ldo);
      rsrc = make_rsrc(seg_base, (uint32_t)op_rows_valid * (uint32_t)rowbytes);
      set_offsets();
      list_on = false;   // the outlier columns, in order
      lds_barrier();   // every wave has read its factors
      issue_pair(0);
      issue_pair(2);
      run_steps(rowbytes / BK, kF16);
    } else {
      lds_barrier();   // every wave has read its factors
      dense_segment();
    }
    lds_barrier();
    store_scales();
  }
  // every wave is done with the stage buffers before the epilogue reuses them
  if (Y) lds_barrier();

  // ---- epilogue
  // Lane (l16, lq), accumulator r of tile (a, b) (the D layout of the 16 x 16
  // MFMAs):
  //   token   = m0 + wm*WM + b*16 + l16
  //   feature = n0 + wn*WN + a*16 + 4*lq + r
  if (WITH_C) {
    const bool n4 = (N & 3) == 0;
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const int64_t tok = m0 + wm * WM + b * 16 + l16;
        if (tok >= M) continue;
        const int64_t f = n0 + wn * WN + a * 16 + 4 * lq;
        int32_t* dst = C + tok * N + f;
        if (n4 && f + 3 < N) {
          *reinterpret_cast<int4*>(dst) =
              make_int4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (f + e < N) dst[e] = acc[a][b][e];
        }
      }
  }
  if (!Y) return;

  // ---- fp16 output
  // Four 16-feature slices at a time go through this wave's part of the (now
  // idle) stage buffers: lane (l16, lq) packs its 4 features of token
  // b*16 + l16 to fp16 and writes them as 8 bytes of a [token][64 features]
  // row. The rows are read back contiguously, so 8 consecutive lanes store
  // one whole 128-byte row segment of Y: write misses reach memory as full
  // lines rather than as 8-byte pieces of 16 different rows.
  constexpr int OUT_ROW = Cfg::OUT_ROW;
  static_assert(TN % 4 == 0, "slices are stored in fours");
  int8_t* s_out = lds + Cfg::OUT0 + wave * (WM * OUT_ROW);
  const bool n8 = (N & 7) == 0;
  auto stage_tile = [&](int a, int b, const v4f32& y) {
    const uint32_t p0 = f2h2(y[0], y[1]);
    const uint32_t p1 = f2h2(y[2], y[3]);
    const int row = b * 16 + l16;
    const int col = (a & 3) * 32 + 8 * lq;   // byte offset in the row
    *reinterpret_cast<uint2*>(s_out + row * OUT_ROW + col) = make_uint2(p0, p1);
  };
  auto flush_four = [&](int a0) {
    // a0 = 4i: slices a0 .. a0+3 = features wn*WN + a0*16 + [0, 64)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t f = n0 + wn * WN + a0 * 16 + 8 * (lane & 7);
    // Streaming stores: Y is written once and not read back by this kernel,
    // so it should not displace operand lines in the caches.
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // (uniform) every row and feature of the 64-wide slab in range: all the
    // rows are read from LDS first, then stored, so that the stores do not
    // each wait for their own read
    const bool whole = n8 && n0 + wn * WN + a0 * 16 + 64 <= N && m0 + wm * WM + WM <= M;
    if (whole) {
      u32x4 v[WM / 8];
#pragma unroll
      for (int it = 0; it < WM / 8; ++it)
        v[it] = *reinterpret_cast<const u32x4*>(s_out + (it * 8 + (lane >> 3)) * OUT_ROW +
                                                16 * (lane & 7));
      uint16_t* dst = Y + (m0 + wm * WM + (lane >> 3)) * N + f;
#pragma unroll
      for (int it = 0; it < WM / 8; ++it)
        __builtin_nontemporal_store(v[it], reinterpret_cast<u32x4*>(dst + (int64_t)it * 8 * N));
    } else {
#pragma unroll 4
      for (int it = 0; it < WM / 8; ++it) {
        const int row = it * 8 + (lane >> 3);
        const uint4 v = *reinterpret_cast<const uint4*>(s_out + row * OUT_ROW + 16 * (lane & 7));
        const int64_t tok = m0 + wm * WM + row;
        if (tok < M) {
          uint16_t* dst = Y + tok * N + f;
          if (n8 && f + 7 < N) {
            __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (f + e < N) dst[e] = (uint16_t)half_of(v, e);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // LDS outlier fragments of v_mfma_f32_16x16x16_f16: 4 fp16 (t = 4*lq ..
  // 4*lq+3) of row l16 of a 16-row slice; the same lane -> t assignment on
  // the weight and the token side.
  auto wo_frag = [&](int a) -> v4f16 {
    return *reinterpret_cast<const v4f16*>(s_wo + (wn * WN + a * 16 + l16) * 16 + lq * 4);
  };
  auto xo_frag = [&](int b) -> v4f16 {
    return *reinterpret_cast<const v4f16*>(s_xo + (wm * WM + b * 16 + l16) * 16 + lq * 4);
  };

  // Fragments of outlier chunks beyond the first (more than 16 outlier
  // columns), built straight from global memory: the weight columns are read
  // from Wf when the weight is kept in fp16, else recovered from Wq as
  // fp16(fl32(fl32(q * sw) / 127)); the activations are read from Xo. Slow,
  // but it keeps the per-slice register footprint small.
  auto wo_frag_g = [&](int a, int t0) -> v4f16 {
    v4f16 w;
    const int64_t f = n0 + wn * WN + a * 16 + l16;
    const float swf = f < N ? sw[f] : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t0 + lq * 4 + e;
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
  auto xo_frag_g = [&](int b, int t0) -> v4f16 {
    const int64_t tok = m0 + wm * WM + b * 16 + l16;
    if (tok >= M) return v4f16{};
    return __builtin_bit_cast(v4f16, *reinterpret_cast<const uint2*>(Xo + tok * ldo + t0 + lq * 4));
  };

  // One 16-feature slice a at a time, its TM token tiles in VGPRs: dequantize
  // y = C * (sx/127) * (sw/127), add the fp16 outlier product on
  // v_mfma_f32_16x16x16_f16 (first 16 columns from the LDS-staged fragments,
  // further chunks from global memory), add the bias, store.
  // The LDS values a slice uses are read one slice ahead (the token-side ones
  // once): the compiler cannot move these reads past the staging stores of
  // the slice before, so read at the slice itself each would wait for its
  // own LDS round trip. The loop is instantiated with and without the bias
  // add, chosen by a uniform branch on the argument, so that without a bias
  // no instruction is spent on it.
  auto slices = [&](auto with_bias) __attribute__((always_inline)) {
    constexpr bool WB = decltype(with_bias)::value;
    const bool o_lds = n_o > 0 && !seg2;
    float ax_b[TM];
    v4f16 xo_b[TM];
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      ax_b[b] = s_ax[wm * WM + b * 16 + l16];
      xo_b[b] = o_lds ? xo_frag(b) : v4f16{};
    }
    float fw_n[4], bv_n[4];
    load_fw(0, fw_n, WB ? bv_n : nullptr);
    v4f16 wa_n = o_lds ? wo_frag(0) : v4f16{};
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      float fw[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        fw[r] = fw_n[r];
        bv[r] = WB ? bv_n[r] : 0.0f;
      }
      const v4f16 wa_lds = wa_n;
      if (a + 1 < TN) {
        load_fw(a + 1, fw_n, WB ? bv_n : nullptr);
        if (o_lds) wa_n = wo_frag(a + 1);
      }
      v4f32 y[TM];
      if (seg2) {
        // already dequantized, with the outlier product added (dense: still
        // without the factor sw/127)
#pragma unroll
        for (int b = 0; b < TM; ++b) {
          y[b] = __builtin_bit_cast(v4f32, acc[a][b]);
          if (dense && Wf == nullptr) {
#pragma unroll
            for (int r = 0; r < 4; ++r) y[b][r] = y[b][r] * fw[r];
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < TM; ++b) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[b][r] = (float)acc[a][b][r] * ax_b[b] * fw[r];
        }
      }
      if (o_lds) {
#pragma unroll
        for (int b = 0; b < TM; ++b)
          y[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(wa_lds, xo_b[b], y[b], 0, 0, 0);
      }
      for (int t0 = 16; t0 < (seg2 ? 0 : n_o); t0 += 16) {
        const v4f16 wa = wo_frag_g(a, t0);
#pragma unroll
        for (int b = 0; b < TM; ++b)
          y[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(wa, xo_frag_g(b, t0), y[b], 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        if constexpr (WB) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[b][r] += bv[r];
        }
        stage_tile(a, b, y[b]);
      }
      if ((a & 3) == 3) flush_four(a - 3);
    }
  };
  if (bias)
    slices(std::integral_constant<bool, true>{});
  else
    slices(std::integral_constant<bool, false>{});
}

template <class Cfg>
hipError_t launch_gemm_t(const int8_t* Xq, const int8_t* Wq, const float* sx, const float* sw,
                         int64_t M, int64_t N, int64_t K, const uint16_t* Xo, const int32_t* cols,
                         const int32_t* n_out, const uint16_t* bias, uint16_t* Y, int32_t* C,
                         const uint16_t* Wo, int wo_cols, const uint16_t* Wf, const uint16_t* Xd,
                         const uint32_t* bmp, const int32_t* kbl, hipStream_t s) {
  const dim3 grid((unsigned)(((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN)));
  const dim3 block(Cfg::THREADS);
  if (C) {
    // parity mode: the epilogue outlier path only
    hipLaunchKernelGGL((k_gemm_i8<Cfg, kInt32>), grid, block, 0, s, Xq, Wq, sx, sw, (int)M, (int)N,
                       (int)K, Xo, cols, n_out, bias, Y, C, nullptr, 0, Wf, nullptr, nullptr,
                       nullptr);
    return hipGetLastError();
  }
  // The outlier count is only known on the device: with a second segment
  // possible, its mode is launched too and the one whose case it is not
  // returns at once.
  hipLaunchKernelGGL((k_gemm_i8<Cfg, kPlain>), grid, block, 0, s, Xq, Wq, sx, sw, (int)M, (int)N,
                     (int)K, Xo, cols, n_out, bias, Y, C, Wo, wo_cols, Wf, Xd, bmp, nullptr);
  if (Wo) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_i8<Cfg, kOutlierSeg>), grid, block, 0, s, Xq, Wq, sx, sw, (int)M,
                       (int)N, (int)K, Xo, cols, n_out, bias, Y, C, Wo, wo_cols, Wf, Xd, bmp,
                       kbl);
  }
  if (Xd && bmp) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (Wf)
      hipLaunchKernelGGL((k_gemm_i8<Cfg, kDenseSegW>), grid, block, 0, s, Xq, Wq, sx, sw, (int)M,
                         (int)N, (int)K, Xo, cols, n_out, bias, Y, C, Wo, wo_cols, Wf, Xd, bmp,
                         kbl);
    else
      hipLaunchKernelGGL((k_gemm_i8<Cfg, kDenseSeg>), grid, block, 0, s, Xq, Wq, sx, sw, (int)M,
                         (int)N, (int)K, Xo, cols, n_out, bias, Y, C, Wo, wo_cols, Wf, Xd, bmp,
                         kbl);
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
                       const uint16_t* Wo, int wo_cols, const uint16_t* Wf,
                       const uint16_t* Xd, const uint32_t* bmp, const int32_t* kbl,
                       hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // (K == 0 goes to the tiled kernel, whose empty main loop leaves only the
  // epilogue: Y = bias, or 0)
  if (gemv_applies(M) && K > 0)
    return launch_gemv(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_out, bias, Y, C, Wf, s);
  // 256 x 256 tiles when they give every CU at least one; otherwise the
  // 128 x 128 tiles (four times as many, two blocks per CU).
  const int64_t tiles_large = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles_large >= kLargeTileMin)
    return launch_gemm_t<CfgLarge>(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_out, bias, Y, C, Wo,
                                   wo_cols, Wf, Xd, bmp, kbl, s);
  return launch_gemm_t<CfgSmall>(Xq, Wq, sx, sw, M, N, K, Xo, cols, n_out, bias, Y, C, Wo, wo_cols,
                                 Wf, Xd, bmp, kbl, s);
}

}  // namespace i8mm
