// Device helpers shared by the i8mm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

typedef int32_t v4i32 __attribute__((ext_vector_type(4)));
typedef int32_t v16i32 __attribute__((ext_vector_type(16)));
typedef float v16f32 __attribute__((ext_vector_type(16)));
typedef _Float16 v8f16 __attribute__((ext_vector_type(8)));
typedef _Float16 v4f16 __attribute__((ext_vector_type(4)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp16 bits <-> fp32. The widening conversion is exact; the narrowing one
// rounds to nearest even (the default rounding mode of the hardware).
__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// Two narrowing conversions at once (lo in bits 0-15, hi in 16-31): one
// v_cvt_pk_f16_f32, with the same rounding as f2h.
typedef float v2f32 __attribute__((ext_vector_type(2)));
typedef _Float16 v2f16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2h2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f32{lo, hi}, v2f16));
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

// Wave-wide maximum with DPP moves (VALU, no LDS round trips): a running
// maximum over each 16-lane row by row_shr 1, 2, 4, 8 leaves the row's
// maximum in its last lane; the four row maxima are read out as scalars.
// The result is uniform across the wave.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  // row_shr:n is DPP control 0x110 + n; bound_ctrl makes shifted-in lanes 0
  // (the identity of an unsigned maximum)
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);
  v = v > t ? v : t;
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// Inclusive prefix sum over the 64 lanes with DPP adds (no LDS round trips):
// within each 16-lane row by row_shr 1, 2, 4, 8 (lanes shifted in read 0),
// then row 0's last lane is added to row 1 and row 2's to row 3
// (row_bcast:15), and lane 31's total to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return v;
}

// OR over the four lanes of each quad (quad_perm [1,0,3,2], then [2,3,0,1]).
__device__ __forceinline__ uint32_t quad_or_dpp(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Half element e (0..7) of a 16-byte chunk.
__device__ __forceinline__ uint32_t half_of(const uint4& v, int e) {
  uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// int8 codes of 8 fp16 elements with the scale s: y = fl32(x * s); y + 1.5 *
// 2^23 rounds to the nearest integer with ties to even (the addend is even
// and |y| <= 127 < 2^22), so the low byte of its bit pattern is the two's
// complement code rne(y). No clamp is needed: s = fl32(127 / a) and
// abs(x) <= a give abs(y) <= 127 up to one rounding, and rne of that is
// within [-127, 127]. Returns the 8 codes packed little-endian.
__device__ __forceinline__ uint2 codes8_rne(const uint4& t, float s) {
  const float magic = 12582912.0f;
  uint32_t r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = h2f(half_of(t, e)) * s;
    r[e] = __builtin_bit_cast(uint32_t, y + magic);
  }
  const uint32_t lo01 = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);
  const uint32_t lo23 = __builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(r[5], r[4], 0x0c0c0400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(r[7], r[6], 0x0c0c0400u);
  return make_uint2(__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                    __builtin_amdgcn_perm(hi23, hi01, 0x05040100u));
}

// Buffer descriptor over [base, base + bytes): loads past `bytes` return 0,
// stores past it are dropped. The fields go through readfirstlane so the
// descriptor lives in SGPRs (callers pass wave-uniform values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// operations complete (lgkmcnt(0), gfx9 encoding), then s_barrier, with no
// fence on global memory, so nothing in flight there is waited for. The
// empty asm statements keep the compiler from moving memory accesses across
// the barrier.
__device__ __forceinline__ void lds_only_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool kLdsOnly>
__device__ __forceinline__ void block_sync() {
  if constexpr (kLdsOnly) lds_only_barrier();
  else __syncthreads();
}

// Outlier bitmap helpers for blocks of kBlockThreads threads.
constexpr int kBlockThreads = 256;

// Exclusive prefix of popcount over the bitmap words, in LDS. Returns the
// total (the outlier count n). All threads of the block must call it.
// kLdsOnly: its barriers order LDS only (no fence on global memory).
template <bool kLdsOnly = false>
__device__ inline int bitmap_prefix(const uint32_t* sbm, uint32_t* spre, int nwords, int* sred) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (nwords + kBlockThreads - 1) / kBlockThreads;
  const int w0 = tid * per;
  const int w1 = min(nwords, w0 + per);
  int local = 0;
  for (int w = w0; w < w1; ++w) local += __popc(sbm[w]);
  int incl = wave_inclusive_scan(local, lane);
  if (lane == 63) sred[wave] = incl;
  block_sync<kLdsOnly>();
  int wave_off = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kBlockThreads / kWave; ++i) {
    wave_off += i < wave ? sred[i] : 0;
    total += sred[i];
  }
  int run = wave_off + incl - local;
  for (int w = w0; w < w1; ++w) {
    spre[w] = (uint32_t)run;
    run += __popc(sbm[w]);
  }
  block_sync<kLdsOnly>();
  return total;
}

// Writes cols[p] = k for the p-th set bit k (ascending) and *n_out.
__device__ inline void write_cols(const uint32_t* sbm, const uint32_t* spre, int nwords, int n,
                           int32_t* __restrict__ cols, int32_t* __restrict__ n_out) {
  if (cols) {
    for (int w = threadIdx.x; w < nwords; w += kBlockThreads) {
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

// The 64-column k-blocks that hold at least one normal (non-outlier) column:
// kbl[0] = their count, kbl[1 ..] = their indices, ascending. Columns past K
// count as outlier columns. The int8 GEMM visits only these blocks when many
// columns are outliers (an all-outlier block has only zero codes). Wave 0 of
// the block, 64 k-blocks per pass; sbm holds the bitmap.
__device__ inline void write_kblocks(const uint32_t* sbm, int64_t K, int32_t* __restrict__ kbl) {
  if (!kbl || threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int nkb = (int)((K + 63) / 64);
  int base = 0;
  for (int kb0 = 0; kb0 < nkb; kb0 += kWave) {
    const int kb = kb0 + lane;
    bool act = false;
    if (kb < nkb) {
      const int valid = (int)(K - (int64_t)kb * 64 < 64 ? K - (int64_t)kb * 64 : 64);
      const uint32_t m0 = valid >= 32 ? 0xffffffffu : (1u << valid) - 1u;
      act = (sbm[2 * kb] & m0) != m0;
      if (valid > 32) {
        const uint32_t m1 = valid >= 64 ? 0xffffffffu : (1u << (valid - 32)) - 1u;
        act = act || (sbm[2 * kb + 1] & m1) != m1;
      }
    }
    const uint64_t b = __ballot(act);
    if (act) kbl[1 + base + __popcll(b & ((1ull << lane) - 1ull))] = kb;
    base += __popcll(b);
  }
  if (lane == 0) kbl[0] = base;
}

}  // namespace i8mm
