// sa_device.h -- small device helpers shared by the kernels of libsinkattn.
#pragma once

#include "sa_internal.h"

namespace sa {

// Document holding token t: the largest n < D with cu[n] <= t, for 0 <= t < T.
// Empty documents (cu[n] == cu[n+1]) are skipped because the search keeps the
// last index whose start is <= t.
__device__ inline int doc_of_token(const int32_t* __restrict__ cu, int D, int t) {
  int lo = 0, hi = D - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Document of token t for the lanes of one wave, called by all 64 lanes, with
// every lane's t inside [t_lo, t_hi] (wave-uniform bounds in [0, T)).  Lanes
// 0-31 narrow down the document of t_lo and lanes 32-63 that of t_hi: each
// lane tests one of 32 evenly spaced document starts per level and a ballot
// keeps the last one that passes (cu is non-decreasing), so up to 1,024
// documents take two dependent loads and up to 32,768 three, where a binary
// search takes 10 or 15.  Each lane then searches between the two results,
// which for a wave's few consecutive tokens are mostly the same document.
__device__ inline int doc_of_token_wave(const int32_t* __restrict__ cu, int D, int t, int t_lo,
                                        int t_hi) {
  const int lane = __lane_id();
  const int half = lane >> 5, sub = lane & 31;
  const int tq = half ? t_hi : t_lo;
  int lo = 0, hi = D - 1;  // cu[lo] <= tq (cu[0] == 0); uniform within a half
  for (;;) {
    const bool busy = hi > lo;
    if (!__any(busy)) break;
    const int step = (hi - lo + 32) / 32;
    const int idx = lo + sub * step;
    const bool le = busy && idx <= hi && cu[idx] <= tq;
    const unsigned long long m = __ballot(le);
    const unsigned mh = half ? (unsigned)(m >> 32) : (unsigned)m;
    if (busy) {
      // (a count of 0 is possible only for a malformed cu with cu[0] > t;
      // clamping keeps every read in bounds whatever cu holds)
      lo += max(__popc(mh) - 1, 0) * step;
      hi = min(hi, lo + step - 1);
    }
  }
  int a = __shfl(lo, 0), b = __shfl(lo, 32);
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (cu[mid] <= t) a = mid;
    else b = mid - 1;
  }
  return a;
}

// Minimum / maximum of x over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = min(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = max(x, __shfl_xor(x, m));
  return x;
}

// sin and cos of the NeoX RoPE angle p * inv_freq (flint.layers,
// FlintAttention._apply_rope).  The product is formed and reduced modulo 2*pi
// in fp64 so positions up to 2^31 keep a fp32-accurate angle; the reduced
// angle then goes through the accurate fp32 sincos.
__device__ inline void rope_sincos(int p, double inv_freq, float* s, float* c) {
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  double ang = (double)p * inv_freq;
  ang -= two_pi * rint(ang * inv_two_pi);
  sincosf((float)ang, s, c);
}

// sin and cos of the RoPE angle for the bf16 paths: the angle is carried in
// revolutions (p * inv_freq / 2pi), reduced to [-1/2, 1/2] in fp64, and fed
// to v_sin_f32 / v_cos_f32, which take revolutions.  Their error (~1e-6) is far
// below the bf16 rounding the rotated vector gets next.
__device__ inline void rope_sincos_rev(int p, double inv_freq_rev, float* s, float* c) {
  double r = (double)p * inv_freq_rev;
  r -= rint(r);
  const float rf = (float)r;
  *s = __builtin_amdgcn_sinf(rf);
  *c = __builtin_amdgcn_cosf(rf);
}

// Workgroup barrier that leaves outstanding global loads (LDS copies of later
// tiles, operand loads) in flight: it waits only for the wave's own LDS
// accesses (lgkmcnt(0)), whose results the code before it has consumed or
// stored.  The memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void barrier_keep_copies() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- RoPE angles of a block of query tokens --------------------------------
// The G query heads of a token rotate by the same angles, so a workgroup
// writes (cos, sin) of each (token, frequency) pair of its tokens once into an
// LDS table and every lane reads its 32 pairs from there.  Row r (token a + r)
// is kRopeRow bytes: 64 pairs and 16 bytes more, so that the rows of the
// different tokens a wave reads start 4 banks apart.
constexpr int kRopeRow = 64 * 8 + 16;

// Fill rows [0, rows) of the table for the tokens a + r < a_end of a document
// that starts at doc_start (positions a + r - doc_start), head_dim 128:
// thread tid computes frequency i = tid % 64, theta^(-i/64) in revolutions,
// for rows tid / 64, tid / 64 + nthreads / 64, ...
__device__ inline void rope_table(char* tab, int tid, int nthreads, int rows, int a, int a_end,
                                  int doc_start, double theta) {
  const int i = tid & 63;
  const double invf = pow(theta, -(double)i / 64.0) * kInvTwoPi;
  for (int r = tid >> 6; r < rows && a + r < a_end; r += nthreads >> 6) {
    float sn, cs;
    rope_sincos_rev(a + r - doc_start, invf, &sn, &cs);
    *reinterpret_cast<float2*>(tab + r * kRopeRow + 8 * i) = make_float2(cs, sn);
  }
}

// Rotate the 64 channels a lane holds (x[8kk + e] = channel 16kk + 8hf + e,
// NeoX partners kk and kk + 4) by the angles of table row `row`.
__device__ __forceinline__ void rope_from_table(const char* row, int hf, float (&x)[64]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    // pairs 16kk + 8hf + e, e < 8: four 16-byte reads of (cos, sin, cos, sin)
    const char* p = row + 128 * kk + 64 * hf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 cs = *reinterpret_cast<const float4*>(p + 16 * j);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * j + u;
        const float c = u ? cs.z : cs.x, sn = u ? cs.w : cs.y;
        const float x1 = x[8 * kk + e], x2 = x[8 * (kk + 4) + e];
        x[8 * kk + e] = x1 * c - x2 * sn;
        x[8 * (kk + 4) + e] = x2 * c + x1 * sn;
      }
    }
  }
}

// Layout of the key/value tiles the prologue writes and the attention kernel
// copies verbatim into LDS (64 keys per tile, 16-byte chunks XOR-swizzled so
// the MFMA operand reads, 32 lanes on 32 rows at one column, hit distinct
// banks for a 32- or 64-bank LDS):
//   k_hat tile: 64 rows (keys) x 256 B; chunk c (channels 8c..8c+7) of row r
//               sits at chunk position c ^ kswz(r)
//   V^T tile:   128 rows (channels) x 128 B; chunk c (8 keys) of row r sits at
//               chunk position c ^ vswz(r)
// vswz keeps positions distinct over any 8 consecutive rows and the pairs
// (row parity, position) distinct over any 16.
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// max / sum of x over the lane pair (l, l ^ 32): v_permlane32_swap exchanges
// the upper half of one operand with the lower half of the other, so with x
// in both operands each lane ends up holding x[l] and x[l ^ 32].
__device__ __forceinline__ float lane_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- band masks ------------------------------------------------------------
// Register r of a lane's 32x32 MFMA accumulator holds row 8(r/4) + r%4 + 4hf
// (hf = lane / 32) of its block.  A mask is built once per lane and block as
// a word whose bit k says whether row offset k (from the lane's first row) is
// visible; the visible rows of a causal, window or document band always form
// one run of offsets.

// Bits lo .. hi of a word, none when hi < lo (0 <= lo <= 31 when hi >= lo,
// hi <= 31).  The shift counts are masked so that both sides of the final
// select are defined and the compiler forms a select, not a branch.
__device__ __forceinline__ unsigned bit_run(int lo, int hi) {
  const unsigned run = ((2u << ((hi - lo) & 31)) - 1u) << (lo & 31);
  return hi >= lo ? run : 0u;
}

// s when bit k of vis is set, -inf otherwise: a sign-extended bit extract
// (v_bfe_i32) and a bit select (v_bitop3).  No lane mask is formed, so there
// is neither a VCC dependency chain nor scalar-unit work per score.
__device__ __forceinline__ float keep_if(unsigned vis, int k, float s) {
  const unsigned on = (unsigned)((int)(vis << (31 - k)) >> 31);
  return __uint_as_float((__float_as_uint(s) & on) | (~on & 0xff800000u));
}

// ---- 16-bit element helpers (E = bf16 or f16) -----------------------------

// C += A B on the 32x32x16 MFMA of the element type (fp32 accumulation).
template <typename E>
__device__ __forceinline__ f32x16 mfma32(vec8<E> a, vec8<E> b, f32x16 c) {
  if constexpr (is_f16<E>) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// c + a0 b0 + a1 b1 in fp32 (v_dot2_f32_{bf16,f16}).
template <typename E>
__device__ __forceinline__ float dot2(vec2<E> a, vec2<E> b, float c) {
  if constexpr (is_f16<E>) return __builtin_amdgcn_fdot2(a, b, c, false);
  else return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// A softmax reference point (log2 domain) that E represents exactly, so an
// MFMA step with E operands can subtract it without error.  fp16 tops out at
// 65504: references are held within +-2^15 there (scores and sinks beyond
// about 22,700 in natural-log units are outside the fp16 path's range).
template <typename E>
__device__ __forceinline__ float ref_round(float x) {
  if constexpr (is_f16<E>) return (float)(E)fminf(fmaxf(x, -32768.f), 32768.f);
  else return (float)(E)x;
}

// ---- AGPR-resident accumulation by inline-asm MFMA -------------------------
// C += A B into an accumulator the compiler keeps in AGPRs.  The compiler
// cannot see the hazards of these inline-asm MFMAs: the caller inserts the
// two wait states an MFMA needs after VALU code wrote a or b (mfma32_acc_nop,
// or an explicit s_nop 1), and agpr_fence() before VALU code touches an
// accumulator an MFMA just wrote.
template <typename E>
__device__ __forceinline__ void mfma32_acc(f32x16& acc, vec8<E> a, vec8<E> b) {
  if constexpr (is_f16<E>)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The same with the two wait states a VALU write of a or b needs first.
template <typename E>
__device__ __forceinline__ void mfma32_acc_nop(f32x16& acc, vec8<E> a, vec8<E> b) {
  if constexpr (is_f16<E>)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Zero an AGPR accumulator with an MFMA of zero operands, so that every
// definition of the accumulator is an AGPR one and the register allocator
// never moves it through VGPRs (s_nop 1: the zero operand was just written
// by VALU code).
template <typename E>
__device__ __forceinline__ void zero_acc(f32x16& acc, vec8<E> zero) {
  if constexpr (is_f16<E>)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %1, 0" : "=a"(acc) : "v"(zero));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(zero));
}

// Wait states before VALU code reads or writes accumulators that an
// inline-asm MFMA wrote.
__device__ __forceinline__ void agpr_fence() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// One 16-byte MFMA operand (8 elements) from LDS or global memory.
template <typename E>
__device__ __forceinline__ vec8<E> rd(const char* p) {
  return *reinterpret_cast<const vec8<E>*>(p);
}

}  // namespace sa
