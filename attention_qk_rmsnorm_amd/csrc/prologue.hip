// prologue.hip -- first stage of the forward pass.
//
// 16-bit path (bf16 or fp16 k, v and images; fp32 arithmetic), one launch:
//   * blocks 0 and 1 build the varlen work schedules from cu_seqlens, one per
//     attention tile configuration (query blocks of 128/G and 256/G tokens):
//     the number of query blocks of every document, their exclusive prefix,
//     and the table of (document, block) items the attention grid walks,
//     longest-running (highest position) blocks first.
//   * every other block takes 64 consecutive tokens (one key tile) of one kv
//     head and
//       - applies per-head RMSNorm and, when enabled, NeoX RoPE to K
//         (flint.layers FlintAttention: q_norm / k_norm, _apply_rope; positions
//         are document-local), writing k_hat [Hkv][t_pad][128] in the input's
//         16-bit type;
//       - writes V transposed, one [128][64] block per key tile (keys permuted
//         inside groups of 16, see below) so the PV product reads its operand
//         with one 16-byte LDS load.
//     Both are written as the exact byte image the attention kernel keeps in
//     LDS (16-byte chunks swizzled, see sa_device.h), so its tile copy is a
//     straight 16 KiB memcpy.
//     Padding keys [T, t_pad) and document padding (tokens past a
//     document's real end, cu_end) are written as zeros.
// fp32 debug path: RMSNorm (+RoPE) of K into k_hat fp32 [T][Hkv][d], and a
// copy of V beside it, so the attention stage reads only the workspace.
#include "sa_device.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kLdsPrefix = 4096;  // documents whose prefix fits in LDS

// Varlen schedule.  sched[0] = number of items; items (int2 at sched + 4) hold
// (document, block index in document) in descending order of block position.
// s_scan (kThreads ints) and s_pref (kLdsPrefix ints) are LDS arrays; prefix_g
// is global scratch of D + 1 ints used when D + 1 > kLdsPrefix.
__device__ void build_schedule(const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_end,
                               int D, int m_tok,
                               int32_t* __restrict__ sched, int64_t items_ub,
                               int32_t* __restrict__ prefix_g, int* s_scan, int* s_pref) {
  const int tid = threadIdx.x;
  const bool in_lds = D + 1 <= kLdsPrefix;
  int* pref = in_lds ? s_pref : prefix_g;
  int running = 0;
  for (int base = 0; base < D; base += kThreads) {
    const int n = base + tid;
    int cnt = 0;
    if (n < D) {
      const int len = cu_end[n] - cu[n];
      cnt = len > 0 ? (len + m_tok - 1) / m_tok : 0;
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    if (n < D) pref[n] = running + s_scan[tid] - cnt;
    running += s_scan[kThreads - 1];
    __syncthreads();
  }
  // A malformed cu_seqlens could ask for more items than the grid covers;
  // never write past the table.
  if (running > items_ub) running = (int)items_ub;
  if (tid == 0) {
    pref[D] = running;
    sched[0] = running;
  }
  __threadfence_block();
  __syncthreads();
  int2* items = reinterpret_cast<int2*>(sched + 4);
  for (int j = tid; j < running; j += kThreads) {
    int lo = 0, hi = D - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= j) lo = mid;
      else hi = mid - 1;
    }
    items[running - 1 - j] = make_int2(lo, j - pref[lo]);
  }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void prologue_16_kernel(
    const E* __restrict__ k, const E* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_end,
    const float* __restrict__ knorm_w, int T, int D,
    int Hkv, int64_t t_pad, int m_tok, int m_tok_wide, float eps, double theta,
    int use_rope, E* __restrict__ khat, E* __restrict__ vt,
    int32_t* __restrict__ sched, int32_t* __restrict__ sched_wide) {
  // One LDS buffer: the V tile of a key-tile block, or the scan and prefix
  // arrays of the two schedule blocks (so the key-tile blocks, nearly all of
  // the grid, do not reserve the schedule's arrays: 8 blocks fit on a CU).
  constexpr int kVBytes = kKeyTile * (kHeadDim + 8) * (int)sizeof(E);
  constexpr int kSchedBytes = (kThreads + kLdsPrefix) * (int)sizeof(int);
  __shared__ __attribute__((aligned(16))) char s_mem[kVBytes > kSchedBytes ? kVBytes : kSchedBytes];
  if (blockIdx.x < 2) {
    const bool wide = blockIdx.x == 1;
    const int mt = wide ? m_tok_wide : m_tok;
    const int64_t items_ub = T / mt + D;
    int32_t* sc = wide ? sched_wide : sched;
    int* s_scan = reinterpret_cast<int*>(s_mem);
    build_schedule(cu, cu_end, D, mt, sc, items_ub, sc + 4 + 2 * items_ub, s_scan,
                   s_scan + kThreads);
    return;
  }
  __shared__ double s_invf[64];
  auto s_v = reinterpret_cast<E(*)[kHeadDim + 8]>(s_mem);

  const int tid = threadIdx.x;
  const int blk = blockIdx.x - 2;
  const int tile = blk / Hkv;
  const int g = blk - tile * Hkv;
  const int t0 = tile * kKeyTile;

  // inv_freq_i / 2pi with inv_freq_i = theta^(-2i/128), i < 64: NeoX pairs
  // channel i with i + 64 (wave 1: wave 0 runs the document search below)
  if (use_rope && tid >= 64 && tid < 128)
    s_invf[tid - 64] = pow(theta, -(double)(tid - 64) / 64.0) * kInvTwoPi;

  // The tile's V and K rows go out first: the document lookup below takes a
  // few dependent loads, and without this the rows would be requested only
  // after it.  The loads are unconditional -- a token at or past T reads row
  // T - 1 -- so that no register merge makes the compiler wait for them
  // here; rows of padding keys and of document padding are zeroed once the
  // documents are known (s_real).
  uint4 vval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int t = min(t0 + (c >> 4), T - 1);
    vval[i] = *reinterpret_cast<const uint4*>(v + ((size_t)t * Hkv + g) * kHeadDim + (c & 15) * 8);
  }
  // K rows: 8 lanes per token; lane c holds channels 8c..8c+7 and 64+8c..64+8c+7
  vec8<E> krow[2][2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int t = min(t0 + (tid >> 3) + 32 * it, T - 1);
    const E* kp = k + ((size_t)t * Hkv + g) * kHeadDim;
    krow[it][0] = *reinterpret_cast<const vec8<E>*>(kp + 8 * (tid & 7));
    krow[it][1] = *reinterpret_cast<const vec8<E>*>(kp + 64 + 8 * (tid & 7));
  }
  // the norm weights of the lane's channels, with the rows
  float wk[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wk[e] = knorm_w[8 * (tid & 7) + e];
    wk[8 + e] = knorm_w[64 + 8 * (tid & 7) + e];
  }

  // Documents of the tile's tokens.  cu[d0 .. d0 + 64] and cu_end[d0 ..
  // d0 + 63] go to LDS, where each token finds its own document, its start
  // and whether it is real.  With at most 64 documents d0 = 0 and the LDS
  // copy holds every start.  Otherwise wave 0 first finds the document d0 of
  // the first token (the largest d < D with cu[d] <= t0) level by level: each
  // lane tests one of 64 evenly spaced candidates and a ballot keeps the last
  // one that passes (cu is non-decreasing), so D <= 4096 takes two dependent
  // loads instead of a binary search's 12; a tile that crosses more than 64
  // document starts (empty documents) falls back to a search in memory.
  __shared__ int s_d0;
  __shared__ int s_cu[kKeyTile + 1];
  __shared__ int s_end[kKeyTile];
  __shared__ int s_real[kKeyTile];  // token inside [0, T) and not document padding
  __shared__ int s_pos0[kKeyTile];  // start of the token's document (RoPE positions)
  if (D > kKeyTile) {
    if (tid < 64) {
      int lo = 0, hi = D - 1;  // cu[lo] <= t0 (cu[0] == 0)
      const int tq = min(t0, T - 1);
      while (hi > lo) {
        const int step = (hi - lo + 64) / 64;
        const int idx = lo + tid * step;
        const bool le = idx <= hi && cu[idx] <= tq;
        const int cnt = __popcll(__ballot(le));
        // (cnt is 0 only for a malformed cu with cu[0] > t0; clamping keeps
        // every read in bounds whatever cu holds)
        lo += max(cnt - 1, 0) * step;
        hi = min(hi, lo + step - 1);
      }
      if (tid == 0) s_d0 = lo;
    }
    __syncthreads();
  }
  const int d0 = D > kKeyTile ? s_d0 : 0;
  if (tid <= kKeyTile) s_cu[tid] = d0 + tid <= D ? cu[d0 + tid] : INT_MAX;
  if (tid >= 128 && tid < 128 + kKeyTile) {
    const int j = tid - 128;
    s_end[j] = d0 + j < D ? cu_end[d0 + j] : 0;
  }
  __syncthreads();
  if (tid < kKeyTile) {
    const int t = t0 + tid;
    int real = 0, pos0 = 0;
    if (t < T) {
      const int jmax = min(kKeyTile, D - 1 - d0);  // documents d0 .. d0 + jmax
      if (jmax == kKeyTile && s_cu[kKeyTile] <= t) {
        const int d = doc_of_token(cu, D, t);
        pos0 = cu[d];
        real = t < cu_end[d];
      } else {
        int a = 0, b = jmax;  // largest j <= jmax with s_cu[j] <= t
        while (a < b) {
          const int mid = (a + b + 1) >> 1;
          if (s_cu[mid] <= t) a = mid;
          else b = mid - 1;
        }
        pos0 = s_cu[a];
        real = t < s_end[a];
      }
    }
    s_real[tid] = real;
    s_pos0[tid] = pos0;
  }
  __syncthreads();

  // V tile [64 tokens][128] into LDS
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int tt = c >> 4, cc = c & 15;
    // (a mask per word: a select of the whole vector goes through scratch)
    const unsigned m = s_real[tt] ? 0xFFFFFFFFu : 0u;
    const uint4 val = make_uint4(vval[i].x & m, vval[i].y & m, vval[i].z & m, vval[i].w & m);
    *reinterpret_cast<uint4*>(&s_v[tt][cc * 8]) = val;
  }
  __syncthreads();

#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int tt = (tid >> 3) + 32 * it;
    const int c = tid & 7;
    const int t = t0 + tt;
    const bool real = s_real[tt];
    float x[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = real ? (float)krow[it][0][e] : 0.f;
      x[8 + e] = real ? (float)krow[it][1][e] : 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss += x[e] * x[e];
    ss += __shfl_xor(ss, 1, 8);
    ss += __shfl_xor(ss, 2, 8);
    ss += __shfl_xor(ss, 4, 8);
    // rows that are not real stay zero (no 0 * inf when eps == 0)
    const float inv = real ? 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps) : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] *= inv * wk[e];
      x[8 + e] *= inv * wk[8 + e];
    }
    if (use_rope && real) {
      const int p = t - s_pos0[tt];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rope_sincos_rev(p, s_invf[8 * c + e], &sn, &cs);
        const float a = x[e], b = x[8 + e];
        x[e] = a * cs - b * sn;
        x[8 + e] = b * cs + a * sn;
      }
    }
    vec8<E> lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = (E)x[e];
      hi[e] = (E)x[8 + e];
    }
    // row t of the tile image: chunk c at position c ^ kswz(t)
    E* kh = khat + ((size_t)g * t_pad + t) * kHeadDim;
    *reinterpret_cast<vec8<E>*>(kh + 8 * (c ^ kswz(t))) = lo;
    *reinterpret_cast<vec8<E>*>(kh + 8 * ((c + 8) ^ kswz(t))) = hi;
  }

  // V^T rows: lane (d, 8-position chunk) writes 16 contiguous bytes of row d.
  // Inside each group of 16 keys, position q holds key q with bits 2 and 3
  // swapped (0-3, 8-11, 4-7, 12-15): the order in which the attention
  // kernel's PV MFMA takes its A operand, so that operand is one 16-byte read.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pidx = tid + kThreads * i;
    const int tc = pidx & 7, d = pidx >> 3;
    const int kbase16 = 16 * (tc >> 1) + 4 * (tc & 1);
    vec8<E> col;
#pragma unroll
    for (int e = 0; e < 8; ++e) col[e] = s_v[kbase16 + 8 * (e >> 2) + (e & 3)][d];
    // tile-major image: tile (g, tile) is 128 rows x 64 keys, chunk tc of
    // row d at position tc ^ vswz(d)
    E* vrow = vt + (((size_t)g * (t_pad / kKeyTile) + tile) * kHeadDim + d) * kKeyTile;
    *reinterpret_cast<vec8<E>*>(vrow + 8 * (tc ^ vswz(d))) = col;
  }
}

template <int HD>
__global__ __launch_bounds__(kThreads) void prologue_f32_kernel(
    const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_end,
    const float* __restrict__ knorm_w, int T, int D,
    int Hkv, float eps, double theta, int use_rope, float* __restrict__ khat,
    float* __restrict__ vcopy) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)T * Hkv) return;
  const int t = (int)(idx / Hkv);
  const bool real = t < cu_end[doc_of_token(cu, D, t)];  // else document padding
  const float* kp = k + idx * HD;
  float x[HD];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < HD; ++i) {
    x[i] = real ? kp[i] : 0.f;
    ss += x[i] * x[i];
  }
  const float inv = real ? 1.0f / sqrtf(ss * (1.0f / HD) + eps) : 0.f;
#pragma unroll
  for (int i = 0; i < HD; ++i) x[i] *= inv * knorm_w[i];
  if (use_rope) {
    const int p = t - cu[doc_of_token(cu, D, t)];
    for (int i = 0; i < HD / 2; ++i) {
      float sn, cs;
      rope_sincos(p, pow(theta, -2.0 * i / HD), &sn, &cs);
      const float a = x[i], b = x[i + HD / 2];
      x[i] = a * cs - b * sn;
      x[i + HD / 2] = b * cs + a * sn;
    }
  }
  float* kh = khat + idx * HD;
  const float* vp = v + idx * HD;
  float* vc = vcopy + idx * HD;
#pragma unroll
  for (int i = 0; i < HD; ++i) {
    kh[i] = x[i];
    vc[i] = real ? vp[i] : 0.f;
  }
}

}  // namespace

template <typename E>
hipError_t launch_prologue_16(const E* k, const E* v, const int32_t* cu,
                                const int32_t* cu_end, const float* knorm_w, int T, int D, int Hkv,
                                int64_t t_pad, int m_tok, int m_tok_wide, double eps,
                                double theta, int use_rope, E* khat, E* vt,
                                int32_t* sched, int32_t* sched_wide, hipStream_t stream) {
  const int64_t n_tiles = t_pad / kKeyTile;
  const int64_t grid = 2 + n_tiles * Hkv;
  prologue_16_kernel<E><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      k, v, cu, cu_end, knorm_w, T, D, Hkv, t_pad, m_tok, m_tok_wide, (float)eps, theta, use_rope,
      khat, vt, sched, sched_wide);
  return hipGetLastError();
}

#define SA_INSTANTIATE(E)                                                                    \
  template hipError_t launch_prologue_16<E>(const E*, const E*, const int32_t*,            \
                                              const int32_t*, const float*, int, int, int,   \
                                              int64_t, int, int, double, double, int, E*, E*, \
                                              int32_t*, int32_t*, hipStream_t);
SA_INSTANTIATE(bf16)
SA_INSTANTIATE(f16)
#undef SA_INSTANTIATE

hipError_t launch_prologue_f32(const float* k, const float* v, const int32_t* cu,
                               const int32_t* cu_end, const float* knorm_w, int T, int D, int Hkv, int d,
                               double eps, double theta, int use_rope, float* khat,
                               float* vcopy, hipStream_t stream) {
  const int64_t n = (int64_t)T * Hkv;
  const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
  if (d == 128)
    prologue_f32_kernel<128><<<grid, kThreads, 0, stream>>>(
        k, v, cu, cu_end, knorm_w, T, D, Hkv, (float)eps, theta, use_rope, khat, vcopy);
  else
    prologue_f32_kernel<64><<<grid, kThreads, 0, stream>>>(
        k, v, cu, cu_end, knorm_w, T, D, Hkv, (float)eps, theta, use_rope, khat, vcopy);
  return hipGetLastError();
}

}  // namespace sa
