// attn_bf16.hip -- sink-aware GQA attention forward, bf16 in/out, gfx950 MFMA.
//
// Computes, for every (token t, query head h) of a packed THD batch
//   out = sum_{j visible} exp(s_j - M) v_j / (exp(sink_h - M) + sum_j exp(s_j - M))
//   lse = M + log(denominator)
// with s_j = scale * <q_hat, k_hat_j> (flint.layers FlintAttention.forward: causal
// attention with a zero-value sink category; _FlintSinkParameters: unscaled fp32
// logits), keys j <= t of the same document and, for a window W > 0,
// t - W < j (flint.config: the window counts the current token).
//
// Workgroup = 4 waves = one query block of one kv head g: tokens
// [a, a + 128/G) of one document, times the G query heads that read kv head g.
// Each wave owns 32 (token, head) columns.  RMSNorm and RoPE of the wave's
// queries are done once at the start, in fp32, straight into bf16 MFMA
// operands.  The key loop walks 64-key tiles of k_hat and V^T (written by the
// prologue), copied global -> LDS by global_load_lds_dwordx4 (no VGPR
// staging) into one of two buffers while the other is consumed; the tile is
// shared by all 4 waves, i.e. by the 8 query heads of the group at 4 tokens
// per wave.  Per tile and wave:
//   S^T[key][col] = K Q^T      2 x 8 v_mfma_f32_32x32x16_bf16
//   online softmax in the log2 domain, the sink seeding the running max and
//   denominator; band masks only on tiles that cross a document, causal or
//   window edge; tiles outside the band are never visited
//   O^T[d][col] += V^T P^T     16 v_mfma_f32_32x32x16_bf16 (P rounded to bf16)
// MFMA operand layouts (32x32x16, wave64): A lane l holds A[l%32][8(l/32)..+7],
// B lane l holds B[8(l/32)..+7][l%32], and accumulator register r of lane l is
// C[8(r/4) + 4(l/32) + r%4][l%32].  With S^T in that layout a lane holds 16 keys
// of one query column, so a column's max needs a single exchange with lane l^32
// and every O^T entry of a lane belongs to one column.
#include "sa_device.h"

namespace sa {

namespace {

constexpr int kThreads = kWaves * 64;
constexpr int kTileK = kKeyTile * kHeadDim * 2;   // bytes of one k_hat tile (16 KiB)
constexpr int kTileV = kHeadDim * kKeyTile * 2;   // bytes of one V^T tile (16 KiB)
constexpr int kBuf = kTileK + kTileV;             // one LDS buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // log2-domain slack before the running max moves

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tile layouts.  One global_load_lds_dwordx4 writes 64 lanes x 16 B
// contiguously, so rows cannot be padded; 16-byte chunks are XOR-swizzled
// instead so the MFMA operand reads (32 lanes on 32 rows, one column) spread
// over all banks (for a 32- or 64-bank LDS):
//   k_hat tile: row r = key (256 B), chunk c stored at c ^ (r & 15)
//   V^T tile:   row r = channel (128 B), chunk c stored at c ^ vswz(r)
// vswz(r) = (r & 7) ^ ((r >> 3) & 1) keeps chunk positions distinct over any
// 8 consecutive rows and the (row parity, chunk) pairs distinct over 16 rows.
__device__ __forceinline__ int vswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Issue the direct-to-LDS copy of the 64-key tile at kt into buffer `buf`:
// 4 + 4 16-byte loads per thread; chunk C = 256 i + tid lands at byte 16 C.
__device__ __forceinline__ void issue_tile(const bf16* __restrict__ kbase,
                                           const bf16* __restrict__ vbase, int64_t t_pad,
                                           int kt, int tid, char* buf) {
  char* wbase = buf + (tid >> 6) * 1024;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int C = kThreads * i + tid;
    const int rk = C >> 4, ck = (C & 15) ^ (rk & 15);
    __builtin_amdgcn_global_load_lds(kbase + (size_t)(kt + rk) * kHeadDim + ck * 8,
                                     (lds_void*)(wbase + 4096 * i), 16, 0, 0);
    const int rv = C >> 3, cv = (C & 7) ^ vswz(rv);
    __builtin_amdgcn_global_load_lds(vbase + (size_t)rv * t_pad + kt + cv * 8,
                                     (lds_void*)(wbase + kTileK + 4096 * i), 16, 0, 0);
  }
}

// Per-lane state of one wave's 32 query columns.
struct ColState {
  bf16x8 qf[8];     // Q^T B operands, channels 16kk + 8hf .. +7
  f32x16 o[4];      // O^T accumulators, channels 32dd + ...
  float m_run;      // reference max (log2 domain, scaled scores)
  float l_part;     // this lane's share of the denominator
};

// One 64-key tile for one wave: S^T = K Q^T, masked online softmax with the
// sink-seeded state, O^T += V^T P^T.  `buf` is the LDS buffer holding the tile.
template <int BUF>
__device__ __forceinline__ void attend_tile(const char* lds, const int (&koff)[8],
                                            const int (&voff)[4], ColState& st, int kt,
                                            int col, int hf, int tok, bool tok_ok, int tw0,
                                            int tw1, int doc_start, int window, float c_log2) {
  const char* buf = lds + BUF * kBuf;
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(buf + kb * 32 * 256 + koff[kk]);
      s[kb] = mfma32(ka, st.qf[kk], s[kb]);
    }
  }

  // band mask, only on tiles that cross a document, causal or window edge
  const bool full = kt >= doc_start && kt + kKeyTile - 1 <= tw0 &&
                    (window < 0 || kt > tw1 - 1 - window);
  if (!full) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int u = kt + kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
        const bool vis = tok_ok && u >= doc_start && u <= tok && (window < 0 || u > tok - window);
        s[kb][r] = vis ? s[kb][r] : -INFINITY;
      }
  }
  // column max of the raw scores (both lane halves hold keys of a column)
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * c_log2;

  // Lazy rescale: the reference point m_run moves only when a score exceeds
  // it by more than kLazy (log2 units), so weights stay <= 2^kLazy and the
  // O / l rescale runs on the few tiles where the max jumps.  The result is
  // the same softmax; lse uses the reference actually kept.
  const bool grow = mx > st.m_run + kLazy;
  if (__any(grow)) {
    const float m_new = grow ? mx : st.m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m_run - m_new) : 1.f;
    st.m_run = m_new;
    st.l_part *= alpha;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[dd][r] *= alpha;
  }
  const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;

  // P = exp2(s * scale * log2e - m) straight into bf16 B operands; the
  // denominator sums the same bf16 weights the PV product uses.
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      // B operand: k-slot 8hf + e <-> key kb*32 + 16sp + 8(e/4) + 4hf + e%4;
      // the prologue stored V^T keys in exactly this order inside each group
      // of 16, so the A operand is one 16-byte read.
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[e] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][8 * sp + e], c_log2, -m_use));
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pb[e], pb[e + 1]};
        st.l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, st.l_part, false);
      }
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(buf + kTileK + dd * 4096 +
                                                           voff[2 * kb + sp]);
        st.o[dd] = mfma32(va, pb, st.o[dd]);
      }
    }
}

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ khat,
    const bf16* __restrict__ vt, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ sched, const float* __restrict__ sinks,
    const float* __restrict__ qnorm_w, bf16* __restrict__ out, float* __restrict__ lse,
    int T, int Hq, int Hkv, int G, int log2G, int64_t t_pad, int window, int use_rope,
    float eps, double theta, float c_log2, int xcd_per) {
  // ---- work item: blocks of one kv head stay on one group of XCDs --------
  const int bid = blockIdx.x;
  int g, item;
  if (xcd_per > 0) {
    const int xcd = bid & 7;
    g = xcd / xcd_per;
    item = (bid >> 3) * xcd_per + (xcd - g * xcd_per);
  } else {
    g = bid % Hkv;
    item = bid / Hkv;
  }
  const int n_items = sched[0];
  if (item >= n_items) return;
  const int2 it = reinterpret_cast<const int2*>(sched + 4)[item];
  const int doc = it.x;
  const int doc_start = max(cu[doc], 0);
  const int doc_end = min(cu[doc + 1], T);
  const int m_tok = (kWaves * kColsPerWave) >> log2G;
  const int tpw = kColsPerWave >> log2G;  // tokens per wave
  const int a = doc_start + it.y * m_tok;
  const int a_end = min(a + m_tok, doc_end);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int tok = a + wave * tpw + (col >> log2G);
  const int hq = g * G + (col & (G - 1));
  const bool tok_ok = tok < a_end;
  const int tw0 = a + wave * tpw;                 // this wave's tokens [tw0, tw1)
  const int tw1 = min(tw0 + tpw, a_end);

  __shared__ double s_invf[64];
  __shared__ __attribute__((aligned(1024))) char lds[2 * kBuf];

  // ---- key range of the block: [lo, hi), visited in 64-aligned tiles ------
  const int hi = a_end;
  const int lo = window > 0 ? max(doc_start, a - window + 1) : doc_start;
  const int wlo = window > 0 ? max(doc_start, tw0 - window + 1) : doc_start;
  const int kt_lo = lo & ~(kKeyTile - 1);
  const bf16* kbase = khat + (size_t)g * t_pad * kHeadDim;
  const bf16* vbase = vt + (size_t)g * kHeadDim * t_pad;
  // the first tile's copy overlaps the Q prologue
  if (kt_lo < hi) issue_tile(kbase, vbase, t_pad, kt_lo, tid, lds);

  if (use_rope && tid < 64) s_invf[tid] = pow(theta, -(double)tid / 64.0) * kInvTwoPi;
  __syncthreads();

  ColState st;
  // ---- Q: load, RMSNorm, RoPE, round to bf16 B operands --------------------
  // lane holds channels 16kk + 8hf + e (kk < 8, e < 8) of its column; NeoX
  // partners i and i + 64 (kk and kk + 4) sit in the same lane.
  {
    float x[64];
    if (tok_ok) {
      const bf16* qp = q + ((size_t)tok * Hq + hq) * kHeadDim + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * kk + e] = (float)v8[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 32);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * kk + e] *= inv * qnorm_w[16 * kk + 8 * hf + e];
    if (use_rope && tok_ok) {
      const int p = tok - doc_start;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float sn, cs;
          rope_sincos_rev(p, s_invf[16 * kk + 8 * hf + e], &sn, &cs);
          const float x1 = x[8 * kk + e], x2 = x[8 * (kk + 4) + e];
          x[8 * kk + e] = x1 * cs - x2 * sn;
          x[8 * (kk + 4) + e] = x2 * cs + x1 * sn;
        }
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.qf[kk][e] = (bf16)x[8 * kk + e];
  }

  // running state in the log2 domain: m = max(sink, scores) * log2(e) scaled,
  // l = partial denominator of this lane's keys (the sink's 1 in half 0 only)
  st.m_run = sinks[hq] * kLog2e;
  st.l_part = hf == 0 ? 1.f : 0.f;
#pragma unroll
  for (int dd = 0; dd < 4; ++dd)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[dd][r] = 0.f;

  // swizzled LDS byte offsets of this lane's operand reads inside a buffer
  int koff[8], voff[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = col * 256 + (((2 * kk + hf) ^ (col & 15)) << 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) voff[j] = col * 128 + (((2 * j + hf) ^ vswz(col)) << 4);

  // ---- key loop, two tiles per trip so buffer offsets are immediates ------
  for (int kt = kt_lo; kt < hi;) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (kt >= hi) break;
      // wait for this tile's copy, then let everyone past the barrier: the
      // other buffer's readers (previous tile) are done too
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if (kt + kKeyTile < hi) issue_tile(kbase, vbase, t_pad, kt + kKeyTile, tid, lds + (b ^ 1) * kBuf);
      const bool active = (tw0 < tw1) && (kt < tw1) && (kt + kKeyTile > wlo);
      if (active) {
        if (b == 0)
          attend_tile<0>(lds, koff, voff, st, kt, col, hf, tok, tok_ok, tw0, tw1, doc_start,
                         window, c_log2);
        else
          attend_tile<1>(lds, koff, voff, st, kt, col, hf, tok, tok_ok, tw0, tw1, doc_start,
                         window, c_log2);
      }
      kt += kKeyTile;
    }
  }

  // ---- epilogue: out = O / l in bf16, lse = ln2 * (m + log2 l) -------------
  const float l = st.l_part + __shfl_xor(st.l_part, 32);
  if (tok_ok) {
    const float inv_l = 1.0f / l;
    bf16* op = out + ((size_t)tok * Hq + hq) * kHeadDim + 4 * hf;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(st.o[dd][4 * rq + e] * inv_l);
        *reinterpret_cast<bf16x4*>(op + 32 * dd + 8 * rq) = w;
      }
    if (lse != nullptr && hf == 0) lse[(size_t)hq * T + tok] = (st.m_run + __log2f(l)) * kLn2;
  }
}

}  // namespace

hipError_t launch_attention_bf16(const bf16* q, const bf16* khat, const bf16* vt,
                                 const int32_t* cu, const int32_t* sched,
                                 const float* sinks, const float* qnorm_w, bf16* out,
                                 float* lse, int T, int D, int Hq, int Hkv,
                                 int64_t t_pad, int64_t items_ub, int window,
                                 int use_rope, double eps, double theta,
                                 double scale, hipStream_t stream) {
  const int G = Hq / Hkv;
  int log2G = 0;
  while ((1 << log2G) < G) ++log2G;
  // XCD-aware order: when Hkv divides the 8 XCDs, kv head g runs on XCDs
  // [g * 8/Hkv, (g+1) * 8/Hkv) so the blocks streaming one head's keys share L2.
  int xcd_per = 0;
  int64_t grid;
  if (Hkv <= 8 && 8 % Hkv == 0) {
    xcd_per = 8 / Hkv;
    grid = 8 * ((items_ub + xcd_per - 1) / xcd_per);
  } else {
    grid = items_ub * Hkv;
  }
  if (grid <= 0) return hipSuccess;
  const float c_log2 = (float)(scale * 1.4426950408889634);
  attn_fwd_bf16_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      q, khat, vt, cu, sched, sinks, qnorm_w, out, lse, T, Hq, Hkv, G, log2G, t_pad,
      window, use_rope, (float)eps, theta, c_log2, xcd_per);
  return hipGetLastError();
}

}  // namespace sa
