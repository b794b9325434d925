// attn_narrow.hip -- sink-aware GQA attention forward, narrow tiles (32 query
// columns per wave, two workgroups per CU), 16-bit in/out (bf16, or fp16 for the
// fp16 I/O variant), gfx950 MFMA.  The kernel is a template over
// the element type E; everything below says "E" where the two differ only in
// the type of the operands (v_mfma_f32_32x32x16_bf16 or _f16).
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
// queries are done once at the start, in fp32, straight into E MFMA
// operands.  The key loop walks 64-key tiles of k_hat and V^T (written by the
// prologue), copied global -> LDS by global_load_lds_dwordx4 (no VGPR
// staging) into one of two buffers while the other is consumed; the tile is
// shared by all 4 waves, i.e. by the 8 query heads of the group at 4 tokens
// per wave.  Per tile and wave:
//   S^T[key][col] = K Q^T - m_ref   2 x (8 + 1) v_mfma_f32_32x32x16_E: Q is
//   pre-scaled by scale * log2(e), and a ninth step with A = a column of ones
//   and B = -m_ref subtracts the column's reference max inside the MFMA, so
//   the weights need one v_exp_f32 each and no other VALU op
//   online softmax in the log2 domain, the sink seeding the running max and
//   denominator; band masks only on tiles that cross a document, causal or
//   window edge; tiles outside the band are never visited
//   O^T[d][col] += V^T P^T     16 v_mfma_f32_32x32x16_E (P rounded to E)
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

typedef __attribute__((address_space(3))) void lds_void;

// Copy the 64-key tile at kt into LDS buffer `buf`: the prologue wrote k_hat
// and V^T as the exact LDS image (see sa_device.h), so this is a straight
// 2 x 16 KiB copy by global_load_lds_dwordx4 -- chunk 256 i + tid of each
// image lands at byte 16 (256 i + tid) -- with no VGPR staging.
__device__ __forceinline__ void issue_tile(const char* __restrict__ ktile,
                                           const char* __restrict__ vtile, int tid, int wave,
                                           char* buf) {
  char* wbase = buf + wave * 1024;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_global_load_lds(ktile + 4096 * i + 16 * tid,
                                     (lds_void*)(wbase + 4096 * i), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vtile + 4096 * i + 16 * tid,
                                     (lds_void*)(wbase + kTileK + 4096 * i), 16, 0, 0);
  }
}

// Per-lane state of one wave's 32 query columns.
template <typename E>
struct ColState {
  vec8<E> qf[8];    // Q^T B operands, channels 16kk + 8hf .. +7
  f32x16 o[4];      // O^T accumulators, channels 32dd + ...
  vec8<E> ones_a;   // A operand of the reference step: A[key][0] = 1
  vec8<E> negm_b;   // B operand of the reference step: B[0][col] = -m_ref
  float m_ref;      // reference max (log2 domain, E-representable, or -inf)
  float l_part;     // this lane's share of the denominator
};

// B operand that makes the reference MFMA step subtract m_ref from every
// score of the column: lanes 0-31 hold k-slot 0 of their column.
template <typename E>
__device__ __forceinline__ vec8<E> neg_ref_operand(float m_ref, int hf) {
  vec8<E> b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (E)0.f;
  if (hf == 0 && m_ref != -INFINITY) b[0] = (E)(-m_ref);
  return b;
}

// One 64-key tile for one wave: S^T = K Q^T, masked online softmax with the
// sink-seeded state, O^T += V^T P^T.  LDS operand reads are issued one step
// ahead of the MFMAs that consume them; sched_barrier keeps the compiler from
// sinking them back next to their use.  HALVES says which 32-key halves hold
// a key any of the wave's tokens can see (bit 0: keys kt .. kt + 31, bit 1:
// kt + 32 .. kt + 63): a dead half gets no MFMAs, exps or PV steps, which is
// exact, as its weights would all be zero.  On short documents a block's first
// tile often starts half a tile before the document and its last ends half a
// tile past the wave's tokens.
template <typename E, int BUF, int HALVES>
__device__ __forceinline__ void attend_tile(const char* lds, const int (&koff)[8],
                                            const int (&voff)[4], ColState<E>& st, int kt,
                                            int hf, int tok, bool tok_ok, int tw0, int tw1,
                                            int doc_start, int window) {
  const char* kbuf = lds + BUF * kBuf;
  const char* vbuf = kbuf + kTileK;
  auto rd = [](const char* p) { return *reinterpret_cast<const vec8<E>*>(p); };

  constexpr bool kL0 = HALVES & 1, kL1 = HALVES & 2;
  // PV steps [kJ0, kJ1): step j covers keys 16j .. 16j + 15
  constexpr int kJ0 = kL0 ? 0 : 2, kJ1 = kL1 ? 4 : 2;

  // ---- S^T = K Q^T: two 32-key chains, K fragments one step ahead --------
  f32x16 s0, s1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = kL0 ? 0.f : -INFINITY;
    s1[r] = kL1 ? 0.f : -INFINITY;
  }
  vec8<E> a0, a1;
  if constexpr (kL0) a0 = rd(kbuf + koff[0]);
  if constexpr (kL1) a1 = rd(kbuf + 8192 + koff[0]);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    vec8<E> n0 = a0, n1 = a1;
    if (kk < 7) {
      if constexpr (kL0) n0 = rd(kbuf + koff[kk + 1]);
      if constexpr (kL1) n1 = rd(kbuf + 8192 + koff[kk + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kL0) s0 = mfma32(a0, st.qf[kk], s0);
    if constexpr (kL1) s1 = mfma32(a1, st.qf[kk], s1);
    a0 = n0;
    a1 = n1;
  }
  // reference step: every score of a column minus m_ref (exact: m_ref is an
  // E value), so the accumulators hold s * scale * log2e - m_ref
  if constexpr (kL0) s0 = mfma32(st.ones_a, st.negm_b, s0);
  if constexpr (kL1) s1 = mfma32(st.ones_a, st.negm_b, s1);
  // V fragments of the first PV step, read while the softmax runs
  vec8<E> va[4];
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) va[dd] = rd(vbuf + dd * 4096 + voff[kJ0]);
  __builtin_amdgcn_sched_barrier(0);

  // ---- band mask, only on tiles that cross a document, causal or window edge
  const bool full = kt >= doc_start && kt + kKeyTile - 1 <= tw0 &&
                    (window < 0 || kt > tw1 - 1 - window);
  if (!full) {
    // accumulator register r of chain i holds key kt + 32i + 4hf + k(r),
    // k(r) = 8(r/4) + r%4 in [0, 27]; the key is visible iff lo <= key <= tok
    // (lo = document start, or tok - W + 1 under a window)
    const int lo = window < 0 ? doc_start : max(doc_start, tok - window + 1);
    unsigned vis[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int base = kt + 32 * i + 4 * hf;
      vis[i] = bit_run(max(lo - base, 0), tok_ok ? min(tok - base, 27) : -1);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = (r >> 2) * 8 + (r & 3);
      if constexpr (kL0) s0[r] = keep_if(vis[0], k, s0[r]);
      if constexpr (kL1) s1[r] = keep_if(vis[1], k, s1[r]);
    }
  }
  // column max of the raw scores (the lane pair l, l^32 holds one column)
  float mx = -INFINITY;
  if constexpr (kL0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[r]);
  }
  if constexpr (kL1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
  }
  mx = lane_pair_max(mx);  // relative to the reference (or absolute while none)

  // Lazy rescale: the reference point m_run moves only when a score exceeds
  // it by more than kLazy (log2 units), so weights stay <= 2^kLazy and the
  // O / l rescale runs on the few tiles where the max jumps.  The result is
  // the same softmax; lse uses the reference actually kept.
  const bool no_ref = st.m_ref == -INFINITY;
  const bool grow = no_ref ? mx > -INFINITY : mx > kLazy;
  if (__any(grow)) {
    const float m_eff = no_ref ? 0.f : st.m_ref;         // what the step subtracted
    const float m_new = grow ? ref_round<E>(m_eff + mx) : st.m_ref;
    const float delta = grow ? m_new - m_eff : 0.f;
    const float alpha = grow ? (no_ref ? 0.f : __builtin_amdgcn_exp2f(st.m_ref - m_new)) : 1.f;
    st.m_ref = m_new;
    st.negm_b = neg_ref_operand<E>(m_new, hf);
    st.l_part *= alpha;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[dd][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (kL0) s0[r] -= delta;
      if constexpr (kL1) s1[r] -= delta;
    }
  }

  // ---- P = exp2(s * scale * log2e - m) into E B operands; O^T += V^T P^T.
  // Step j covers keys 16j..16j+15 (j = 2 kb + sp): B operand k-slot 8hf + e
  // <-> key 16j + 8(e/4) + 4hf + e%4, which is the order the prologue stored
  // V^T keys in, so the A operand is one 16-byte read.  The denominator sums
  // the same rounded weights the PV product uses.
  const vec2<E> ones = {(E)1.0f, (E)1.0f};
  auto weights = [&](int j) {
    const f32x16& sv = (j < 2) ? s0 : s1;
    const int base = 8 * (j & 1);
    vec8<E> pb;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pb[e] = (E)__builtin_amdgcn_exp2f(sv[base + e]);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const vec2<E> pr = {pb[e], pb[e + 1]};
      st.l_part = dot2<E>(pr, ones, st.l_part);
    }
    return pb;
  };
  vec8<E> pb = weights(kJ0);
#pragma unroll
  for (int j = kJ0; j < kJ1; ++j) {
    vec8<E> vn[4];
    if (j + 1 < kJ1) {
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) vn[dd] = rd(vbuf + dd * 4096 + voff[j + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) st.o[dd] = mfma32(va[dd], pb, st.o[dd]);
    if (j + 1 < kJ1) {
      pb = weights(j + 1);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) va[dd] = vn[dd];
    }
  }
}

// RoPE of the queries: none, from an LDS table of the block's tokens (G >= 8,
// where a token's G heads share its angles), or per lane.  A template
// argument rather than a run-time flag, so that the code without RoPE has no
// branches around the rotation and no register copies where they rejoin.
enum RopeMode { kRopeNone = 0, kRopeTable = 1, kRopeLane = 2 };

template <typename E, int RM>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_narrow_kernel(
    const E* __restrict__ q, const E* __restrict__ khat,
    const E* __restrict__ vt, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_end, const int32_t* __restrict__ sched, const float* __restrict__ sinks,
    const float* __restrict__ qnorm_w, E* __restrict__ out, float* __restrict__ lse,
    int T, int Hq, int Hkv, int G, int log2G, int64_t t_pad, int window,
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
  const int doc_end = min(cu_end[doc], T);  // real end (document padding follows)
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
  __shared__ __attribute__((aligned(16))) char s_rope[16 * kRopeRow];

  // ---- key range of the block: [lo, hi), visited in 64-aligned tiles ------
  const int hi = a_end;
  const int lo = window > 0 ? max(doc_start, a - window + 1) : doc_start;
  const int wlo = window > 0 ? max(doc_start, tw0 - window + 1) : doc_start;
  const int kt_lo = lo & ~(kKeyTile - 1);
  // byte images of this kv head's tiles: tile kt/64 at 16 KiB * (kt/64)
  const char* kimg = reinterpret_cast<const char*>(khat + (size_t)g * t_pad * kHeadDim);
  const char* vimg = reinterpret_cast<const char*>(vt + (size_t)g * t_pad * kHeadDim);
  // wave index as a uniform value with a known range [0, 4): the range lets
  // the compiler prove the next tile's LDS copy does not alias the buffer
  // being read, so it does not wait for that copy before the reads
  const int wave_u = __builtin_amdgcn_readfirstlane(wave) & (kWaves - 1);
  // RoPE angles: a table of the block's tokens (kRopeTable, G >= 8, so the
  // block's 128 / G tokens fit the table), or per lane from the frequencies
  // in s_invf (kRopeLane)
  if constexpr (RM == kRopeLane) {
    if (tid < 64) s_invf[tid] = pow(theta, -(double)tid / 64.0) * kInvTwoPi;
    __syncthreads();
  }

  ColState<E> st;
  // ---- Q: load, RMSNorm, RoPE, round to E B operands -----------------------
  // lane holds channels 16kk + 8hf + e (kk < 8, e < 8) of its column; NeoX
  // partners i and i + 64 (kk and kk + 4) sit in the same lane.  The wave's 32
  // rows are copied global -> LDS by global_load_lds_dwordx4 into the second
  // tile buffer (not used before the key loop's first barrier), four whole
  // rows per instruction, and each lane then reads the pieces of its own
  // column from there.  Instruction j fills rows 4j .. 4j + 3 (1 KiB) and lane
  // l writes its 16 bytes at byte 16 l of that, i.e. row r = 4j + l / 16 at
  // position l % 16; lane l therefore fetches chunk (l % 16) ^ (r % 16) of
  // row r, so that chunk k of row r sits at position k ^ (r % 16).  Rows are
  // addressed by 32-bit offsets from the wave's first (token, head) row.
  // The copies go out before the first tile's copy, and the wait before the
  // reads covers both.
  char* stg = lds + kBuf + wave_u * (32 * 256);
  // Column r of the wave is (token tw0 + r / G, head g G + r % G); its row
  // sits r * 256 + (r / G) * (Hq - G) * 256 bytes past the wave's first row.
  // A column past the block's tokens reads the wave's first row instead (its
  // norm factor is zero below), or, in a wave without tokens, the block's.
  // The wave's token count and base token are wave-uniform; readfirstlane
  // makes them scalars for the compiler.
  const int tpw_live = __builtin_amdgcn_readfirstlane(tw1 - tw0);  // tokens of this wave (may be <= 0)
  const int t_base = __builtin_amdgcn_readfirstlane(tpw_live > 0 ? tw0 : a);
  const uint32_t gap = (uint32_t)(Hq - G) * (kHeadDim * (uint32_t)sizeof(E));
  {
    const char* qwave = reinterpret_cast<const char*>(q + ((size_t)t_base * Hq + g * G) * kHeadDim);
    // with G >= 4 the token r / G = (4j + lane/16) / G = 4j / G of row group j
    // is the same for the whole wave (G is a power of two), so the row offset
    // is a per-lane constant plus a uniform term and the bounds test is uniform
    const uint32_t lane_off = ((uint32_t)(lane >> 4) << 8) | ((uint32_t)((lane & 15) ^ (lane >> 4)) << 4);
    if (G >= 4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // row 4j + lane/16, chunk position (lane%16) ^ (r%16) with
        // r%16 = 4(j%4) + lane/16; a row past the tokens reads row 0
        const int tq = (4 * j) >> log2G;
        const uint32_t off = tq < tpw_live
                                 ? (uint32_t)(1024 * j) + (uint32_t)tq * gap + (lane_off ^ ((j & 3) << 6))
                                 : (lane_off & 0xF0u) ^ ((uint32_t)(j & 3) << 6);
        __builtin_amdgcn_global_load_lds(qwave + off, (lds_void*)(stg + 1024 * j), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 4 * j + (lane >> 4);
        const int tq = r >> log2G;
        uint32_t off = tq < tpw_live ? (uint32_t)r * 256 + (uint32_t)tq * gap : 0u;
        off += (uint32_t)((lane & 15) ^ (r & 15)) << 4;
        __builtin_amdgcn_global_load_lds(qwave + off, (lds_void*)(stg + 1024 * j), 16, 0, 0);
      }
    }
  }
  {
    float w[64];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) w[8 * kk + e] = qnorm_w[16 * kk + 8 * hf + e];
    __builtin_amdgcn_sched_barrier(0);
    // the first tile's copy overlaps the Q prologue
    if (kt_lo < hi)
      issue_tile(kimg + (size_t)kt_lo * 256, vimg + (size_t)kt_lo * 256, tid, wave_u, lds);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RM == kRopeTable) {
      rope_table(s_rope, tid, kThreads, m_tok, a, a_end, doc_start, theta);
      barrier_keep_copies();
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the q rows (and the first tile) landed
    vec8<E> qraw[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qraw[kk] = *reinterpret_cast<const vec8<E>*>(stg + col * 256 + (((2 * kk + hf) ^ (col & 15)) << 4));

    float x[64];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * kk + e] = (float)qraw[kk][e];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
    ss = lane_pair_sum(ss);
    // the norm factor carries scale * log2(e) (RoPE is linear, so the order
    // does not matter), and a padding column, which loaded a real token's
    // row, gets a zero factor: zero operands
    const float inv = tok_ok ? c_log2 / sqrtf(ss * (1.0f / kHeadDim) + eps) : 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] *= inv * w[i];
    if constexpr (RM == kRopeTable) {
      if (tok_ok) rope_from_table(s_rope + (tok - a) * kRopeRow, hf, x);
    } else if constexpr (RM == kRopeLane) {
      if (tok_ok) {
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
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.qf[kk][e] = (E)x[8 * kk + e];
  }

  // running state in the log2 domain: m = max(sink, scores) * log2(e) scaled,
  // l = partial denominator of this lane's keys (the sink's 1 in half 0 only)
  {
    const float sl = sinks[hq] * kLog2e;
    st.m_ref = sl == -INFINITY ? -INFINITY : ref_round<E>(sl);
    st.l_part = (hf == 0 && sl != -INFINITY) ? __builtin_amdgcn_exp2f(sl - st.m_ref) : 0.f;
    st.negm_b = neg_ref_operand<E>(st.m_ref, hf);
#pragma unroll
    for (int e = 0; e < 8; ++e) st.ones_a[e] = (E)0.f;
    if (hf == 0) st.ones_a[0] = (E)1.f;
  }
  // O^T starts at zero: four MFMAs of zero operands on the otherwise idle
  // matrix cores, instead of 64 VALU moves; the fence keeps them after the Q
  // prologue, whose 128 live floats per lane leave no room for O
  __builtin_amdgcn_sched_barrier(0);
  {
    f32x16 zc;
#pragma unroll
    for (int r = 0; r < 16; ++r) zc[r] = 0.f;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      vec8<E> z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = (E)0.f;
      // an opaque copy per product, so the compiler keeps four MFMAs rather
      // than one and 48 register copies of its result
      asm volatile("" : "+v"(z));
      st.o[dd] = mfma32(z, z, zc);
    }
  }

  // swizzled LDS byte offsets of this lane's operand reads inside a buffer
  int koff[8], voff[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = col * 256 + (((2 * kk + hf) ^ kswz(col)) << 4);
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
      if (kt + kKeyTile < hi)
        issue_tile(kimg + (size_t)(kt + kKeyTile) * 256, vimg + (size_t)(kt + kKeyTile) * 256, tid,
                   wave_u, lds + (b ^ 1) * kBuf);
      // the wave's visible keys are [wlo, tw1 - 1]; a tile that reaches them
      // has at least one live half
      const bool active = (tw0 < tw1) && (kt < tw1) && (kt + kKeyTile > wlo);
      if (active) {
        const bool live0 = kt + 31 >= wlo, live1 = kt + 32 < tw1;
#define SA_TILE(B, H) \
  attend_tile<E, B, H>(lds, koff, voff, st, kt, hf, tok, tok_ok, tw0, tw1, doc_start, window)
        if (b == 0) {
          if (live0 && live1) SA_TILE(0, 3);
          else if (live0) SA_TILE(0, 1);
          else SA_TILE(0, 2);
        } else {
          if (live0 && live1) SA_TILE(1, 3);
          else if (live0) SA_TILE(1, 1);
          else SA_TILE(1, 2);
        }
#undef SA_TILE
      }
      kt += kKeyTile;
    }
  }

  // ---- epilogue: out = O / l in E, lse = ln2 * (m + log2 l) ----------------
  // A lane holds 4-channel pieces of one output row, so storing from the
  // accumulators would write 16 bytes into each of 32 rows per instruction.
  // The wave's 32 rows go through LDS instead -- the tile buffer the last tile
  // did not use: no copy is in flight into it, and every wave has passed the
  // barrier of the last tile, so no wave still reads it -- and each store
  // instruction then writes 4 whole 256-byte rows.  Row r sits at r * 256 with
  // its 16-byte chunk c at position c ^ (r % 16).
  const float l = lane_pair_sum(st.l_part);
  const int n_tiles = kt_lo < hi ? (hi - kt_lo + kKeyTile - 1) / kKeyTile : 0;
  char* obuf = lds + (n_tiles & 1) * kBuf + wave * (32 * 256);
  {
    const float inv_l = 1.0f / l;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        // channels 32dd + 8rq + 4hf .. + 3: chunk 4dd + rq, bytes 8hf .. + 7
        vec4<E> w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (E)(st.o[dd][4 * rq + e] * inv_l);
        const int pos = ((4 * dd + rq) ^ (col & 15)) << 4;
        *reinterpret_cast<vec4<E>*>(obuf + col * 256 + pos + 8 * hf) = w;
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  {
    // rows addressed by 32-bit offsets from the wave's first row, as the Q copy
    char* owave = reinterpret_cast<char*>(out + ((size_t)t_base * Hq + g * G) * kHeadDim);
    // an opaque copy of the lane index: the row terms below are the Q copy's
    // again, and without it the compiler keeps those alive through the key
    // loop instead of recomputing them, which costs registers it does not have
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // row r = 4j + lane/16 of the wave, chunk lane % 16; as in the Q copy, the
    // token r / G of row group j is uniform when G >= 4
    if (G >= 4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 4 * j + (ln >> 4), c = ln & 15;
        const vec8<E> v = *reinterpret_cast<const vec8<E>*>(obuf + r * 256 + ((c ^ (r & 15)) << 4));
        const int tq = (4 * j) >> log2G;
        if (tq < tpw_live)
          *reinterpret_cast<vec8<E>*>(owave + (uint32_t)r * 256 + (uint32_t)tq * gap + 16 * c) = v;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 4 * j + (ln >> 4), c = ln & 15;
        const vec8<E> v = *reinterpret_cast<const vec8<E>*>(obuf + r * 256 + ((c ^ (r & 15)) << 4));
        const int tq = r >> log2G;
        if (tq < tpw_live)
          *reinterpret_cast<vec8<E>*>(owave + (uint32_t)r * 256 + (uint32_t)tq * gap + 16 * c) = v;
      }
    }
  }
  if (tok_ok && lse != nullptr && hf == 0)
    lse[(size_t)hq * T + tok] = (st.m_ref + __log2f(l)) * kLn2;
}

}  // namespace

template <typename E>
hipError_t launch_attention_narrow(const E* q, const E* khat, const E* vt,
                                 const int32_t* cu, const int32_t* cu_end, const int32_t* sched,
                                 const float* sinks, const float* qnorm_w, E* out,
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
  // the block's 128 / G tokens fit the 16-row angle table from G = 8 on
  const int rm = !use_rope ? kRopeNone : ((kWaves * kColsPerWave) >> log2G) <= 16 ? kRopeTable
                                                                                   : kRopeLane;
#define SA_LAUNCH(RMV)                                                                        \
  attn_fwd_narrow_kernel<E, RMV><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(        \
      q, khat, vt, cu, cu_end, sched, sinks, qnorm_w, out, lse, T, Hq, Hkv, G, log2G, t_pad, \
      window, (float)eps, theta, c_log2, xcd_per)
  if (rm == kRopeNone) SA_LAUNCH(kRopeNone);
  else if (rm == kRopeTable) SA_LAUNCH(kRopeTable);
  else SA_LAUNCH(kRopeLane);
#undef SA_LAUNCH
  return hipGetLastError();
}

#define SA_INSTANTIATE(E)                                                                    \
  template hipError_t launch_attention_narrow<E>(const E*, const E*, const E*, const int32_t*, \
                                               const int32_t*, const int32_t*, const float*,   \
                                               const float*, E*, float*, int, int, int, int,   \
                                               int64_t, int64_t, int, int, double, double,     \
                                               double, hipStream_t);
SA_INSTANTIATE(bf16)
SA_INSTANTIATE(f16)
#undef SA_INSTANTIATE

}  // namespace sa
