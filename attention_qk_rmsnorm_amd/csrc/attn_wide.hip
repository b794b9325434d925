// attn_wide.hip -- sink-aware GQA attention forward, 16-bit in/out (bf16,
// or fp16 for the fp16 I/O variant: a template over the element type E),
// gfx950 MFMA, wide tiles (64 query columns per wave, one workgroup per CU).
//
// Computes, for every (token t, query head h) of a packed THD batch
//   out = sum_{j visible} exp(s_j - M) v_j / (exp(sink_h - M) + sum_j exp(s_j - M))
//   lse = M + log(denominator)
// with s_j = scale * <q_hat, k_hat_j> (flint.layers FlintAttention.forward: causal
// attention with a zero-value sink category; _FlintSinkParameters: unscaled fp32
// logits), keys j <= t of the same document and, for a window W > 0,
// t - W < j (flint.config: the window counts the current token).
//
// Workgroup = 4 waves (one per SIMD) = one query block of one kv head g:
// tokens [a, a + 256/G) of one document, times the G query heads that read kv
// head g.  Each wave owns 64 (token, head) columns as two 32-column blocks, so
// every K or V^T operand read from LDS feeds two MFMAs: half the LDS traffic
// per MFMA of the narrow configuration.  RMSNorm and RoPE of the wave's
// queries are done once at the start, in fp32, straight into E MFMA
// operands pre-scaled by scale * log2(e), which then live in AGPRs.
//
// Keys are walked in 64-key tiles of k_hat and V^T, which the prologue wrote
// as exact LDS images; global_load_lds_dwordx4 copies them into three LDS
// slots (tiles j, j + 1 in use, j + 2 landing; one barrier per tile).  The
// loop is software-pipelined inside each wave in 32-key half tiles: while the
// VALU forms the weights of half tile u, the matrix core computes the scores
// of half tile u + 1; then O accumulates half tile u's values.
//   S^T[key][col] = K Q^T - m_ref   8 v_mfma_f32_32x32x16_E per 32-key x
//                                   32-column block; the chain starts from a
//                                   tile of -m_ref, so a weight is one v_exp
//   O^T[d][col] += V^T P^T          P rounded to E; O in AGPRs
// The reference each weight is taken against is fixed for the whole key loop:
// the larger of the sink and the token's score against its own key (always
// visible).  Weights may exceed 1 -- exp2 of up to 90 keeps bf16 weights and
// the fp32 sums finite and exact to their usual relative precision -- so the
// loop never rescales O.  A block where some denominator passes 2^90 (a score
// more than 90 log2 units above the reference), or some O accumulator is not
// finite (values beyond about 2^38 times such weights), hands itself to a
// second launch that finds the exact row max with a scores-only pass first.  fp16
// weights overflow past 2^16 instead: such a weight rounds to inf, its
// denominator is no longer finite, and the same rerun takes the block.  Band
// masks run only on half tiles that cross a document, causal or window edge;
// tiles outside the block's band are never visited.
// MFMA operand layouts (32x32x16, wave64): A lane l holds A[l%32][8(l/32)..+7],
// B lane l holds B[8(l/32)..+7][l%32], and accumulator register r of lane l is
// C[8(r/4) + 4(l/32) + r%4][l%32].  With S^T in that layout a lane holds 16 keys
// of one query column per block, and every O^T entry of a lane belongs to one
// column.
#include "sa_device.h"

namespace sa {

namespace {

constexpr int kThreads = kWaves * 64;
constexpr int kTileK = kKeyTile * kHeadDim * 2;   // bytes of one k_hat tile (16 KiB)
constexpr int kTileV = kHeadDim * kKeyTile * 2;   // bytes of one V^T tile (16 KiB)
// LDS: three slots of (k_hat tile, V^T tile): tiles j and j + 1 in use while
// tile j + 2 lands
constexpr int kSlot = kTileK + kTileV;
constexpr int kSlots = 3;
constexpr int kLds = kSlots * kSlot;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRedo = 0x1p90f;  // denominator bound that sends a block to its exact pass

typedef __attribute__((address_space(3))) void lds_void;

// O^T lives in AGPRs: the accumulators are touched only by the inline-asm
// MFMAs of sa_device.h (mfma32_acc), their zeroing (zero_acc) and the
// epilogue (after agpr_fence()), which leaves the 256 VGPRs to the scores,
// weights and operands.

// Copy one 16 KiB tile image into LDS at dst: chunk 256 i + tid of the image
// lands at byte 16 (256 i + tid), by global_load_lds_dwordx4.
__device__ __forceinline__ void copy_image(const char* __restrict__ src, int tid, int wave,
                                           char* dst) {
  char* wbase = dst + wave * 1024;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds(src + 4096 * i + 16 * tid, (lds_void*)(wbase + 4096 * i),
                                     16, 0, 0);
}

// Per-lane state of one wave's 64 query columns (column block cb = 0, 1).
template <typename E>
struct WaveState {
  vec8<E> qf[2][8];  // Q^T B operands, channels 16kk + 8hf .. +7
  f32x16 o[2][4];    // O^T accumulators (AGPRs), channels 32dd + ...
  f32x16 negm[2];    // -m_ref splat: the score MFMA chains start from it
  float m_ref[2];    // reference (log2 domain)
  float l_part[2];   // this lane's share of the denominator
};

// Where a wave's columns sit, for the band mask.
struct Cols {
  int tok[2];
  bool ok[2];
  int tw0, tw1;  // the wave's tokens [tw0, tw1)
  int doc_start, window, hf;
};

// Does the 32-key half tile at kh need the band mask?
__device__ __forceinline__ bool half_full(int kh, const Cols& c) {
  return kh >= c.doc_start && kh + 31 <= c.tw0 && (c.window < 0 || kh > c.tw1 - 1 - c.window);
}

__device__ __forceinline__ void mask_half(int kh, const Cols& c, f32x16 (&s)[2]) {
  // accumulator register r holds key kh + 4hf + k(r), k(r) = 8(r/4) + r%4;
  // key u is visible to token t iff lo <= u <= t (lo = document start, or
  // t - W + 1 under a window), i.e. lo - base <= k(r) <= t - base.  The
  // masked scores go straight to v_exp_f32 in the key loop.
  const int base = kh + 4 * c.hf;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int t = c.tok[cb];
    const int lo = c.window < 0 ? c.doc_start : max(c.doc_start, t - c.window + 1);
    // (a padding column sees nothing: an empty run)
    const unsigned vis = bit_run(max(lo - base, 0), c.ok[cb] ? min(t - base, 27) : -1);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[cb][r] = keep_if(vis, (r >> 2) * 8 + (r & 3), s[cb][r]);
  }
}

// Weights of keys 16jj .. 16jj + 15 of a half tile for column block cb:
// B operand k-slot 8hf + e <-> key 16jj + 8(e/4) + 4hf + e%4, the order the
// prologue stored V^T keys in.
// (elements 2q, 2q + 1 only: the exps are spread over the score MFMAs, two
// behind each, about as many issue cycles as the MFMA itself)
template <typename E>
__device__ __forceinline__ void weights_pair(const f32x16& sv, int jj, int q, vec8<E>& pb) {
#pragma unroll
  for (int e = 2 * q; e < 2 * q + 2; ++e) pb[e] = (E)__builtin_amdgcn_exp2f(sv[8 * jj + e]);
}

template <typename E>
__device__ __forceinline__ void add_denominator(const vec8<E>& pb, float& l) {
  const vec2<E> ones = {(E)1.0f, (E)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const vec2<E> pr = {pb[e], pb[e + 1]};
    l = dot2<E>(pr, ones, l);
  }
}

// Scores of the half tile H of k_hat slot SLOT: s[cb] = K_H Q_cb^T - m_ref[cb]
// (the chain starts from the -m_ref splat).
template <int SLOT, int H, typename E>
__device__ __forceinline__ void score_half(const char* lds, const int (&koff)[8],
                                           const WaveState<E>& st, f32x16 (&s)[2]) {
  const char* kbuf = lds + SLOT * kSlot + H * 8192;
  s[0] = st.negm[0];
  s[1] = st.negm[1];
  vec8<E> a = rd<E>(kbuf + koff[0]);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    vec8<E> n = a;
    if (kk < 7) n = rd<E>(kbuf + koff[kk + 1]);
    __builtin_amdgcn_sched_barrier(0);
    s[0] = mfma32(a, st.qf[0][kk], s[0]);
    s[1] = mfma32(a, st.qf[1][kk], s[1]);
    a = n;
  }
}

// One pipelined half-tile step.  sc holds the current half tile's scores
// (masked, relative to the reference); its values are in V^T slot VS, keys
// 32 VH .. 32 VH + 31.  Phase A forms sc's weights while the MFMAs compute the
// next half tile's scores into sn (k_hat slot KS, half KH); phase B accumulates
// O^T += V^T P^T and the denominator, then masks sn if it crosses an edge.
// When there is no next half tile (next == false) sn is still computed, from
// valid LDS, and ignored.
template <int VS, int VH, int KS, int KH, int KSN, int KHN, typename E>
__device__ __forceinline__ void half_step(const char* lds, const int (&koff)[8],
                                          const int (&voff)[4], WaveState<E>& st,
                                          f32x16 (&sc)[2], f32x16 (&sn)[2], vec8<E> (&kf)[8],
                                          bool next, int kh_next, const Cols& c) {
  // ---- phase A: weights of this half || scores of the next half ----------
  // All eight K fragments of the half tile, then the first PV step's V^T
  // fragments, are read up front: with one wave per SIMD nothing else hides
  // LDS latency, so each MFMA waits only for its own fragment.
  const char* vbuf = lds + VS * kSlot + kTileK;
  vec8<E> va[4], vn[4];
  vec8<E> p[2][2];
  {
    // kf: this half tile's K fragments (K slot KS, half KH), read during the
    // previous half step.  Both PV steps' V^T fragments are read here, after
    // the first score MFMA: the compiler waits for every LDS read in flight
    // before an MFMA whose operand an LDS read returns, so reads issued just
    // before the score chain (which needs kf) or in the middle of the PV
    // steps would be waited for there; issued here, they land behind 15 score
    // MFMAs, and phase B's K reads land behind the PV MFMAs
    sn[0] = st.negm[0];  // the chains start from -m_ref: no separate subtraction
    sn[1] = st.negm[1];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      // two weights behind each MFMA: group g = kk / 2 (cb = g / 2,
      // jj = g % 2), elements 4 (kk % 2) .. + 3.  Four exps take longer to
      // issue than one MFMA runs, so four behind one MFMA of the pair would
      // hold back the next
      const int g = kk >> 1;
      __builtin_amdgcn_sched_barrier(0);
      sn[0] = mfma32(kf[kk], st.qf[0][kk], sn[0]);
      if (kk == 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) va[dd] = rd<E>(vbuf + dd * 4096 + voff[2 * VH]);
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) vn[dd] = rd<E>(vbuf + dd * 4096 + voff[2 * VH + 1]);
      }
      weights_pair<E>(sc[g >> 1], g & 1, 2 * (kk & 1), p[g >> 1][g & 1]);
      __builtin_amdgcn_sched_barrier(0);
      sn[1] = mfma32(kf[kk], st.qf[1][kk], sn[1]);
      weights_pair<E>(sc[g >> 1], g & 1, 2 * (kk & 1) + 1, p[g >> 1][g & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- phase B: O^T += V^T P^T for this half || reduce the next half -----
  // the weights were just written by VALU code; the inline-asm MFMAs below
  // read them, and the compiler does not count wait states for inline asm
  asm volatile("s_nop 1");
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      mfma32_acc(st.o[0][dd], va[dd], p[0][jj]);
      mfma32_acc(st.o[1][dd], va[dd], p[1][jj]);
      if (jj == 0 && dd == 0) {
        // the next half step's K fragments (K slot KSN, half KHN), behind
        // the first MFMAs
        const char* knext = lds + KSN * kSlot + KHN * 8192;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) kf[kk] = rd<E>(knext + koff[kk]);
      }
    }
    add_denominator(p[0][jj], st.l_part[0]);
    add_denominator(p[1][jj], st.l_part[1]);
    __builtin_amdgcn_sched_barrier(0);
    if (jj == 0) {
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) va[dd] = vn[dd];
    }
  }
  if (next && !half_full(kh_next, c)) mask_half(kh_next, c, sn);
}

// Scores-only pass over the block's tiles (k_hat images only, both K slots):
// the exact max of every column, in the log2 domain, reduced over the lane
// pair.  Run only for blocks whose fixed reference proved too low.
template <typename E>
__device__ __forceinline__ void max_pass(char* lds, const int (&koff)[8], const WaveState<E>& st,
                                         const char* kimg, int kt_lo, int n_tiles, int tid,
                                         int wave_u, const Cols& c, float (&mx)[2]) {
  mx[0] = mx[1] = -INFINITY;
  copy_image(kimg + (size_t)kt_lo * 256, tid, wave_u, lds);
  for (int j = 0; j < n_tiles;) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (j >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      const int kt = kt_lo + j * kKeyTile;
      if (j + 1 < n_tiles)
        copy_image(kimg + (size_t)(kt + kKeyTile) * 256, tid, wave_u, lds + (b ^ 1) * kSlot);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x16 sh[2];
        if (b == 0) {
          if (h == 0) score_half<0, 0>(lds, koff, st, sh);
          else score_half<0, 1>(lds, koff, st, sh);
        } else {
          if (h == 0) score_half<1, 0>(lds, koff, st, sh);
          else score_half<1, 1>(lds, koff, st, sh);
        }
        if (!half_full(kt + 32 * h, c)) mask_half(kt + 32 * h, c, sh);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx[cb] = fmaxf(mx[cb], sh[cb][r]);
      }
      ++j;
    }
  }
  mx[0] = lane_pair_max(mx[0]);
  mx[1] = lane_pair_max(mx[1]);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

// One 64-key tile in LDS slot SL: its second half's scores, then the next
// tile's first half (slot SN).  After the last tile that second step still
// runs its MFMAs on whatever slot SN holds (nothing copies into it then) and
// ignores the result, which keeps a single code path.
template <int SL, int SN, typename E>
__device__ __forceinline__ void tile_steps(const char* lds, const int (&koff)[8],
                                           const int (&voff)[4], WaveState<E>& st,
                                           f32x16 (&sA)[2], f32x16 (&sB)[2], vec8<E> (&kf)[8],
                                           int kt, bool has_next_tile, const Cols& c) {
  half_step<SL, 0, SL, 1, SN, 0>(lds, koff, voff, st, sA, sB, kf, true, kt + 32, c);
  half_step<SL, 1, SN, 0, SN, 1>(lds, koff, voff, st, sB, sA, kf, has_next_tile,
                                 kt + kKeyTile, c);
}

// The block's key loop against the fixed references in st: l_part and O^T.
// Tile j sits in LDS slot j % 3.  At the top of tile j every wave is done with
// tile j - 1, whose slot then takes tile j + 2; tile j + 1 (needed halfway
// through tile j) was copied during tile j - 1, so one barrier per tile.
template <typename E>
__device__ __forceinline__ void attend_pass(char* lds, const int (&koff)[8], const int (&voff)[4],
                                            WaveState<E>& st, const char* kimg, const char* vimg,
                                            int kt_lo, int n_tiles, int tid, int wave_u,
                                            const Cols& c, bool copies_issued) {
  auto kimg_at = [&](int j) { return kimg + (size_t)(kt_lo + j * kKeyTile) * 256; };
  auto vimg_at = [&](int j) { return vimg + (size_t)(kt_lo + j * kKeyTile) * 256; };
  if (!copies_issued) {
    copy_image(kimg_at(0), tid, wave_u, lds);
    copy_image(vimg_at(0), tid, wave_u, lds + kTileK);
    if (n_tiles > 1) {
      copy_image(kimg_at(1), tid, wave_u, lds + kSlot);
      copy_image(vimg_at(1), tid, wave_u, lds + kSlot + kTileK);
    }
  }
  f32x16 sA[2], sB[2];
  // ---- first half tile's scores (slot 0) ---------------------------------
  if (n_tiles > 1) __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): tile 0 landed
  else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
  __syncthreads();
  score_half<0, 0>(lds, koff, st, sA);
  if (!half_full(kt_lo, c)) mask_half(kt_lo, c, sA);
  vec8<E> kf[8];  // K fragments of the next half tile to score (slot 0, half 1)
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kf[kk] = rd<E>(lds + 8192 + koff[kk]);

  for (int j = 0; j < n_tiles;) {
#pragma unroll
    for (int b = 0; b < kSlots; ++b) {
      if (j >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile j + 1 landed
      __syncthreads();
      if (j + 2 < n_tiles) {
        copy_image(kimg_at(j + 2), tid, wave_u, lds + ((b + 2) % kSlots) * kSlot);
        copy_image(vimg_at(j + 2), tid, wave_u, lds + ((b + 2) % kSlots) * kSlot + kTileK);
      }
      const int kt = kt_lo + j * kKeyTile;
      const bool more = j + 1 < n_tiles;
      if (b == 0) tile_steps<0, 1>(lds, koff, voff, st, sA, sB, kf, kt, more, c);
      else if (b == 1) tile_steps<1, 2>(lds, koff, voff, st, sA, sB, kf, kt, more, c);
      else tile_steps<2, 0>(lds, koff, voff, st, sA, sB, kf, kt, more, c);
      ++j;
    }
  }
}

// EXACT = false: the main launch, with the fixed references; a block whose
// denominators left the safe range marks itself in redo[] and writes nothing.
// EXACT = true: the follow-up launch; only marked blocks run, with the exact
// row max found by a scores-only pass first.
template <bool EXACT, typename E>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_wide_kernel(
    const E* __restrict__ q, const E* __restrict__ khat,
    const E* __restrict__ vt, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_end, const int32_t* __restrict__ sched, const float* __restrict__ sinks,
    const float* __restrict__ qnorm_w, E* __restrict__ out, float* __restrict__ lse,
    int32_t* __restrict__ redo, int T, int Hq, int Hkv, int G, int log2G, int64_t t_pad,
    int window, int use_rope, float eps, double theta, float c_log2, int xcd_per,
    int exact_all) {
  // ---- work item: blocks of one kv head stay on one group of XCDs --------
  const int bid = blockIdx.x;
  if (EXACT && redo[bid] == 0) return;
  if (!EXACT && exact_all) {
    if (threadIdx.x == 0) redo[bid] = 1;
    return;
  }
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
  if (item >= n_items) {
    if (!EXACT && threadIdx.x == 0) redo[bid] = 0;
    return;
  }
  const int2 it = reinterpret_cast<const int2*>(sched + 4)[item];
  const int doc = it.x;
  const int doc_start = max(cu[doc], 0);
  const int doc_end = min(cu_end[doc], T);  // real end (document padding follows)
  const int m_tok = (kWaves * kColsPerWaveWide) >> log2G;
  const int tpw = kColsPerWaveWide >> log2G;  // tokens per wave
  const int a = doc_start + it.y * m_tok;
  const int a_end = min(a + m_tok, doc_end);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;

  Cols c;
  c.tw0 = a + wave * tpw;
  c.tw1 = min(c.tw0 + tpw, a_end);
  c.doc_start = doc_start;
  c.window = window;
  c.hf = hf;
  int hq[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int wc = 32 * cb + col;  // column inside the wave
    c.tok[cb] = c.tw0 + (wc >> log2G);
    c.ok[cb] = c.tok[cb] < a_end;
    hq[cb] = g * G + (wc & (G - 1));
  }

  __shared__ double s_invf[64];
  __shared__ int s_bad;
  __shared__ __attribute__((aligned(1024))) char lds[kLds];

  // ---- key range of the block: [lo, hi), visited in 64-aligned tiles ------
  const int hi = a_end;
  const int lo = window > 0 ? max(doc_start, a - window + 1) : doc_start;
  const int kt_lo = lo & ~(kKeyTile - 1);
  const int n_tiles = (hi - kt_lo + kKeyTile - 1) / kKeyTile;  // >= 1: a < a_end
  // byte images of this kv head's tiles: tile kt/64 at 16 KiB * (kt/64)
  const char* kimg = reinterpret_cast<const char*>(khat + (size_t)g * t_pad * kHeadDim);
  const char* vimg = reinterpret_cast<const char*>(vt + (size_t)g * t_pad * kHeadDim);
  // wave index as a uniform value with a known range [0, 4): the range lets
  // the compiler prove a tile copy does not alias the slots being read, so it
  // does not wait for that copy before the reads
  const int wave_u = __builtin_amdgcn_readfirstlane(wave) & (kWaves - 1);
  // RoPE angles: a table of the block's tokens in the third LDS slot (its
  // first copy is issued after the key loop's first barrier) when it fits,
  // i.e. for G >= 8; otherwise each lane computes its own from the
  // frequencies in s_invf
  const bool rope_tab = use_rope && m_tok * kRopeRow <= kSlot;
  if (tid == 0) s_bad = 0;  // read after the key loop's barriers
  if (use_rope && !rope_tab) {
    if (tid < 64) s_invf[tid] = pow(theta, -(double)tid / 64.0) * kInvTwoPi;
    __syncthreads();
  }

  WaveState<E> st;
  float sink_raw[2], self_score[2];
  // ---- Q: load, RMSNorm, RoPE, scale, round to E B operands ---------------
  // lane holds channels 16kk + 8hf + e (kk < 8, e < 8) of its columns; NeoX
  // partners i and i + 64 (kk and kk + 4) sit in the same lane.  The global
  // loads go out before the first tiles' copies; the compiler's wait before
  // the prologue covers those copies as well (with a copy into LDS in flight
  // it waits for the vector memory counter to reach zero).
  {
    vec8<E> qraw[2][8], kself[2][8];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const E* qp = q + ((size_t)(c.ok[cb] ? c.tok[cb] : a) * Hq + hq[cb]) * kHeadDim + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) qraw[cb][kk] = *reinterpret_cast<const vec8<E>*>(qp + 16 * kk);
    }
    float w[64];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) w[8 * kk + e] = qnorm_w[16 * kk + 8 * hf + e];
    sink_raw[0] = sinks[hq[0]];
    sink_raw[1] = sinks[hq[1]];
    if (!EXACT) {
      // the token's own k_hat row (chunk 2kk + hf at position (2kk + hf) ^ (t & 15))
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int ts = c.ok[cb] ? c.tok[cb] : a;
        const char* kp = kimg + (size_t)ts * 256;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          kself[cb][kk] = *reinterpret_cast<const vec8<E>*>(kp + (((2 * kk + hf) ^ (ts & 15)) << 4));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the first copies (k_hat 0, V^T 0, k_hat 1) overlap the Q prologue
    if (!EXACT) {
      copy_image(kimg + (size_t)kt_lo * 256, tid, wave_u, lds);
      copy_image(vimg + (size_t)kt_lo * 256, tid, wave_u, lds + kTileK);
      if (n_tiles > 1) {
        copy_image(kimg + (size_t)(kt_lo + kKeyTile) * 256, tid, wave_u, lds + kSlot);
        copy_image(vimg + (size_t)(kt_lo + kKeyTile) * 256, tid, wave_u, lds + kSlot + kTileK);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (rope_tab) {
      rope_table(lds + 2 * kSlot, tid, kThreads, m_tok, a, a_end, doc_start, theta);
      barrier_keep_copies();
    }

#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float x[64];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * kk + e] = (float)qraw[cb][kk][e];
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
      ss = lane_pair_sum(ss);
      // the norm factor carries scale * log2(e) (RoPE is linear, so the order
      // does not matter), and a padding column, which loaded a real token's
      // row, gets a zero factor: zero operands and a zero self score
      const float inv = c.ok[cb] ? c_log2 / sqrtf(ss * (1.0f / kHeadDim) + eps) : 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] *= inv * w[i];
      if (use_rope && c.ok[cb]) {
        if (rope_tab) {
          rope_from_table(lds + 2 * kSlot + (c.tok[cb] - a) * kRopeRow, hf, x);
        } else {
          const int p = c.tok[cb] - doc_start;
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
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) st.qf[cb][kk][e] = (E)x[8 * kk + e];
        // park the Q operands in AGPRs (MFMAs read them from there), which
        // leaves the VGPRs to the scores, weights and operand prefetch
        asm volatile("" : "+a"(st.qf[cb][kk]));
      }
      if (!EXACT) {
        float dot = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) dot += x[8 * kk + e] * (float)kself[cb][kk][e];
        self_score[cb] = lane_pair_sum(dot);
      }
    }
  }

  // swizzled LDS byte offsets of this lane's operand reads inside a slot
  int koff[8], voff[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = col * 256 + (((2 * kk + hf) ^ kswz(col)) << 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) voff[j] = col * 128 + (((2 * j + hf) ^ vswz(col)) << 4);

  // ---- references (log2 domain) ---------------------------------------------
  // main launch: max(sink, the token's own score); follow-up: the exact row max
  float mref[2];
  if (EXACT) {
#pragma unroll
    for (int r = 0; r < 16; ++r) st.negm[0][r] = st.negm[1][r] = 0.f;
    max_pass(lds, koff, st, kimg, kt_lo, n_tiles, tid, wave_u, c, mref);
  } else {
    mref[0] = self_score[0];
    mref[1] = self_score[1];
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float sl = sink_raw[cb] * kLog2e;
    const float m = fmaxf(sl, mref[cb]);
    st.m_ref[cb] = m == -INFINITY ? 0.f : m;
    st.l_part[cb] = (hf == 0 && sl != -INFINITY) ? __builtin_amdgcn_exp2f(sl - st.m_ref[cb]) : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.negm[cb][r] = -st.m_ref[cb];
  }
  {
    vec8<E> zero;
#pragma unroll
    for (int e = 0; e < 8; ++e) zero[e] = (E)0.f;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) zero_acc(st.o[cb][dd], zero);
  }

  attend_pass(lds, koff, voff, st, kimg, vimg, kt_lo, n_tiles, tid, wave_u, c, !EXACT);

  // ---- epilogue: out = O / l in E, lse = ln2 * (m + log2 l) ----------------
  float l[2];
  bool bad = false;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    l[cb] = lane_pair_sum(st.l_part[cb]);
    bad |= c.ok[cb] && !(l[cb] < kRedo);
  }
  agpr_fence();
  if (!EXACT) {
    // a denominator at or past 2^90 (or not finite) hands the block to the
    // follow-up launch; so does an O accumulator that is not finite, which
    // huge values can cause first (weights up to 2^90 times |v| past about
    // 2^38 overflow fp32 while the denominator is still in range).  The
    // denominator is at least 1 (the reference's own weight), so a finite O
    // gives a finite output.
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int r = 0; r < 16; ++r) bad |= c.ok[cb] && !__builtin_isfinite(st.o[cb][dd][r]);
    if (__any(bad) && lane == 0) s_bad = 1;
    __syncthreads();
    const int block_bad = s_bad;
    if (tid == 0) redo[bid] = block_bad;
    if (block_bad) return;
  }
  // A lane holds 4-channel pieces of its two columns' output rows, so storing
  // from the accumulators would write 16 bytes into each of 32 rows per
  // instruction.  The wave's 64 rows go through LDS instead (16 KiB per wave
  // in the first two slots: past the barrier above, or the one below in the
  // follow-up launch, no wave reads a tile and no copy is in flight), and each
  // store instruction writes 4 whole 256-byte rows.  Row r sits at r * 256
  // with its 16-byte chunk k at position k ^ (r % 16).
  if (EXACT) __syncthreads();
  char* obuf = lds + wave * (64 * 256);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float inv_l = 1.0f / l[cb];
    const int row = 32 * cb + col;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        // channels 32dd + 8rq + 4hf .. + 3: chunk 4dd + rq, bytes 8hf .. + 7
        vec4<E> w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (E)(st.o[cb][dd][4 * rq + e] * inv_l);
        const int pos = ((4 * dd + rq) ^ (row & 15)) << 4;
        *reinterpret_cast<vec4<E>*>(obuf + row * 256 + pos + 8 * hf) = w;
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    // row r = 4j + lane/16 of the wave (column r: token tw0 + r/G, head g G + r%G),
    // chunk lane % 16
    const int r = 4 * j + (lane >> 4), k = lane & 15;
    const vec8<E> v = *reinterpret_cast<const vec8<E>*>(obuf + r * 256 + ((k ^ (r & 15)) << 4));
    const int tr = c.tw0 + (r >> log2G);
    if (tr < a_end)
      *reinterpret_cast<vec8<E>*>(out + ((size_t)tr * Hq + g * G + (r & (G - 1))) * kHeadDim +
                                  8 * k) = v;
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
    if (c.ok[cb] && lse != nullptr && hf == 0)
      lse[(size_t)hq[cb] * T + c.tok[cb]] = (st.m_ref[cb] + __log2f(l[cb])) * kLn2;
}

}  // namespace

template <typename E>
hipError_t launch_attention_wide(const E* q, const E* khat, const E* vt,
                                      const int32_t* cu, const int32_t* cu_end,
                                      const int32_t* sched,
                                      const float* sinks, const float* qnorm_w, E* out,
                                      float* lse, int32_t* redo, int T, int D, int Hq,
                                      int Hkv, int64_t t_pad, int64_t items_ub, int window,
                                      int use_rope, double eps, double theta, double scale,
                                      bool exact_all, hipStream_t stream) {
  const int G = Hq / Hkv;
  int log2G = 0;
  while ((1 << log2G) < G) ++log2G;
  // XCD-aware order: when Hkv divides the 8 XCDs, kv head g runs on XCDs
  // [g * 8/Hkv, (g+1) * 8/Hkv) so the blocks streaming one head's keys share L2.
  // The grid size is also the size of the redo table (wide_grid).
  const int xcd_per = (Hkv <= 8 && 8 % Hkv == 0) ? 8 / Hkv : 0;
  const int64_t grid = wide_grid(items_ub, Hkv);
  if (grid <= 0) return hipSuccess;
  const float c_log2 = (float)(scale * 1.4426950408889634);
  // main launch, then the follow-up that reruns the blocks it marked
  attn_fwd_wide_kernel<false, E><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      q, khat, vt, cu, cu_end, sched, sinks, qnorm_w, out, lse, redo, T, Hq, Hkv, G, log2G, t_pad,
      window, use_rope, (float)eps, theta, c_log2, xcd_per, exact_all ? 1 : 0);
  attn_fwd_wide_kernel<true, E><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      q, khat, vt, cu, cu_end, sched, sinks, qnorm_w, out, lse, redo, T, Hq, Hkv, G, log2G, t_pad,
      window, use_rope, (float)eps, theta, c_log2, xcd_per, 0);
  return hipGetLastError();
}

#define SA_INSTANTIATE(E)                                                                     \
  template hipError_t launch_attention_wide<E>(                                          \
      const E*, const E*, const E*, const int32_t*, const int32_t*, const int32_t*,           \
      const float*, const float*, E*, float*, int32_t*, int, int, int, int, int64_t, int64_t, \
      int, int, double, double, double, bool, hipStream_t);
SA_INSTANTIATE(bf16)
SA_INSTANTIATE(f16)
#undef SA_INSTANTIATE

}  // namespace sa
