// bwd.hip -- backward pass of the sink-aware GQA attention, 16-bit in/out
// (bf16, or fp16 for the fp16 I/O variant: the kernels are templates over the
// element type E), gfx950 MFMA.
//
// Gradients of L = sum(dout * out) for the forward of attn_narrow.hip / attn_wide.hip
// (flint.layers FlintAttention: the sinks are trainable fp32 logits,
// _FlintSinkParameters, and the q_norm / k_norm weights are RMSNorm
// parameters).  Per (token t, query head h) with weights P_u = exp(s_u - lse)
// and p_sink = exp(sink_h - lse) (lse saved by the forward):
//   D = dout . out,  dS_u = P_u (dout . v_u - D),  dsink_h = -sum_t p_sink D
//   dv_u = sum P_u dout,  dk_hat_u = scale sum dS_u q_hat,  dq_hat = scale sum dS_u k_hat_u
// then the transposed NeoX rotation and the RMSNorm backward
//   dx = w dy r - x r^3 (sum_c w_c dy_c x_c) / d,  dw += dy x r,  r = (mean(x^2)+eps)^-1/2.
//
// Kernels (one launch each, in this order):
//   bwd_keys_kernel    per 64-key tile: k_hat rows and V rows as LDS row
//                      images
//   bwd_cols_kernel    per 32-column tile (32/G tokens x the G heads of one kv
//                      head): q_hat * scale * log2(e) and dout as row images,
//                      -lse*log2(e) and -D per column, and the tile's share of
//                      dsink
//   bwd_dkdv_kernel    per 128-key block (a wave holds 32 keys' K and V rows
//                      as MFMA operands): walks the column tiles that see the
//                      keys; S = q K^T, P, dP - D = dout V^T - D, dS; dV^T +=
//                      dout^T P, dK^T += q^T dS (AGPR accumulators, the
//                      transposed operands by LDS transpose reads); epilogue:
//                      dv, and dk through the rotation and norm backward
//   bwd_dq_kernel      per 256- or 128-column block (8 or 4 waves of 32
//                      columns): walks the key tiles the columns see;
//                      S^T = K q^T, P^T, dP^T - D, dS^T; dq^T += K^T dS^T;
//                      epilogue: dq through the rotation and norm backward
//   bwd_reduce_kernel  dsinks and both norm-weight gradients from per-tile and
//                      per-block partial sums, in a fixed order
// MFMA operand layouts (32x32x16, wave64): A lane l holds A[l%32][8(l/32)..+7],
// B lane l holds B[8(l/32)..+7][l%32], accumulator register r of lane l is
// C[8(r/4) + 4(l/32) + r%4][l%32].  A 16-step of an accumulator taken as an
// operand (registers 8j..8j+7) covers rows 16j + 8(e/4) + 4(l/32) + e%4, which
// is the order the transpose reads deliver the rows of a row image in.
#include "sa_device.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) void lds_void;

// ---- workspace images ------------------------------------------------------
// Row images only: 256-byte rows of 128 16-bit channels, 16-byte chunk c of
// row r at chunk position c ^ bswz(r).  MFMA operands that run over the rows
// (the transposed products) come from the same images through the LDS
// transpose read.
// key tile (64 keys of one kv head), 32 KiB: k_hat rows | V rows
constexpr int kKT = 16384;                 // one 64-row image
constexpr int kKeyTileBytes = 2 * kKT;
// column tile (32 columns of one kv head), 16.25 KiB: q rows | dout rows |
// (-lse*log2e)[32], (-D)[32]
constexpr int kCT = 8192;                  // one 32-row image
constexpr int kColLd = 2 * kCT;
constexpr int kColTileBytes = 2 * kCT + 256;
// dK/dV workgroups keep a ring of this many column tiles in LDS; one tile
// copy is this many global_load_lds instructions per wave (four of the two
// row images, one of the -lse / -D block)
constexpr int kColBufs = 8;
constexpr int kColCopyOps = 2 * kCT / (16 * kThreads) + 1;
static_assert(kColCopyOps * (kColBufs - 2) < 64, "vmcnt holds 6 bits");

// s_waitcnt vmcnt(N) (other counters untouched); N < 64
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Chunk swizzle of the backward's row images.  Rows are 256 B, so every row
// starts on LDS bank 0 and only the chunk position decides the banks.  The
// MFMA operand read takes one chunk from each of 16 aligned rows: bswz is a
// permutation of 0..15 over them.  The transpose read takes 4 consecutive
// chunks from each of 4 aligned rows: bits 2-3 of bswz differ across those
// rows.  Both reads are therefore free of bank conflicts.
__device__ __forceinline__ int bswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// LDS transpose read (ds_read_b64_tr_b16): in every group of 16 lanes, lane
// 4a + b receives, as its elements 0..3, element b of the 8 bytes read by
// lanes a, a + 4, a + 8 and a + 12 of the group.  Two such reads make one
// MFMA operand of 8 16-bit elements.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;
template <typename E>
__device__ __forceinline__ vec8<E> rd_tr(const char* p0, const char* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_char*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_char*)p1);
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(vec8<E>, v);
}

// Per-lane offsets of the transpose reads for an A operand A[m][k] with
// m = 32 dd + (lane % 32) a channel and k running over 16 rows 16 j .. of a
// row image, in the order the accumulator layout hands out its rows: slot
// 4h + e of lane half hf is row 16 j + 8 h + 4 hf + e.  Reading lane l (in
// its 16-lane group: e = (l % 16) / 4, a = l % 4, G = (l / 16) % 2) fetches
// row 16 j + 8 h + 4 hf + e, channels 32 dd + 16 G + 4a .. + 3, i.e. 8 bytes
// of chunk 4 dd + 2 G + a / 2.  The offset is 4096 j + tr_off(dd, h).
__device__ __forceinline__ int tr_off(int lane, int dd, int h) {
  const int hf = lane >> 5, e = (lane >> 2) & 3, a = lane & 3, G = (lane >> 4) & 1;
  const int r = 8 * h + 4 * hf + e;  // row within the 16-row step (bswz only sees bits 0-3)
  const int c = 4 * dd + 2 * G + (a >> 1);
  return r * 256 + ((c ^ bswz(r)) << 4) + 8 * (a & 1);
}

// Copy nbytes (a multiple of 4096) from global to LDS with global_load_lds.
// The LDS destination goes through readfirstlane as a plain 32-bit address,
// so the compiler keeps no alias information for the copy and adds no waits
// of its own for it: every reader of a copied tile waits with an explicit
// vmcnt and a barrier (with alias information the compiler, unable to follow
// the ring across loop iterations, waits for all copies in flight).
__device__ __forceinline__ void copy_lds(const char* __restrict__ src, int nbytes, int tid,
                                         int nthreads, char* dst) {
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_char*)dst;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int off = 0; off < nbytes; off += 16 * nthreads) {
    const uint32_t a = __builtin_amdgcn_readfirstlane(base + off + 1024 * w);
    __builtin_amdgcn_global_load_lds(src + off + 16 * tid, (lds_void*)(uintptr_t)a, 16, 0, 0);
  }
}

// Copy one column tile: the two row images with every lane, then the 256-byte
// -lse / -D block with lanes 0-3 of every wave (64 bytes per wave).
__device__ __forceinline__ void copy_col_tile(const char* __restrict__ src, int tid, char* dst) {
  copy_lds(src, 2 * kCT, tid, kThreads, dst);
  const uint32_t base = (uint32_t)(uintptr_t)(lds_char*)dst;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t a = __builtin_amdgcn_readfirstlane(base + kColLd + 64 * w);
  if ((tid & 63) < 4)
    __builtin_amdgcn_global_load_lds(src + kColLd + 64 * w + 16 * (tid & 63),
                                     (lds_void*)(uintptr_t)a, 16, 0, 0);
}

// Rows of 128 16-bit channels staged in LDS: row r at r * 256, its 16-byte
// chunk k at position k ^ (r % 16).  A lane of the MFMA accumulator layout
// holds 4-channel pieces of one row (channels 32dd + 8rq + 4hf .. + 3: chunk
// 4dd + rq, bytes 8hf .. + 7); global memory is read and written 4 whole
// rows per instruction (row 4j + lane/16, chunk lane % 16) and the pieces go
// through LDS, instead of 32 rows x 8 bytes per instruction.
__device__ __forceinline__ int stage_pos(int r, int k) { return r * 256 + ((k ^ (r & 15)) << 4); }

// Backward of the rotation and the RMSNorm for one head vector held by a lane
// pair: lane half hf holds the gradient w.r.t. the normalised, rotated vector
// for channels 32dd + 8rq + 4hf + e at dy[16dd + 4rq + e] (dd, rq, e < 4).
// The raw input row is staged row `row` of `rows`, and dx replaces it there
// (in place: each piece is read before it is written); w is the norm weight,
// pos the document position (rope only).  ok: the row is a real token (a
// padding row may hold anything and gets a zero gradient).  dx is zero when
// !ok, and dy x r (zero when !ok) goes to wsum in dy's order.
template <typename E>
__device__ __forceinline__ void norm_rope_bwd_staged(float (&dy)[64], char* rows, int row,
                                                     const float* __restrict__ w, bool ok,
                                                     bool rope, int pos, const double* s_invf,
                                                     float eps, int hf, float (&wsum)[64]) {
  auto piece = [&](int dd, int rq) {
    return reinterpret_cast<vec4<E>*>(rows + stage_pos(row, 4 * dd + rq) + 8 * hf);
  };
  if (rope && ok) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {  // channel 32dd + 8rq + 4hf + e (dd < 2), partner + 64
      const int dd = i >> 4, rq = (i >> 2) & 3, e = i & 3;
      float sn, cs;
      rope_sincos_rev(pos, s_invf[32 * dd + 8 * rq + 4 * hf + e], &sn, &cs);
      const float a = dy[i], b = dy[i + 32];
      dy[i] = a * cs + b * sn;
      dy[i + 32] = b * cs - a * sn;
    }
  }
  float ss = 0.f, wdx = 0.f;
#pragma unroll
  for (int dd = 0; dd < 4; ++dd)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const vec4<E> xv = *piece(dd, rq);
      const f32x4 wv = *reinterpret_cast<const f32x4*>(w + 32 * dd + 8 * rq + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = ok ? (float)xv[e] : 0.f;
        ss += x * x;
        wdx += wv[e] * dy[16 * dd + 4 * rq + e] * x;
      }
    }
  ss = lane_pair_sum(ss);
  wdx = lane_pair_sum(wdx);
  const float r = ok ? 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps) : 0.f;
  const float coef = r * r * r * wdx * (1.0f / kHeadDim);
#pragma unroll
  for (int dd = 0; dd < 4; ++dd)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const vec4<E> xv = *piece(dd, rq);  // read again rather than held in registers
      const f32x4 wv = *reinterpret_cast<const f32x4*>(w + 32 * dd + 8 * rq + 4 * hf);
      vec4<E> o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = ok ? (float)xv[e] : 0.f, g = dy[16 * dd + 4 * rq + e];
        o[e] = (E)(ok ? wv[e] * g * r - x * coef : 0.f);
        wsum[16 * dd + 4 * rq + e] = g * x * r;
      }
      *piece(dd, rq) = o;
    }
}

// LDS writes and reads of one wave in program order (the rows a lane reads
// were written by other lanes of the same wave)
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ============================================================================
// bwd_keys_kernel: one block per (64-key tile, kv head)
// ============================================================================
template <typename E>
__global__ __launch_bounds__(kThreads) void bwd_keys_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_end, const float* __restrict__ knorm_w, int T, int D,
    int Hkv, int n_kt, float eps, double theta, int use_rope, char* __restrict__ keys) {
  __shared__ double s_invf[64];
  __shared__ int s_real[kKeyTile];  // inside [0, T) and not document padding
  __shared__ int s_pos0[kKeyTile];  // start of the token's document (RoPE positions)
  const int tid = threadIdx.x;
  const int tile = blockIdx.x / Hkv, g = blockIdx.x - tile * Hkv;
  const int t0 = tile * kKeyTile;
  char* img = keys + ((size_t)g * n_kt + tile) * kKeyTileBytes;
  // (wave 1: wave 0 looks up the documents)
  if (use_rope && tid >= 64 && tid < 128)
    s_invf[tid - 64] = pow(theta, -(double)(tid - 64) / 64.0) * kInvTwoPi;
  if (tid < kKeyTile) {
    const int t = t0 + tid, t_hi = min(t0 + kKeyTile, T) - 1;
    const int n = t0 < T ? doc_of_token_wave(cu, D, min(t, t_hi), min(t0, t_hi), t_hi) : 0;
    s_real[tid] = t < T && t < cu_end[n];
    s_pos0[tid] = t < T ? cu[n] : 0;
  }
  __syncthreads();
  // V rows straight into the V image
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int r = idx >> 4, c = idx & 15;
    const int t = t0 + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (s_real[r]) val = *reinterpret_cast<const uint4*>(v + ((size_t)t * Hkv + g) * kHeadDim + 8 * c);
    *reinterpret_cast<uint4*>(img + kKT + r * 256 + 16 * (c ^ bswz(r))) = val;
  }
  // K rows: RMSNorm (+RoPE), 8 lanes per token (channels 8c.. and 64+8c..)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = (tid >> 3) + 32 * it;
    const int c = tid & 7;
    const int t = t0 + r;
    const bool real = s_real[r];
    float x[16];
    if (real) {
      const E* kp = k + ((size_t)t * Hkv + g) * kHeadDim;
      const vec8<E> lo = *reinterpret_cast<const vec8<E>*>(kp + 8 * c);
      const vec8<E> hi = *reinterpret_cast<const vec8<E>*>(kp + 64 + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = (float)lo[e];
        x[8 + e] = (float)hi[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss += x[e] * x[e];
    ss += __shfl_xor(ss, 1, 8);
    ss += __shfl_xor(ss, 2, 8);
    ss += __shfl_xor(ss, 4, 8);
    const float inv = real ? 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps) : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] *= inv * knorm_w[8 * c + e];
      x[8 + e] *= inv * knorm_w[64 + 8 * c + e];
    }
    if (use_rope && real) {
      const int p = t - s_pos0[r];
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
    *reinterpret_cast<vec8<E>*>(img + r * 256 + 16 * (c ^ bswz(r))) = lo;
    *reinterpret_cast<vec8<E>*>(img + r * 256 + 16 * ((c + 8) ^ bswz(r))) = hi;
  }
}

// ============================================================================
// bwd_cols_kernel: one block per (32-column tile, kv head)
// ============================================================================
template <typename E>
__global__ __launch_bounds__(kThreads) void bwd_cols_kernel(
    const E* __restrict__ q, const E* __restrict__ out, const E* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_end,
    const float* __restrict__ qnorm_w, int T, int D, int Hq,
    int Hkv, int G, int log2G, int n_ct, float eps, double theta, int use_rope, float c_log2,
    char* __restrict__ cols, float* __restrict__ dsink_part) {
  __shared__ double s_invf[64];
  __shared__ float s_sink[32];
  const int tid = threadIdx.x;
  const int ct = blockIdx.x / Hkv, g = blockIdx.x - ct * Hkv;
  const int tpt = 32 >> log2G;
  char* img = cols + ((size_t)g * n_ct + ct) * kColTileBytes;
  // (wave 1, so that wave 0's document lookup below does not wait behind it)
  if (use_rope && tid >= 64 && tid < 128)
    s_invf[tid - 64] = pow(theta, -(double)(tid - 64) / 64.0) * kInvTwoPi;
  __syncthreads();

  // column col = 8 lanes: lane c holds channels 8c.. and 64+8c..
  const int col = tid >> 3, c = tid & 7;
  const int t = ct * tpt + (col >> log2G);
  const int h = g * G + (col & (G - 1));
  // the token's document; wave w holds columns 8w .. 8w + 7, so its tokens lie
  // in [ct * tpt + (8w >> log2G), ct * tpt + ((8w + 7) >> log2G)]
  const int w8 = (tid >> 6) * 8;
  const int tw_lo = min(ct * tpt + (w8 >> log2G), T - 1);
  const int tw_hi = min(ct * tpt + ((w8 + 7) >> log2G), T - 1);
  const int n = doc_of_token_wave(cu, D, min(t, T - 1), tw_lo, tw_hi);
  // a real query: inside [0, T) and not document padding (padded rows have no
  // gradient: their out is the constant 0)
  const bool ok = t < T && t < cu_end[n];
  float x[16], y[16], o[16];
  if (ok) {
    const size_t row = ((size_t)t * Hq + h) * kHeadDim;
    const vec8<E> ql = *reinterpret_cast<const vec8<E>*>(q + row + 8 * c);
    const vec8<E> qh = *reinterpret_cast<const vec8<E>*>(q + row + 64 + 8 * c);
    const vec8<E> dl = *reinterpret_cast<const vec8<E>*>(dout + row + 8 * c);
    const vec8<E> dh = *reinterpret_cast<const vec8<E>*>(dout + row + 64 + 8 * c);
    const vec8<E> ol = *reinterpret_cast<const vec8<E>*>(out + row + 8 * c);
    const vec8<E> oh = *reinterpret_cast<const vec8<E>*>(out + row + 64 + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = (float)ql[e];
      x[8 + e] = (float)qh[e];
      y[e] = (float)dl[e];
      y[8 + e] = (float)dh[e];
      o[e] = (float)ol[e];
      o[8 + e] = (float)oh[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = y[e] = o[e] = 0.f;
  }
  // q_hat: RMSNorm (+RoPE), then * scale * log2(e) for the exp2 softmax
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    ss += x[e] * x[e];
    dot += y[e] * o[e];
  }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    ss += __shfl_xor(ss, m, 8);
    dot += __shfl_xor(dot, m, 8);
  }
  const float inv = ok ? 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps) : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] *= inv * qnorm_w[8 * c + e];
    x[8 + e] *= inv * qnorm_w[64 + 8 * c + e];
  }
  if (use_rope && ok) {
    const int p = t - cu[n];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sn, cs;
      rope_sincos_rev(p, s_invf[8 * c + e], &sn, &cs);
      const float a = x[e], b = x[8 + e];
      x[e] = a * cs - b * sn;
      x[8 + e] = b * cs + a * sn;
    }
  }
  vec8<E> ql, qh, dl, dh;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ql[e] = (E)(x[e] * c_log2);
    qh[e] = (E)(x[8 + e] * c_log2);
    dl[e] = (E)y[e];
    dh[e] = (E)y[8 + e];
  }
  // row images
  *reinterpret_cast<vec8<E>*>(img + col * 256 + 16 * (c ^ bswz(col))) = ql;
  *reinterpret_cast<vec8<E>*>(img + col * 256 + 16 * ((c + 8) ^ bswz(col))) = qh;
  *reinterpret_cast<vec8<E>*>(img + kCT + col * 256 + 16 * (c ^ bswz(col))) = dl;
  *reinterpret_cast<vec8<E>*>(img + kCT + col * 256 + 16 * ((c + 8) ^ bswz(col))) = dh;
  // per column: -lse*log2e, -D, and the sink's share -p_sink * D
  if (c == 0) {
    float* ld = reinterpret_cast<float*>(img + kColLd);
    const float l = ok ? lse[(size_t)h * T + t] : INFINITY;
    ld[col] = -l * kLog2e;
    ld[32 + col] = -dot;
    s_sink[col] = ok ? -__expf(sinks[h] - l) * dot : 0.f;
  }
  __syncthreads();
  // dsink share of this tile per head of the group (tokens in order)
  if (tid < G) {
    float acc = 0.f;
    for (int j = 0; j < tpt; ++j) acc += s_sink[j * G + tid];
    dsink_part[((size_t)g * n_ct + ct) * G + tid] = acc;
  }
}

// ============================================================================
// bwd_dkdv_kernel: one block per (128-key block, kv head); 4 waves, one per SIMD
// ============================================================================
template <typename E>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const E* __restrict__ k, const char* __restrict__ keys, const char* __restrict__ cols,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_end,
    const float* __restrict__ knorm_w, int T, int D, int Hkv,
    int log2G, int n_kt, int n_ct, int window, int use_rope, float eps, double theta,
    E* __restrict__ dk, E* __restrict__ dv, float* __restrict__ dwk_part) {
  // the ring: one array per slot, so that the compiler can tell a copy into
  // one slot from reads of another (with one array and computed offsets it
  // waits for every copy in flight before reading)
  __shared__ __attribute__((aligned(256))) char ring0[kColTileBytes];
  __shared__ __attribute__((aligned(256))) char ring1[kColTileBytes];
  __shared__ __attribute__((aligned(256))) char ring2[kColTileBytes];
  __shared__ __attribute__((aligned(256))) char ring3[kColTileBytes];
  __shared__ __attribute__((aligned(256))) char ring4[kColTileBytes];
  __shared__ __attribute__((aligned(256))) char ring5[kColTileBytes];
  __shared__ __attribute__((aligned(256))) char ring6[kColTileBytes];
  __shared__ __attribute__((aligned(256))) char ring7[kColTileBytes];
  static_assert(kColBufs == 8, "one array per ring slot");
  auto slot = [&](int b) -> char* {
    switch (b) {
      case 0: return ring0;
      case 1: return ring1;
      case 2: return ring2;
      case 3: return ring3;
      case 4: return ring4;
      case 5: return ring5;
      case 6: return ring6;
      default: return ring7;
    }
  };
  __shared__ double s_invf[64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int kb = blockIdx.x / Hkv, g = blockIdx.x - kb * Hkv;
  const int kb0 = kb * 128;
  const int tpt = 32 >> log2G;
  if (use_rope && tid < 64) s_invf[tid] = pow(theta, -(double)tid / 64.0) * kInvTwoPi;

  // this lane's key (column of S) and the wave's key range
  const int u = kb0 + 32 * wave + col;
  const bool u_ok = u < T;
  const int uc = u_ok ? u : T - 1;
  const int ua = kb0 + 32 * wave, ub = min(ua + 31, T - 1);
  // the key's document by one wave-level lookup (lanes past T look up the
  // wave's last key); the latest token that sees the key is
  // min(document's real end, u + W) - 1, below u for document padding
  const int n_u = doc_of_token_wave(cu, D, uc, min(ua, T - 1), ub);
  const int u_start = cu[n_u];
  int u_last = -1;  // visible tokens [u, u_last]
  if (u_ok) {
    const int e = cu_end[n_u];
    u_last = (window > 0 && u + window < e ? u + window : e) - 1;
  }
  const bool u_real = u_ok && u_last >= u;  // else document padding: no gradient
  const int ua_last = __shfl(u_last, 0);  // lane 0 holds key ua
  // the block's column tiles: tokens [kb0, last viewer of its last key]; the
  // last viewer is non-decreasing in the key, so that is the block's maximum
  // (a block of padding keys only still walks one, fully masked, tile)
  __shared__ int s_last[4];
  const int w_last = wave_max(u_last);
  if (lane == 0) s_last[wave] = w_last;
  __syncthreads();
  const int t_hi = max(max(max(s_last[0], s_last[1]), max(s_last[2], s_last[3])), kb0);
  const int c_lo = kb0 / tpt, c_hi = t_hi / tpt;
  const char* ctiles = cols + (size_t)g * n_ct * kColTileBytes;

  // K and V rows of this lane's key as B operands (channels 16kk + 8hf ..)
  vec8<E> kB[8], vB[8];
  if (ua + 31 < T) {
    // (every key of the wave is below T, wave-uniform) the wave's 32 rows of
    // both images are 8 KiB runs: read as whole 1 KiB pieces (rows 4j ..
    // 4j + 3 per load) and handed to the lanes that hold each row's operand
    // pieces through ring slot `wave`, which the tile copies fill only after
    // the barrier below
    const char* kimg = keys + ((size_t)g * n_kt + (ua >> 6)) * kKeyTileBytes + (ua & 63) * 256;
    vec8<E> ki[8], vi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ki[j] = rd<E>(kimg + 1024 * j + 16 * lane);
      vi[j] = rd<E>(kimg + kKT + 1024 * j + 16 * lane);
    }
    // row r of the staged runs is key ua + r; its chunk positions follow the
    // image's swizzle of row (ua & 63) + r, and ua & 63 is 0 or 32
    char* stg = slot(wave);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<vec8<E>*>(stg + 1024 * j + 16 * lane) = ki[j];
      *reinterpret_cast<vec8<E>*>(stg + 8192 + 1024 * j + 16 * lane) = vi[j];
    }
    wave_lds_fence();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int pos = ((2 * kk + hf) ^ bswz(col)) << 4;
      kB[kk] = *reinterpret_cast<const vec8<E>*>(stg + col * 256 + pos);
      vB[kk] = *reinterpret_cast<const vec8<E>*>(stg + 8192 + col * 256 + pos);
    }
  } else {
    const char* kimg = keys + ((size_t)g * n_kt + (uc >> 6)) * kKeyTileBytes;
    const int r = uc & 63;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int pos = ((2 * kk + hf) ^ bswz(r)) << 4;
      kB[kk] = rd<E>(kimg + r * 256 + pos);
      vB[kk] = rd<E>(kimg + kKT + r * 256 + pos);
    }
  }
  // land them before the tile copies start (a later wait would drain those),
  // and let every wave finish reading its staged rows before the copies
  // overwrite the slots
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(kB[kk]), "v"(vB[kk]));
  __syncthreads();
  f32x16 acc_dv[4], acc_dk[4];
  {
    vec8<E> zero;
#pragma unroll
    for (int e = 0; e < 8; ++e) zero[e] = (E)0.f;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      zero_acc(acc_dv[dd], zero);
      zero_acc(acc_dk[dd], zero);
    }
  }
  // LDS read offsets: operand reads of the row images (row = column) and
  // transpose reads (k over the columns, m over channels)
  int roff[8], toff[4][2];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) roff[kk] = col * 256 + (((2 * kk + hf) ^ bswz(col)) << 4);
#pragma unroll
  for (int dd = 0; dd < 4; ++dd)
#pragma unroll
    for (int h = 0; h < 2; ++h) toff[dd][h] = tr_off(lane, dd, h);

  // The walk runs from the last tile down: the key blocks of a causal
  // document all end at the document's last token, so blocks running at the
  // same time read the same tiles and share them in L2.  Tiles are copied
  // kColBufs - 1 ahead into a ring of kColBufs LDS buffers.
  // The walk is software-pipelined by one tile: while the scores of tile i + 1
  // run on the matrix cores, the vector units turn tile i's scores into P and
  // dS, two elements per score step; then tile i's dV and dK products follow.
  // Every LDS operand is read one step ahead of its MFMA, and scheduling
  // fences keep that order (left alone, the compiler reads each operand just
  // before its use and waits out the LDS latency at every MFMA).
  // Tiles are copied kColBufs - 2 ahead of the one being scored into a ring
  // of kColBufs LDS slots (tile i in slot i % kColBufs).  Past the last tile
  // the copies repeat tile c_lo into slots no later step reads, so every step
  // waits for the same count.  Tiles this wave's keys cannot see are not skipped: the
  // element mask zeroes them (the waves of a block share every step).
  const int n_tiles = c_hi - c_lo + 1;
  auto copy_tile = [&](int i, char* dst) {
    const int c = i < n_tiles ? c_hi - i : c_lo;
    copy_col_tile(ctiles + (size_t)c * kColTileBytes, tid, dst);
  };
  // -lse*log2e and -D of the 16 columns this lane's accumulator rows hold:
  // the starting values of the score accumulators
  auto init_scores = [&](const char* buf, f32x16& s, f32x16& dp) {
    const float* ld = reinterpret_cast<const float*>(buf + kColLd);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(ld + 8 * a + 4 * hf);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(ld + 32 + 8 * a + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[4 * a + e] = l4[e];
        dp[4 * a + e] = d4[e];
      }
    }
  };
  // the element mask of tile c when some (column, key) pair is not visible
  auto mask = [&](int c, f32x16& s) {
    const int ta = c * tpt, tb = ta + tpt - 1;
    if (ta >= ub && tb <= ua_last) return;  // all visible (wave-uniform)
    // column offset o in [0, 32) of the tile is token ta + (o >> log2G), seen
    // by key u iff u <= token <= u_last: the offsets of one run, from
    // (u - ta) << log2G to ((u_last - ta + 1) << log2G) - 1; register r of
    // this lane holds offset 4hf + 8(r/4) + r%4
    // (d0 and d1 are clamped before the shifts; a key no column sees, or a
    // padding key, gets an empty run)
    const int d0 = min(max(u - ta, 0), 32), d1 = u_ok ? min(u_last - ta, 31) : -1;
    const unsigned vis =
        bit_run(d0 << log2G, d1 >= 0 ? min(((d1 + 1) << log2G) - 1, 31) : -1) >> (4 * hf);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = keep_if(vis, 8 * (r >> 2) + (r & 3), s[r]);
  };
  // elements 2m, 2m + 1 of P and dS = P (dP - D), packed as B operands
  auto grads2 = [&](int m, const f32x16& s, const f32x16& dp, vec8<E> (&pb)[2],
                    vec8<E> (&sb)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * m + h;
      const float p = __builtin_amdgcn_exp2f(s[e]);
      pb[e >> 3][e & 7] = (E)p;
      sb[e >> 3][e & 7] = (E)(p * dp[e]);
    }
  };
  // scores of the tile in nbuf (into s_n, dp_n) while P and dS of the
  // finished scores (s_c, dp_c) are formed; then dV^T += dout^T P and
  // dK^T += q^T dS for the finished tile in cbuf.  has_next == false: no next
  // tile (nbuf unused).  Both are compile-time at every call.
  auto step = [&](bool has_next, const char* nbuf, const char* cbuf, const f32x16& s_c,
                  const f32x16& dp_c, f32x16& s_n, f32x16& dp_n) {
    // 16 MFMA pairs: k < 8 scores of the next tile (q and dout rows of
    // nbuf), k >= 8 the products of the finished tile (dout^T and q^T of
    // cbuf); the operands of pair k are read kReadAhead pairs earlier
    constexpr int kReadAhead = 3;
    auto operands = [&](int k, vec8<E>& x, vec8<E>& y) {
      if (k < 8) {
        x = rd<E>(nbuf + roff[k]);
        y = rd<E>(nbuf + kCT + roff[k]);
      } else {
        // step m = 2 dd + j: dout^T and q^T for channels 32 dd.., columns 16 j..
        const int m = k - 8, dd = m >> 1, j = m & 1;
        x = rd_tr<E>(cbuf + kCT + 4096 * j + toff[dd][0], cbuf + kCT + 4096 * j + toff[dd][1]);
        y = rd_tr<E>(cbuf + 4096 * j + toff[dd][0], cbuf + 4096 * j + toff[dd][1]);
      }
    };
    vec8<E> pb[2], sb[2];
    vec8<E> ox[16], oy[16];
    if (has_next) init_scores(nbuf, s_n, dp_n);
#pragma unroll
    for (int k = 0; k < kReadAhead; ++k)
      if (has_next || k >= 8) operands(k, ox[k], oy[k]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int kn = k + kReadAhead;
      if (kn < 16 && (has_next || kn >= 8)) operands(kn, ox[kn], oy[kn]);
      if (k < 8) {
        grads2(k, s_c, dp_c, pb, sb);
        // pin the two new elements here (otherwise they sink to their use)
        asm volatile("" : "+v"(pb[k >> 2]), "+v"(sb[k >> 2]));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (k < 8) {
        if (has_next) {
          s_n = mfma32(ox[k], kB[k], s_n);
          dp_n = mfma32(oy[k], vB[k], dp_n);
        }
      } else {
        const int m = k - 8, dd = m >> 1, j = m & 1;
        if (dd == 0) {
          mfma32_acc_nop(acc_dv[dd], ox[k], pb[j]);
          mfma32_acc_nop(acc_dk[dd], oy[k], sb[j]);
        } else {
          mfma32_acc(acc_dv[dd], ox[k], pb[j]);
          mfma32_acc(acc_dk[dd], oy[k], sb[j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 sx[2], dpx[2];  // scores of the tile being finished / being formed
#pragma unroll
  for (int i = 0; i < kColBufs - 1; ++i) copy_tile(i, slot(i));
  wait_vmcnt<(kColBufs - 2) * kColCopyOps>();  // tile 0 landed
  barrier_keep_copies();
  {
    vec8<E> qa[8], da[8];
    init_scores(slot(0), sx[0], dpx[0]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qa[kk] = rd<E>(slot(0) + roff[kk]);
      da[kk] = rd<E>(slot(0) + kCT + roff[kk]);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      sx[0] = mfma32(qa[kk], kB[kk], sx[0]);
      dpx[0] = mfma32(da[kk], vB[kk], dpx[0]);
    }
  }
  // steady state, unrolled by the ring size (slots are compile-time) and by
  // two for the score registers
  int i = 0;
  for (; i + 1 < n_tiles;) {
#pragma unroll
    for (int b = 0; b < kColBufs; ++b) {  // i % kColBufs == b
      if (i + 1 >= n_tiles) break;
      const int x = b & 1;  // scores of tile i in sx[x]
      mask(c_hi - i, sx[x]);
      // tile i + 1 landed; tiles i + 2 .. i + kColBufs - 2 may be in flight
      wait_vmcnt<(kColBufs - 3) * kColCopyOps>();
      barrier_keep_copies();
      copy_tile(i + kColBufs - 1, slot((b + kColBufs - 1) % kColBufs));
      step(true, slot((b + 1) % kColBufs), slot(b), sx[x], dpx[x], sx[x ^ 1], dpx[x ^ 1]);
      ++i;
    }
  }
  // the last tile (i == n_tiles - 1); its scores sit in sx[i & 1]
  {
    f32x16 dummy_s, dummy_dp;
    // Each case may leave the accumulators in other registers than the next
    // one, and the compiler then copies them where the cases join.  It cannot
    // see that the inline-asm MFMAs wrote them, so the fence provides the wait
    // states an AGPR read needs after an MFMA write.
#define SA_LAST_TILE(B, X)                                    \
  mask(c_hi - i, sx[X]);                                      \
  step(false, slot(0), slot(B), sx[X], dpx[X], dummy_s, dummy_dp); \
  agpr_fence();
    switch (i % kColBufs) {  // the parity of the slot is the parity of i
      case 0: SA_LAST_TILE(0, 0) break;
      case 1: SA_LAST_TILE(1, 1) break;
      case 2: SA_LAST_TILE(2, 0) break;
      case 3: SA_LAST_TILE(3, 1) break;
      case 4: SA_LAST_TILE(4, 0) break;
      case 5: SA_LAST_TILE(5, 1) break;
      case 6: SA_LAST_TILE(6, 0) break;
      default: SA_LAST_TILE(7, 1) break;
    }
#undef SA_LAST_TILE
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  agpr_fence();

  // ---- epilogue: lane holds channels 32dd + 8(r/4) + 4hf + r%4 of key u ----
  // Each wave stages its 32 keys' rows in ring slot 2 + wave (past the
  // barrier above no copy is in flight and no wave reads a tile): dv rows in
  // the first 8 KiB, k rows (then dk in place) in the second.
  char* vrows = slot(2 + wave);
  char* krows = vrows + 32 * 256;
  // row r of the wave: key ua + r (ua = kb0 + 32 wave)
  // dv: the accumulation is the gradient
#pragma unroll
  for (int dd = 0; dd < 4; ++dd)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      vec4<E> w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (E)acc_dv[dd][4 * rq + e];
      *reinterpret_cast<vec4<E>*>(vrows + stage_pos(col, 4 * dd + rq) + 8 * hf) = w;
    }
  // k rows of the wave's keys, 4 whole rows per load (keys past T read key T - 1)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + (lane >> 4), kc = lane & 15;
    const int ur = min(ua + r, T - 1);
    *reinterpret_cast<vec8<E>*>(krows + stage_pos(r, kc)) =
        *reinterpret_cast<const vec8<E>*>(k + ((size_t)ur * Hkv + g) * kHeadDim + 8 * kc);
  }
  wave_lds_fence();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + (lane >> 4), kc = lane & 15;
    if (ua + r < T)
      *reinterpret_cast<vec8<E>*>(dv + ((size_t)(ua + r) * Hkv + g) * kHeadDim + 8 * kc) =
          *reinterpret_cast<const vec8<E>*>(vrows + stage_pos(r, kc));
  }
  // dk_hat = ln2 * acc (q was scaled by scale*log2e); rotate back; RMSNorm
  // bwd; dy x r per channel into LDS rows [key][channel] for the weight sum
  {
    float dy[64];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int r = 0; r < 16; ++r) dy[16 * dd + r] = acc_dk[dd][r] * kLn2;
    const int pos = u_real && use_rope ? u - u_start : 0;
    float wsum[64];
    norm_rope_bwd_staged<E>(dy, krows, col, knorm_w, u_real, use_rope != 0, pos, s_invf, eps,
                            hf, wsum);
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4), kc = lane & 15;
      if (ua + r < T)
        *reinterpret_cast<vec8<E>*>(dk + ((size_t)(ua + r) * Hkv + g) * kHeadDim + 8 * kc) =
            *reinterpret_cast<const vec8<E>*>(krows + stage_pos(r, kc));
    }
    // the weight gradient sums dy x r over the block's keys in a fixed order,
    // one wave (32 keys) at a time through LDS rows [key][channel]
    static_assert(32 * 129 * 4 <= kColTileBytes, "one wave's rows fit a ring slot");
    float* red = reinterpret_cast<float*>(ring0);
    float acc = 0.f;
#pragma unroll
    for (int round = 0; round < 4; ++round) {
      if (wave == round) {
        float* row = red + col * 129;
#pragma unroll
        for (int i = 0; i < 64; ++i) row[32 * (i >> 4) + 8 * ((i >> 2) & 3) + 4 * hf + (i & 3)] = wsum[i];
      }
      __syncthreads();
      if (tid < kHeadDim)
        for (int kr = 0; kr < 32; ++kr) acc += red[kr * 129 + tid];
      __syncthreads();
    }
    if (tid < kHeadDim) dwk_part[(size_t)blockIdx.x * kHeadDim + tid] = acc;
  }
}

// ============================================================================
// bwd_dq_kernel: one block per (WAVES x 32-column block, kv head).  Two
// configurations: 8 waves with a ring of 4 key tiles (128 KiB of LDS, one
// block per CU) for long key walks, and 4 waves with a ring of 2 (64 KiB, two
// blocks per CU) for short documents, where a block's set-up and epilogue
// latencies are as long as its key loop and a second block hides them.
// ============================================================================
template <int WAVES>
struct DqConfig {
  static_assert(WAVES == 4 || WAVES == 8, "two configurations");
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kBufs = WAVES == 8 ? 4 : 2;  // ring of key tiles in LDS
  static constexpr int kCopyOps = kKeyTileBytes / (16 * kThreads);  // copies per wave per tile
  static_assert(kCopyOps * (kBufs - 2) < 64, "vmcnt holds 6 bits");
};

template <typename E, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 8 / WAVES) void bwd_dq_kernel(
    const E* __restrict__ q, const char* __restrict__ keys, const char* __restrict__ cols,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_end,
    const float* __restrict__ qnorm_w, int T, int D, int Hq,
    int Hkv, int G, int log2G, int n_kt, int n_ct, int window, int use_rope, float eps,
    double theta, float scale, E* __restrict__ dq, float* __restrict__ dwq_part) {
  using Cfg = DqConfig<WAVES>;
  constexpr int kDqWaves = WAVES, kDqThreads = Cfg::kThreads, kKeyBufs = Cfg::kBufs;
  constexpr int kKeyCopyOps = Cfg::kCopyOps;
  // the ring of key tiles, one array per slot (see the dK/dV kernel)
  __shared__ __attribute__((aligned(1024))) char ring0[kKeyTileBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[kKeyTileBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[kKeyBufs > 2 ? kKeyTileBytes : 16];
  __shared__ __attribute__((aligned(1024))) char ring3[kKeyBufs > 2 ? kKeyTileBytes : 16];
  auto slot = [&](int b) -> char* {
    return b == 0 ? ring0 : b == 1 ? ring1 : b == 2 ? ring2 : ring3;
  };
  __shared__ double s_invf[64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int n_qb = (n_ct + kDqWaves - 1) / kDqWaves;
  // longest blocks (latest tokens) first
  const int qb = n_qb - 1 - (int)(blockIdx.x / Hkv), g = blockIdx.x % Hkv;
  const int tpt = 32 >> log2G;
  const int ct = qb * kDqWaves + wave;  // this wave's column tile

  // this lane's column: token t, head h
  const int t = ct * tpt + (col >> log2G);
  const int h = g * G + (col & (G - 1));
  const bool t_in = ct < n_ct && t < T;
  // Documents by one wave-level lookup per lane (lanes past T look up the
  // wave's last token), then everything else by reductions: t_lo, the first
  // key token t sees, is non-decreasing in t, so the wave's real tokens
  // [ta, tb] and their first keys are minima and maxima over its lanes, and
  // the block's over its waves.
  const int w_first = min(ct * tpt, T - 1), w_last = min(ct * tpt + tpt - 1, T - 1);
  const int n_t = doc_of_token_wave(cu, D, t_in ? t : w_last, w_first, w_last);
  const bool t_ok = t_in && t < cu_end[n_t];  // a real query
  const int t_start = cu[n_t];
  const int t_lo = t_ok ? (window > 0 ? max(t_start, t - window + 1) : t_start)
                        : 1 << 30;  // visible keys [t_lo, t]
  const int ta = wave_min(t_ok ? t : INT_MAX), tb = wave_max(t_ok ? t : -1);
  const bool wave_ok = ta <= tb;
  const int wa_lo = wave_ok ? wave_min(t_ok ? t_lo : INT_MAX) : 0;
  const int wb_lo = wave_ok ? wave_max(t_ok ? t_lo : -1) : 0;
  __shared__ int s_span[kDqWaves][3];
  if (lane == 0) {
    s_span[wave][0] = ta;
    s_span[wave][1] = tb;
    s_span[wave][2] = wave_ok ? wa_lo : INT_MAX;
  }
  __syncthreads();
  // the block's real tokens [a0, a1] and the first key they see; a block of
  // document padding only (block-uniform) writes zero dq and no weight
  // gradient, and leaves
  int a0 = INT_MAX, a1 = -1, lo = INT_MAX;
#pragma unroll
  for (int w = 0; w < kDqWaves; ++w) {
    a0 = min(a0, s_span[w][0]);
    a1 = max(a1, s_span[w][1]);
    lo = min(lo, s_span[w][2]);
  }
  if (a0 > a1) {
    if (t_in) {
      E* dz = dq + ((size_t)t * Hq + h) * kHeadDim + 4 * hf;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *reinterpret_cast<uint2*>(dz + 32 * (i >> 2) + 8 * (i & 3)) = make_uint2(0, 0);
    }
    if (tid < kHeadDim) dwq_part[(size_t)blockIdx.x * kHeadDim + tid] = 0.f;
    return;
  }
  if (use_rope && tid < 64) s_invf[tid] = pow(theta, -(double)tid / 64.0) * kInvTwoPi;
  // the block's key range: the keys its real tokens see (document padding
  // sees none)
  const int kt_lo = lo & ~(kKeyTile - 1);
  const int n_tiles = (a1 + 1 - kt_lo + kKeyTile - 1) / kKeyTile;
  const char* ktiles = keys + (size_t)g * n_kt * kKeyTileBytes;

  // q (scaled) and dout rows of this lane's column as B operands, -lse*log2e, -D
  vec8<E> qB[8], dB[8];
  float nlse = -INFINITY, nD = 0.f;
  {
    const int ctc = min(ct, n_ct - 1);
    const char* cimg = cols + ((size_t)g * n_ct + ctc) * kColTileBytes;
    if constexpr (WAVES == 4) {
      // Both row images of the wave's column tile are read as whole 1 KiB
      // runs (image rows 4j .. 4j + 3 per load) and handed to the lanes that
      // hold each row's operand pieces through this wave's 8 KiB of ring slot
      // 1, which no copy fills before the key loop's first barrier: first
      // the q image, then, in place, the dout image (the q operand
      // reads are complete before the dout rows overwrite them).  Short blocks
      // spend a good part of their life here.
      vec8<E> qi[8], di[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qi[j] = rd<E>(cimg + 1024 * j + 16 * lane);
        di[j] = rd<E>(cimg + kCT + 1024 * j + 16 * lane);
      }
      char* stg = ring1 + wave * 8192;
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<vec8<E>*>(stg + 1024 * j + 16 * lane) = qi[j];
      wave_lds_fence();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        qB[kk] = *reinterpret_cast<const vec8<E>*>(stg + col * 256 + (((2 * kk + hf) ^ bswz(col)) << 4));
      wave_lds_fence();
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<vec8<E>*>(stg + 1024 * j + 16 * lane) = di[j];
      wave_lds_fence();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        dB[kk] = *reinterpret_cast<const vec8<E>*>(stg + col * 256 + (((2 * kk + hf) ^ bswz(col)) << 4));
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int off = col * 256 + (((2 * kk + hf) ^ bswz(col)) << 4);
        qB[kk] = rd<E>(cimg + off);
        dB[kk] = rd<E>(cimg + kCT + off);
      }
    }
    if (t_ok) {
      nlse = reinterpret_cast<const float*>(cimg + kColLd)[col];
      nD = reinterpret_cast<const float*>(cimg + kColLd)[32 + col];
    }
    // land them before the tile copies start (a later wait would drain those)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(qB[kk]), "v"(dB[kk]));
    asm volatile("" ::"v"(nlse), "v"(nD));
  }
  f32x16 acc[4];
  {
    vec8<E> zero;
#pragma unroll
    for (int e = 0; e < 8; ++e) zero[e] = (E)0.f;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) zero_acc(acc[dd], zero);
  }
  // operand reads of the key images (row = key) and transpose reads of k_hat
  // (k over the keys, m over channels)
  int koff[8], toff[4][2];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = col * 256 + (((2 * kk + hf) ^ bswz(col)) << 4);
#pragma unroll
  for (int dd = 0; dd < 4; ++dd)
#pragma unroll
    for (int h = 0; h < 2; ++h) toff[dd][h] = tr_off(lane, dd, h);
  f32x16 nl16, nd16;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    nl16[r] = nlse;
    nd16[r] = nD;
  }

  // Key tiles are copied kKeyBufs - 1 ahead into a ring of kKeyBufs LDS
  // slots; the slot of each unrolled step is a compile-time constant (see the
  // dK/dV kernel).  Past the last tile the copies repeat the first tile into
  // slots no later step reads, so every step waits for the same count.
  auto copy_tile = [&](int j, char* dst) {
    const int t_idx = (kt_lo >> 6) + (j < n_tiles ? j : 0);
    copy_lds(ktiles + (size_t)t_idx * kKeyTileBytes, kKeyTileBytes, tid, kDqThreads, dst);
  };
#pragma unroll
  for (int j = 0; j < kKeyBufs - 1; ++j) copy_tile(j, slot(j));
  auto tile = [&](const char* buf, int kt) {
    // keys of the tile this wave's tokens cannot see: skip (wave-uniform)
    if (!wave_ok || kt > tb || kt + kKeyTile - 1 < wa_lo) return;
    const bool full = kt + kKeyTile - 1 <= ta && kt >= wb_lo;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // S^T[key][col] * log2e - lse*log2e and dP^T - D for 32 keys
      f32x16 s = nl16, dp = nd16;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s = mfma32(rd<E>(buf + kh * 8192 + koff[kk]), qB[kk], s);
        dp = mfma32(rd<E>(buf + kKT + kh * 8192 + koff[kk]), dB[kk], dp);
      }
      if (!full) {
        // key kt + 32kh + 4hf + 8(r/4) + r%4 is visible iff t_lo <= key <= t
        // (t_lo is past every key for a padding token)
        const int base = kt + 32 * kh + 4 * hf;
        const unsigned vis = bit_run(max(t_lo - base, 0), min(t - base, 27));
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = keep_if(vis, 8 * (r >> 2) + (r & 3), s[r]);
      }
      vec8<E> sb[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sb[jj][e] = (E)(__builtin_amdgcn_exp2f(s[8 * jj + e]) * dp[8 * jj + e]);
      // dq^T[ch][col] += K^T[ch][key] dS^T[key][col]
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          // K^T for channels 32 dd.., keys 32 kh + 16 jj..
          const char* kt_rows = buf + 4096 * (2 * kh + jj);
          const vec8<E> a = rd_tr<E>(kt_rows + toff[dd][0], kt_rows + toff[dd][1]);
          if (dd == 0)
            mfma32_acc_nop(acc[dd], a, sb[jj]);
          else
            mfma32_acc(acc[dd], a, sb[jj]);
        }
    }
  };
  for (int j = 0; j < n_tiles;) {
#pragma unroll
    for (int b = 0; b < kKeyBufs; ++b) {  // j % kKeyBufs == b
      if (j >= n_tiles) break;
      // tile j landed; tiles j + 1 .. j + kKeyBufs - 2 may be in flight
      wait_vmcnt<(kKeyBufs - 2) * kKeyCopyOps>();
      barrier_keep_copies();
      copy_tile(j + kKeyBufs - 1, slot((b + kKeyBufs - 1) % kKeyBufs));
      tile(slot(b), kt_lo + j * kKeyTile);
      ++j;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  agpr_fence();

  // ---- epilogue: dq_hat = scale * acc; rotate back; RMSNorm bwd ------------
  // Each wave stages its 32 columns' q rows (then dq in place) in LDS, 8 KiB
  // per wave in slots 0 and 1 (past the barrier above no copy is in flight
  // and no wave reads a tile).  Row r of the wave is column r: token
  // ct tpt + r / G, head g G + r % G.
  char* qrows = slot(wave >> 2) + (wave & 3) * (32 * 256);
  const bool ct_in = ct < n_ct;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + (lane >> 4), kc = lane & 15;
    const int tr = ct * tpt + (r >> log2G), hr = g * G + (r & (G - 1));
    const int trc = ct_in && tr < T ? tr : 0;
    *reinterpret_cast<vec8<E>*>(qrows + stage_pos(r, kc)) =
        *reinterpret_cast<const vec8<E>*>(q + ((size_t)trc * Hq + hr) * kHeadDim + 8 * kc);
  }
  wave_lds_fence();
  float wsum[64];
  {
    float dy[64];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int r = 0; r < 16; ++r) dy[16 * dd + r] = acc[dd][r] * scale;
    const int pos = t_ok && use_rope ? t - t_start : 0;
    norm_rope_bwd_staged<E>(dy, qrows, col, qnorm_w, t_ok, use_rope != 0, pos, s_invf, eps, hf,
                            wsum);
  }
  wave_lds_fence();
  // dq rows of every column in the grid (zero for document padding)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + (lane >> 4), kc = lane & 15;
    const int tr = ct * tpt + (r >> log2G), hr = g * G + (r & (G - 1));
    if (ct_in && tr < T)
      *reinterpret_cast<vec8<E>*>(dq + ((size_t)tr * Hq + hr) * kHeadDim + 8 * kc) =
          *reinterpret_cast<const vec8<E>*>(qrows + stage_pos(r, kc));
  }
  // The weight gradient sums dy x r over the block's columns in a fixed
  // order: every wave writes its 32 rows of 128 sums (16 KiB per wave, two
  // waves per 32 KiB ring slot; float4 chunk k of row r at position k ^ r),
  // then thread (part, channel c) adds rows 0 .. 31 of waves 2 part and
  // 2 part + 1, and the WAVES / 2 parts are added in order.
  constexpr int kParts = kDqWaves / 2;
  __shared__ float s_quarter[kParts][kHeadDim];
  __syncthreads();  // every wave is done with its staged rows
  {
    float* wrows = reinterpret_cast<float*>(slot(wave >> 1) + (wave & 1) * (32 * 512));
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        // channels 32dd + 8rq + 4hf .. + 3: float4 chunk 8dd + 2rq + hf
        const int kc = 8 * dd + 2 * rq + hf;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = wsum[16 * dd + 4 * rq + e];
        *reinterpret_cast<f32x4*>(wrows + col * 128 + ((kc ^ col) << 2)) = v;
      }
  }
  __syncthreads();
  {
    static_assert(kDqThreads == kParts * kHeadDim, "one part of 128 channels per 2 waves");
    const int c = tid & (kHeadDim - 1), quarter = tid >> 7;
    float part = 0.f;
#pragma unroll
    for (int w = 2 * quarter; w < 2 * quarter + 2; ++w) {
      const float* wrows = reinterpret_cast<const float*>(slot(w >> 1) + (w & 1) * (32 * 512));
      for (int cr = 0; cr < 32; ++cr) part += wrows[cr * 128 + ((((c >> 2) ^ cr) << 2) | (c & 3))];
    }
    s_quarter[quarter][c] = part;
  }
  __syncthreads();
  if (tid < kHeadDim) {
    float sum = s_quarter[0][tid];
#pragma unroll
    for (int pt = 1; pt < kParts; ++pt) sum += s_quarter[pt][tid];
    dwq_part[(size_t)blockIdx.x * kHeadDim + tid] = sum;
  }
}

// ============================================================================
// bwd_reduce_kernel: one block per output (Hq sinks, then 128 + 128 norm
// weight channels); thread i sums partials i, i + 256, ... and a tree in LDS
// adds the 256 sums, so the order is fixed and the result deterministic
// ============================================================================
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(
    const float* __restrict__ dsink_part, const float* __restrict__ dwq_part,
    const float* __restrict__ dwk_part, int Hq, int G, int n_ct, int n_qblk, int n_kblk,
    float* __restrict__ dsinks, float* __restrict__ dqnorm_w, float* __restrict__ dknorm_w) {
  __shared__ float s_red[kThreads];
  const int tid = threadIdx.x;
  const int o = blockIdx.x;
  const float* src;
  size_t stride;
  int n;
  float* dst;
  if (o < Hq) {
    const int g = o / G;
    src = dsink_part + (size_t)g * n_ct * G + (o - g * G);
    stride = G;
    n = n_ct;
    dst = dsinks + o;
  } else if (o < Hq + kHeadDim) {
    src = dwq_part + (o - Hq);
    stride = kHeadDim;
    n = n_qblk;
    dst = dqnorm_w + (o - Hq);
  } else {
    src = dwk_part + (o - Hq - kHeadDim);
    stride = kHeadDim;
    n = n_kblk;
    dst = dknorm_w + (o - Hq - kHeadDim);
  }
  float acc = 0.f;
  for (int i = tid; i < n; i += kThreads) acc += src[(size_t)i * stride];
  s_red[tid] = acc;
  __syncthreads();
#pragma unroll
  for (int m = kThreads / 2; m > 0; m >>= 1) {
    if (tid < m) s_red[tid] += s_red[tid + m];
    __syncthreads();
  }
  if (tid == 0) *dst = s_red[0];
}

}  // namespace

BwdWorkspace plan_bwd_workspace(int64_t T, int64_t D, int Hq, int Hkv) {
  BwdWorkspace w;
  if (T <= 0) return w;
  const int G = Hq / Hkv;
  const int tpt = 32 / G;
  w.n_kt = (T + kKeyTile - 1) / kKeyTile;
  w.n_ct = (T + tpt - 1) / tpt;
  w.n_kblk = (int64_t)((T + 127) / 128) * Hkv;
  // the dQ partial sums are sized for the smaller (4-wave) blocks, which
  // need more of them; the 8-wave blocks use the first half
  w.n_qblk = (int64_t)((w.n_ct + 3) / 4) * Hkv;
  size_t off = 0;
  w.keys_off = off;
  off += (size_t)Hkv * w.n_kt * kKeyTileBytes;
  w.cols_off = off = round_up(off, 256);
  off += (size_t)Hkv * w.n_ct * kColTileBytes;
  w.dsink_off = off = round_up(off, 256);
  off += sizeof(float) * (size_t)Hkv * w.n_ct * G;
  w.dwq_off = off = round_up(off, 256);
  off += sizeof(float) * (size_t)w.n_qblk * kHeadDim;
  w.dwk_off = off = round_up(off, 256);
  off += sizeof(float) * (size_t)w.n_kblk * kHeadDim;
  w.ends_off = off = round_up(off, 256);
  off += sizeof(int32_t) * (size_t)(D + 1);
  w.total = round_up(off, 256);
  return w;
}

template <typename E>
hipError_t launch_bwd(const E* q, const E* k, const E* v, const int32_t* cu,
                           const int32_t* cu_end, const float* sinks, const float* qnorm_w, const float* knorm_w,
                           const E* out, const float* lse, const E* dout, E* dq,
                           E* dk, E* dv, float* dsinks, float* dqnorm_w,
                           float* dknorm_w, int T, int D, int Hq, int Hkv, int window,
                           int use_rope, double eps, double theta, double scale, char* ws,
                           const BwdWorkspace& w, int dq_waves, hipStream_t stream) {
  const int G = Hq / Hkv;
  int log2G = 0;
  while ((1 << log2G) < G) ++log2G;
  char* keys = ws + w.keys_off;
  char* cols = ws + w.cols_off;
  float* dsink_part = reinterpret_cast<float*>(ws + w.dsink_off);
  float* dwq_part = reinterpret_cast<float*>(ws + w.dwq_off);
  float* dwk_part = reinterpret_cast<float*>(ws + w.dwk_off);
  const float c_log2 = (float)(scale * 1.4426950408889634);
  bwd_keys_kernel<E><<<dim3((unsigned)(w.n_kt * Hkv)), dim3(kThreads), 0, stream>>>(
      k, v, cu, cu_end, knorm_w, T, D, Hkv, (int)w.n_kt, (float)eps, theta, use_rope, keys);
  bwd_cols_kernel<E><<<dim3((unsigned)(w.n_ct * Hkv)), dim3(kThreads), 0, stream>>>(
      q, out, dout, lse, sinks, cu, cu_end, qnorm_w, T, D, Hq, Hkv, G, log2G, (int)w.n_ct, (float)eps,
      theta, use_rope, c_log2, cols, dsink_part);
  bwd_dkdv_kernel<E><<<dim3((unsigned)w.n_kblk), dim3(kThreads), 0, stream>>>(
      k, keys, cols, cu, cu_end, knorm_w, T, D, Hkv, log2G, (int)w.n_kt, (int)w.n_ct, window, use_rope,
      (float)eps, theta, dk, dv, dwk_part);
  const int64_t n_qblk = (w.n_ct + dq_waves - 1) / dq_waves * Hkv;
  if (dq_waves == 4)
    bwd_dq_kernel<E, 4><<<dim3((unsigned)n_qblk), dim3(4 * 64), 0, stream>>>(
        q, keys, cols, cu, cu_end, qnorm_w, T, D, Hq, Hkv, G, log2G, (int)w.n_kt, (int)w.n_ct,
        window, use_rope, (float)eps, theta, (float)scale, dq, dwq_part);
  else
    bwd_dq_kernel<E, 8><<<dim3((unsigned)n_qblk), dim3(8 * 64), 0, stream>>>(
        q, keys, cols, cu, cu_end, qnorm_w, T, D, Hq, Hkv, G, log2G, (int)w.n_kt, (int)w.n_ct,
        window, use_rope, (float)eps, theta, (float)scale, dq, dwq_part);
  bwd_reduce_kernel<<<dim3(Hq + 2 * kHeadDim), dim3(kThreads), 0, stream>>>(
      dsink_part, dwq_part, dwk_part, Hq, G, (int)w.n_ct, (int)n_qblk, (int)w.n_kblk,
      dsinks, dqnorm_w, dknorm_w);
  return hipGetLastError();
}

#define SA_INSTANTIATE(E)                                                                     \
  template hipError_t launch_bwd<E>(                                                     \
      const E*, const E*, const E*, const int32_t*, const int32_t*, const float*,             \
      const float*, const float*, const E*, const float*, const E*, E*, E*, E*, float*,       \
      float*, float*, int, int, int, int, int, int, double, double, double, char*,            \
      const BwdWorkspace&, int, hipStream_t);
SA_INSTANTIATE(bf16)
SA_INSTANTIATE(f16)
#undef SA_INSTANTIATE

}  // namespace sa
