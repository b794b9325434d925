// sink_attn_api.hip -- host side of the C ABI declared in include/sink_attn.h:
// argument checks, workspace carve-up and kernel launches.  Every check runs
// before the first HIP call, so a rejected call enqueues nothing (mirroring
// flint.layers _validate_backend and attention.utils, which reject a backend
// or layout they cannot consume instead of falling back).
#include "sink_attn.h"

#include <math.h>

#include <atomic>
#include <mutex>

#include "sa_device.h"

// Device memory sink_attn_fwd_noalloc works in, in place of a caller's
// workspace.  Each device the library runs on holds its own copy for the life
// of the process.  Host code never uses this name as an address (on the host
// it is only a handle the runtime maps to a device address): the entry point
// asks the runtime once per device for that device's address
// (scratch_address below) and every later use goes through that pointer.
static __device__ __align__(256) char scratch[SINK_ATTN_NOALLOC_SCRATCH_BYTES];

namespace sa {

Workspace plan_workspace(int64_t T, int64_t D, int Hq, int Hkv, int d, int dtype) {
  Workspace w;
  if (T <= 0) return w;
  w.t_pad = round_up(T, kKeyTile);
  size_t off = 0;
  if (dtype != SINK_ATTN_F32) {  // 16-bit (bf16 or fp16) images
    const int G = Hq / Hkv;
    w.items_ub = T / tokens_per_block(G) + D;
    w.items_ub_wide = T / tokens_per_block_wide(G) + D;
    w.khat_off = off;
    off += (size_t)Hkv * w.t_pad * kHeadDim * sizeof(bf16);
    off = round_up(off, 256);
    w.vt_off = off;
    off += (size_t)Hkv * kHeadDim * w.t_pad * sizeof(bf16);
    off = round_up(off, 256);
    w.sched_off = off;
    off += sizeof(int32_t) * sched_ints(w.items_ub, D);
    off = round_up(off, 256);
    w.sched_wide_off = off;
    off += sizeof(int32_t) * sched_ints(w.items_ub_wide, D);
    off = round_up(off, 256);
    w.redo_off = off;
    off += sizeof(int32_t) * wide_grid(w.items_ub_wide, Hkv);
  } else {
    w.khat_off = off;
    off += (size_t)T * Hkv * d * sizeof(float);
    off = round_up(off, 256);
    w.vt_off = off;
    off += (size_t)T * Hkv * d * sizeof(float);
  }
  w.ends_off = off = round_up(off, 256);
  off += sizeof(int32_t) * (size_t)(D + 1);
  w.total = round_up(off, 256);
  return w;
}

namespace {

__global__ void doc_ends_kernel(const int32_t* __restrict__ cu,
                                const int32_t* __restrict__ cu_padded, int D,
                                int32_t* __restrict__ ends) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n < D) ends[n] = cu_padded[n] + (cu[n + 1] - cu[n]);
}

// Padding rows of the output: out = 0 and lse = sinks[h] (their softmax holds
// the sink alone).  A workgroup covers kFillTokens tokens: it finds which are
// padding, then clears their rows with coalesced row-wide stores of V (16
// bytes when the output is 16-byte aligned, else 4).
constexpr int kFillTokens = 8;

template <typename V>
__global__ __launch_bounds__(256) void pad_fill_kernel(
    const int32_t* __restrict__ starts, const int32_t* __restrict__ ends, int D, int T, int Hq,
    int row_words, const float* __restrict__ sinks, V* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ int s_pad[kFillTokens];
  const int t0 = blockIdx.x * kFillTokens;
  if (threadIdx.x < kFillTokens) {
    const int t = t0 + (int)threadIdx.x;
    s_pad[threadIdx.x] = t < T && t >= ends[doc_of_token(starts, D, t)];
  }
  __syncthreads();
  V zero;
  memset(&zero, 0, sizeof(zero));
  for (int i = 0; i < kFillTokens; ++i) {
    if (!s_pad[i]) continue;
    V* row = out + (size_t)(t0 + i) * row_words;
    for (int w = threadIdx.x; w < row_words; w += blockDim.x) row[w] = zero;
  }
  if (lse != nullptr)
    for (int idx = threadIdx.x; idx < kFillTokens * Hq; idx += blockDim.x) {
      const int i = idx % kFillTokens, h = idx / kFillTokens;
      if (s_pad[i]) lse[(size_t)h * T + t0 + i] = sinks[h];
    }
}

}  // namespace

hipError_t launch_doc_ends(const int32_t* cu, const int32_t* cu_padded, int D, int32_t* ends,
                           hipStream_t stream) {
  doc_ends_kernel<<<dim3((unsigned)((D + 255) / 256)), dim3(256), 0, stream>>>(cu, cu_padded,
                                                                               D, ends);
  return hipGetLastError();
}

hipError_t launch_pad_fill(const int32_t* starts, const int32_t* ends, int D, int T, int Hq,
                           int d, int dtype, const float* sinks, void* out, float* lse,
                           hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((T + kFillTokens - 1) / kFillTokens);
  const size_t row_bytes = (size_t)Hq * d * (dtype == SINK_ATTN_F32 ? 4 : 2);
  if (row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0)
    pad_fill_kernel<uint4><<<dim3(grid), dim3(256), 0, stream>>>(
        starts, ends, D, T, Hq, (int)(row_bytes / 16), sinks, static_cast<uint4*>(out), lse);
  else
    pad_fill_kernel<uint32_t><<<dim3(grid), dim3(256), 0, stream>>>(
        starts, ends, D, T, Hq, (int)(row_bytes / 4), sinks, static_cast<uint32_t*>(out), lse);
  return hipGetLastError();
}

namespace {

// BSHD attention mask [batch][seq] (nonzero = real token) to padded THD
// boundaries in two launches.  mask_rows_kernel: one workgroup per row counts
// its real tokens and checks that the padding trails (the first padding
// position comes after the last real one); it leaves the count in
// cu[b + 1], or -1 - count for a row whose padding does not trail.
__global__ __launch_bounds__(256) void mask_rows_kernel(const uint8_t* __restrict__ mask,
                                                        int seq, int32_t* __restrict__ cu) {
  __shared__ int s_count, s_first_pad, s_last_real;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    s_count = 0;
    s_first_pad = seq;
    s_last_real = -1;
  }
  __syncthreads();
  const uint8_t* row = mask + (size_t)b * seq;
  int count = 0, first_pad = seq, last_real = -1;
  for (int i = threadIdx.x; i < seq; i += blockDim.x) {
    if (row[i]) {
      ++count;
      last_real = i;
    } else {
      first_pad = min(first_pad, i);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    count += __shfl_xor(count, o);
    first_pad = min(first_pad, __shfl_xor(first_pad, o));
    last_real = max(last_real, __shfl_xor(last_real, o));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&s_count, count);
    atomicMin(&s_first_pad, first_pad);
    atomicMax(&s_last_real, last_real);
  }
  __syncthreads();
  if (threadIdx.x == 0) cu[b + 1] = s_first_pad < s_last_real ? -1 - s_count : s_count;
}

// mask_seqlens_scan_kernel: one workgroup turns the row counts into prefix
// sums (cu_seqlens), writes the slot starts b * seq (cu_seqlens_padded) and
// the number of rows whose padding does not trail.
__global__ __launch_bounds__(256) void mask_seqlens_scan_kernel(int batch, int seq,
                                                                int32_t* __restrict__ cu,
                                                                int32_t* __restrict__ cu_padded,
                                                                int32_t* __restrict__ bad_rows) {
  __shared__ int s_scan[256];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  int carry = 0, bad = 0;
  for (int base = 0; base < batch; base += 256) {
    const int b = base + tid;
    int v = 0;
    if (b < batch) {
      v = cu[b + 1];
      if (v < 0) {
        v = -1 - v;
        ++bad;
      }
    }
    s_scan[tid] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan (Hillis-Steele)
      const int add = tid >= o ? s_scan[tid - o] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    if (b < batch) {
      cu[b + 1] = carry + s_scan[tid];
      cu_padded[b + 1] = (b + 1) * seq;
    }
    carry += s_scan[255];
    __syncthreads();
  }
  if (tid == 0) {
    cu[0] = 0;
    cu_padded[0] = 0;
  }
  atomicAdd(&s_bad, bad);
  __syncthreads();
  if (tid == 0) *bad_rows = s_bad;
}

}  // namespace

}  // namespace sa

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks common to every entry point.
int check_desc(const sink_attn_desc* d) {
  if (d == nullptr) return SINK_ATTN_EINVAL;
  if (d->total_tokens < 0 || d->num_docs < 0 || d->num_q_heads <= 0 ||
      d->num_kv_heads <= 0 || d->head_dim <= 0 || d->max_seqlen < 0 ||
      d->tile_config < sa::kTileAuto || d->tile_config > sa::kTileWideExact)
    return SINK_ATTN_EINVAL;
  if (d->num_q_heads % d->num_kv_heads != 0) return SINK_ATTN_EINVAL;
  if (d->total_tokens > 0 && d->num_docs == 0) return SINK_ATTN_EINVAL;
  if (d->total_tokens > INT32_MAX - 2 * sa::kKeyTile) return SINK_ATTN_EINVAL;
  if (!(d->rms_eps >= 0.0) || !isfinite(d->rms_eps)) return SINK_ATTN_EINVAL;
  if (!(d->rope_theta > 0.0) || !isfinite(d->rope_theta)) return SINK_ATTN_EINVAL;
  if (!isfinite(d->softmax_scale)) return SINK_ATTN_EINVAL;
  if (d->dtype == SINK_ATTN_BF16 || d->dtype == SINK_ATTN_F16) {
    if (d->head_dim != sa::kHeadDim) return SINK_ATTN_EUNSUPPORTED;
    const int G = d->num_q_heads / d->num_kv_heads;
    if (G > sa::kMaxGroup || (G & (G - 1)) != 0) return SINK_ATTN_EUNSUPPORTED;
  } else if (d->dtype == SINK_ATTN_F32) {
    if (d->head_dim != 64 && d->head_dim != 128) return SINK_ATTN_EUNSUPPORTED;
  } else {
    return SINK_ATTN_EUNSUPPORTED;
  }
  return SINK_ATTN_OK;
}

int check_workspace(const sink_attn_desc* d, const sa::Workspace& w) {
  if (w.total == 0) return SINK_ATTN_OK;
  if (d->workspace == nullptr || d->workspace_bytes < w.total) return SINK_ATTN_EWORKSPACE;
  if (!aligned(d->workspace, 256)) return SINK_ATTN_EWORKSPACE;
  return SINK_ATTN_OK;
}

uintptr_t io_align(const sink_attn_desc* d) { return d->dtype == SINK_ATTN_F32 ? 4 : 16; }

sa::Workspace plan(const sink_attn_desc* d) {
  return sa::plan_workspace(d->total_tokens, d->num_docs, d->num_q_heads, d->num_kv_heads,
                            d->head_dim, d->dtype);
}

// 16-bit tile configuration of a call.  Wide tiles (64 columns per wave, one
// workgroup per CU, half the LDS operand traffic per MFMA) win once a query
// block visits many key tiles; narrow ones (32 columns, two workgroups per
// CU, shorter blocks) win on short documents and narrow windows.  The
// automatic choice estimates the mean number of keys a query sees from the
// mean document length L = T / D (the host does not read cu_seqlens): L / 2
// when causal or when the window reaches past L, W - W^2 / 2L for a window
// W < L (the first W tokens of a document see fewer than W keys).
int64_t mean_keys(const sink_attn_desc* d, int32_t window) {
  const int64_t mean_len = (int64_t)d->total_tokens / d->num_docs;
  const int64_t w = window;
  return w > 0 && w < mean_len ? w - w * w / (2 * mean_len) : mean_len / 2;
}
// Mean keys per query from which the automatic choice takes the wide
// attention tiles.  Both configurations timed on one box over causal
// documents of 1,024 to 32,768 tokens and windows of 1,024 to 3,072 keys:
// wide 3-16 % faster from 1,024 keys on; from ~700 to 1,024 either one by up
// to 5 %; narrow up to 8 % faster at 512.
constexpr int64_t kWideKeys = 1024;
// The backward's dQ kernel takes 8-wave workgroups (one per CU, a 4-slot key
// ring) from kDqWideKeys mean keys per query, or from kDqMidKeys when the
// 8-wave grid still has kDqMinBlocks workgroups (eight rounds of the CUs);
// 4-wave ones (two per CU, a 2-slot ring) otherwise.  Timed on one box: 8
// waves 1-7 % faster on 23,417- and 32,768-token batches from 512 mean keys
// on and on one 8,192-token causal document; 4 waves 2-7 % faster on the
// 12,450-token Sliding batch (687 keys) and on 512 short documents (108).
constexpr int64_t kDqWideKeys = 2048;
constexpr int64_t kDqMidKeys = 512;
constexpr int64_t kDqMinBlocks = 2048;

int select_tile(const sink_attn_desc* d, int32_t window) {
  if (d->tile_config != sa::kTileAuto) return d->tile_config;
  if (d->num_docs <= 0) return sa::kTileNarrow;
  return mean_keys(d, window) >= kWideKeys ? sa::kTileWide : sa::kTileNarrow;
}

// Workgroup size of the backward's dQ kernel (4 or 8 waves, see above);
// tile_config narrow / wide force either.  In a padded batch T counts the
// padding, so only the first rule applies there (the 12,450 real tokens of
// the Sliding lengths in 8 slots of 4,096: 4 waves 3 % faster).
int dq_waves(const sink_attn_desc* d, int32_t window, bool padded) {
  if (d->tile_config == sa::kTileNarrow) return 4;
  if (d->tile_config != sa::kTileAuto) return 8;
  if (d->num_docs <= 0) return 4;
  const int64_t keys = mean_keys(d, window);
  // workgroups of the 8-wave grid: 256 query columns each
  const int64_t blocks = (int64_t)d->total_tokens * d->num_q_heads / 256;
  if (keys >= kDqWideKeys) return 8;
  return !padded && keys >= kDqMidKeys && blocks >= kDqMinBlocks ? 8 : 4;
}

double softmax_scale(const sink_attn_desc* d) {
  return d->softmax_scale > 0.0 ? d->softmax_scale : 1.0 / sqrt((double)d->head_dim);
}

// Argument checks of each stage; check_ws = false leaves out the workspace
// (the no-alloc entry point supplies its own).
int check_prologue(const sink_attn_desc* d, const void* k, const void* v,
                   const int32_t* cu, const float* knorm_w, int32_t use_rope,
                   bool check_ws = true) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (use_rope != 0 && use_rope != 1) return SINK_ATTN_EINVAL;
  if (cu == nullptr || !aligned(cu, 4)) return SINK_ATTN_EINVAL;
  if (d->total_tokens == 0) return SINK_ATTN_OK;
  if (k == nullptr || v == nullptr || knorm_w == nullptr) return SINK_ATTN_EINVAL;
  const uintptr_t al = io_align(d);
  if (!aligned(k, al) || !aligned(v, al) || !aligned(knorm_w, 4)) return SINK_ATTN_EINVAL;
  return check_ws ? check_workspace(d, plan(d)) : SINK_ATTN_OK;
}

int check_attention(const sink_attn_desc* d, const void* q, const int32_t* cu,
                    const float* sinks, const float* qnorm_w, int32_t window,
                    int32_t use_rope, const void* out, const float* lse,
                    bool check_ws = true) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (window == 0) return SINK_ATTN_EINVAL;
  if (use_rope != 0 && use_rope != 1) return SINK_ATTN_EINVAL;
  if (cu == nullptr || !aligned(cu, 4)) return SINK_ATTN_EINVAL;
  if (d->total_tokens == 0) return SINK_ATTN_OK;
  if (q == nullptr || sinks == nullptr || qnorm_w == nullptr || out == nullptr)
    return SINK_ATTN_EINVAL;
  const uintptr_t al = io_align(d);
  if (!aligned(q, al) || !aligned(out, al) || !aligned(sinks, 4) || !aligned(qnorm_w, 4) ||
      (lse != nullptr && !aligned(lse, 4)))
    return SINK_ATTN_EINVAL;
  return check_ws ? check_workspace(d, plan(d)) : SINK_ATTN_OK;
}

template <typename E>
hipError_t prologue16(const sink_attn_desc* d, const void* k, const void* v, const int32_t* cu,
                      const int32_t* cu_end, const float* knorm_w, int32_t use_rope,
                      hipStream_t stream) {
  const sa::Workspace w = plan(d);
  char* ws = static_cast<char*>(d->workspace);
  const int G = d->num_q_heads / d->num_kv_heads;
  return sa::launch_prologue_16<E>(
      static_cast<const E*>(k), static_cast<const E*>(v), cu, cu_end, knorm_w, d->total_tokens,
      d->num_docs, d->num_kv_heads, w.t_pad, sa::tokens_per_block(G),
      sa::tokens_per_block_wide(G), d->rms_eps, d->rope_theta, use_rope,
      reinterpret_cast<E*>(ws + w.khat_off), reinterpret_cast<E*>(ws + w.vt_off),
      reinterpret_cast<int32_t*>(ws + w.sched_off),
      reinterpret_cast<int32_t*>(ws + w.sched_wide_off), stream);
}

template <typename E>
hipError_t attention16(const sink_attn_desc* d, int tile, const void* q, const int32_t* cu,
                       const int32_t* cu_end, const float* sinks, const float* qnorm_w,
                       int32_t window, int32_t use_rope, void* out, float* lse,
                       hipStream_t stream) {
  const sa::Workspace w = plan(d);
  char* ws = static_cast<char*>(d->workspace);
  if (tile == sa::kTileWide || tile == sa::kTileWideExact)
    return sa::launch_attention_wide<E>(
        static_cast<const E*>(q), reinterpret_cast<const E*>(ws + w.khat_off),
        reinterpret_cast<const E*>(ws + w.vt_off), cu, cu_end,
        reinterpret_cast<const int32_t*>(ws + w.sched_wide_off), sinks, qnorm_w,
        static_cast<E*>(out), lse, reinterpret_cast<int32_t*>(ws + w.redo_off),
        d->total_tokens, d->num_docs, d->num_q_heads, d->num_kv_heads, w.t_pad,
        w.items_ub_wide, window, use_rope, d->rms_eps, d->rope_theta, softmax_scale(d),
        tile == sa::kTileWideExact, stream);
  return sa::launch_attention_narrow<E>(
      static_cast<const E*>(q), reinterpret_cast<const E*>(ws + w.khat_off),
      reinterpret_cast<const E*>(ws + w.vt_off), cu, cu_end,
      reinterpret_cast<const int32_t*>(ws + w.sched_off), sinks, qnorm_w, static_cast<E*>(out),
      lse, d->total_tokens, d->num_docs, d->num_q_heads, d->num_kv_heads, w.t_pad, w.items_ub,
      window, use_rope, d->rms_eps, d->rope_theta, softmax_scale(d), stream);
}

int launch_prologue(const sink_attn_desc* d, const void* k, const void* v,
                    const int32_t* cu, const int32_t* cu_end, const float* knorm_w,
                    int32_t use_rope, hipStream_t stream) {
  const sa::Workspace w = plan(d);
  char* ws = static_cast<char*>(d->workspace);
  hipError_t e;
  if (d->dtype == SINK_ATTN_BF16) {
    e = prologue16<sa::bf16>(d, k, v, cu, cu_end, knorm_w, use_rope, stream);
  } else if (d->dtype == SINK_ATTN_F16) {
    e = prologue16<sa::f16>(d, k, v, cu, cu_end, knorm_w, use_rope, stream);
  } else {
    e = sa::launch_prologue_f32(static_cast<const float*>(k), static_cast<const float*>(v), cu,
                                cu_end, knorm_w, d->total_tokens, d->num_docs, d->num_kv_heads,
                                d->head_dim, d->rms_eps, d->rope_theta, use_rope,
                                reinterpret_cast<float*>(ws + w.khat_off),
                                reinterpret_cast<float*>(ws + w.vt_off), stream);
  }
  return e == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_ELAUNCH;
}

int launch_attention(const sink_attn_desc* d, const void* q, const int32_t* cu,
                     const int32_t* cu_end, const float* sinks, const float* qnorm_w,
                     int32_t window, int32_t use_rope, void* out, float* lse,
                     hipStream_t stream) {
  const sa::Workspace w = plan(d);
  char* ws = static_cast<char*>(d->workspace);
  hipError_t e;
  if (d->dtype == SINK_ATTN_BF16) {
    e = attention16<sa::bf16>(d, select_tile(d, window), q, cu, cu_end, sinks, qnorm_w, window,
                              use_rope, out, lse, stream);
  } else if (d->dtype == SINK_ATTN_F16) {
    e = attention16<sa::f16>(d, select_tile(d, window), q, cu, cu_end, sinks, qnorm_w, window,
                             use_rope, out, lse, stream);
  } else {
    e = sa::launch_attention_f32(
        static_cast<const float*>(q), reinterpret_cast<const float*>(ws + w.khat_off),
        reinterpret_cast<const float*>(ws + w.vt_off), cu, cu_end, sinks, qnorm_w,
        static_cast<float*>(out), lse,
        d->total_tokens, d->num_docs, d->num_q_heads, d->num_kv_heads, d->head_dim, window,
        use_rope, d->rms_eps, d->rope_theta, softmax_scale(d), stream);
  }
  return e == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_ELAUNCH;
}

sa::BwdWorkspace plan_bwd(const sink_attn_desc* d) {
  return sa::plan_bwd_workspace(d->total_tokens, d->num_docs, d->num_q_heads, d->num_kv_heads);
}

int check_bwd(const sink_attn_desc* d, const void* q, const void* k, const void* v,
              const int32_t* cu, const float* sinks, const float* qnorm_w,
              const float* knorm_w, int32_t window, int32_t use_rope, const void* out,
              const float* lse, const void* dout, const void* dq, const void* dk,
              const void* dv, const float* dsinks, const float* dqnorm_w,
              const float* dknorm_w) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (d->dtype == SINK_ATTN_F32) return SINK_ATTN_EUNSUPPORTED;
  if (window == 0) return SINK_ATTN_EINVAL;
  if (use_rope != 0 && use_rope != 1) return SINK_ATTN_EINVAL;
  if (cu == nullptr || !aligned(cu, 4)) return SINK_ATTN_EINVAL;
  if (sinks == nullptr || qnorm_w == nullptr || knorm_w == nullptr || dsinks == nullptr ||
      dqnorm_w == nullptr || dknorm_w == nullptr)
    return SINK_ATTN_EINVAL;
  const float* f32s[] = {sinks, qnorm_w, knorm_w, dsinks, dqnorm_w, dknorm_w};
  for (const float* p : f32s)
    if (!aligned(p, 4)) return SINK_ATTN_EINVAL;
  if (d->total_tokens == 0) return SINK_ATTN_OK;
  const void* io[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* p : io)
    if (p == nullptr || !aligned(p, 16)) return SINK_ATTN_EINVAL;
  if (lse == nullptr || !aligned(lse, 4)) return SINK_ATTN_EINVAL;
  const sa::BwdWorkspace w = plan_bwd(d);
  if (d->workspace == nullptr || d->workspace_bytes < w.total || !aligned(d->workspace, 256))
    return SINK_ATTN_EWORKSPACE;
  return SINK_ATTN_OK;
}

// Zero-token calls still define the parameter gradients: zero them.
__global__ void zero_f32_kernel(float* a, int na, float* b, int nb, float* c, int nc) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < na) a[i] = 0.f;
  if (i < nb) b[i] = 0.f;
  if (i < nc) c[i] = 0.f;
}

// Document boundaries the kernels use: starts (D + 1 entries, searched to
// find a token's document) and real ends (D entries).  Unpadded THD: both
// from cu_seqlens.  Padded THD: starts = cu_seqlens_padded, ends computed
// into the workspace from the real lengths.
struct Docs {
  const int32_t* starts;
  const int32_t* ends;
};

hipError_t doc_bounds(const sink_attn_desc* d, const int32_t* cu, const int32_t* cu_padded,
                      size_t ends_off, hipStream_t s, Docs* out) {
  if (cu_padded == nullptr) {
    *out = Docs{cu, cu + 1};
    return hipSuccess;
  }
  int32_t* ends = reinterpret_cast<int32_t*>(static_cast<char*>(d->workspace) + ends_off);
  *out = Docs{cu_padded, ends};
  return sa::launch_doc_ends(cu, cu_padded, d->num_docs, ends, s);
}

int check_fwd(const sink_attn_desc* desc, const void* q, const void* k, const void* v,
              const int32_t* cu_seqlens, const int32_t* cu_padded, const float* sinks,
              const float* qnorm_w, const float* knorm_w, int32_t window, int32_t use_rope,
              const void* out, const float* lse, bool check_ws) {
  int rc = check_prologue(desc, k, v, cu_seqlens, knorm_w, use_rope, check_ws);
  if (rc != SINK_ATTN_OK) return rc;
  rc = check_attention(desc, q, cu_seqlens, sinks, qnorm_w, window, use_rope, out, lse,
                       check_ws);
  if (rc != SINK_ATTN_OK) return rc;
  if (cu_padded != nullptr && !aligned(cu_padded, 4)) return SINK_ATTN_EINVAL;
  return SINK_ATTN_OK;
}

// The forward's launches, after check_fwd passed.
int fwd_launch(const sink_attn_desc* desc, const void* q, const void* k, const void* v,
               const int32_t* cu_seqlens, const int32_t* cu_padded, const float* sinks,
               const float* qnorm_w, const float* knorm_w, int32_t window, int32_t use_rope,
               void* out, float* lse, void* stream) {
  if (desc->total_tokens == 0) return SINK_ATTN_OK;
  int rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Docs docs;
  if (doc_bounds(desc, cu_seqlens, cu_padded, plan(desc).ends_off, s, &docs) != hipSuccess)
    return SINK_ATTN_ELAUNCH;
  rc = launch_prologue(desc, k, v, docs.starts, docs.ends, knorm_w, use_rope, s);
  if (rc != SINK_ATTN_OK) return rc;
  rc = launch_attention(desc, q, docs.starts, docs.ends, sinks, qnorm_w, window, use_rope, out,
                        lse, s);
  if (rc != SINK_ATTN_OK || cu_padded == nullptr || desc->dtype == SINK_ATTN_F32) return rc;
  // the fp32 kernel writes padding rows itself; the 16-bit kernels never visit them
  return sa::launch_pad_fill(docs.starts, docs.ends, desc->num_docs, desc->total_tokens,
                             desc->num_q_heads, desc->head_dim, desc->dtype, sinks, out, lse,
                             s) == hipSuccess
             ? SINK_ATTN_OK
             : SINK_ATTN_ELAUNCH;
}

int fwd_impl(const sink_attn_desc* desc, const void* q, const void* k, const void* v,
             const int32_t* cu_seqlens, const int32_t* cu_padded, const float* sinks,
             const float* qnorm_w, const float* knorm_w, int32_t window, int32_t use_rope,
             void* out, float* lse, void* stream) {
  const int rc = check_fwd(desc, q, k, v, cu_seqlens, cu_padded, sinks, qnorm_w, knorm_w,
                           window, use_rope, out, lse, true);
  if (rc != SINK_ATTN_OK) return rc;
  return fwd_launch(desc, q, k, v, cu_seqlens, cu_padded, sinks, qnorm_w, knorm_w, window,
                    use_rope, out, lse, stream);
}

// ---- forward without a caller workspace (sink_attn_fwd_noalloc) -----------
// `scratch` (top of this file) is the memory it works in.

constexpr int kMaxScratchDevices = 64;
std::atomic<char*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device that runs the work of `stream` (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  if (stream == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(stream, &d);
  *dev = d;
  return e;
}

// Address of `scratch` on device dev: looked up on the first call for that
// device with the device current (the caller's current device is restored),
// then kept.
hipError_t scratch_address(int dev, char** addr) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  char* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = 0;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      void* sym = nullptr;
      e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t back = hipSetDevice(cur);
        if (e == hipSuccess) e = back;
      }
      if (e != hipSuccess) return e;
      if (sym == nullptr || !aligned(sym, 256)) return hipErrorInvalidSymbol;
      p = static_cast<char*>(sym);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return hipSuccess;
}

int bwd_impl(const sink_attn_desc* desc, const void* q, const void* k, const void* v,
             const int32_t* cu_seqlens, const int32_t* cu_padded, const float* sinks,
             const float* qnorm_w, const float* knorm_w, int32_t window, int32_t use_rope,
             const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
             float* dsinks, float* dqnorm_w, float* dknorm_w, void* stream) {
  const int rc = check_bwd(desc, q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window,
                           use_rope, out, lse, dout, dq, dk, dv, dsinks, dqnorm_w, dknorm_w);
  if (rc != SINK_ATTN_OK) return rc;
  if (cu_padded != nullptr && !aligned(cu_padded, 4)) return SINK_ATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Hq = desc->num_q_heads, dh = desc->head_dim;
  if (desc->total_tokens == 0) {
    const int n = Hq > dh ? Hq : dh;
    zero_f32_kernel<<<dim3((n + 255) / 256), dim3(256), 0, s>>>(dsinks, Hq, dqnorm_w, dh,
                                                                 dknorm_w, dh);
    return hipGetLastError() == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_ELAUNCH;
  }
  const sa::BwdWorkspace w = plan_bwd(desc);
  Docs docs;
  if (doc_bounds(desc, cu_seqlens, cu_padded, w.ends_off, s, &docs) != hipSuccess)
    return SINK_ATTN_ELAUNCH;
  auto run = [&](auto elem) {
    using E = decltype(elem);
    return sa::launch_bwd<E>(
        static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v),
        docs.starts, docs.ends, sinks, qnorm_w, knorm_w, static_cast<const E*>(out), lse,
        static_cast<const E*>(dout), static_cast<E*>(dq), static_cast<E*>(dk),
        static_cast<E*>(dv), dsinks, dqnorm_w, dknorm_w, desc->total_tokens, desc->num_docs,
        Hq, desc->num_kv_heads, window, use_rope, desc->rms_eps, desc->rope_theta,
        softmax_scale(desc), static_cast<char*>(desc->workspace), w,
        dq_waves(desc, window, cu_padded != nullptr), s);
  };
  const hipError_t e = desc->dtype == SINK_ATTN_F16 ? run(sa::f16{}) : run(sa::bf16{});
  return e == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_ELAUNCH;
}

}  // namespace

extern "C" {

size_t sink_attn_workspace_bytes(const sink_attn_desc* desc) {
  if (check_desc(desc) != SINK_ATTN_OK) return 0;
  return plan(desc).total;
}

int sink_attn_prologue(const sink_attn_desc* desc, const void* k, const void* v,
                       const int32_t* cu_seqlens, const float* knorm_w, int32_t use_rope,
                       void* stream) {
  const int rc = check_prologue(desc, k, v, cu_seqlens, knorm_w, use_rope);
  if (rc != SINK_ATTN_OK || desc->total_tokens == 0) return rc;
  return launch_prologue(desc, k, v, cu_seqlens, cu_seqlens + 1, knorm_w, use_rope,
                         static_cast<hipStream_t>(stream));
}

int sink_attn_attention(const sink_attn_desc* desc, const void* q,
                        const int32_t* cu_seqlens, const float* sinks,
                        const float* qnorm_w, int32_t window, int32_t use_rope, void* out,
                        float* lse, void* stream) {
  const int rc = check_attention(desc, q, cu_seqlens, sinks, qnorm_w, window, use_rope, out,
                                 lse);
  if (rc != SINK_ATTN_OK || desc->total_tokens == 0) return rc;
  return launch_attention(desc, q, cu_seqlens, cu_seqlens + 1, sinks, qnorm_w, window,
                          use_rope, out, lse, static_cast<hipStream_t>(stream));
}

int sink_attn_fwd(const sink_attn_desc* desc, const void* q, const void* k, const void* v,
                  const int32_t* cu_seqlens, const float* sinks, const float* qnorm_w,
                  const float* knorm_w, int32_t window, int32_t use_rope, void* out,
                  float* lse, void* stream) {
  return fwd_impl(desc, q, k, v, cu_seqlens, nullptr, sinks, qnorm_w, knorm_w, window,
                  use_rope, out, lse, stream);
}

int sink_attn_fwd_padded(const sink_attn_desc* desc, const void* q, const void* k,
                         const void* v, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_padded, const float* sinks,
                         const float* qnorm_w, const float* knorm_w, int32_t window,
                         int32_t use_rope, void* out, float* lse, void* stream) {
  if (cu_seqlens_padded == nullptr) return SINK_ATTN_EINVAL;
  return fwd_impl(desc, q, k, v, cu_seqlens, cu_seqlens_padded, sinks, qnorm_w, knorm_w,
                  window, use_rope, out, lse, stream);
}

int sink_attn_fwd_noalloc(const sink_attn_desc* desc, const void* q, const void* k,
                          const void* v, const int32_t* cu_seqlens, const float* sinks,
                          const float* qnorm_w, const float* knorm_w, int32_t window,
                          int32_t use_rope, void* out, float* lse, void* stream) {
  int rc = check_fwd(desc, q, k, v, cu_seqlens, nullptr, sinks, qnorm_w, knorm_w, window,
                     use_rope, out, lse, false);
  if (rc != SINK_ATTN_OK) return rc;
  const size_t need = plan(desc).total;
  if (need > SINK_ATTN_NOALLOC_SCRATCH_BYTES) return SINK_ATTN_ESCRATCH;
  if (desc->total_tokens == 0) return SINK_ATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  char* ws = nullptr;
  if (stream_device(s, &dev) != hipSuccess || scratch_address(dev, &ws) != hipSuccess)
    return SINK_ATTN_ELAUNCH;
  sink_attn_desc d = *desc;
  d.workspace = ws;
  d.workspace_bytes = SINK_ATTN_NOALLOC_SCRATCH_BYTES;
  return fwd_launch(&d, q, k, v, cu_seqlens, nullptr, sinks, qnorm_w, knorm_w, window,
                    use_rope, out, lse, stream);
}

size_t sink_attn_bwd_workspace_bytes(const sink_attn_desc* desc) {
  if (check_desc(desc) != SINK_ATTN_OK || desc->dtype == SINK_ATTN_F32) return 0;
  return plan_bwd(desc).total;
}

int sink_attn_bwd(const sink_attn_desc* desc, const void* q, const void* k, const void* v,
                  const int32_t* cu_seqlens, const float* sinks, const float* qnorm_w,
                  const float* knorm_w, int32_t window, int32_t use_rope, const void* out,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  float* dsinks, float* dqnorm_w, float* dknorm_w, void* stream) {
  return bwd_impl(desc, q, k, v, cu_seqlens, nullptr, sinks, qnorm_w, knorm_w, window,
                  use_rope, out, lse, dout, dq, dk, dv, dsinks, dqnorm_w, dknorm_w, stream);
}

int sink_attn_bwd_padded(const sink_attn_desc* desc, const void* q, const void* k,
                         const void* v, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_padded, const float* sinks,
                         const float* qnorm_w, const float* knorm_w, int32_t window,
                         int32_t use_rope, const void* out, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* dsinks,
                         float* dqnorm_w, float* dknorm_w, void* stream) {
  if (cu_seqlens_padded == nullptr) return SINK_ATTN_EINVAL;
  return bwd_impl(desc, q, k, v, cu_seqlens, cu_seqlens_padded, sinks, qnorm_w, knorm_w,
                  window, use_rope, out, lse, dout, dq, dk, dv, dsinks, dqnorm_w, dknorm_w,
                  stream);
}

int sink_attn_mask_to_seqlens(const uint8_t* attention_mask, int32_t batch, int32_t seq,
                              int32_t* cu_seqlens, int32_t* cu_seqlens_padded,
                              int32_t* bad_rows, void* stream) {
  if (batch < 0 || seq < 0 || (int64_t)batch * seq > INT32_MAX - 2 * sa::kKeyTile)
    return SINK_ATTN_EINVAL;
  if (cu_seqlens == nullptr || cu_seqlens_padded == nullptr || bad_rows == nullptr ||
      !aligned(cu_seqlens, 4) || !aligned(cu_seqlens_padded, 4) || !aligned(bad_rows, 4))
    return SINK_ATTN_EINVAL;
  if ((int64_t)batch * seq > 0 && attention_mask == nullptr) return SINK_ATTN_EINVAL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (batch > 0)  // (seq = 0: every row counts 0 and reads nothing)
    sa::mask_rows_kernel<<<dim3((unsigned)batch), dim3(256), 0, st>>>(attention_mask, seq,
                                                                       cu_seqlens);
  sa::mask_seqlens_scan_kernel<<<dim3(1), dim3(256), 0, st>>>(batch, seq, cu_seqlens,
                                                              cu_seqlens_padded, bad_rows);
  return hipGetLastError() == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_ELAUNCH;
}

int sink_attn_tile_config(const sink_attn_desc* desc, int32_t window) {
  const int rc = check_desc(desc);
  if (rc != SINK_ATTN_OK) return rc;
  if (window == 0) return SINK_ATTN_EINVAL;
  if (desc->dtype == SINK_ATTN_F32) return 0;
  return select_tile(desc, window);
}

const char* sink_attn_status_string(int status) {
  switch (status) {
    case SINK_ATTN_OK: return "success";
    case SINK_ATTN_EINVAL: return "invalid argument";
    case SINK_ATTN_EUNSUPPORTED: return "unsupported configuration";
    case SINK_ATTN_EWORKSPACE: return "workspace missing, too small or misaligned";
    case SINK_ATTN_ELAUNCH: return "kernel launch failed";
    case SINK_ATTN_ESCRATCH:
      return "call needs more than the no-alloc scratch (SINK_ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int sink_attn_version(void) { return 500; }

}  // extern "C"
