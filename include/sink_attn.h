/*
 * sink_attn.h -- C ABI of the MI355X (gfx950) sink-aware grouped-query
 * attention forward pass: per-head RMSNorm and NeoX RoPE on Q and K, then
 * causal or sliding-window attention over packed variable-length documents
 * with one learned fp32 sink logit per query head -- and its backward pass.
 *
 * Sources (NeMo AutoModel API reference pages):
 *   "flint.layers"     FlintAttention: separate Q/K/V, per-head RMSNorm,
 *                      selective NeoX RoPE (_apply_rope rotates corresponding
 *                      channels of the two halves of each head), forward()
 *                      computes causal attention with a zero-value sink
 *                      category over document-local zero-based positions;
 *                      _FlintSinkParameters: unscaled FP32 logits, one per
 *                      query head, that enter only the softmax denominator.
 *   "flint.config"     FlintConfig: head_dim 128, 32 query / 4 KV heads,
 *                      rms_norm_eps 1e-6; full layers have no RoPE, sliding
 *                      layers rotate all channels; the window counts the
 *                      current token.
 *   "flint.layers"     (backward) the sinks are trainable parameters
 *                      (_FlintSinkParameters) and q_norm / k_norm are RMSNorm
 *                      modules with weights, so a training step needs the
 *                      gradients of q, k, v, the sinks and both weights.
 *   "flint.layers"     (padding) FlintAttention.forward attention_mask:
 *                      padded queries and keys are excluded from the real
 *                      attention while the sink stays valid; BSHD supports
 *                      trailing padding, other padding uses THD packing.
 *   "attention.utils"  (padding) packed inputs may carry cu_seqlens_padded
 *                      beside cu_seqlens, both int32 [documents + 1].
 *   "attention.utils"  preprocess_args_and_kwargs_for_attn: THD tensors
 *                      [tokens, heads, head_dim], K and V share a layout,
 *                      int32 cu_seqlens [documents + 1], a positive left
 *                      window counts visible keys including the current token
 *                      and a negative one is unbounded; a layout that cannot
 *                      be consumed is rejected with an error.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, on the
 *     device that owns `stream`.  The library never allocates, frees or
 *     synchronises, never writes q, k or v, and keeps no state between calls
 *     (one exception: the device array of sink_attn_fwd_noalloc, below).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns at once.  Buffers must stay alive until it completes.
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns a negative status and enqueues nothing.  There is no fallback to
 *     another path.
 *   - Layouts are THD and contiguous: q and out [T, Hq, d]; k and v
 *     [T, Hkv, d]; lse [Hq, T]; query head h reads kv head h / (Hq / Hkv).
 *   - Document n holds tokens [cu_seqlens[n], cu_seqlens[n+1]); a token's
 *     position is its index inside its document.  cu_seqlens must start at 0,
 *     be non-decreasing and end at T (empty documents are allowed); this is
 *     not checked on the device.
 *   - Key j of a document is visible to query i of the same document iff
 *     j <= i and, when window > 0, i - window < j.  window < 0 is unbounded
 *     (causal); window == 0 is rejected.
 *   - out = sum_j softmax weight * v_j where the softmax includes one extra
 *     category per query head whose logit is sinks[h] (used as given, not
 *     multiplied by softmax_scale) and whose value is zero.
 *     lse[h, i] = log of the full denominator, sink included (natural log).
 *   - Accuracy of the 16-bit paths against an exact (fp64) evaluation of the
 *     same definition: max-abs 2e-2 and mean-abs 2e-3 on out and lse for
 *     bf16 storage (4e-3 and 3e-4 for fp16) at Flint's settings -- scores
 *     scale * <q_hat, k_hat> of unit-RMS heads with norm weights near 1 and
 *     the default scale 1/sqrt(128).  The rounding of q_hat and k_hat to the
 *     storage type moves a score by up to 2 * 2^-9 (bf16; 2^-11 fp16) of
 *     scale * sum_i |q_hat_i k_hat_i|, so that error grows in proportion to
 *     softmax_scale and to the product of the two norm weights: at a scale
 *     of 0.2 (1.8 times the default) one bf16 case measured 0.022.  The fp32
 *     path agrees within 1e-5.
 */
#ifndef SINK_ATTN_H
#define SINK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SINK_ATTN_OK = 0,
  SINK_ATTN_EINVAL = -1,        /* invalid argument: null pointer, bad size, window == 0 */
  SINK_ATTN_EUNSUPPORTED = -2,  /* well-formed but not provided (head_dim, dtype, group) */
  SINK_ATTN_EWORKSPACE = -3,    /* workspace missing or smaller than required */
  SINK_ATTN_ELAUNCH = -4,       /* a kernel launch failed (hipGetLastError) */
  SINK_ATTN_ESCRATCH = -5       /* sink_attn_fwd_noalloc: the call needs more device
                                   memory than SINK_ATTN_NOALLOC_SCRATCH_BYTES */
} sink_attn_status;

typedef enum {
  SINK_ATTN_BF16 = 0,  /* q, k, v, out bf16; fp32 arithmetic and accumulation */
  SINK_ATTN_F32 = 1,   /* q, k, v, out fp32; fp32 arithmetic throughout (debug path) */
  SINK_ATTN_F16 = 2    /* q, k, v, out fp16: the fp16 I/O variant (flint.config,
                          attention_compute_dtype = 'fp16': an fp16 QKV and
                          kernel-output boundary).  Same kernels and limits as
                          bf16 with fp16 MFMA operands (q_hat, k_hat, V, the
                          weights P; dS and dout in the backward), fp32
                          arithmetic and accumulation.  fp16's range bounds
                          the softmax references: sinks and scores must stay
                          within about 22,700 (natural-log units). */
} sink_attn_dtype;

/* Attention tile configuration of the 16-bit paths.  Both compute the same
 * function to the same tolerance; they differ in speed.  Narrow: each wave
 * holds 32 (token, head) query columns, two workgroups share a compute unit;
 * best for short documents and narrow windows.  Wide: 64 columns per wave,
 * one workgroup per compute unit, half the LDS operand traffic per matrix
 * instruction; best when every query sees thousands of keys (long causal
 * documents, wide windows).  The fp32 path has a single configuration and
 * ignores the setting.  In the backward, narrow selects dQ workgroups of
 * 128 query columns (two per compute unit) and wide of 256 (one per compute
 * unit); automatic takes the latter when a query sees at least 2,048 keys on
 * average, or at least 512 in an unpadded batch of T * num_q_heads >= 524,288
 * (the estimate of sink_attn_tile_config).  dq, dk, dv and dsinks do not
 * depend on the setting; dqnorm_w is summed over the dQ workgroups, so its
 * rounding does. */
typedef enum {
  SINK_ATTN_TILE_AUTO = 0,
  SINK_ATTN_TILE_NARROW = 1,
  SINK_ATTN_TILE_WIDE = 2,
  /* Wide tiles with every query block taking the path normally reserved for
   * blocks whose scores rise more than 90 log2 units above the token's own
   * score: a scores-only pass for the exact row max first.  Same results,
   * slower; for testing that path. */
  SINK_ATTN_TILE_WIDE_EXACT = 3
} sink_attn_tile_config_t;

/* Shapes and settings of one call.  Plain data; the library keeps no pointer
 * to it after a call returns. */
typedef struct {
  int32_t total_tokens;   /* T = cu_seqlens[num_docs] >= 0 */
  int32_t num_docs;       /* D >= 0; cu_seqlens has D + 1 entries */
  int32_t num_q_heads;    /* Hq > 0 */
  int32_t num_kv_heads;   /* Hkv > 0, Hq % Hkv == 0 */
  int32_t head_dim;       /* d: 128 (bf16, fp16 and fp32) or 64 (fp32 only) */
  int32_t dtype;          /* sink_attn_dtype of q, k, v and out */
  int32_t max_seqlen;     /* optional hint (0 = unknown); not needed, not trusted */
  int32_t tile_config;    /* sink_attn_tile_config_t: 0 automatic (use this), 1-3 force */
  double rms_eps;         /* RMSNorm epsilon, added to mean(x^2); 1e-6 for Flint */
  double rope_theta;      /* RoPE base; inv_freq_i = theta^(-2i/d) */
  double softmax_scale;   /* <= 0 selects 1/sqrt(head_dim) */
  void* workspace;        /* device scratch of >= sink_attn_workspace_bytes(desc) */
  size_t workspace_bytes; /* bytes available at workspace (256-byte aligned) */
} sink_attn_desc;

/* Bytes of device workspace a call with this descriptor needs (0 when T == 0).
 * Not on the pages: the library's own scratch (normalised keys, the value
 * layout the attention stage reads, the work schedule), which the caller
 * allocates so that the library never allocates device memory.
 * Depends only on total_tokens, num_docs, num_q_heads, num_kv_heads, head_dim
 * and dtype (not on tile_config).
 * Returns 0 for a NULL or invalid descriptor. */
size_t sink_attn_workspace_bytes(const sink_attn_desc* desc);

/* The whole forward pass: normalised/rotated Q and K, band-limited attention
 * with the sink, out and lse.  Equivalent to sink_attn_prologue followed by
 * sink_attn_attention on the same stream.
 * Defined by "flint.layers" FlintAttention.forward (causal attention with a
 * zero-value sink category over document-local positions), FlintAttention's
 * q_norm / k_norm and _apply_rope, _FlintSinkParameters (unscaled fp32
 * logits, one per query head), "flint.config" FlintConfig (sliding window
 * counting the current token; RoPE on sliding layers only; rms_norm_eps) and
 * "attention.utils" preprocess_args_and_kwargs_for_attn (THD layout,
 * cu_seqlens, window_size).
 *   q [T,Hq,d], k [T,Hkv,d], v [T,Hkv,d]   inputs in desc->dtype (16-byte aligned)
 *   cu_seqlens  int32 [D+1]
 *   sinks       fp32 [Hq], unscaled logits (finite, or -inf to disable a head's sink)
 *   qnorm_w     fp32 [d], RMSNorm weight shared by all query heads
 *   knorm_w     fp32 [d], RMSNorm weight shared by all kv heads
 *   window      > 0 sliding window counting the current token, < 0 causal
 *   use_rope    1: NeoX RoPE on Q and K at document positions; 0: none
 *   out         [T,Hq,d] in desc->dtype (16-byte aligned), fully written
 *   lse         fp32 [Hq,T] or NULL (not written) */
int sink_attn_fwd(const sink_attn_desc* desc, const void* q, const void* k,
                  const void* v, const int32_t* cu_seqlens, const float* sinks,
                  const float* qnorm_w, const float* knorm_w, int32_t window,
                  int32_t use_rope, void* out, float* lse, void* stream);

/* First stage of sink_attn_fwd: RMSNorm (+ RoPE) of K into the workspace, the
 * value layout the attention stage reads, and the varlen work schedule derived
 * from cu_seqlens.  Writes only the workspace.
 * Defined by "flint.layers" FlintAttention (k_norm, _apply_rope: the two
 * halves of each head rotated together) and "attention.utils"
 * preprocess_args_and_kwargs_for_attn (cu_seqlens document boundaries). */
int sink_attn_prologue(const sink_attn_desc* desc, const void* k, const void* v,
                       const int32_t* cu_seqlens, const float* knorm_w,
                       int32_t use_rope, void* stream);

/* Second stage of sink_attn_fwd: RMSNorm (+ RoPE) of Q fused with the
 * attention itself.  Reads the workspace a preceding sink_attn_prologue with
 * the same descriptor, k, v, cu_seqlens, knorm_w and use_rope filled.
 * Defined by "flint.layers" FlintAttention.forward (the sink category) with
 * q_norm and _apply_rope, and _FlintSinkParameters. */
int sink_attn_attention(const sink_attn_desc* desc, const void* q,
                        const int32_t* cu_seqlens, const float* sinks,
                        const float* qnorm_w, int32_t window, int32_t use_rope,
                        void* out, float* lse, void* stream);

/* The tile configuration (SINK_ATTN_TILE_NARROW, _WIDE or _WIDE_EXACT) that
 * sink_attn_attention would use for this descriptor and window, 0 for the fp32
 * path, or a negative status for an invalid descriptor or window == 0.
 * Not on the pages: a choice between two kernels of this library that
 * compute the same function.  The
 * automatic choice takes the wide tiles when a query sees at least 1,024
 * keys on average, estimated from the mean document length L = T / D: L / 2
 * when causal or when the window is at least L, W - W^2 / 2L for a window
 * W < L.  Reads no device memory. */
int sink_attn_tile_config(const sink_attn_desc* desc, int32_t window);

/* Padded THD.  Defined by "flint.layers" FlintAttention.forward
 * (attention_mask: padded queries and keys leave the real attention, the
 * sink stays valid) and "attention.utils" (packed inputs may carry
 * cu_seqlens_padded beside cu_seqlens).
 * cu_seqlens holds the real document lengths (as prefix sums)
 * and cu_seqlens_padded, also int32 [D+1], where each document starts in the
 * packed tensors: document n's real tokens are
 *   [cu_seqlens_padded[n], cu_seqlens_padded[n] + cu_seqlens[n+1] - cu_seqlens[n])
 * and the rest of [cu_seqlens_padded[n], cu_seqlens_padded[n+1]) is padding;
 * desc->total_tokens = cu_seqlens_padded[D] counts the padding.  Positions
 * run from 0 at each document's first token.  Padding tokens are excluded as
 * keys and as queries: a padding query's softmax holds the sink alone, so its
 * out row is 0 and its lse is sinks[h].  Whatever the inputs hold at padding
 * rows (even NaN) does not reach the real rows.  The boundaries are not
 * checked on the device: cu_seqlens_padded must start at 0, be
 * non-decreasing, end at T, and leave every document room for its real
 * tokens.  Otherwise as sink_attn_fwd (same workspace size). */
int sink_attn_fwd_padded(const sink_attn_desc* desc, const void* q, const void* k,
                         const void* v, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_padded, const float* sinks,
                         const float* qnorm_w, const float* knorm_w, int32_t window,
                         int32_t use_rope, void* out, float* lse, void* stream);

/* Padded-THD boundaries of a BSHD attention mask ("flint.layers"
 * FlintAttention.forward: BSHD takes trailing padding, other padding is
 * packed as THD): attention_mask is a device
 * uint8 [batch][seq] (nonzero = real token) whose rows must be a run of real
 * tokens followed by padding (trailing padding, as Transformer Engine's BSHD
 * takes; other padding has to be packed as THD).  Writes cu_seqlens and
 * cu_seqlens_padded (int32 [batch+1] each; row b starts at b * seq) so that
 * [batch, seq, heads, d] tensors, viewed as [batch * seq, heads, d], run
 * through the padded-THD entry points; writes into *bad_rows (device int32)
 * the number of rows whose padding does not trail (those boundaries are then
 * meaningless; check it before use).  Every pointer is a device pointer. */
int sink_attn_mask_to_seqlens(const uint8_t* attention_mask, int32_t batch, int32_t seq,
                              int32_t* cu_seqlens, int32_t* cu_seqlens_padded,
                              int32_t* bad_rows, void* stream);

/* Bytes of device workspace sink_attn_bwd needs for this descriptor (0 when
 * T == 0, for the fp32 path, or for an invalid descriptor).  Not on the
 * pages: the backward's own scratch (key and column tile images, partial
 * sums), which the caller allocates.  The forward's
 * workspace can be reused once the forward has completed; the backward does
 * not read what the forward left there. */
size_t sink_attn_bwd_workspace_bytes(const sink_attn_desc* desc);

/* Backward pass of sink_attn_fwd (bf16 and fp16): the gradients of
 * L = sum(dout * out) with respect to every input of the forward.
 * Defined by the forward's pages plus "flint.layers" _FlintSinkParameters
 * (the sinks are trainable parameters) and FlintAttention's q_norm / k_norm
 * (RMSNorm modules with weights).
 *   q, k, v, cu_seqlens, sinks, qnorm_w, knorm_w, window, use_rope
 *               exactly as passed to the forward
 *   out [T,Hq,d] (desc->dtype) and lse fp32 [Hq,T]: what that forward wrote (lse is
 *               required here)
 *   dout        [T,Hq,d] desc->dtype, the gradient of the loss with respect to out
 *   dq [T,Hq,d], dk [T,Hkv,d], dv [T,Hkv,d]   desc->dtype, fully overwritten
 *   dsinks fp32 [Hq], dqnorm_w fp32 [d], dknorm_w fp32 [d]   overwritten, not
 *               accumulated (zero when T == 0)
 * desc->workspace must hold sink_attn_bwd_workspace_bytes(desc) bytes
 * (256-byte aligned); every 16-bit tensor 16-byte aligned.  Gradients through
 * the softmax use D = dout . out per (token, head) with the stored out.  The
 * sums over tokens (dsinks, norm weights) are added in a fixed order: equal
 * inputs give bitwise equal outputs.  fp32 descriptors return
 * SINK_ATTN_EUNSUPPORTED. */
int sink_attn_bwd(const sink_attn_desc* desc, const void* q, const void* k,
                  const void* v, const int32_t* cu_seqlens, const float* sinks,
                  const float* qnorm_w, const float* knorm_w, int32_t window,
                  int32_t use_rope, const void* out, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, float* dsinks,
                  float* dqnorm_w, float* dknorm_w, void* stream);

/* Backward of sink_attn_fwd_padded: as sink_attn_bwd, with padded-THD
 * boundaries ("flint.layers" FlintAttention.forward attention_mask).  Padding rows of dq, dk and dv are written as zeros; padding
 * rows contribute nothing to dsinks and the norm-weight gradients. */
int sink_attn_bwd_padded(const sink_attn_desc* desc, const void* q, const void* k,
                         const void* v, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_padded, const float* sinks,
                         const float* qnorm_w, const float* knorm_w, int32_t window,
                         int32_t use_rope, const void* out, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* dsinks,
                         float* dqnorm_w, float* dknorm_w, void* stream);

/* Device memory the library keeps for sink_attn_fwd_noalloc: 80 MiB, once per
 * device it runs on, held until the process ends.  That covers a forward of
 * up to about 40,000 tokens at 4 kv heads and head_dim 128 in bf16 or fp16
 * (sink_attn_workspace_bytes(desc) <= this). */
#define SINK_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)

/* sink_attn_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results as sink_attn_fwd (bitwise), except that
 * desc->workspace and desc->workspace_bytes are ignored: the call runs in a
 * device array of SINK_ATTN_NOALLOC_SCRATCH_BYTES that the library holds,
 * and never allocates or frees anything itself.
 *   - A descriptor whose sink_attn_workspace_bytes() exceeds
 *     SINK_ATTN_NOALLOC_SCRATCH_BYTES returns SINK_ATTN_ESCRATCH and enqueues
 *     nothing; argument errors return as for sink_attn_fwd.
 *   - The array of the stream's device is looked up on the first call on
 *     that device (hipGetSymbolAddress, which is not an allocation);
 *     SINK_ATTN_ELAUNCH if that fails.
 *   - Every call on one device uses that device's one array, which keeps the
 *     last call's contents (a call rewrites all it reads, so nothing needs
 *     clearing).  Calls whose stream work overlaps on one device -- different
 *     streams, or host threads without ordering -- race on the array and give
 *     undefined results; order them on one stream. */
int sink_attn_fwd_noalloc(const sink_attn_desc* desc, const void* q, const void* k,
                          const void* v, const int32_t* cu_seqlens, const float* sinks,
                          const float* qnorm_w, const float* knorm_w, int32_t window,
                          int32_t use_rope, void* out, float* lse, void* stream);

/* Static text for a status code (never NULL).  Errors are returned, never
 * worked around ("flint.layers" _validate_backend rejects an unsupported
 * backend; "attention.utils" raises when a layout cannot be consumed). */
const char* sink_attn_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch (not on the pages). */
int sink_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_H */
