// sa_internal.h -- types, constants and launch wrappers shared by the HIP
// translation units of libsinkattn.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
// The 16-bit paths are templates over the storage/operand element E: bf16
// (__bf16) or fp16 (_Float16).  Both feed the same MFMA shape
// (v_mfma_f32_32x32x16_{bf16,f16}) with fp32 accumulation.
template <typename E> using vec8 = E __attribute__((ext_vector_type(8)));
template <typename E> using vec4 = E __attribute__((ext_vector_type(4)));
template <typename E> using vec2 = E __attribute__((ext_vector_type(2)));
template <typename E> constexpr bool is_f16 = __is_same(E, _Float16);
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;     // head_dim of the bf16 MFMA path
constexpr int kKeyTile = 64;      // keys per LDS tile; tiles start at multiples of 64
constexpr int kWaves = 4;         // waves per attention workgroup
constexpr int kColsPerWave = 32;  // narrow tiles: (token, head) query columns per wave
constexpr int kColsPerWaveWide = 64;  // wide tiles: columns per wave
constexpr int kMaxGroup = 32;     // largest Hq / Hkv of the bf16 path
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// bf16 attention tile configurations (sink_attn_desc.tile_config).
constexpr int kTileAuto = 0;
constexpr int kTileNarrow = 1;  // 32 columns per wave, two workgroups per CU
constexpr int kTileWide = 2;    // 64 columns per wave, one workgroup per CU
constexpr int kTileWideExact = 3;  // wide, every block through the exact-max pass

// Query tokens one attention workgroup covers for a GQA group size G:
// kWaves * columns per wave = tokens * G.
inline int tokens_per_block(int G) { return kWaves * kColsPerWave / G; }
inline int tokens_per_block_wide(int G) { return kWaves * kColsPerWaveWide / G; }

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Workspace carve-up (all offsets 256-byte aligned).
struct Workspace {
  int64_t t_pad = 0;         // keys padded to a multiple of kKeyTile
  int64_t items_ub = 0;      // upper bound on (document, query block) items, narrow tiles
  int64_t items_ub_wide = 0; // the same for wide tiles
  size_t khat_off = 0;       // bf16: k_hat tile images [Hkv][t_pad/64][64][128]; f32: [T][Hkv][d]
  size_t vt_off = 0;         // bf16: V^T tile images [Hkv][t_pad/64][128][64]; f32: V copy [T][Hkv][d]
  size_t sched_off = 0;      // narrow schedule: int32 n_items, int2 items[items_ub], prefix
  size_t sched_wide_off = 0; // wide schedule, same format
  size_t redo_off = 0;       // int32 per wide workgroup: rerun with the exact row max
  size_t ends_off = 0;       // int32 [D]: real end of every document (padded THD)
  size_t total = 0;
};

// Schedule table size in int32 for items_ub items and D documents.
inline int64_t sched_ints(int64_t items_ub, int64_t D) { return 4 + 2 * items_ub + D + 1; }

// Wide-tile grid size (also the redo table size) for items_ub items.
inline int64_t wide_grid(int64_t items_ub, int Hkv) {
  return (Hkv <= 8 && 8 % Hkv == 0) ? 8 * ((items_ub + 8 / Hkv - 1) / (8 / Hkv))
                                    : items_ub * Hkv;
}

Workspace plan_workspace(int64_t T, int64_t D, int Hq, int Hkv, int d, int dtype);

// Backward workspace (bf16): per kv head, 48 KiB key-tile images (64 keys:
// k_hat rows, V rows, K^T) and 36 KiB column-tile images (32 query columns:
// scaled q_hat rows, dout rows, their transposes, -lse and -D), then fp32
// partial sums of dsink (per column tile and head) and of the two norm-weight
// gradients (per dK/dV and dQ workgroup).
struct BwdWorkspace {
  int64_t n_kt = 0;    // 64-key tiles per kv head
  int64_t n_ct = 0;    // 32-column tiles per kv head (32 / G tokens each)
  int64_t n_kblk = 0;  // dK/dV workgroups (128 keys x kv head)
  int64_t n_qblk = 0;  // dQ partial-sum rows: 4-wave workgroups (128 columns x kv head)
  size_t keys_off = 0, cols_off = 0, dsink_off = 0, dwq_off = 0, dwk_off = 0;
  size_t ends_off = 0;  // int32 [D]: real end of every document (padded THD)
  size_t total = 0;
};

BwdWorkspace plan_bwd_workspace(int64_t T, int64_t D, int Hq, int Hkv);

// Padded THD support (sink_attn_api.hip): real document ends from
// cu_seqlens (real lengths) and cu_seqlens_padded (starts), and the output rows
// of padding tokens (out = 0, lse = the sink).
hipError_t launch_doc_ends(const int32_t* cu, const int32_t* cu_padded, int D, int32_t* ends,
                           hipStream_t stream);
hipError_t launch_pad_fill(const int32_t* starts, const int32_t* ends, int D, int T, int Hq,
                           int d, int dtype, const float* sinks, void* out, float* lse,
                           hipStream_t stream);

// ---- launch wrappers (return hipGetLastError after the launches) ----------

// The 16-bit launch wrappers are instantiated for E = bf16 and E = f16.
template <typename E>
hipError_t launch_prologue_16(const E* k, const E* v, const int32_t* cu,
                                const int32_t* cu_end, const float* knorm_w, int T, int D, int Hkv,
                                int64_t t_pad, int m_tok, int m_tok_wide, double eps,
                                double theta, int use_rope, E* khat, E* vt,
                                int32_t* sched, int32_t* sched_wide, hipStream_t stream);

template <typename E>
hipError_t launch_attention_narrow(const E* q, const E* khat, const E* vt,
                                 const int32_t* cu, const int32_t* cu_end, const int32_t* sched,
                                 const float* sinks, const float* qnorm_w, E* out,
                                 float* lse, int T, int D, int Hq, int Hkv,
                                 int64_t t_pad, int64_t items_ub, int window,
                                 int use_rope, double eps, double theta,
                                 double scale, hipStream_t stream);

template <typename E>
hipError_t launch_attention_wide(const E* q, const E* khat, const E* vt,
                                      const int32_t* cu, const int32_t* cu_end,
                                      const int32_t* sched,
                                      const float* sinks, const float* qnorm_w, E* out,
                                      float* lse, int32_t* redo, int T, int D, int Hq,
                                      int Hkv, int64_t t_pad, int64_t items_ub, int window,
                                      int use_rope, double eps, double theta, double scale,
                                      bool exact_all, hipStream_t stream);

template <typename E>
hipError_t launch_bwd(const E* q, const E* k, const E* v, const int32_t* cu,
                           const int32_t* cu_end, const float* sinks, const float* qnorm_w, const float* knorm_w,
                           const E* out, const float* lse, const E* dout, E* dq,
                           E* dk, E* dv, float* dsinks, float* dqnorm_w,
                           float* dknorm_w, int T, int D, int Hq, int Hkv, int window,
                           int use_rope, double eps, double theta, double scale, char* ws,
                           const BwdWorkspace& w, int dq_waves, hipStream_t stream);

hipError_t launch_prologue_f32(const float* k, const float* v, const int32_t* cu,
                               const int32_t* cu_end, const float* knorm_w, int T, int D, int Hkv, int d,
                               double eps, double theta, int use_rope, float* khat,
                               float* vcopy, hipStream_t stream);

hipError_t launch_attention_f32(const float* q, const float* khat, const float* v,
                                const int32_t* cu, const int32_t* cu_end, const float* sinks,
                                const float* qnorm_w, float* out, float* lse, int T,
                                int D, int Hq, int Hkv, int d, int window, int use_rope,
                                double eps, double theta, double scale,
                                hipStream_t stream);

}  // namespace sa
