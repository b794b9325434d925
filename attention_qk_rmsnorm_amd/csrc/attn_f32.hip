// attn_f32.hip -- fp32 debug path of the sink-aware GQA attention forward.
//
// Same computation as the bf16 path (flint.layers FlintAttention.forward with
// the _FlintSinkParameters sink category), with fp32 inputs, arithmetic and
// outputs and no bf16 rounding anywhere: one thread per (token, query head)
// normalises and rotates its query, then walks its visible keys in order with
// an online softmax seeded by the sink.  Correctness reference for the fp32
// tolerance, not a fast path.
#include "sa_device.h"

namespace sa {

namespace {

constexpr int kThreads = 128;

template <int HD>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ khat,
    const float* __restrict__ v, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_end, const float* __restrict__ sinks, const float* __restrict__ qnorm_w,
    float* __restrict__ out, float* __restrict__ lse, int T, int D, int Hq, int Hkv,
    int window, int use_rope, float eps, double theta, float scale) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)T * Hq) return;
  const int t = (int)(idx / Hq);
  const int h = (int)(idx - (int64_t)t * Hq);
  const int g = h / (Hq / Hkv);
  const int doc = doc_of_token(cu, D, t);
  const int doc_start = cu[doc];

  // RMSNorm (+ NeoX RoPE) of the query row
  float x[HD];
  float ss = 0.f;
  const float* qp = q + idx * HD;
#pragma unroll
  for (int i = 0; i < HD; ++i) {
    x[i] = qp[i];
    ss += x[i] * x[i];
  }
  const float inv = 1.0f / sqrtf(ss * (1.0f / HD) + eps);
#pragma unroll
  for (int i = 0; i < HD; ++i) x[i] *= inv * qnorm_w[i];
  if (use_rope) {
    const int p = t - doc_start;
    for (int i = 0; i < HD / 2; ++i) {
      float sn, cs;
      rope_sincos(p, pow(theta, -2.0 * i / HD), &sn, &cs);
      const float a = x[i], b = x[i + HD / 2];
      x[i] = a * cs - b * sn;
      x[i + HD / 2] = b * cs + a * sn;
    }
  }

  // online softmax over visible keys, natural-log domain, sink as the seed
  float m = sinks[h];
  float l = 1.f;
  float acc[HD];
#pragma unroll
  for (int i = 0; i < HD; ++i) acc[i] = 0.f;
  const int lo = window > 0 ? max(doc_start, t - window + 1) : doc_start;
  // a document-padding row sees no key: only the sink (out = 0, lse = sink)
  const int hi = t < cu_end[doc] ? t : lo - 1;
  for (int u = lo; u <= hi; ++u) {
    const float* kp = khat + ((int64_t)u * Hkv + g) * HD;
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < HD; ++i) dot += x[i] * kp[i];
    const float s = dot * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float p = expf(s - m_new);
    l = l * alpha + p;
    const float* vp = v + ((int64_t)u * Hkv + g) * HD;
#pragma unroll
    for (int i = 0; i < HD; ++i) acc[i] = acc[i] * alpha + p * vp[i];
    m = m_new;
  }
  float* op = out + idx * HD;
  const float inv_l = 1.0f / l;
#pragma unroll
  for (int i = 0; i < HD; ++i) op[i] = acc[i] * inv_l;
  if (lse != nullptr) lse[(int64_t)h * T + t] = m + logf(l);
}

}  // namespace

hipError_t launch_attention_f32(const float* q, const float* khat, const float* v,
                                const int32_t* cu, const int32_t* cu_end, const float* sinks,
                                const float* qnorm_w, float* out, float* lse, int T,
                                int D, int Hq, int Hkv, int d, int window, int use_rope,
                                double eps, double theta, double scale,
                                hipStream_t stream) {
  const int64_t n = (int64_t)T * Hq;
  const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
  if (d == 128)
    attn_fwd_f32_kernel<128><<<grid, kThreads, 0, stream>>>(
        q, khat, v, cu, cu_end, sinks, qnorm_w, out, lse, T, D, Hq, Hkv, window, use_rope,
        (float)eps, theta, (float)scale);
  else
    attn_fwd_f32_kernel<64><<<grid, kThreads, 0, stream>>>(
        q, khat, v, cu, cu_end, sinks, qnorm_w, out, lse, T, D, Hq, Hkv, window, use_rope,
        (float)eps, theta, (float)scale);
  return hipGetLastError();
}

}  // namespace sa
