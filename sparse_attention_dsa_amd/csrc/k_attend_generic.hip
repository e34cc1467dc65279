// Absorbed MLA over the picked latents, any shape and format (the path for shapes without a
// matrix-core kernel). DSA resource page, attend; ttnn.transformer.sparse_sdpa operation line:
//   logit_j = sm_scale * (q_nope[h] . c_j[0:R] + q_pe[h] . c_j[R:R+P]),
//   out[h]  = sum_j softmax(logit)_j * c_j[0:R]
// With an attention sink (ttnn.transformer.sparse_sdpa, attention_sink) the softmax denominator
// gains e^{sm_scale * sink[h]}. Queries and output are fp32, bf16 or plain e4m3 (the output in
// the queries' format).
// One workgroup per (row, head): logits of all picks (one pick per thread, a serial dot in fp32),
// an exact max / sum over the row, then one output column per thread.
#include "dsa_internal.hpp"

namespace {

constexpr int kThreads = 256;

// Element e of a latent row decoded to fp32 (e < R: latent part; R <= e < R+P: rope part).
template <int LFMT>
__device__ __forceinline__ float latent_elem(const uint8_t* row, int e, int R) {
  if constexpr (LFMT == DSA_FMT_F32) {
    return reinterpret_cast<const float*>(row)[e];
  } else if constexpr (LFMT == DSA_FMT_BF16) {
    return dsa::bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[e]);
  } else {
    if (e < R) {
      const float sc = reinterpret_cast<const float*>(row + R)[e >> 7];
      return dsa::fp8_to_f32(row[e]) * sc;
    }
    const uint16_t* rope = reinterpret_cast<const uint16_t*>(row + R + 4 * (R >> 7));
    return dsa::bf16_to_f32(rope[e - R]);
  }
}

template <int QFMT>
__device__ __forceinline__ float q_elem(const void* q, int64_t i) {
  if constexpr (QFMT == DSA_FMT_F32) return static_cast<const float*>(q)[i];
  else if constexpr (QFMT == DSA_FMT_BF16) return dsa::bf16_to_f32(static_cast<const uint16_t*>(q)[i]);
  else return dsa::fp8_to_f32(static_cast<const uint8_t*>(q)[i]);
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <int QFMT, int LFMT>
__global__ void __launch_bounds__(kThreads)
attend_generic(DevPlan p, const int32_t* __restrict__ sel, const void* __restrict__ q_nope,
               const void* __restrict__ q_pe, const uint8_t* __restrict__ pool, float sm_scale,
               const float* __restrict__ sink, void* __restrict__ out, int topk, int H, int R, int P,
               int64_t row_bytes) {
  extern __shared__ float smem[];
  float* qv = smem;                      // [R + P]
  float* logit = smem + R + P;           // [topk]
  int* rowoff = reinterpret_cast<int*>(logit + topk);  // [topk] token index in the pool, -1 none
  __shared__ float red[kThreads / 64];

  const int t = blockIdx.x, h = blockIdx.y;
  dsa_span sp;
  dsa::row_span(p.spans, p.n_spans, t, &sp);
  const int pos = sp.ctx_start + (t - sp.q_start);
  for (int e = threadIdx.x; e < R; e += kThreads) qv[e] = q_elem<QFMT>(q_nope, (int64_t(t) * H + h) * R + e);
  for (int e = threadIdx.x; e < P; e += kThreads) qv[R + e] = q_elem<QFMT>(q_pe, (int64_t(t) * H + h) * P + e);
  __syncthreads();

  float mx = -__builtin_inff();
  for (int i = threadIdx.x; i < topk; i += kThreads) {
    const int j = sel[int64_t(t) * topk + i];
    float l = -__builtin_inff();
    int tok = -1;
    if (j >= 0 && j <= pos) {
      int off;
      const int page = dsa::page_of(p, sp, j, &off);
      tok = page * p.page_size + off;
      const uint8_t* row = pool + int64_t(tok) * row_bytes;
      float acc = 0.0f;
      for (int e = 0; e < R + P; ++e) acc = fmaf(qv[e], latent_elem<LFMT>(row, e, R), acc);
      l = acc * sm_scale;
    }
    logit[i] = l;
    rowoff[i] = tok;
    mx = fmaxf(mx, l);
  }
  mx = block_reduce(mx, red, true);
  // the sink joins the max (for range) and the denominator, never the numerator
  const float sk = sink != nullptr && sink[h] != -__builtin_inff() ? sink[h] * sm_scale : -__builtin_inff();
  if (mx == -__builtin_inff()) mx = sk;           // nothing picked: every e below is 0
  else mx = fmaxf(mx, sk);
  float sum = 0.0f;
  for (int i = threadIdx.x; i < topk; i += kThreads) {
    const float e = rowoff[i] >= 0 ? __expf(logit[i] - mx) : 0.0f;
    logit[i] = e;
    sum += e;
  }
  sum = block_reduce(sum, red, false);  // also orders the logit[] writes before the reads below
  if (sk != -__builtin_inff()) sum += __expf(sk - mx);
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  for (int d = threadIdx.x; d < R; d += kThreads) {
    float acc = 0.0f;
    for (int i = 0; i < topk; ++i) {
      const int tok = rowoff[i];
      if (tok >= 0) acc = fmaf(logit[i], latent_elem<LFMT>(pool + int64_t(tok) * row_bytes, d, R), acc);
    }
    const float o = acc * inv;
    const int64_t oi = (int64_t(t) * H + h) * R + d;
    if constexpr (QFMT == DSA_FMT_F32) static_cast<float*>(out)[oi] = o;
    else if constexpr (QFMT == DSA_FMT_BF16) static_cast<uint16_t*>(out)[oi] = dsa::f32_to_bf16(o);
    else static_cast<uint8_t*>(out)[oi] = uint8_t(dsa::f32_to_e4m3(o));
  }
}

template <int QFMT, int LFMT>
hipError_t launch_attend_generic_t(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                   const int32_t* sel, const void* qn, const void* qp,
                                   const void* pool, float sm_scale, const float* sink, void* out,
                                   hipStream_t st) {
  const dsa_config& c = h->cfg;
  size_t lds = size_t(c.kv_lora_rank + c.rope_dim + 2 * c.topk) * 4;
  hipLaunchKernelGGL((attend_generic<QFMT, LFMT>), dim3(in.n_rows, c.n_heads), dim3(kThreads), lds,
                     st, p, sel, qn, qp, static_cast<const uint8_t*>(pool), sm_scale, sink, out, c.topk,
                     c.n_heads, c.kv_lora_rank, c.rope_dim, h->latent_row_bytes);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_generic(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                 const int32_t* sel, const void* qn, const void* qp,
                                 const void* pool, float sm_scale, const float* sink, void* out,
                                 hipStream_t st) {
  const int qf = h->cfg.q_fmt, lf = h->cfg.latent_fmt;
#define DSA_CASE(Q, L) \
  if (qf == Q && lf == L) \
    return launch_attend_generic_t<Q, L>(h, p, in, sel, qn, qp, pool, sm_scale, sink, out, st);
  DSA_CASE(DSA_FMT_F32, DSA_FMT_F32)
  DSA_CASE(DSA_FMT_F32, DSA_FMT_BF16)
  DSA_CASE(DSA_FMT_F32, DSA_FMT_FP8)
  DSA_CASE(DSA_FMT_BF16, DSA_FMT_F32)
  DSA_CASE(DSA_FMT_BF16, DSA_FMT_BF16)
  DSA_CASE(DSA_FMT_BF16, DSA_FMT_FP8)
  DSA_CASE(DSA_FMT_FP8, DSA_FMT_F32)
  DSA_CASE(DSA_FMT_FP8, DSA_FMT_BF16)
  DSA_CASE(DSA_FMT_FP8, DSA_FMT_FP8)
#undef DSA_CASE
  return hipErrorInvalidValue;
}
