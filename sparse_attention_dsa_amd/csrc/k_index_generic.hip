// Indexer score, any shape and format (the path for shapes without a matrix-core kernel):
//   s[t][j] = sum_h w[t][h] * relu(q[t][h] . k_j),  j = 0 .. position(t)
// (DSA resource page: module description and index_topk). One thread per (row, key); the row's
// queries and weights sit in LDS as fp32; dots accumulate in fp32 over d, 16 heads at a time.
// An fp8 key is e4m3(code) * scale: the scale multiplies the finished dot.
#include "dsa_internal.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kHeadGroup = 16;

template <int KFMT>
__device__ __forceinline__ void load8(const uint8_t* src, float* v) {
  if constexpr (KFMT == DSA_FMT_F32) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
    float4 a = s4[0], b = s4[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else if constexpr (KFMT == DSA_FMT_BF16) {
    uint4 u = *reinterpret_cast<const uint4*>(src);
    uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w4[i] << 16);
      v[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
    }
  } else {
    uint2 u = *reinterpret_cast<const uint2*>(src);
    uint32_t w2[2] = {u.x, u.y};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b) v[4 * i + b] = dsa::fp8_to_f32((w2[i] >> (8 * b)) & 0xFF);
  }
}

template <int QFMT, int KFMT>
__global__ void __launch_bounds__(kThreads)
index_scores_generic(DevPlan p, const void* __restrict__ qv, const float* __restrict__ w,
                     const uint8_t* __restrict__ pool, float* __restrict__ scores, int64_t ld,
                     int H, int D, int64_t page_bytes, int fill_masked) {
  extern __shared__ float smem[];
  float* qs = smem;             // [H][D]
  float* ws = smem + H * D;     // [H]
  const int t = blockIdx.y;
  dsa_span sp;
  dsa::row_span(p.spans, p.n_spans, t, &sp);
  const int pos = sp.ctx_start + (t - sp.q_start);
  const int j0 = blockIdx.x * kThreads;
  float* out = scores + int64_t(t) * ld;
  if (j0 > pos) {
    if (fill_masked)
      for (int j = j0 + threadIdx.x; j < ld && j < j0 + kThreads; j += kThreads) out[j] = -__builtin_inff();
    return;
  }
  for (int i = threadIdx.x; i < H * D; i += kThreads) {
    if constexpr (QFMT == DSA_FMT_F32)
      qs[i] = static_cast<const float*>(qv)[int64_t(t) * H * D + i];
    else
      qs[i] = dsa::bf16_to_f32(static_cast<const uint16_t*>(qv)[int64_t(t) * H * D + i]);
  }
  for (int i = threadIdx.x; i < H; i += kThreads) ws[i] = w[int64_t(t) * H + i];
  __syncthreads();

  const int j = j0 + threadIdx.x;
  if (j >= ld) return;
  if (j > pos) {
    if (fill_masked) out[j] = -__builtin_inff();
    return;
  }
  int off;
  const int page = dsa::page_of(p, sp, j, &off);
  const uint8_t* pg = pool + int64_t(page) * page_bytes;
  constexpr int esize = KFMT == DSA_FMT_F32 ? 4 : KFMT == DSA_FMT_BF16 ? 2 : 1;
  const uint8_t* key = pg + int64_t(off) * D * esize;
  float scale = 1.0f;
  if constexpr (KFMT == DSA_FMT_FP8)
    scale = reinterpret_cast<const float*>(pg + int64_t(p.page_size) * D)[off];

  float total = 0.0f;
  for (int h0 = 0; h0 < H; h0 += kHeadGroup) {
    float acc[kHeadGroup];
#pragma unroll
    for (int i = 0; i < kHeadGroup; ++i) acc[i] = 0.0f;
    for (int d = 0; d < D; d += 8) {
      float kv[8];
      load8<KFMT>(key + d * esize, kv);
#pragma unroll
      for (int hh = 0; hh < kHeadGroup; ++hh) {
        if (h0 + hh < H) {
          const float* qh = qs + (h0 + hh) * D + d;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[hh] = fmaf(qh[i], kv[i], acc[hh]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < kHeadGroup; ++hh)
      if (h0 + hh < H) total = fmaf(ws[h0 + hh], fmaxf(acc[hh] * scale, 0.0f), total);
  }
  out[j] = total;
}

template <int QFMT, int KFMT>
hipError_t launch_generic(const dsa_handle* h, const DevPlan& p, const PlanInfo& in, const void* q,
                          const float* w, const void* pool, float* scores, int64_t ld, bool fill,
                          hipStream_t st) {
  const dsa_config& c = h->cfg;
  const int64_t cols = fill ? ld : in.max_visible;
  dim3 grid(unsigned((cols + kThreads - 1) / kThreads), unsigned(in.n_rows));
  size_t lds = size_t(c.n_index_heads) * (c.index_dim + 1) * sizeof(float);
  hipLaunchKernelGGL((index_scores_generic<QFMT, KFMT>), grid, dim3(kThreads), lds, st, p, q, w,
                     static_cast<const uint8_t*>(pool), scores, ld, c.n_index_heads, c.index_dim,
                     h->index_page_bytes, fill ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores_generic(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                       const void* q, const float* w, const void* pool,
                                       float* scores, int64_t ld, bool fill, hipStream_t st) {
  const int qf = h->cfg.index_q_fmt, kf = h->cfg.index_key_fmt;
#define DSA_CASE(Q, K) \
  if (qf == Q && kf == K) return launch_generic<Q, K>(h, p, in, q, w, pool, scores, ld, fill, st);
  DSA_CASE(DSA_FMT_F32, DSA_FMT_F32)
  DSA_CASE(DSA_FMT_F32, DSA_FMT_BF16)
  DSA_CASE(DSA_FMT_F32, DSA_FMT_FP8)
  DSA_CASE(DSA_FMT_BF16, DSA_FMT_F32)
  DSA_CASE(DSA_FMT_BF16, DSA_FMT_BF16)
  DSA_CASE(DSA_FMT_BF16, DSA_FMT_FP8)
#undef DSA_CASE
  return hipErrorInvalidValue;
}
