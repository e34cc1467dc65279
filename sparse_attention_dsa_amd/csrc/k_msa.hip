// Block-sparse MSA: block selection from token scores, and GQA over the picked blocks (page
// "Sparse attention (DSA and block-sparse MSA)", table "Two shapes, three checkpoints": the top
// 16 blocks of 128 tokens, over plain GQA). The token scores come from the DSA score kernels.
//
// msa_block_topk: one workgroup per row. Each group of BLOCK/4 lanes takes one block, four
// scores a lane, and reduces their order keys to the group's last lane on the DPP network; a
// block's key is (order key of its best visible score) << 32 | ~block, unique per block, larger
// for a better score and, among equal scores, for the lower block. Each block's rank is then the
// number of larger keys, counted against every block of the row in LDS, and the blocks ranked
// below topk are written at their rank.
//
// msa_attend: one workgroup per (row, query head): the row's picked positions, their logits
// against the head's KV head in fp32, an exact max and sum, then the V-weighted sum with the
// threads spread over output columns.
#include "dsa_internal.hpp"

namespace {

constexpr int kThreads = 256;

// Largest value over each group of G consecutive lanes (G = 8, 16, 32 or 64), left in the
// group's last lane: shifts within 16-lane rows, then the broadcasts across rows.
template <int G>
__device__ __forceinline__ uint32_t group_max_last(uint32_t x) {
  x = max(x, dsa::dpp_zero_fill<0x111, 0xF>(x));
  x = max(x, dsa::dpp_zero_fill<0x112, 0xF>(x));
  x = max(x, dsa::dpp_zero_fill<0x114, 0xF>(x));
  if constexpr (G >= 16) x = max(x, dsa::dpp_zero_fill<0x118, 0xF>(x));
  if constexpr (G >= 32) x = max(x, dsa::dpp_zero_fill<0x142, 0xA>(x));
  if constexpr (G >= 64) x = max(x, dsa::dpp_zero_fill<0x143, 0xC>(x));
  return x;
}

template <int BLOCK>
__global__ void __launch_bounds__(kThreads)
msa_block_topk(DevPlan p, const float* __restrict__ scores, int64_t ld, int topk,
               int32_t* __restrict__ sel) {
  extern __shared__ uint64_t comp[];        // composite key of each block of the row
  constexpr int kLanes = BLOCK / 4;         // lanes per block, four scores each
  constexpr int kPerPass = kThreads / kLanes;
  constexpr int kOwn = 4;                   // blocks a thread ranks per pass
  const int t = blockIdx.x;
  dsa_span sp;
  dsa::row_span(p.spans, p.n_spans, t, &sp);
  const int pos = sp.ctx_start + (t - sp.q_start);
  const int nb = pos / BLOCK + 1;
  const float* row = scores + int64_t(t) * ld;
  const int gl = threadIdx.x % kLanes;

  for (int b0 = 0; b0 < nb; b0 += kPerPass) {
    const int b = b0 + int(threadIdx.x) / kLanes;
    uint32_t k = 0u;
    if (b < nb) {
      const int j = b * BLOCK + 4 * gl;
#pragma unroll
      for (int e = 0; e < 4; ++e) k = max(k, dsa::order_key(row[min(j + e, pos)]));   // past the row: its last score again
    }
    k = group_max_last<kLanes>(k);
    if (b < nb && gl == kLanes - 1) comp[b] = (uint64_t(k) << 32) | uint64_t(~uint32_t(b));
  }
  __syncthreads();
  int32_t* out = sel + int64_t(t) * topk;
  for (int b0 = 0; b0 < nb; b0 += kThreads * kOwn) {
    uint64_t c[kOwn];
    int rank[kOwn];
#pragma unroll
    for (int i = 0; i < kOwn; ++i) {
      const int b = b0 + threadIdx.x + kThreads * i;
      c[i] = b < nb ? comp[b] : ~uint64_t(0);
      rank[i] = 0;
    }
    for (int o = 0; o < nb; ++o) {          // every thread reads the same entry: one broadcast
      const uint64_t x = comp[o];
#pragma unroll
      for (int i = 0; i < kOwn; ++i) rank[i] += x > c[i] ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < kOwn; ++i) {
      const int b = b0 + threadIdx.x + kThreads * i;
      if (b < nb && rank[i] < topk) out[rank[i]] = b;
    }
  }
  for (int i = nb + threadIdx.x; i < topk; i += kThreads) out[i] = -1;
}

template <int QFMT>
__device__ __forceinline__ float elem(const void* base, int64_t i) {
  if constexpr (QFMT == DSA_FMT_F32) return static_cast<const float*>(base)[i];
  else return dsa::bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <int QFMT>
__global__ void __launch_bounds__(kThreads)
msa_attend(DevPlan p, const int32_t* __restrict__ sel, const void* __restrict__ q,
           const uint8_t* __restrict__ pool, float sm_scale, void* __restrict__ out, int topk,
           int block, int H, int n_kv, int d, int64_t row_bytes) {
  extern __shared__ float smem[];
  const int n_slots = topk * block;
  float* qv = smem;                               // [d] this head's query
  float* logit = qv + d;                          // [n_slots] logits, then weights
  int* tok = reinterpret_cast<int*>(logit + n_slots);   // [n_slots] pool token, -1 none
  float* part = reinterpret_cast<float*>(tok + n_slots); // [kThreads] partial output sums
  __shared__ float red[kThreads / 64];
  constexpr int E = QFMT == DSA_FMT_F32 ? 4 : 2;

  const int t = blockIdx.x, h = blockIdx.y;
  const int kh = h / (H / n_kv);
  dsa_span sp;
  dsa::row_span(p.spans, p.n_spans, t, &sp);
  const int pos = sp.ctx_start + (t - sp.q_start);
  for (int e = threadIdx.x; e < d; e += kThreads) qv[e] = elem<QFMT>(q, (int64_t(t) * H + h) * d + e);
  for (int i = threadIdx.x; i < n_slots; i += kThreads) {
    const int b = sel[int64_t(t) * topk + i / block];
    const int j = b * block + i % block;
    int tk = -1;
    if (b >= 0 && j <= pos) {
      int off;
      const int pg = dsa::page_of(p, sp, j, &off);
      tk = pg * p.page_size + off;
    }
    tok[i] = tk;
  }
  __syncthreads();

  // logits of this head's KV head: K of KV head kh starts kh*d elements into the row
  float mx = -__builtin_inff();
  for (int i = threadIdx.x; i < n_slots; i += kThreads) {
    float l = -__builtin_inff();
    if (tok[i] >= 0) {
      // 16-byte pieces (d is a multiple of 8 and every row offset a multiple of 16 bytes)
      const uint4* k4 = reinterpret_cast<const uint4*>(pool + int64_t(tok[i]) * row_bytes + int64_t(kh) * d * E);
      float acc = 0.0f;
      for (int c = 0; c < d * E / 16; ++c) {
        const uint4 v = k4[c];
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        if constexpr (QFMT == DSA_FMT_F32) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = fmaf(qv[4 * c + r], __uint_as_float(wv[r]), acc);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc = fmaf(qv[8 * c + 2 * r], __uint_as_float(wv[r] << 16), acc);
            acc = fmaf(qv[8 * c + 2 * r + 1], __uint_as_float(wv[r] & 0xFFFF0000u), acc);
          }
        }
      }
      l = acc * sm_scale;
    }
    logit[i] = l;
    mx = fmaxf(mx, l);
  }
  mx = block_reduce(mx, red, true);
  float sum = 0.0f;
  for (int i = threadIdx.x; i < n_slots; i += kThreads) {
    const float e = tok[i] >= 0 ? __expf(logit[i] - mx) : 0.0f;
    logit[i] = e;
    sum += e;
  }
  sum = block_reduce(sum, red, false);            // also orders the weight writes before the reads
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;

  // V of KV head kh: (n_kv + kh) * d elements into the row. Threads take one output column
  // and one share of the picked positions; the shares are added through LDS.
  const int nparts = kThreads / d;
  const int col = threadIdx.x % d, share = threadIdx.x / d;
  float acc = 0.0f;
  if (share < nparts) {
    for (int i = share; i < n_slots; i += nparts) {
      const int tk = tok[i];
      if (tk >= 0) {
        const uint8_t* vrow = pool + int64_t(tk) * row_bytes + int64_t(n_kv + kh) * d * E;
        acc = fmaf(logit[i], elem<QFMT>(vrow, col), acc);
      }
    }
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < d) {
    float o = 0.0f;
    for (int s = 0; s < nparts; ++s) o += part[s * d + threadIdx.x];
    o *= inv;
    const int64_t oi = (int64_t(t) * H + h) * d + threadIdx.x;
    if constexpr (QFMT == DSA_FMT_F32) static_cast<float*>(out)[oi] = o;
    else static_cast<uint16_t*>(out)[oi] = dsa::f32_to_bf16(o);
  }
}

}  // namespace

size_t msa_select_lds_bytes(const dsa_msa_config& c, const PlanInfo& in) {
  return size_t(in.max_visible / c.block_size + 1) * 8;
}

size_t msa_attend_lds_bytes(const dsa_msa_config& c) {
  return size_t(c.head_dim + 2 * c.topk_blocks * c.block_size + kThreads) * 4;
}

hipError_t launch_msa_block_topk(const dsa_msa_handle* h, const DevPlan& p, const PlanInfo& in,
                                 const float* scores, int64_t ld, int32_t* sel, hipStream_t st) {
  const dsa_msa_config& c = h->cfg;
  const size_t lds = msa_select_lds_bytes(c, in);
  const dim3 grid(unsigned(in.n_rows));
#define DSA_MSA_TOPK(B) \
  case B: hipLaunchKernelGGL(msa_block_topk<B>, grid, dim3(kThreads), lds, st, p, scores, ld, c.topk_blocks, sel); break;
  switch (c.block_size) {
    DSA_MSA_TOPK(32)
    DSA_MSA_TOPK(64)
    DSA_MSA_TOPK(128)
    DSA_MSA_TOPK(256)
    default: return hipErrorInvalidValue;
  }
#undef DSA_MSA_TOPK
  return hipGetLastError();
}

hipError_t launch_msa_attend(const dsa_msa_handle* h, const DevPlan& p, const PlanInfo& in,
                             const int32_t* sel, const void* q, const void* pool, float sm_scale,
                             void* out, hipStream_t st) {
  const dsa_msa_config& c = h->cfg;
  const size_t lds = msa_attend_lds_bytes(c);
  const dim3 grid(unsigned(in.n_rows), unsigned(c.n_heads));
  if (c.q_fmt == DSA_FMT_F32)
    hipLaunchKernelGGL(msa_attend<DSA_FMT_F32>, grid, dim3(kThreads), lds, st, p, sel, q,
                       static_cast<const uint8_t*>(pool), sm_scale, out, c.topk_blocks, c.block_size,
                       c.n_heads, c.n_kv_heads, c.head_dim, h->gqa_row_bytes);
  else
    hipLaunchKernelGGL(msa_attend<DSA_FMT_BF16>, grid, dim3(kThreads), lds, st, p, sel, q,
                       static_cast<const uint8_t*>(pool), sm_scale, out, c.topk_blocks, c.block_size,
                       c.n_heads, c.n_kv_heads, c.head_dim, h->gqa_row_bytes);
  return hipGetLastError();
}
