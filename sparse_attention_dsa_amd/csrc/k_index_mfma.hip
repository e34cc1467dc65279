// Indexer score on the matrix cores, 64 heads x 128 dims, bf16 queries, bf16 or fp8 keys:
//   s[t][j] = sum_h w[t][h] * relu(q[t][h] . k_j),  j = 0 .. position(t)
// (DSA resource page: module description, index_topk.)
//
// One workgroup (4 waves) scores KPB consecutive keys of one row. Per 16-key tile a wave runs
// 16 v_mfma_f32_16x16x32_bf16: heads are M (4 tiles of 16), keys are N, dims are K (4 steps of
// 32). The row's queries stay in VGPRs as the A operand for the whole block. Keys stream from
// HBM straight into B-operand registers: lane l owns key l%16 and the 32 consecutive dims
// 32*(l/16) .. +32 (64 bytes of bf16 or 32 bytes of fp8, converted to bf16 exactly in
// registers); the A operand uses the same dim order, so the contraction is unchanged. The
// epilogue (relu, head weight, sum over heads) runs on the accumulators: each lane sums its 16
// heads, two cross-lane adds finish the 64. An fp8 key is e4m3(code) * scale; the scale is >= 0
// and multiplies the finished sum (relu(c*x) = c*relu(x) for c >= 0).
// Each block also writes the min and max order key of its scores for the top-k select.
#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int H = 64, D = 128;
constexpr int kWaves = 4;
constexpr int KPB = kScoreBlock;                   // keys per block
constexpr int kTilesPerWave = KPB / (kWaves * 16);
constexpr int kQPitch = D + 8;                     // bf16 elements per q row in LDS (padded)

template <int KFMT>
struct Raw {
  // bf16: 64 bytes of one key (4 x 16 B); fp8: 32 bytes (2 x 16 B) and the key's scale
  u32x4 v[KFMT == DSA_FMT_BF16 ? 4 : 2];
  float scale;
};

template <int KFMT>
__device__ __forceinline__ void load_tile(Raw<KFMT>& r, const uint8_t* __restrict__ pool,
                                          const int* __restrict__ pages_lds, int first_list,
                                          int page_start, int log2_ps, int ps_mask, int64_t page_bytes,
                                          int j, int lane_grp) {
  const int slot = page_start + j;
  const int page = pages_lds[(slot >> log2_ps) - first_list];
  const int off = slot & ps_mask;
  const uint8_t* pg = pool + int64_t(page) * page_bytes;
  if constexpr (KFMT == DSA_FMT_BF16) {
    const u32x4* src = reinterpret_cast<const u32x4*>(pg + int64_t(off) * (D * 2) + lane_grp * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = __builtin_nontemporal_load(src + i);
    r.scale = 1.0f;
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(pg + int64_t(off) * D + lane_grp * 32);
    r.v[0] = __builtin_nontemporal_load(src);
    r.v[1] = __builtin_nontemporal_load(src + 1);
    r.scale = reinterpret_cast<const float*>(pg + ((int64_t(ps_mask) + 1) * D))[off];
  }
}

// B fragment for k-step ks (dims 32*grp + 8*ks .. +8 of the lane's key).
template <int KFMT>
__device__ __forceinline__ bf16x8 b_frag(const Raw<KFMT>& r, int ks) {
  if constexpr (KFMT == DSA_FMT_BF16) {
    return __builtin_bit_cast(bf16x8, r.v[ks]);
  } else {
    const uint32_t lo = r.v[ks >> 1][(ks & 1) * 2], hi = r.v[ks >> 1][(ks & 1) * 2 + 1];
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <int KFMT>
__global__ void __launch_bounds__(kWaves * 64)
index_scores_mfma(DevPlan p, const uint16_t* __restrict__ q, const float* __restrict__ w,
                  const uint8_t* __restrict__ pool, float* __restrict__ scores, int64_t ld,
                  int64_t page_bytes, int log2_ps, uint32_t* __restrict__ blk_minmax, int nb_max,
                  int fill_masked) {
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[H * kQPitch];
  __shared__ int pages_lds[KPB + 2];
  __shared__ uint32_t red[2 * kWaves];

  const int t = blockIdx.y;
  const int s = dsa::find_span(p.spans, p.n_spans, t);
  const dsa_span sp = p.spans[s];
  const int pos = sp.ctx_start + (t - sp.q_start);
  const int n = pos + 1;
  const int kb = blockIdx.x * KPB;
  float* out = scores + int64_t(t) * ld;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  if (kb >= n) {
    if (fill_masked)
      for (int j = kb + threadIdx.x; j < ld && j < kb + KPB; j += kWaves * 64) out[j] = -__builtin_inff();
    return;
  }
  const int ps_mask = (1 << log2_ps) - 1;
  const int kend = min(n, kb + KPB);
  const int first_list = (sp.page_start + kb) >> log2_ps;
  const int last_list = (sp.page_start + kend - 1) >> log2_ps;

  // stage the row's queries and this block's page ids
  {
    const u32x4* qs = reinterpret_cast<const u32x4*>(q + int64_t(t) * H * D);
    for (int i = threadIdx.x; i < H * D / 8; i += kWaves * 64) {
      const int h = i / (D / 8), c = i % (D / 8);
      *reinterpret_cast<u32x4*>(q_lds + h * kQPitch + c * 8) = qs[i];
    }
    for (int i = threadIdx.x; i <= last_list - first_list; i += kWaves * 64) {
      int pg = p.page_table[sp.page_offset + first_list + i];
      pages_lds[i] = pg < 0 ? 0 : (pg >= p.pool_pages ? p.pool_pages - 1 : pg);
    }
  }
  __syncthreads();

  const int grp = lane >> 4, col = lane & 15;
  // A operand: head 16*mt + col, dims 32*grp + 8*ks .. +8
  bf16x8 a[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      a[mt][ks] = *reinterpret_cast<const bf16x8*>(q_lds + (16 * mt + col) * kQPitch + 32 * grp + 8 * ks);
  // head weights of the accumulator rows this lane holds: head 16*mt + 4*grp + v
  float wr[16];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) wr[mt * 4 + v] = w[int64_t(t) * H + 16 * mt + 4 * grp + v];

  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  auto tile_key = [&](int it) { return kb + (it * kWaves + wave) * 16 + col; };

  auto compute = [&](const Raw<KFMT>& r, int it) {
    const int j = tile_key(it);
    f32x4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b = b_frag<KFMT>(r, ks);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][ks], b, acc[mt], 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) part = fmaf(wr[mt * 4 + v], fmaxf(acc[mt][v], 0.0f), part);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    part *= r.scale;
    if (j < kend) {
      if (grp == 0) out[j] = part;
      const uint32_t k = dsa::order_key(part);
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
  };

  auto load = [&](Raw<KFMT>& r, int it) {
    const int j = min(tile_key(it), kend - 1);   // keys past the row load a valid key, unused
    load_tile<KFMT>(r, pool, pages_lds, first_list, sp.page_start, log2_ps, ps_mask, page_bytes, j, grp);
  };

  // tiles of this wave that hold at least one key of the row; a ring of kDepth tiles in flight
  const int n_tiles = min(kWaves * kTilesPerWave, (kend - kb + 15) / 16);
  const int n_it = (n_tiles - wave + kWaves - 1) / kWaves;    // this wave's tiles: it*kWaves + wave
  constexpr int kDepth = KFMT == DSA_FMT_FP8 ? 8 : 6;
  Raw<KFMT> ring[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (d < n_it) load(ring[d], d);
  for (int it = 0; it < n_it; it += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (it + d < n_it) {
        compute(ring[d], it + d);
        if (it + d + kDepth < n_it) load(ring[d], it + d + kDepth);
      }
    }
  }
  if (fill_masked)
    for (int j = kend + threadIdx.x; j < kb + KPB && j < ld; j += kWaves * 64) out[j] = -__builtin_inff();

  // block min / max of the order keys
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, uint32_t(__shfl_xor(int(kmin), o)));
    kmax = max(kmax, uint32_t(__shfl_xor(int(kmax), o)));
  }
  if (lane == 0) { red[wave] = kmin; red[kWaves + wave] = kmax; }
  __syncthreads();
  if (threadIdx.x == 0 && blk_minmax) {
    uint32_t mn = red[0], mx = red[kWaves];
    for (int i = 1; i < kWaves; ++i) { mn = min(mn, red[i]); mx = max(mx, red[kWaves + i]); }
    blk_minmax[2 * (int64_t(t) * nb_max + blockIdx.x)] = mn;
    blk_minmax[2 * (int64_t(t) * nb_max + blockIdx.x) + 1] = mx;
  }
}

}  // namespace

int index_mfma_keys_per_block() { return KPB; }

bool index_mfma_supported(const dsa_config& c) {
  const bool pow2 = c.page_size > 0 && (c.page_size & (c.page_size - 1)) == 0;
  return c.n_index_heads == H && c.index_dim == D && c.index_q_fmt == DSA_FMT_BF16 &&
         (c.index_key_fmt == DSA_FMT_BF16 || c.index_key_fmt == DSA_FMT_FP8) && pow2;
}

hipError_t launch_index_scores_mfma(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                    const void* q, const float* w, const void* pool, float* scores,
                                    int64_t ld, bool fill, uint32_t* blk_minmax, int nb_max,
                                    hipStream_t st) {
  const dsa_config& c = h->cfg;
  int log2_ps = 0;
  while ((1 << log2_ps) < c.page_size) ++log2_ps;
  const int64_t cols = fill ? ld : in.max_visible;
  dim3 grid(unsigned((cols + KPB - 1) / KPB), unsigned(in.n_rows));
  if (c.index_key_fmt == DSA_FMT_BF16)
    hipLaunchKernelGGL(index_scores_mfma<DSA_FMT_BF16>, grid, dim3(kWaves * 64), 0, st, p,
                       static_cast<const uint16_t*>(q), w, static_cast<const uint8_t*>(pool), scores,
                       ld, h->index_page_bytes, log2_ps, blk_minmax, nb_max, fill ? 1 : 0);
  else
    hipLaunchKernelGGL(index_scores_mfma<DSA_FMT_FP8>, grid, dim3(kWaves * 64), 0, st, p,
                       static_cast<const uint16_t*>(q), w, static_cast<const uint8_t*>(pool), scores,
                       ld, h->index_page_bytes, log2_ps, blk_minmax, nb_max, fill ? 1 : 0);
  return hipGetLastError();
}
