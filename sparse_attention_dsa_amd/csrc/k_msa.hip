// Block-sparse MSA: block selection from token scores, and GQA over the picked blocks (page
// "Sparse attention (DSA and block-sparse MSA)", table "Two shapes, three checkpoints": the top
// 16 blocks of 128 tokens, over plain GQA). The token scores come from the DSA score kernels.
//
// Selection, two launches:
//   msa_block_keys: many workgroups per row, 4,096 scores each. Each group of BLOCK/4 lanes
//     takes one block (one float4 a lane) and reduces the order keys of its visible scores to
//     the group's last lane on the DPP network. A block's key is
//     (order key of its best visible score) << 32 | ~block: unique per block, larger for a better
//     score and, among equal scores, for the lower block.
//   msa_block_rank: each lane owns one block of a row and counts the row's larger keys, read
//     in LDS tiles and split over 16 waves; a block whose count is below topk is written at
//     that count.
// When every row is a decode row, the score kernel itself writes the best order key of each
// 32-key group, msa_block_keys is skipped, and msa_block_rank forms the block keys from those.
//
// Attention, two launches:
//   msa_attend_split: one workgroup per (row, KV head, group of up to 16 query heads, picked
//     block). The block's K and V rows go straight from the pool into LDS (global_load_lds, every
//     load in flight at once; chunks of tokens when a block does not fit), the group's logits
//     are formed in fp32 against the one K tile, and a per-head running max and sum weigh the V
//     rows. The partial output, max and sum go to the workspace.
//   msa_attend_mfma: the same grid and partials for bf16 caches of head_dim 64/128/256 and
//     blocks of up to 128 tokens, with Q.K^T and P.V on the matrix cores (P in bf16).
//   msa_combine: one workgroup per (row, query head) merges the picked blocks' partials.
// msa_block_keys, msa_block_rank (from keys) and msa_attend_mfma issue the loads that do not
// depend on the row's position before looking the row up in the plan, so that the lookup's
// memory round trip overlaps them.
#include "dsa_internal.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kKeyPasses = 4;            // float4 loads per thread in msa_block_keys
constexpr int kKeyScores = kKeyPasses * kThreads * 4;   // scores per msa_block_keys workgroup
constexpr int kRankTile = 2048;          // keys per LDS tile in msa_block_rank
constexpr int kRankWaves = 16;           // waves of an msa_block_rank workgroup
constexpr int kMaxGroup = 16;            // query heads per attention workgroup
constexpr int kMaxPieces = 16;           // 16-byte K/V pieces a thread stages per chunk
constexpr int kMaxUnits = 4;             // (head, piece) output units a thread accumulates

__device__ __forceinline__ int row_position(const DevPlan& p, int t, dsa_span* sp) {
  dsa::row_span(p.spans, p.n_spans, t, sp);
  return sp->ctx_start + (t - sp->q_start);
}

// grid (rows, ceil(blocks of the longest row / (kKeyScores / BLOCK)))
template <int BLOCK>
__global__ void __launch_bounds__(kThreads)
msa_block_keys(DevPlan p, const float* __restrict__ scores, int64_t ld, uint64_t* __restrict__ keys,
               int64_t kld) {
  constexpr int kLanes = BLOCK / 4;                  // lanes per block, one float4 each
  constexpr int kPerPass = kThreads / kLanes;        // blocks per pass of the workgroup
  const int t = blockIdx.x;
  const int b0 = int(blockIdx.y) * kPerPass * kKeyPasses;
  const float* row = scores + int64_t(t) * ld;
  const int gl = threadIdx.x % kLanes;
  // The loads go out before the row's position is known (one memory round trip fewer): a
  // float4 starting below ld lies inside the row (ld is a multiple of 4). Elements past the
  // row's own position are loaded but never used.
  float4 v[kKeyPasses];
#pragma unroll
  for (int i = 0; i < kKeyPasses; ++i) {
    const int j = (b0 + i * kPerPass + int(threadIdx.x) / kLanes) * BLOCK + 4 * gl;
    v[i] = j < ld ? *reinterpret_cast<const float4*>(row + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  dsa_span sp;
  const int pos = row_position(p, t, &sp);
  const int nb = pos / BLOCK + 1;
  if (b0 >= nb) return;
  uint64_t* out = keys + int64_t(t) * kld;
#pragma unroll
  for (int i = 0; i < kKeyPasses; ++i) {
    const int b = b0 + i * kPerPass + int(threadIdx.x) / kLanes;
    const int j = b * BLOCK + 4 * gl;
    uint32_t k = 0u;
    if (j <= pos) k = dsa::order_key(v[i].x);
    if (j + 1 <= pos) k = max(k, dsa::order_key(v[i].y));
    if (j + 2 <= pos) k = max(k, dsa::order_key(v[i].z));
    if (j + 3 <= pos) k = max(k, dsa::order_key(v[i].w));
    k = dsa::group_max_last<kLanes>(k);
    if (b < nb && gl == kLanes - 1) out[b] = (uint64_t(k) << 32) | uint64_t(~uint32_t(b));
  }
}

// grid (rows, ceil(blocks of the longest row / 64)). Lane i of every wave owns block
// 64 y + i; the 16 waves split the row's keys between them and add their counts in LDS.
// RUNS: the block keys are formed here from the score kernel's best order key of every 32-key
// group (runs, kld of them a row) instead of read from msa_block_keys' output (keys).
template <bool RUNS>
__global__ void __launch_bounds__(64 * kRankWaves)
msa_block_rank(DevPlan p, int block, const uint64_t* __restrict__ keys,
               const uint32_t* __restrict__ runs, int64_t kld, int topk, int32_t* __restrict__ sel) {
  constexpr int kN = 64 * kRankWaves;
  static_assert(kRankTile == 2 * kN, "the first tile is prefetched two keys a thread");
  __shared__ uint64_t tile[kRankTile];
  __shared__ int partial[kRankWaves][64];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = int(blockIdx.y) * 64 + lane;
  const uint64_t* rk = keys + int64_t(t) * kld;
  const uint32_t* rr = runs + int64_t(t) * kld;
  // keys: the own key and the first tile's keys go out before the row's block count is known
  // (reads below kld stay inside the row's keys; those past its blocks are not used)
  uint64_t own = 0, pre0 = 0, pre1 = 0;
  if constexpr (!RUNS) {
    own = b < kld ? rk[b] : 0;
    pre0 = int(threadIdx.x) < kld ? rk[threadIdx.x] : 0;
    pre1 = int(threadIdx.x) + kN < kld ? rk[threadIdx.x + kN] : 0;
  }
  dsa_span sp;
  const int pos = row_position(p, t, &sp);
  const int nb = pos / block + 1;
  // runs: block o's key from its 32-key groups that start at or before the row's position
  // (rows of the runs buffer are 32-byte aligned, so a block's 4 or 8 groups are whole vectors)
  auto key_of = [&](int o) -> uint64_t {
    const int r = block >> 5;
    const int lim = pos / 32 - o * r;          // groups 0 .. lim of the block are visible
    uint32_t k = 0u;
    if (r == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(rr + 4 * o);
      k = v.x;
      if (lim >= 1) k = max(k, v.y);
      if (lim >= 2) k = max(k, v.z);
      if (lim >= 3) k = max(k, v.w);
    } else if (r == 8) {
      const uint4 a = *reinterpret_cast<const uint4*>(rr + 8 * o);
      const uint4 c = *reinterpret_cast<const uint4*>(rr + 8 * o + 4);
      const uint32_t g[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      k = g[0];
#pragma unroll
      for (int i = 1; i < 8; ++i)
        if (lim >= i) k = max(k, g[i]);
    } else {
      for (int i = 0; i < r; ++i)
        if (i <= lim) k = max(k, rr[o * r + i]);
    }
    return (uint64_t(k) << 32) | uint64_t(~uint32_t(o));
  };
  int32_t* out = sel + int64_t(t) * topk;
  if (blockIdx.y == 0)
    for (int i = nb + threadIdx.x; i < topk; i += kN) out[i] = -1;
  if (int(blockIdx.y) * 64 >= nb) return;
  const uint64_t mine = b < nb ? (RUNS ? key_of(b) : own) : ~uint64_t(0);
  int rank = 0;
  for (int o0 = 0; o0 < nb; o0 += kRankTile) {
    const int n = min(kRankTile, nb - o0);
    const int nr = (n + 8 * kRankWaves - 1) / (8 * kRankWaves) * (8 * kRankWaves);
    __syncthreads();                          // the previous tile is consumed
    if (RUNS) {
      for (int i = threadIdx.x; i < nr; i += kN) tile[i] = i < n ? key_of(o0 + i) : 0;   // 0 is below every key
    } else if (o0 == 0) {
      tile[threadIdx.x] = int(threadIdx.x) < n ? pre0 : 0;
      tile[threadIdx.x + kN] = int(threadIdx.x) + kN < n ? pre1 : 0;
    } else {
      for (int i = threadIdx.x; i < nr; i += kN) tile[i] = i < n ? rk[o0 + i] : 0;
    }
    __syncthreads();
    const int per = nr / kRankWaves;          // a multiple of 8
    for (int i = wave * per; i < (wave + 1) * per; i += 8) {   // the wave's lanes read the same entries
#pragma unroll
      for (int e = 0; e < 8; ++e) rank += tile[i + e] > mine ? 1 : 0;
    }
  }
  partial[wave][lane] = rank;
  __syncthreads();
  if (wave == 0) {
    int r = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) r += partial[w][lane];
    if (b < nb && r < topk) out[r] = b;
  }
}

// 16 bytes from global memory into LDS at m0 + 16 x lane (the lanes of a wave fill consecutive
// slots), without passing through registers.
__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
// Wait for every vector-memory operation of the wave (loads into LDS included), then a compiler
// barrier so that no LDS read is hoisted above it.
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Elements of one 16-byte piece as floats: 8 bf16 or 4 fp32.
template <int QFMT>
__device__ __forceinline__ void unpack(const uint4& v, float* f) {
  if constexpr (QFMT == DSA_FMT_F32) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f[2 * r] = __uint_as_float(w[r] << 16);
      f[2 * r + 1] = __uint_as_float(w[r] & 0xFFFF0000u);
    }
  }
}

template <int QFMT>
__device__ __forceinline__ float elem(const void* base, int64_t i) {
  if constexpr (QFMT == DSA_FMT_F32) return static_cast<const float*>(base)[i];
  else return dsa::bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
}

__device__ __forceinline__ float wave_max_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// LDS layout of msa_attend_split, in bytes from the start of the dynamic area.
struct SplitLds {
  int trow;    // [block] int64 pool row of each visible token of the block
  int q;       // [gh][d] f32
  int s;       // [gh][tc] f32 logits, then weights
  int ml;      // [3][gh] f32 running max, running sum, rescale of the chunk
  int total;
};

// The K/V tile comes first: tc token rows of 2 x pieces x 16 bytes (the token's K pieces, then
// its V pieces). Inside each half, piece c of token k sits in slot (c + k) mod pieces, so that
// lanes reading one piece of consecutive tokens hit different banks. The area also holds the
// partial sums of the token parts at the end (kThreads x 8 floats), hence its minimum size.
__host__ __device__ inline SplitLds split_lds(int d, int elem_bytes, int block, int gh, int tc) {
  SplitLds l;
  int kv_bytes = 2 * tc * (d * elem_bytes / 16) * 16;
  kv_bytes = kv_bytes < kThreads * 8 * 4 ? kThreads * 8 * 4 : kv_bytes;
  l.trow = kv_bytes;
  l.q = l.trow + block * 8;
  l.s = l.q + gh * d * 4;
  l.ml = l.s + gh * tc * 4;
  l.total = (l.ml + 3 * gh * 4 + 15) & ~15;
  return l;
}

// grid (rows, n_kv x head groups, topk). CPT: pieces per head row when known at compile time
// (16 for bf16 x 128 dims), else 0 (taken from d).
template <int QFMT, int CPT>
__global__ void __launch_bounds__(kThreads)
msa_attend_split(DevPlan p, const int32_t* __restrict__ sel, const void* __restrict__ q,
                 const uint8_t* __restrict__ pool, float sm_scale, float* __restrict__ part_o,
                 float2* __restrict__ part_ml, int topk, int block, int H, int n_kv, int d,
                 int64_t row_bytes, int gh, int tc) {
  constexpr int E = QFMT == DSA_FMT_F32 ? 4 : 2;
  constexpr int EPU = 16 / E;                         // elements per 16-byte piece
  extern __shared__ uint4 smem4[];
  const int cpt = CPT > 0 ? CPT : d / EPU;            // pieces per head row
  const int rowp = 2 * cpt;                           // pieces per token row of the K/V tile
  const SplitLds L = split_lds(d, E, block, gh, tc);
  uint8_t* base = reinterpret_cast<uint8_t*>(smem4);
  const uint4* tile = smem4;                          // [tc][K pieces | V pieces], rotated
  const uint32_t tile_lds = uint32_t(reinterpret_cast<uintptr_t>(smem4));
  int64_t* trow = reinterpret_cast<int64_t*>(base + L.trow);
  float* qv = reinterpret_cast<float*>(base + L.q);
  float* sc = reinterpret_cast<float*>(base + L.s);
  float* mrun = reinterpret_cast<float*>(base + L.ml);
  float* lrun = mrun + gh;
  float* alpha = lrun + gh;

  const int G = H / n_kv;
  const int n_hg = (G + gh - 1) / gh;
  const int t = blockIdx.x, kh = int(blockIdx.y) / n_hg, hg = int(blockIdx.y) % n_hg;
  const int s = blockIdx.z;
  const int h0 = kh * G + hg * gh;                    // first query head of the workgroup
  const int ng = min(gh, G - hg * gh);
  dsa_span sp;
  const int pos = row_position(p, t, &sp);
  const int blk = sel[int64_t(t) * topk + s];
  const int64_t first = int64_t(blk) * block;
  // visible tokens of the block: positions first .. min(pos, first + block - 1)
  const int n_valid = (blk < 0 || first > pos) ? 0 : int(min(int64_t(block), int64_t(pos) - first + 1));
  const int64_t pbase = int64_t(t) * H + h0;
  if (n_valid == 0) {                                 // nothing to attend: an empty partial
    if (int(threadIdx.x) < ng) part_ml[(pbase + threadIdx.x) * topk + s] = make_float2(-__builtin_inff(), 0.0f);
    return;
  }
  for (int i = threadIdx.x; i < n_valid; i += kThreads) {
    int off;
    const int pg = dsa::page_of(p, sp, int(first) + i, &off);
    trow[i] = int64_t(pg) * p.page_size + off;
  }
  for (int i = threadIdx.x; i < ng * d; i += kThreads) qv[i] = elem<QFMT>(q, pbase * d + i);
  for (int g = threadIdx.x; g < ng; g += kThreads) {
    mrun[g] = -__builtin_inff();
    lrun[g] = 0.0f;
  }

  // output units (head g, piece c); token parts when there are fewer units than threads
  const int units = ng * cpt;
  const int parts = units >= kThreads ? 1 : kThreads / units;
  const int part = int(threadIdx.x) / units < parts ? int(threadIdx.x) / units : -1;
  float acc[kMaxUnits][EPU];
#pragma unroll
  for (int u = 0; u < kMaxUnits; ++u)
#pragma unroll
    for (int e = 0; e < EPU; ++e) acc[u][e] = 0.0f;

  const int groups = kThreads / tc;                   // thread groups over a chunk's tokens
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* kv_base = pool + int64_t(kh) * d * E;
  const int64_t v_off = int64_t(n_kv) * d * E;
  __syncthreads();

  for (int c0 = 0; c0 < n_valid; c0 += tc) {
    const int nt = min(tc, n_valid - c0);
    // stage K and V of the chunk: slot i of the tile is piece i of the chunk's row-major
    // [token][K | V] order after the rotation; a wave's 64 lanes fill 64 consecutive slots
    const int npieces = nt * rowp;
    const uint32_t wave_lds =
        uint32_t(__builtin_amdgcn_readfirstlane(int(tile_lds + 16u * (threadIdx.x & ~63u))));
    const uint8_t* src[kMaxPieces];                  // every address first: the row reads batch
#pragma unroll
    for (int r = 0; r < kMaxPieces; ++r) {
      const int i = threadIdx.x + r * kThreads;
      const int tok = min(i, npieces - 1) / rowp, j = i - tok * rowp;
      const int isv = j >= cpt, jj = j - (isv ? cpt : 0);
      const int rot = tok % cpt;
      const int c = jj >= rot ? jj - rot : jj - rot + cpt;
      src[r] = kv_base + trow[c0 + tok] * row_bytes + (isv ? v_off : 0) + c * 16;
    }
#pragma unroll
    for (int r = 0; r < kMaxPieces; ++r)
      if (int(threadIdx.x) + r * kThreads < npieces) dma16(src[r], wave_lds + uint32_t(16 * r * kThreads));
    wait_vm_all();
    __syncthreads();

    // logits: thread (token, head subset), four heads at a time against its K row
    {
      const int tok = threadIdx.x % tc, gq = threadIdx.x / tc;
      if (tok < nt) {
        const int rot = tok % cpt;
        for (int g0 = gq; g0 < ng; g0 += 4 * groups) {
          float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          for (int c = 0; c < cpt; ++c) {
            float kf[EPU];
            const int slot = c + rot < cpt ? c + rot : c + rot - cpt;
            unpack<QFMT>(tile[tok * rowp + slot], kf);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int g = min(g0 + i * groups, ng - 1);
              const float* qq = qv + g * d + c * EPU;
#pragma unroll
              for (int e = 0; e < EPU; ++e) a[i] = fmaf(qq[e], kf[e], a[i]);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int g = g0 + i * groups;
            if (g < ng) sc[g * tc + tok] = a[i] * sm_scale;
          }
        }
      }
    }
    __syncthreads();

    // running max and sum per head; the chunk's logits become weights
    for (int g = wave; g < ng; g += kThreads / 64) {
      float cm = -__builtin_inff();
      for (int i = lane; i < nt; i += 64) cm = fmaxf(cm, sc[g * tc + i]);
      cm = wave_max_f(cm);
      const float m_old = mrun[g];
      const float m_new = fmaxf(m_old, cm);
      float ls = 0.0f;
      for (int i = lane; i < nt; i += 64) {
        const float e = __expf(sc[g * tc + i] - m_new);
        sc[g * tc + i] = e;
        ls += e;
      }
      ls = wave_sum_f(ls);
      if (lane == 0) {
        const float a = m_old == -__builtin_inff() ? 0.0f : __expf(m_old - m_new);
        mrun[g] = m_new;
        lrun[g] = lrun[g] * a + ls;
        alpha[g] = a;
      }
    }
    __syncthreads();

    // weighted V rows: each unit rescales its sum, then adds its part's tokens
    if (part >= 0) {
#pragma unroll
      for (int u = 0; u < kMaxUnits; ++u) {
        const int unit = parts > 1 ? int(threadIdx.x) % units : int(threadIdx.x) + u * kThreads;
        if (parts > 1 ? u == 0 : unit < units) {
          const int g = unit / cpt, c = unit - g * cpt;
          const float a = alpha[g];
#pragma unroll
          for (int e = 0; e < EPU; ++e) acc[u][e] *= a;
          auto v_piece = [&](int tok) {
            const int rot = tok % cpt;
            return tile[tok * rowp + cpt + (c + rot < cpt ? c + rot : c + rot - cpt)];
          };
          int tok = part;
          for (; tok + 3 * parts < nt; tok += 4 * parts) {     // four tokens' reads in flight
            float w[4];
            uint4 vp[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              w[k] = sc[g * tc + tok + k * parts];
              vp[k] = v_piece(tok + k * parts);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              float vf[EPU];
              unpack<QFMT>(vp[k], vf);
#pragma unroll
              for (int e = 0; e < EPU; ++e) acc[u][e] = fmaf(w[k], vf[e], acc[u][e]);
            }
          }
          for (; tok < nt; tok += parts) {
            const float w = sc[g * tc + tok];
            float vf[EPU];
            unpack<QFMT>(v_piece(tok), vf);
#pragma unroll
            for (int e = 0; e < EPU; ++e) acc[u][e] = fmaf(w, vf[e], acc[u][e]);
          }
        }
      }
    }
    __syncthreads();                                  // the chunk's tiles and weights are consumed
  }

  // the partial: unnormalised output, running max and sum
  if (parts > 1) {
    float* red = reinterpret_cast<float*>(smem4);     // [kThreads][EPU], over the K/V tiles
    if (part >= 0)
#pragma unroll
      for (int e = 0; e < EPU; ++e) red[threadIdx.x * EPU + e] = acc[0][e];
    __syncthreads();
    if (int(threadIdx.x) < units) {
      float o[EPU];
#pragma unroll
      for (int e = 0; e < EPU; ++e) o[e] = acc[0][e];
      for (int q2 = 1; q2 < parts; ++q2)
#pragma unroll
        for (int e = 0; e < EPU; ++e) o[e] += red[(q2 * units + threadIdx.x) * EPU + e];
      const int g = threadIdx.x / cpt, c = threadIdx.x - g * cpt;
      float* dst = part_o + ((pbase + g) * topk + s) * d + c * EPU;
#pragma unroll
      for (int e = 0; e < EPU; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kMaxUnits; ++u) {
      const int unit = threadIdx.x + u * kThreads;
      if (unit < units) {
        const int g = unit / cpt, c = unit - g * cpt;
        float* dst = part_o + ((pbase + g) * topk + s) * d + c * EPU;
#pragma unroll
        for (int e = 0; e < EPU; e += 4)
          *reinterpret_cast<float4*>(dst + e) =
              make_float4(acc[u][e], acc[u][e + 1], acc[u][e + 2], acc[u][e + 3]);
      }
    }
  }
  if (int(threadIdx.x) < ng)
    part_ml[(pbase + threadIdx.x) * topk + s] = make_float2(mrun[threadIdx.x], lrun[threadIdx.x]);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 lds_b128(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(static_cast<uintptr_t>(a));
}
// ds_read_b64_tr_b16: in each group of 16 lanes, lane j addresses row j / 4 of a 4-row block,
// columns 4 (j % 4) .. +3; lane j receives column j of the 16 for the block's 4 rows.
__device__ __forceinline__ bf16x4 lds_tr16(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<bf16x4 __attribute__((address_space(3)))*>(static_cast<uintptr_t>(a)));
}

constexpr int kMfTok = 128;                  // tokens staged by msa_attend_mfma (a whole block)
constexpr int kPPitch = kMfTok + 8;          // bf16 per head row of P in LDS (a 16-byte pad)

// LDS layout of msa_attend_mfma<D> in bytes: the K|V tile (the token rows as msa_attend_split
// lays them out, rotated pieces), P [16 heads][kPPitch] bf16, per-wave head maxima and sums, and
// the pool rows of the block's tokens.
template <int D>
struct MfLds {
  static constexpr int kRow = 4 * D;
  static constexpr int kP = kMfTok * kRow;
  static constexpr int kRed = kP + 16 * kPPitch * 2;
  static constexpr int kTrow = kRed + 2 * 4 * 16 * 4;
  static constexpr int kTotal = kTrow + kMfTok * 8;
};

// grid (rows, n_kv x head groups, topk); bf16, head_dim D (64, 128 or 256), blocks of at most
// 128 tokens, at most 16 query heads per workgroup.
//   Q.K^T  v_mfma_f32_16x16x32_bf16, A = 16 tokens' K rows (LDS), B = the group's queries
//          (VGPRs, zero past the group): wave w scores tokens 32 w .. 32 w + 31.
//   softmax in fp32 over the block (maxima and sums through LDS), in base 2; P rounded to bf16
//          into LDS.
//   P.V    v_mfma_f32_16x16x32_bf16, A = P (heads x 32 tokens, LDS), B = V read transposed from
//          the tile; wave w produces output columns w D/4 .. (w + 1) D/4 - 1 for every head.
template <int D>
__global__ void __launch_bounds__(kThreads)
msa_attend_mfma(DevPlan p, const int32_t* __restrict__ sel, const uint16_t* __restrict__ q,
                const uint8_t* __restrict__ pool, float sm_scale, float* __restrict__ part_o,
                float2* __restrict__ part_ml, int topk, int block, int H, int n_kv,
                int64_t row_bytes, int gh) {
  using L = MfLds<D>;
  constexpr int CPT = D / 8;                          // 16-byte pieces per head row
  constexpr int KS = D / 32;                          // k-steps of Q.K^T
  constexpr int NT = D / 64;                          // 16-column tiles of a wave's P.V share
  constexpr int kPer = kMfTok * 2 * CPT / kThreads;   // DMAs per thread for a full block
  extern __shared__ uint4 smem4[];
  uint8_t* base = reinterpret_cast<uint8_t*>(smem4);
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem4));
  int64_t* trow = reinterpret_cast<int64_t*>(base + L::kTrow);
  float* red_m = reinterpret_cast<float*>(base + L::kRed);   // [4][16]
  float* red_l = red_m + 4 * 16;                             // [4][16]

  const int G = H / n_kv;
  const int n_hg = (G + gh - 1) / gh;
  const int t = blockIdx.x, kh = int(blockIdx.y) / n_hg, hg = int(blockIdx.y) % n_hg;
  const int s = blockIdx.z;
  const int h0 = kh * G + hg * gh;
  const int ng = min(gh, G - hg * gh);
  const int64_t pbase = int64_t(t) * H + h0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 15, g = lane >> 4;
  // the picked block and the queries first: neither depends on the row's place in the plan
  const int blk = sel[int64_t(t) * topk + s];
  // B operand of Q.K^T: head h0 + j, dims 32 ks + 8 g .. +7
  bf16x8 qb[KS];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(q + (pbase + min(j, ng - 1)) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = qrow[4 * ks + g];
      if (j >= ng) v = make_uint4(0u, 0u, 0u, 0u);
      qb[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  dsa_span sp;
  const int pos = row_position(p, t, &sp);
  const int64_t first = int64_t(blk) * block;
  const int n_valid = (blk < 0 || first > pos) ? 0 : int(min(int64_t(block), int64_t(pos) - first + 1));
  if (n_valid == 0) {
    if (int(threadIdx.x) < ng) part_ml[(pbase + threadIdx.x) * topk + s] = make_float2(-__builtin_inff(), 0.0f);
    return;
  }
  const int ntp = (n_valid + 31) & ~31;               // tokens staged: whole k-steps of 32
  for (int i = threadIdx.x; i < ntp; i += kThreads) {   // padding tokens repeat the last one
    int off;
    const int pg = dsa::page_of(p, sp, int(first) + min(i, n_valid - 1), &off);
    trow[i] = int64_t(pg) * p.page_size + off;
  }
  __syncthreads();                                    // trow

  // K and V of the staged tokens into the tile, rotated as in msa_attend_split
  {
    const int npieces = ntp * 2 * CPT;
    const uint8_t* kv_base = pool + int64_t(kh) * D * 2;
    const int64_t v_off = int64_t(n_kv) * D * 2;
    const uint32_t wave_lds =
        uint32_t(__builtin_amdgcn_readfirstlane(int(lds0 + 16u * (threadIdx.x & ~63u))));
    const uint8_t* src[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = threadIdx.x + r * kThreads;
      const int tok = min(i, npieces - 1) / (2 * CPT), jj = i - tok * 2 * CPT;
      const int isv = jj >= CPT;
      const int c = ((jj - (isv ? CPT : 0)) - tok) & (CPT - 1);
      src[r] = kv_base + trow[tok] * row_bytes + (isv ? v_off : 0) + c * 16;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r)
      if (int(threadIdx.x) + r * kThreads < npieces) dma16(src[r], wave_lds + uint32_t(16 * r * kThreads));
  }
  wait_vm_all();
  __syncthreads();

  // Q.K^T for this wave's 32 tokens; logits in base-2 units
  const float scale2 = sm_scale * 1.4426950408889634f;
  const bool active = 32 * wave < ntp;
  float sv[2][4];
  float mloc = -__builtin_inff();
  if (active) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = 32 * wave + 16 * tt + j;        // A row: this lane's token
      const uint32_t rowa = lds0 + uint32_t(tok * L::kRow);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int slot = (4 * ks + g + tok) & (CPT - 1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_b128(rowa + 16 * slot), qb[ks], acc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tk = 32 * wave + 16 * tt + 4 * g + v;     // C row: token, column: head j
        sv[tt][v] = tk < n_valid ? acc[v] * scale2 : -__builtin_inff();
        mloc = fmaxf(mloc, sv[tt][v]);
      }
    }
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  if (g == 0) red_m[wave * 16 + j] = mloc;
  __syncthreads();
  const float m = fmaxf(fmaxf(red_m[j], red_m[16 + j]), fmaxf(red_m[32 + j], red_m[48 + j]));
  float lsum = 0.0f;
  if (active) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      uint32_t pk[2];
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const float p0 = exp2f(sv[tt][v] - m), p1 = exp2f(sv[tt][v + 1] - m);
        lsum += p0 + p1;
        pk[v / 2] = uint32_t(dsa::f32_to_bf16(p0)) | (uint32_t(dsa::f32_to_bf16(p1)) << 16);
      }
      const int tk0 = 32 * wave + 16 * tt + 4 * g;
      *reinterpret_cast<uint2*>(base + L::kP + (j * kPPitch + tk0) * 2) = make_uint2(pk[0], pk[1]);
    }
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (g == 0) red_l[wave * 16 + j] = lsum;
  __syncthreads();                                    // P and the sums are in LDS

  // P.V over the staged k-steps: this wave's NT column tiles
  f32x4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nks = ntp / 32;
  for (int u = 0; u < nks; ++u) {
    const bf16x8 pa = lds_b128(lds0 + uint32_t(L::kP + (j * kPPitch + 32 * u + 8 * g) * 2));
    const int tk = 32 * u + 8 * g + (j >> 2);          // rows of this lane's transposed reads: tk, tk + 4
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int cc = wave * (D / 4) + 16 * nt + 4 * (j & 3);   // first of the lane's 4 columns
      const int c = cc >> 3, cb = (cc & 7) * 2;
      const uint32_t a0 = lds0 + uint32_t(tk * L::kRow + CPT * 16 + ((c + tk) & (CPT - 1)) * 16 + cb);
      const uint32_t a1 = lds0 + uint32_t((tk + 4) * L::kRow + CPT * 16 + ((c + tk + 4) & (CPT - 1)) * 16 + cb);
      const bf16x4 b0 = lds_tr16(a0), b1 = lds_tr16(a1);
      const bf16x8 bv = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, bv, o[nt], 0, 0, 0);
    }
  }
  // C: head 4 g + v, column wave D/4 + 16 nt + j
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = 4 * g + v;
      if (hh < ng)
        part_o[((pbase + hh) * topk + s) * D + wave * (D / 4) + 16 * nt + j] = o[nt][v];
    }
  }
  if (wave == 0 && g == 0 && j < ng) {
    const float l = red_l[j] + red_l[16 + j] + red_l[32 + j] + red_l[48 + j];
    part_ml[(pbase + j) * topk + s] = make_float2(m * 0.6931471805599453f, l);
  }
}

// grid (rows, H); thread e < d owns output element e
template <int QFMT>
__global__ void __launch_bounds__(kThreads)
msa_combine(const float* __restrict__ part_o, const float2* __restrict__ part_ml, int topk, int H,
            int d, void* __restrict__ out) {
  const int64_t row = int64_t(blockIdx.x) * H + blockIdx.y;
  const int e = threadIdx.x;
  if (e >= d) return;
  const float2* ml = part_ml + row * topk;
  const float* po = part_o + row * topk * d + e;
  // sixteen partials' maxima, sums and outputs loaded at once, merged with a running max; an
  // empty partial (max -inf) wrote no output, so its loaded value is never used
  float M = -__builtin_inff(), L = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < topk; s0 += 16) {
    float2 v[16];
    float ov[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int si = min(s0 + i, topk - 1);
      v[i] = ml[si];
      ov[i] = po[int64_t(si) * d];
    }
    float mb = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) mb = fmaxf(mb, s0 + i < topk ? v[i].x : -__builtin_inff());
    const float Mn = fmaxf(M, mb);
    if (Mn == -__builtin_inff()) continue;            // nothing yet
    const float a = M == -__builtin_inff() ? 0.0f : __expf(M - Mn);
    L *= a;
    o *= a;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool use = s0 + i < topk && v[i].x != -__builtin_inff();
      const float w = use ? __expf(v[i].x - Mn) : 0.0f;
      L = fmaf(w, use ? v[i].y : 0.0f, L);
      o = fmaf(w, use ? ov[i] : 0.0f, o);
    }
    M = Mn;
  }
  const float r = L > 0.0f ? o / L : 0.0f;
  if constexpr (QFMT == DSA_FMT_F32) static_cast<float*>(out)[row * d + e] = r;
  else static_cast<uint16_t*>(out)[row * d + e] = dsa::f32_to_bf16(r);
}

// The matrix-core attention takes bf16 caches of head_dim 64, 128 or 256 and blocks of at most
// 128 tokens; every other shape goes to msa_attend_split.
bool msa_mfma_shape(const dsa_msa_config& c) {
  return c.q_fmt == DSA_FMT_BF16 && c.block_size <= kMfTok &&
         (c.head_dim == 64 || c.head_dim == 128 || c.head_dim == 256);
}

// Tile of the attention launch: query heads per workgroup and tokens per chunk (a power of two
// that keeps a chunk's K and V pieces within kMaxPieces per thread).
void attend_tile(const dsa_msa_config& c, int* gh, int* tc) {
  const int G = c.n_heads / c.n_kv_heads;
  *gh = G < kMaxGroup ? G : kMaxGroup;
  const int cpt = c.head_dim * (c.q_fmt == DSA_FMT_F32 ? 4 : 2) / 16;
  int n = c.block_size < 128 ? c.block_size : 128;
  while (n > 1 && n * cpt * 2 > kMaxPieces * kThreads) n /= 2;
  *tc = n;
}

}  // namespace

size_t msa_block_keys_ld(const dsa_msa_config& c, const PlanInfo& in) {
  return size_t(in.max_visible / c.block_size + 1);
}

size_t msa_attend_lds_bytes(const dsa_msa_config& c) {
  int gh, tc;
  attend_tile(c, &gh, &tc);
  return size_t(split_lds(c.head_dim, c.q_fmt == DSA_FMT_F32 ? 4 : 2, c.block_size, gh, tc).total);
}

size_t msa_attend_workspace_bytes(const dsa_msa_config& c, const PlanInfo& in) {
  const size_t parts = size_t(in.n_rows) * c.n_heads * c.topk_blocks;
  return ((parts * c.head_dim * 4 + 255) & ~size_t(255)) + ((parts * 8 + 255) & ~size_t(255));
}

hipError_t msa_prepare(const dsa_msa_config& c) {
  const struct { const void* f; int lds; } mf[] = {
      {reinterpret_cast<const void*>(&msa_attend_mfma<64>), MfLds<64>::kTotal},
      {reinterpret_cast<const void*>(&msa_attend_mfma<128>), MfLds<128>::kTotal},
      {reinterpret_cast<const void*>(&msa_attend_mfma<256>), MfLds<256>::kTotal}};
  for (const auto& k : mf) {
    const hipError_t e = hipFuncSetAttribute(k.f, hipFuncAttributeMaxDynamicSharedMemorySize, k.lds);
    if (e != hipSuccess) return e;
  }
  const int lds = int(msa_attend_lds_bytes(c));
  const void* fns[] = {
      reinterpret_cast<const void*>(&msa_attend_split<DSA_FMT_F32, 0>),
      reinterpret_cast<const void*>(&msa_attend_split<DSA_FMT_F32, 16>),
      reinterpret_cast<const void*>(&msa_attend_split<DSA_FMT_F32, 32>),
      reinterpret_cast<const void*>(&msa_attend_split<DSA_FMT_BF16, 0>),
      reinterpret_cast<const void*>(&msa_attend_split<DSA_FMT_BF16, 16>),
      reinterpret_cast<const void*>(&msa_attend_split<DSA_FMT_BF16, 32>)};
  for (const void* f : fns) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_msa_block_topk(const dsa_msa_handle* h, const DevPlan& p, const PlanInfo& in,
                                 const float* scores, int64_t ld, uint64_t* keys, int32_t* sel,
                                 hipStream_t st) {
  const dsa_msa_config& c = h->cfg;
  const int64_t kld = int64_t(msa_block_keys_ld(c, in));
  const int64_t per_group = kKeyScores / c.block_size;     // blocks per msa_block_keys workgroup
  const dim3 kgrid(unsigned(in.n_rows), unsigned((kld + per_group - 1) / per_group));
#define DSA_MSA_KEYS(B) \
  case B: hipLaunchKernelGGL(msa_block_keys<B>, kgrid, dim3(kThreads), 0, st, p, scores, ld, keys, kld); break;
  switch (c.block_size) {
    DSA_MSA_KEYS(32)
    DSA_MSA_KEYS(64)
    DSA_MSA_KEYS(128)
    DSA_MSA_KEYS(256)
    default: return hipErrorInvalidValue;
  }
#undef DSA_MSA_KEYS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 rgrid(unsigned(in.n_rows), unsigned((kld + 63) / 64));
  hipLaunchKernelGGL(msa_block_rank<false>, rgrid, dim3(64 * kRankWaves), 0, st, p, c.block_size,
                     keys, nullptr, kld, c.topk_blocks, sel);
  return hipGetLastError();
}

// 32-key groups per row of the runs buffer, padded to 8 (32-byte aligned rows)
int64_t msa_runs_ld(const PlanInfo& in) { return ((int64_t(in.max_visible) + 31) / 32 + 7) & ~int64_t(7); }

hipError_t launch_msa_block_rank_runs(const dsa_msa_handle* h, const DevPlan& p,
                                      const PlanInfo& in, const uint32_t* runs, int32_t* sel,
                                      hipStream_t st) {
  const dsa_msa_config& c = h->cfg;
  const int64_t nb = int64_t(msa_block_keys_ld(c, in));
  const dim3 rgrid(unsigned(in.n_rows), unsigned((nb + 63) / 64));
  hipLaunchKernelGGL(msa_block_rank<true>, rgrid, dim3(64 * kRankWaves), 0, st, p, c.block_size,
                     nullptr, runs, msa_runs_ld(in), c.topk_blocks, sel);
  return hipGetLastError();
}

hipError_t launch_msa_attend(const dsa_msa_handle* h, const DevPlan& p, const PlanInfo& in,
                             const int32_t* sel, const void* q, const void* pool, float sm_scale,
                             void* out, void* ws, hipStream_t st) {
  const dsa_msa_config& c = h->cfg;
  int gh, tc;
  attend_tile(c, &gh, &tc);
  const size_t lds = msa_attend_lds_bytes(c);
  const int G = c.n_heads / c.n_kv_heads;
  const int n_hg = (G + gh - 1) / gh;
  const size_t parts = size_t(in.n_rows) * c.n_heads * c.topk_blocks;
  float* part_o = static_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                              ((parts * c.head_dim * 4 + 255) & ~size_t(255)));
  const dim3 grid(unsigned(in.n_rows), unsigned(c.n_kv_heads * n_hg), unsigned(c.topk_blocks));
  const dim3 cgrid(unsigned(in.n_rows), unsigned(c.n_heads));
  const unsigned cthreads = unsigned((c.head_dim + 63) / 64 * 64);
  const uint8_t* pb = static_cast<const uint8_t*>(pool);
  const int cpt = c.head_dim * (c.q_fmt == DSA_FMT_F32 ? 4 : 2) / 16;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
#define DSA_MSA_MFMA(D)                                                                          \
  hipLaunchKernelGGL((msa_attend_mfma<D>), grid, dim3(kThreads), size_t(MfLds<D>::kTotal), st, p, \
                     sel, q16, pb, sm_scale, part_o, part_ml, c.topk_blocks, c.block_size,       \
                     c.n_heads, c.n_kv_heads, h->gqa_row_bytes, gh)
#define DSA_MSA_SPLIT(Q, CPT)                                                                    \
  hipLaunchKernelGGL((msa_attend_split<Q, CPT>), grid, dim3(kThreads), lds, st, p, sel, q, pb,  \
                     sm_scale, part_o, part_ml, c.topk_blocks, c.block_size, c.n_heads,         \
                     c.n_kv_heads, c.head_dim, h->gqa_row_bytes, gh, tc)
  if (c.q_fmt == DSA_FMT_F32) {
    if (cpt == 16) DSA_MSA_SPLIT(DSA_FMT_F32, 16);
    else if (cpt == 32) DSA_MSA_SPLIT(DSA_FMT_F32, 32);
    else DSA_MSA_SPLIT(DSA_FMT_F32, 0);
  } else if (msa_mfma_shape(c)) {
    if (c.head_dim == 64) DSA_MSA_MFMA(64);
    else if (c.head_dim == 128) DSA_MSA_MFMA(128);
    else DSA_MSA_MFMA(256);
  } else {
    if (cpt == 16) DSA_MSA_SPLIT(DSA_FMT_BF16, 16);
    else if (cpt == 32) DSA_MSA_SPLIT(DSA_FMT_BF16, 32);
    else DSA_MSA_SPLIT(DSA_FMT_BF16, 0);
  }
#undef DSA_MSA_SPLIT
#undef DSA_MSA_MFMA
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (c.q_fmt == DSA_FMT_F32)
    hipLaunchKernelGGL(msa_combine<DSA_FMT_F32>, cgrid, dim3(cthreads), 0, st, part_o, part_ml,
                       c.topk_blocks, c.n_heads, c.head_dim, out);
  else
    hipLaunchKernelGGL(msa_combine<DSA_FMT_BF16>, cgrid, dim3(cthreads), 0, st, part_o, part_ml,
                       c.topk_blocks, c.n_heads, c.head_dim, out);
  return hipGetLastError();
}
