// Causal top-k select (DSA resource page: select_topk_causal, index_topk).
// Row t sees scores[t][0 .. position]. It keeps the topk positions of highest score, equal scores
// going to the lower position, and writes them by score descending / position ascending followed
// by -1 entries (a contiguous tail, as ttnn.transformer.sparse_sdpa lays out masked indices).
//
// Every comparison is on the unique 64-bit key (order_key(score) << 32 | ~position), so the result
// does not depend on how the work is split or scheduled. A row is split into chunks of kChunk keys
// so that long decode rows use many workgroups:
//   minmax   min / max order key per 2048-key block (the matrix-core score kernel writes these
//            itself; other score producers run this kernel)
//   hist     per chunk, a kBins-bin histogram linear in the score between the row's min and max
//            (monotone in the score, so a higher bin always holds higher scores)
//   collect  every chunk finds the bin b* where the count from the top reaches topk, and writes
//            the positions in bins above b* (all kept) and in b* (candidates) to the row's buffer
//            at offsets given by prefix sums of the chunk histograms (no atomics across chunks)
//   final    one workgroup per row orders winners + candidates exactly and keeps topk.
// A row whose b* holds more than kCap keys (massive ties) is selected by an exact single-workgroup
// radix select over the whole row instead.
//
// Rows scored one per workgroup by the matrix-core score kernel take a path of one launch
// (select_lists below) over per-block counts and key lists that kernel writes in place of the
// scores; the launches above serve every other score producer and the select-only entry.
#include "dsa_internal.hpp"

namespace {

constexpr int kMinMaxBlock = kScoreBlock;   // keys per min/max entry (the score kernel's block)
constexpr int kChunk = 4096;         // keys per hist / collect workgroup
constexpr int kBins = 256;           // linear histogram bins
constexpr int kCap = 2048;           // candidates kept per row from the threshold bin
constexpr int kSortBins = 4096;      // counting-sort bins in the final stage
constexpr int kFixMax = 64;          // largest counting-sort bin resolved by direct ranking
constexpr int kFinalThreads = 1024;
constexpr int kThreads = 256;

struct RowInfo {
  int b_star;
  int n_above;
  int n_cand;
  int pad;
};

__device__ __forceinline__ uint64_t composite(uint32_t key, int j) {
  return (uint64_t(key) << 32) | uint32_t(~uint32_t(j));
}
__device__ __forceinline__ int comp_pos(uint64_t c) { return int(~uint32_t(c & 0xFFFFFFFFu)); }
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int row_position(const DevPlan& p, int t) {
  dsa_span sp;
  dsa::row_span(p.spans, p.n_spans, t, &sp);
  return sp.ctx_start + (t - sp.q_start);
}
// the same with the plan's first 64 spans already requested (dsa::span_chunk)
__device__ __forceinline__ int row_position_from(const dsa_span& span0, const DevPlan& p, int t) {
  dsa_span sp;
  dsa::row_span_from(span0, p.spans, p.n_spans, t, &sp);
  return sp.ctx_start + (t - sp.q_start);
}

// Linear bin of a score between the row's lo and hi (weakly increasing in s).
struct Binner {
  float lo, inv;
  bool flat;
  __device__ Binner(uint32_t lo_key, uint32_t hi_key) {
    lo = key_to_float(lo_key);
    const float hi = key_to_float(hi_key);
    const float range = hi - lo;
    inv = range > 0.0f ? float(kBins) / range : 0.0f;
    flat = !(range > 0.0f) || !(inv < 3.0e38f);
  }
  __device__ __forceinline__ int operator()(float s) const {
    if (flat) return 0;
    return int(fminf(fmaxf((s - lo) * inv, 0.0f), float(kBins - 1)));  // NaN -> bin 0
  }
};

// The row's min / max order key from the per-block entries: each thread's share (loads only),
// then the workgroup reduction (synchronises the block). minmax_first loads entry threadIdx.x
// before the row's length is known (any entry below nb_max lies in the buffer), so that the load
// overlaps the span lookup; minmax_partial masks it to the row's blocks and loads the rest.
__device__ __forceinline__ uint2 minmax_first(const uint32_t* __restrict__ mm, int64_t t, int nb_max) {
  const int i = threadIdx.x;
  return i < nb_max ? *reinterpret_cast<const uint2*>(mm + 2 * (t * nb_max + i))
                    : make_uint2(0xFFFFFFFFu, 0u);
}
__device__ __forceinline__ void minmax_partial(uint2 first, const uint32_t* __restrict__ mm, int64_t t,
                                               int nb_max, int n, uint32_t* mn, uint32_t* mx) {
  const int nb = (n + kMinMaxBlock - 1) / kMinMaxBlock;
  uint32_t a = int(threadIdx.x) < nb ? first.x : 0xFFFFFFFFu;
  uint32_t b = int(threadIdx.x) < nb ? first.y : 0u;
  for (int i = threadIdx.x + blockDim.x; i < nb; i += blockDim.x) {
    a = min(a, mm[2 * (t * nb_max + i)]);
    b = max(b, mm[2 * (t * nb_max + i) + 1]);
  }
  *mn = a;
  *mx = b;
}
__device__ void minmax_reduce(uint32_t mn, uint32_t mx, uint32_t* lo, uint32_t* hi, uint32_t* red) {
  mn = dsa::wave_min_u32(mn);
  mx = dsa::wave_max_u32(mx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) { red[wave] = mn; red[nw + wave] = mx; }
  __syncthreads();
  mn = red[0]; mx = red[nw];
  for (int i = 1; i < nw; ++i) { mn = min(mn, red[i]); mx = max(mx, red[nw + i]); }
  __syncthreads();
  *lo = mn; *hi = mx;
}
__device__ void row_minmax(uint2 first, const uint32_t* __restrict__ mm, int64_t t, int nb_max, int n,
                           uint32_t* lo, uint32_t* hi, uint32_t* red) {
  uint32_t mn, mx;
  minmax_partial(first, mm, t, nb_max, n, &mn, &mx);
  minmax_reduce(mn, mx, lo, hi, red);
}

// ------------------------------------------------------------------ minmax
__global__ void __launch_bounds__(kThreads)
select_minmax(DevPlan p, const float* __restrict__ scores, int64_t ld, uint32_t* __restrict__ mm,
              int nb_max) {
  __shared__ uint32_t red[2 * kThreads / 64];
  const int t = blockIdx.y;
  const int n = row_position(p, t) + 1;
  const int j0 = blockIdx.x * kMinMaxBlock;
  if (j0 >= n) return;
  const float* row = scores + int64_t(t) * ld;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int j = j0 + threadIdx.x; j < min(n, j0 + kMinMaxBlock); j += kThreads) {
    const uint32_t k = dsa::order_key(row[j]);
    mn = min(mn, k);
    mx = max(mx, k);
  }
  mn = dsa::wave_min_u32(mn);
  mx = dsa::wave_max_u32(mx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[wave] = mn; red[kThreads / 64 + wave] = mx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kThreads / 64; ++i) { mn = min(mn, red[i]); mx = max(mx, red[kThreads / 64 + i]); }
    mn = min(mn, red[0]); mx = max(mx, red[kThreads / 64]);
    mm[2 * (int64_t(t) * nb_max + blockIdx.x)] = mn;
    mm[2 * (int64_t(t) * nb_max + blockIdx.x) + 1] = mx;
  }
}

// ------------------------------------------------------------------ hist
constexpr int kPerThread = kChunk / kThreads;   // scores per thread in hist / collect

__global__ void __launch_bounds__(kThreads)
select_hist(DevPlan p, const float* __restrict__ scores, int64_t ld, int topk,
            const uint32_t* __restrict__ mm, int nb_max, uint32_t* __restrict__ hist, int g_max) {
  constexpr int kW = kThreads / 64;
  __shared__ uint32_t h[kW][kBins];     // one histogram per wave: fewer colliding LDS atomics
  __shared__ uint32_t red[2 * kW];
  const int t = blockIdx.y, g = blockIdx.x;
  // the chunk's scores first (up to ld, masked to the row below), so that their latency overlaps
  // the span lookup and the min / max reduction
  const float* row = scores + int64_t(t) * ld;
  float v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int j = g * kChunk + i * kThreads + threadIdx.x;
    v[i] = j < ld ? row[j] : 0.0f;
  }
  const uint2 mm0 = minmax_first(mm, t, nb_max);
  const int n = row_position(p, t) + 1;
  if (n <= topk || g * kChunk >= n) return;
  for (int i = threadIdx.x; i < kW * kBins; i += kThreads) (&h[0][0])[i] = 0;
  uint32_t lo, hi;
  row_minmax(mm0, mm, t, nb_max, n, &lo, &hi, red);   // synchronises the block
  const Binner bin(lo, hi);
  uint32_t* mine = h[threadIdx.x >> 6];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int j = g * kChunk + i * kThreads + threadIdx.x;
    if (j < n) atomicAdd(&mine[bin(v[i])], 1u);
  }
  __syncthreads();
  uint32_t* dst = hist + (int64_t(t) * g_max + g) * kBins;
  for (int b = threadIdx.x; b < kBins; b += kThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) c += h[w][b];
    dst[b] = c;
  }
}

// ------------------------------------------------------------------ collect
__global__ void __launch_bounds__(kThreads)
select_collect(DevPlan p, const float* __restrict__ scores, int64_t ld, int topk,
               const uint32_t* __restrict__ mm, int nb_max, const uint32_t* __restrict__ hist,
               int g_max, uint64_t* __restrict__ rowbuf, int rowbuf_len, RowInfo* __restrict__ info) {
  static_assert(kBins == kThreads, "one bin per thread");
  constexpr int kW = kThreads / 64;
  __shared__ uint32_t suffix[kBins];     // count of the row in bins >= b
  __shared__ uint32_t red[2 * kW];
  __shared__ uint32_t wsum[kW];
  __shared__ int s_bstar;
  __shared__ uint32_t s_wscan[kW], s_cscan[kW];
  const int t = blockIdx.y, g = blockIdx.x;
  const float* row = scores + int64_t(t) * ld;
  float v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int j = g * kChunk + i * kThreads + threadIdx.x;
    v[i] = j < ld ? row[j] : 0.0f;
  }
  const uint2 mm0 = minmax_first(mm, t, nb_max);
  // this thread's bin of the first 32 chunk histograms, before the row's chunk count is known
  // (entries below g_max lie in the buffer; those past the row are masked below)
  const int b = threadIdx.x;
  const uint32_t* hrow = hist + int64_t(t) * g_max * kBins;
  constexpr int kPre = 32;
  uint32_t x[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) x[i] = i < g_max ? hrow[int64_t(i) * kBins + b] : 0u;
  const int n = row_position(p, t) + 1;
  if (n <= topk || g * kChunk >= n) return;
  const int G = (n + kChunk - 1) / kChunk;
  uint32_t mn, mx;
  minmax_partial(mm0, mm, t, nb_max, n, &mn, &mx);
  // per bin (one per thread): total over the row, and the part in chunks before g
  uint32_t tot = 0, bel = 0;
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const uint32_t xi = i < G ? x[i] : 0u;
    tot += xi;
    bel += i < g ? xi : 0u;
  }
  for (int c0 = kPre; c0 < G; c0 += 16) {
    uint32_t y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = c0 + i < G ? hrow[int64_t(c0 + i) * kBins + b] : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      tot += y[i];
      bel += c0 + i < g ? y[i] : 0u;
    }
  }
  uint32_t lo, hi;
  minmax_reduce(mn, mx, &lo, &hi, red);
  const Binner bin(lo, hi);
  // suffix sums from the top bin down: thread i takes bin 255 - i, in-wave scan, then earlier waves
  {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    static_assert(kBins == 64 * kW, "bins per wave");
    suffix[b] = tot;
    __syncthreads();
    uint32_t x = dsa::wave_incl_sum_u32(suffix[kBins - 1 - threadIdx.x]);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    for (int w = 0; w < wave; ++w) x += wsum[w];
    suffix[kBins - 1 - threadIdx.x] = x;
    __syncthreads();
  }
  {
    const uint32_t above = b + 1 < kBins ? suffix[b + 1] : 0u;
    if (above < uint32_t(topk) && suffix[b] >= uint32_t(topk)) s_bstar = b;
  }
  __syncthreads();
  const int bstar = s_bstar;
  const uint32_t n_above = bstar + 1 < kBins ? suffix[bstar + 1] : 0u;
  const uint32_t n_cand = suffix[bstar] - n_above;
  // this chunk's write offsets: winners and candidates of earlier chunks (block sums)
  const uint32_t wo = dsa::wave_sum_u32(b > bstar ? bel : 0u);
  const uint32_t co = dsa::wave_sum_u32(b == bstar ? bel : 0u);
  if ((threadIdx.x & 63) == 0) { wsum[threadIdx.x >> 6] = wo; red[threadIdx.x >> 6] = co; }
  __syncthreads();
  uint32_t woff = 0, coff = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) { woff += wsum[w]; coff += red[w]; }
  const bool keep_cand = n_cand <= uint32_t(kCap);
  uint64_t* buf = rowbuf + int64_t(t) * rowbuf_len;
  // which of this thread's scores are winners (above b*) and candidates (in b*), then each
  // thread's first slot from a block prefix scan of the counts: no atomics, the stores go out
  // back to back (the order inside the buffer does not matter to the final ordering)
  static_assert(kPerThread <= 32, "flags fit a word");
  uint32_t wmask = 0, cmask = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int j = g * kChunk + i * kThreads + threadIdx.x;
    const int bj = bin(v[i]);
    if (j < n && bj > bstar) wmask |= 1u << i;
    else if (j < n && bj == bstar && keep_cand) cmask |= 1u << i;
  }
  uint32_t wpre, cpre;
  {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t wi = dsa::wave_incl_sum_u32(__popc(wmask));
    const uint32_t ci = dsa::wave_incl_sum_u32(__popc(cmask));
    if (lane == 63) { s_wscan[wave] = wi; s_cscan[wave] = ci; }
    __syncthreads();
    wpre = wi - __popc(wmask);
    cpre = ci - __popc(cmask);
    for (int w = 0; w < wave; ++w) { wpre += s_wscan[w]; cpre += s_cscan[w]; }
  }
  uint64_t* wdst = buf + woff + wpre;
  uint64_t* cdst = buf + n_above + coff + cpre;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int j = g * kChunk + i * kThreads + threadIdx.x;
    const uint64_t c = composite(dsa::order_key(v[i]), j);
    if ((wmask >> i) & 1u) *wdst++ = c;
    if ((cmask >> i) & 1u) *cdst++ = c;
  }
  if (g == 0 && threadIdx.x == 0) {
    RowInfo ri;
    ri.b_star = bstar;
    ri.n_above = int(n_above);
    ri.n_cand = int(n_cand);
    ri.pad = 0;
    info[t] = ri;
  }
}

// ------------------------------------------------------------------ final
__device__ __forceinline__ int block_excl_scan(bool flag, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int in_wave = __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wave_sums[wave] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kFinalThreads / 64; ++w) {
    const int c = wave_sums[w];
    before += (w < wave) ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

// Descending bitonic sort of n (power of two) keys in LDS.
__device__ void bitonic_sort_desc(uint64_t* v, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += kFinalThreads) {
        const int lo = 2 * i - (i & (j - 1));
        const int hi = lo + j;
        const bool desc = (lo & k) == 0;
        const uint64_t a = v[lo], b = v[hi];
        if ((a < b) == desc) { v[lo] = b; v[hi] = a; }
      }
      __syncthreads();
    }
  }
}

// Sorts a[0..cnt) descending in place (LDS); tmp is LDS scratch of cnt entries and a has room
// for cap_pow2 entries. Counting sort on the top 32 bits (linear bins between the smallest and
// largest), then each element's exact rank inside its bin by direct comparison; a bitonic sort
// if some bin is too full for that.
__device__ void sort_desc(uint64_t* a, uint64_t* tmp, int cnt, int cap_pow2, uint32_t* bins,
                          uint32_t* red, int* flag) {
  // the keys' own range (a tight range keeps the bins sparse for the in-bin ranking below)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kFinalThreads / 64;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = threadIdx.x; i < cnt; i += kFinalThreads) {
    const uint32_t k = uint32_t(a[i] >> 32);
    mn = min(mn, k);
    mx = max(mx, k);
  }
  mn = dsa::wave_min_u32(mn);
  mx = dsa::wave_max_u32(mx);
  if (lane == 0) { red[wave] = mn; red[nw + wave] = mx; }
  for (int i = threadIdx.x; i < kSortBins; i += kFinalThreads) bins[i] = 0;
  if (threadIdx.x == 0) *flag = 0;
  __syncthreads();
  mn = red[0]; mx = red[nw];
  for (int i = 1; i < nw; ++i) { mn = min(mn, red[i]); mx = max(mx, red[nw + i]); }
  __syncthreads();
  // bin 0 holds the largest keys. Any binning that never puts a larger key in a later bin gives
  // the exact order (keys are then ranked inside their bin), so a float multiply serves; it is
  // clamped against rounding at the top of the range
  const float fscale = float(kSortBins) / (float(mx - mn) + 1.0f);
  auto binof = [&](uint64_t c) -> int {
    const float u = float(uint32_t(c >> 32) - mn);
    return kSortBins - 1 - min(int(u * fscale), kSortBins - 1);
  };
  for (int i = threadIdx.x; i < cnt; i += kFinalThreads) atomicAdd(&bins[binof(a[i])], 1u);
  __syncthreads();
  for (int i = threadIdx.x; i < kSortBins; i += kFinalThreads)
    if (bins[i] > uint32_t(kFixMax)) *flag = 1;
  __syncthreads();
  if (*flag) {
    for (int i = cnt + threadIdx.x; i < cap_pow2; i += kFinalThreads) a[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(a, cap_pow2);
    return;
  }
  // exclusive prefix of the bin counts (kSortBins / kFinalThreads bins per thread)
  {
    constexpr int per = kSortBins / kFinalThreads;
    uint32_t loc[per];
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) { loc[q] = bins[threadIdx.x * per + q]; sum += loc[q]; }
    const uint32_t x = dsa::wave_incl_sum_u32(sum);
    if (lane == 63) red[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += red[w];
    uint32_t run = before + x - sum;
#pragma unroll
    for (int q = 0; q < per; ++q) { bins[threadIdx.x * per + q] = run; run += loc[q]; }
  }
  __syncthreads();
  // scatter into bin slices (any order inside a slice); afterwards bins[b] is the end of bin b
  for (int i = threadIdx.x; i < cnt; i += kFinalThreads) {
    const uint64_t c = a[i];
    tmp[atomicAdd(&bins[binof(c)], 1u)] = c;
  }
  __syncthreads();
  // exact place inside each slice: the number of larger keys in the slice
  for (int i = threadIdx.x; i < cnt; i += kFinalThreads) {
    const uint64_t c = tmp[i];
    const int b = binof(c);
    const uint32_t start = b > 0 ? bins[b - 1] : 0u, end = bins[b];
    uint32_t rank = 0;
    for (uint32_t e = start; e < end; ++e) rank += tmp[e] > c ? 1u : 0u;
    a[start + rank] = c;
  }
  __syncthreads();
}

// Writes out[i] = the position of the i-th largest of the cnt keys a[0 .. cnt) (LDS) for i < topk,
// -1 past cnt. As sort_desc: a counting sort on the top 32 bits (kSortBins linear bins between the
// smallest and largest key), each key's place inside its bin by direct comparison, a bitonic sort
// when some bin holds more than kFixMax keys. Each thread keeps its KP keys in registers, so that
// every pass issues its LDS operations together, and the places go straight to out.
template <int KP>
__device__ void sort_to_sel(uint64_t* a, uint64_t* tmp, int cnt, int cap_pow2, uint32_t* bins,
                            uint32_t* red, int* flag, int32_t* __restrict__ out, int topk) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int nw = kFinalThreads / 64;
  uint64_t v[KP];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int i = threadIdx.x + kFinalThreads * k;
    v[k] = i < cnt ? a[i] : 0ull;
    if (i < cnt) {
      mn = min(mn, uint32_t(v[k] >> 32));
      mx = max(mx, uint32_t(v[k] >> 32));
    }
  }
  for (int i = threadIdx.x; i < kSortBins; i += kFinalThreads) bins[i] = 0;
  if (threadIdx.x == 0) *flag = 0;
  mn = dsa::wave_min_u32(mn);
  mx = dsa::wave_max_u32(mx);
  if (lane == 0) { red[wave] = mn; red[nw + wave] = mx; }
  dsa::lds_barrier();
  mn = red[0]; mx = red[nw];
#pragma unroll
  for (int w = 1; w < nw; ++w) { mn = min(mn, red[w]); mx = max(mx, red[nw + w]); }
  // bin 0 holds the largest keys (binning as sort_desc)
  const float fscale = float(kSortBins) / (float(mx - mn) + 1.0f);
  auto binof = [&](uint64_t c) -> uint32_t {
    const float u = float(uint32_t(c >> 32) - mn);
    return uint32_t(kSortBins - 1 - min(int(u * fscale), kSortBins - 1));
  };
  // arrival place of each key in its bin; a key past cnt adds 0 at a slot of its own thread
  uint32_t* own = reinterpret_cast<uint32_t*>(tmp);
  uint32_t b[KP], slot[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const bool valid = int(threadIdx.x) + kFinalThreads * k < cnt;
    b[k] = binof(v[k]);
    const uint32_t r = atomicAdd(valid ? &bins[b[k]] : &own[threadIdx.x], valid ? 1u : 0u);
    slot[k] = valid ? r : 0u;
  }
  dsa::lds_barrier();
  // exclusive prefix of the bin counts (kSortBins / kFinalThreads consecutive bins per thread)
  constexpr int per = kSortBins / kFinalThreads;
  uint32_t loc[per];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < per; ++q) { loc[q] = bins[threadIdx.x * per + q]; sum += loc[q]; }
  bool full = false;
#pragma unroll
  for (int q = 0; q < per; ++q) full |= loc[q] > uint32_t(kFixMax);
  if (full) *flag = 1;
  const uint32_t x = dsa::wave_incl_sum_u32(sum);
  if (lane == 63) red[wave] = x;   // red[0 .. nw) were last read before the barrier above
  dsa::lds_barrier();
  if (*flag) {
    // a bin too full for ranking by comparison: sort the whole buffer
    for (int i = cnt + threadIdx.x; i < cap_pow2; i += kFinalThreads) a[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(a, cap_pow2);
    for (int i = threadIdx.x; i < topk; i += kFinalThreads) out[i] = i < cnt ? comp_pos(a[i]) : -1;
    return;
  }
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < nw; ++w) before += w < wave ? red[w] : 0u;
  uint32_t run = before + x - sum;
#pragma unroll
  for (int q = 0; q < per; ++q) { bins[threadIdx.x * per + q] = run; run += loc[q]; }
  dsa::lds_barrier();
  // each key into its bin's slice, then its place there: the number of larger keys in the slice
  uint32_t start[KP], end[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    start[k] = bins[b[k]];
    end[k] = b[k] + 1 < uint32_t(kSortBins) ? bins[b[k] + 1] : uint32_t(cnt);
  }
#pragma unroll
  for (int k = 0; k < KP; ++k)
    if (int(threadIdx.x) + kFinalThreads * k < cnt) tmp[start[k] + slot[k]] = v[k];
  dsa::lds_barrier();
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    if (int(threadIdx.x) + kFinalThreads * k < cnt) {
      uint32_t rank = 0;
      for (uint32_t e = start[k]; e < end[k]; ++e) rank += tmp[e] > v[k] ? 1u : 0u;
      const uint32_t at = start[k] + rank;
      if (at < uint32_t(topk)) out[at] = comp_pos(v[k]);
    }
  }
  for (int i = cnt + threadIdx.x; i < topk; i += kFinalThreads) out[i] = -1;
}

// The topk largest keys of a whole row (n > topk scores), in any order, into a[0 .. topk): an exact
// radix select on the order keys, 8 bits a pass, then the keys above the threshold and the
// lowest positions among those equal to it. One workgroup of kFinalThreads.
__device__ void exact_topk_row(const float* __restrict__ row, int n, int topk, uint64_t* a,
                               uint32_t* bins, uint32_t* red, int* wave_sums, int* flag) {
  uint32_t prefix = 0, mask = 0;
  int remaining = topk;
  const int shifts[4] = {24, 16, 8, 0};
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = shifts[pass];
    for (int i = threadIdx.x; i < 256; i += kFinalThreads) bins[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += kFinalThreads) {
      const uint32_t k = dsa::order_key(row[j]);
      if ((k & mask) == prefix) atomicAdd(&bins[(k >> sh) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + bins[d] >= uint32_t(remaining)) break;
        above += bins[d];
      }
      red[0] = uint32_t(d);
      red[1] = above;
    }
    __syncthreads();
    remaining -= int(red[1]);
    prefix |= red[0] << sh;
    mask |= 0xFFu << sh;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;
  const int n_gt = topk - need_eq;
  if (threadIdx.x == 0) *flag = 0;
  __syncthreads();
  int eq_base = 0;
  for (int j0 = 0; j0 < n; j0 += kFinalThreads) {
    const int j = j0 + threadIdx.x;
    const uint32_t k = j < n ? dsa::order_key(row[j]) : 0u;
    const bool gt = j < n && k > T;
    const bool eq = j < n && k == T;
    if (gt) a[atomicAdd(flag, 1)] = composite(k, j);
    if (eq_base < need_eq) {
      int total;
      const int off = block_excl_scan(eq, wave_sums, &total);
      if (eq && eq_base + off < need_eq) a[n_gt + eq_base + off] = composite(k, j);
      eq_base += total;
    }
  }
}

__global__ void __launch_bounds__(kFinalThreads)
select_final(DevPlan p, const float* __restrict__ scores, int64_t ld, int topk,
             const uint64_t* __restrict__ rowbuf, int rowbuf_len, const RowInfo* __restrict__ info,
             int cap_pow2, int32_t* __restrict__ sel) {
  extern __shared__ uint64_t lds[];
  uint64_t* a = lds;                 // [cap_pow2]
  uint64_t* tmp = lds + cap_pow2;    // [cap_pow2]
  __shared__ uint32_t bins[kSortBins];
  __shared__ uint32_t red[2 * kFinalThreads / 64];
  __shared__ int wave_sums[kFinalThreads / 64];
  __shared__ int flag;
  const int t = blockIdx.x;
  const RowInfo ri = info[t];        // written by the collect step for rows longer than topk
  const int n = row_position(p, t) + 1;
  const float* row = scores + int64_t(t) * ld;
  int32_t* out = sel + int64_t(t) * topk;

  int cnt;
  if (n <= topk) {
    cnt = n;
    for (int i = threadIdx.x; i < n; i += kFinalThreads) a[i] = composite(dsa::order_key(row[i]), i);
  } else {
    if (ri.n_cand > kCap) {
      // massive ties at the threshold: exact radix select over the whole row
      exact_topk_row(row, n, topk, a, bins, red, wave_sums, &flag);
      cnt = topk;
    } else {
      cnt = ri.n_above + ri.n_cand;
      const uint64_t* buf = rowbuf + int64_t(t) * rowbuf_len;
      for (int i = threadIdx.x; i < cnt; i += kFinalThreads) a[i] = buf[i];
    }
  }
  __syncthreads();
  sort_desc(a, tmp, cnt, cap_pow2, bins, red, &flag);
  for (int i = threadIdx.x; i < topk; i += kFinalThreads) out[i] = i < cnt ? comp_pos(a[i]) : -1;
}

// ------------------------------------------------------------------ one launch over block lists
constexpr int kMaxBlocks = 64;     // blocks of a row the search takes (262144 keys); longer rows go exact
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One workgroup per row over the block counts and lists the score kernel wrote (ScoreHist): the
// bin b* where the count from the top reaches topk (a 16-way search over the 2048 bins below the
// row's highest), then the first (keys in bins >= b*) entries of every block's list, ordered
// exactly. The head of every list is requested with the counts, before b* is known. Rows of at
// most topk keys take every key. A row is selected exactly from its scores instead when b* lies
// more than 2047 bins below the highest, a folded
// block's counts are not exact at b*, a block has more keys at or above b* than it listed, bin b*
// holds more keys than the candidate buffer takes, or the row has more than kMaxBlocks blocks.
__global__ void __launch_bounds__(kFinalThreads)
select_lists(DevPlan p, const float* __restrict__ scores, int64_t ld, int topk, ScoreHist hs,
             int cand_len, int cap_pow2, int ge_pitch, int32_t* __restrict__ sel) {
  constexpr int kB = ScoreHist::kBlock, kWin = ScoreHist::kWin;
  constexpr int kNW = kFinalThreads / 64;                 // waves
  constexpr int kPerWave = kMaxBlocks / kNW;              // blocks whose list head a wave loads
  constexpr int kHead = 2;                                // list entries per lane loaded up front
  static_assert(kSortBins % kFinalThreads == 0, "whole bins per thread");
  static_assert(kMaxBlocks * kWin / 8 % kFinalThreads == 0, "whole 16-byte count pieces per thread");
  static_assert(kMaxBlocks == 64, "one block per lane of a wave");
  // phase 1: [gm][ge_pitch] suffix counts; phase 2: [cap_pow2] keys, [cap_pow2] scratch, bins
  extern __shared__ uint64_t lds[];
  uint16_t* ge = reinterpret_cast<uint16_t*>(lds);
  __shared__ uint32_t red[2 * kNW];
  __shared__ int wave_sums[kNW];
  __shared__ int flag;
  __shared__ uint32_t s_lo[kMaxBlocks], s_hi[kMaxBlocks], s_len[kMaxBlocks], s_off[kMaxBlocks];
  __shared__ uint32_t s_hb, s_bits[3], s_total, s_exact;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // ---- every load at once: the row's span (first, so that its lookup waits for it alone), each
  // block's range (first wave), the blocks' counts (the row's gm x 2 KB run in 16-byte pieces,
  // consecutive pieces on consecutive threads), the heads of the wave's blocks' lists
  const dsa_span span0 = dsa::span_chunk(p.spans, p.n_spans, 0);
  asm volatile("" ::: "memory");
  const int gm = min(hs.g_max, kMaxBlocks);
  constexpr int kPieces = kWin / 8;                       // 16-byte pieces of one block's counts
  const int n_pieces = gm * kPieces;
  // Every load below is unconditional (an index past the row's blocks reads its last block and
  // the value is then dropped): on every path the same loads follow the span's, so the wait for
  // the span counts exactly them and does not wait for them.
  const uint4 rng_ld = hs.range[int64_t(t) * hs.g_max + min(int(threadIdx.x), gm - 1)];
  const uint4 rng = int(threadIdx.x) < gm ? rng_ld : make_uint4(1u, 0u, 0u, 0u);
  const u32x4_t* crow = reinterpret_cast<const u32x4_t*>(hs.counts + int64_t(t) * hs.g_max * kWin);
  u32x4_t cw[kMaxBlocks * kPieces / kFinalThreads];
#pragma unroll
  for (int i = 0; i < kMaxBlocks * kPieces / kFinalThreads; ++i) {
    const int q = kFinalThreads * i + int(threadIdx.x);
    const u32x4_t v = crow[min(q, n_pieces - 1)];
    cw[i] = q < n_pieces ? v : u32x4_t{0u, 0u, 0u, 0u};
  }
  const uint64_t* lists = hs.lists + int64_t(t) * hs.g_max * kB;
  uint64_t head[kPerWave][kHead];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j)
#pragma unroll
    for (int r = 0; r < kHead; ++r) {
      const int gb = wave + kNW * j;
      const uint64_t v = lists[int64_t(min(gb, gm - 1)) * kB + lane + 64 * r];
      head[j][r] = gb < gm ? v : 0ull;
    }
  const int n = row_position_from(span0, p, t) + 1;
  const int G = (n + kB - 1) / kB;
  if (threadIdx.x < kMaxBlocks) {
    s_lo[threadIdx.x] = rng.x;
    s_hi[threadIdx.x] = rng.y;
  }
  if (threadIdx.x < 3) s_bits[threadIdx.x] = 0u;
  if (wave == 0) {
    const uint32_t hb = dsa::wave_max_u32(lane < G ? rng.y : 0u);
    if (lane == 0) s_hb = hb;
  }

  if (n <= topk || G > kMaxBlocks) {
    // every block listed all its keys (or the row goes exact)
    if (wave == 0) {
      const uint32_t keys = lane < G ? uint32_t(min(kB, n - kB * lane)) : 0u;
      const bool short_list = __builtin_amdgcn_ballot_w64(lane < G && rng.z != keys) != 0ull;
      s_len[lane] = keys;
      if (lane == 0) {
        s_total = uint32_t(n);
        s_exact = n > topk || short_list ? 1u : 0u;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kMaxBlocks * kPieces / kFinalThreads; ++i) {
      const int q = kFinalThreads * i + int(threadIdx.x);
      if (q < n_pieces) *reinterpret_cast<u32x4_t*>(&ge[(q / kPieces) * ge_pitch + 8 * (q % kPieces)]) = cw[i];
    }
    dsa::lds_barrier();   // the list heads stay in flight
    // f(i): the row's count in bins >= hb - i reaches topk (lane g of a wave sums block g; folded
    // keys make a window's lowest bin a lower bound). f is monotone in i; its first true i over
    // [0, 2048) is narrowed in three rounds in which the 16 waves test the ends of 16 chunks of
    // 128, then 8, then 1 offsets. Offsets past hb (bins below 0) count every key: true.
    const uint32_t hb = s_hb;
    const bool mine = lane < G;
    const uint32_t lo = (mine ? s_lo[lane] : 1u) & 0x7FFFFFFFu, hi = mine ? s_hi[lane] : 0u;
    auto cnt_ge = [&](uint32_t b) -> uint32_t {
      if (!mine || b > hi) return 0u;
      return ge[lane * ge_pitch + (b <= lo ? 0u : b - lo)];
    };
    uint32_t base = 0u;
    bool found = true;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const uint32_t width = r == 0 ? 128u : (r == 1 ? 8u : 1u);
      const uint32_t i = base + width * uint32_t(wave + 1) - 1u;
      const bool ok = i > hb || dsa::wave_sum_u32(cnt_ge(hb - i)) >= uint32_t(topk);
      if (lane == 0 && ok) atomicOr(&s_bits[r], 1u << wave);
      dsa::lds_barrier();
      const uint32_t m = s_bits[r];
      if (m == 0u) { found = false; break; }   // only in the first round: f(2047) is false
      base += width * uint32_t(__builtin_ctz(m));
    }
    if (wave == 0) {
      // lane g: block g's keys in bins >= b*
      const uint32_t bstar = hb - base;
      const bool fold = (rng.x & 0x80000000u) != 0u;
      const uint32_t sv = found ? cnt_ge(bstar) : 0u;
      const uint32_t total = dsa::wave_sum_u32(sv);
      const bool bad = !found ||
                       __builtin_amdgcn_ballot_w64(mine && ((fold && lo >= bstar) || sv > rng.z)) != 0ull;
      s_len[lane] = sv;
      if (lane == 0) {
        s_total = total;
        s_exact = bad || total > uint32_t(cand_len) ? 1u : 0u;
      }
    }
  }
  __syncthreads();
  const bool exact = s_exact != 0u;
  uint64_t* a = lds;
  uint64_t* tmp = lds + cap_pow2;
  uint32_t* bins = reinterpret_cast<uint32_t*>(lds + 2 * cap_pow2);
  int cnt;
  if (!exact) {
    if (wave == 0) {
      const uint32_t v = lane < G ? s_len[lane] : 0u;
      s_off[lane] = dsa::wave_incl_sum_u32(v) - v;
    }
    __syncthreads();
    cnt = int(s_total);
    // each wave copies its blocks' shares: the loaded heads, then the rest of longer shares
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int g = wave + kNW * j;
      if (g < G) {
        const int len = int(s_len[g]), off = int(s_off[g]);
#pragma unroll
        for (int r = 0; r < kHead; ++r)
          if (lane + 64 * r < len) a[off + lane + 64 * r] = head[j][r];
        for (int e = 64 * kHead + lane; e < len; e += 64) a[off + e] = lists[int64_t(g) * kB + e];
      }
    }
  } else {
    exact_topk_row(scores + int64_t(t) * ld, n, topk, a, bins, red, wave_sums, &flag);
    cnt = topk;
  }
  __syncthreads();
  int32_t* out = sel + int64_t(t) * topk;
  // registers for the keys there are (cnt <= cap_pow2 <= 8 * kFinalThreads)
  if (cnt <= 2 * kFinalThreads)
    sort_to_sel<2>(a, tmp, cnt, cap_pow2, bins, red, &flag, out, topk);
  else if (cnt <= 4 * kFinalThreads)
    sort_to_sel<4>(a, tmp, cnt, cap_pow2, bins, red, &flag, out, topk);
  else
    sort_to_sel<8>(a, tmp, cnt, cap_pow2, bins, red, &flag, out, topk);
}

int pow2_at_least(int n) {
  int v = 1;
  while (v < n) v <<= 1;
  return v;
}

struct SelectLayout {
  int nb_max, g_max, rowbuf_len, cap_pow2;
  size_t off_mm, off_hist, off_rowbuf, off_info;
  // one-launch path (rows scored one per workgroup): block counts, ranges and key lists
  int fg_max, cand_len, cand_pow2;
  size_t off_fcounts, off_frange, off_lists, total;
};

// lists: the workspace holds the one-launch path's block lists (select_lists_used)
SelectLayout layout(const dsa_handle* h, const PlanInfo& in, bool lists) {
  SelectLayout L;
  const int topk = h->cfg.topk;
  L.nb_max = (in.max_visible + kMinMaxBlock - 1) / kMinMaxBlock;
  L.g_max = (in.max_visible + kChunk - 1) / kChunk;
  L.rowbuf_len = topk + kCap;
  L.cap_pow2 = pow2_at_least(topk + kCap);
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t T = size_t(in.n_rows);
  L.off_mm = 0;
  L.off_hist = al(L.off_mm + T * L.nb_max * 8);
  L.off_rowbuf = al(L.off_hist + T * L.g_max * kBins * 4);
  L.off_info = al(L.off_rowbuf + T * L.rowbuf_len * 8);
  L.fg_max = (in.max_visible + ScoreHist::kBlock - 1) / ScoreHist::kBlock;
  L.cand_len = topk + kCap;
  L.cand_pow2 = pow2_at_least(L.cand_len);
  L.off_fcounts = al(L.off_info + T * sizeof(RowInfo));
  L.off_frange = al(L.off_fcounts + T * L.fg_max * ScoreHist::kWin * 2);
  L.off_lists = al(L.off_frange + T * L.fg_max * sizeof(uint4));
  L.total = al(L.off_lists + (lists ? T * L.fg_max * ScoreHist::kBlock * 8 : 0));
  return L;
}

}  // namespace

int select_minmax_block() { return kMinMaxBlock; }

bool index_mfma_supported(const dsa_config& c);

// dsa_index_topk takes the one-launch select when every row is scored one per workgroup by the
// matrix-core score kernel (no span long enough to be scored in row groups).
bool select_lists_used(const dsa_handle* h, const PlanInfo& in) {
  return index_mfma_supported(h->cfg) && in.max_q_len < RowGroups::kMinQLen;
}

size_t select_workspace_bytes(const dsa_handle* h, const PlanInfo& in, bool lists) {
  return layout(h, in, lists).total;
}

uint32_t* select_minmax_buffer(const dsa_handle* h, const PlanInfo& in, void* ws, int* nb_max) {
  const SelectLayout L = layout(h, in, false);
  *nb_max = L.nb_max;
  return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.off_mm);
}

// have_minmax: the score producer already wrote the per-block min/max into the workspace.
hipError_t launch_select_topk_ex(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                                 const float* scores, int64_t ld, int32_t* sel, void* ws,
                                 bool have_minmax, hipStream_t st) {
  const SelectLayout L = layout(h, in, false);
  char* base = static_cast<char*>(ws);
  uint32_t* mm = reinterpret_cast<uint32_t*>(base + L.off_mm);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.off_hist);
  uint64_t* rowbuf = reinterpret_cast<uint64_t*>(base + L.off_rowbuf);
  RowInfo* info = reinterpret_cast<RowInfo*>(base + L.off_info);
  const int topk = h->cfg.topk;
  const unsigned T = unsigned(in.n_rows);
  if (in.max_visible > topk) {
    if (!have_minmax)
      hipLaunchKernelGGL(select_minmax, dim3(L.nb_max, T), dim3(kThreads), 0, st, p, scores, ld, mm,
                         L.nb_max);
    hipLaunchKernelGGL(select_hist, dim3(L.g_max, T), dim3(kThreads), 0, st, p, scores, ld, topk, mm,
                       L.nb_max, hist, L.g_max);
    hipLaunchKernelGGL(select_collect, dim3(L.g_max, T), dim3(kThreads), 0, st, p, scores, ld, topk,
                       mm, L.nb_max, hist, L.g_max, rowbuf, L.rowbuf_len, info);
  }
  const size_t lds = size_t(L.cap_pow2) * 8 * 2;
  hipLaunchKernelGGL(select_final, dim3(T), dim3(kFinalThreads), lds, st, p, scores, ld, topk, rowbuf,
                     L.rowbuf_len, info, L.cap_pow2, sel);
  return hipGetLastError();
}

hipError_t launch_select_topk(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                              const float* scores, int64_t ld, int32_t* sel, void* ws, hipStream_t st) {
  return launch_select_topk_ex(h, p, in, scores, ld, sel, ws, false, st);
}

ScoreHist select_hist_buffers(const dsa_handle* h, const PlanInfo& in, void* ws) {
  const SelectLayout L = layout(h, in, true);
  char* base = static_cast<char*>(ws);
  ScoreHist hs;
  hs.counts = reinterpret_cast<uint16_t*>(base + L.off_fcounts);
  hs.range = reinterpret_cast<uint4*>(base + L.off_frange);
  hs.lists = reinterpret_cast<uint64_t*>(base + L.off_lists);
  hs.g_max = L.fg_max;
  hs.topk = h->cfg.topk;
  return hs;
}

// The select over the block counts and lists (and, for rows that need them, the scores) the
// score kernel wrote into ws: one launch.
hipError_t launch_select_lists(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                               const float* scores, int64_t ld, int32_t* sel, void* ws,
                               hipStream_t st) {
  const SelectLayout L = layout(h, in, true);
  const ScoreHist hs = select_hist_buffers(h, in, ws);
  const int ge_pitch = ScoreHist::kWin + 8;   // a block's counts, then 16 bytes to the next bank group
  const size_t ge_bytes = size_t(min(L.fg_max, kMaxBlocks)) * ge_pitch * 2;
  const size_t sort_bytes = size_t(L.cand_pow2) * 8 * 2 + kSortBins * 4;
  const size_t lds = ge_bytes > sort_bytes ? ge_bytes : sort_bytes;
  hipLaunchKernelGGL(select_lists, dim3(unsigned(in.n_rows)), dim3(kFinalThreads), lds, st, p,
                     scores, ld, h->cfg.topk, hs, L.cand_len, L.cand_pow2, ge_pitch, sel);
  return hipGetLastError();
}
