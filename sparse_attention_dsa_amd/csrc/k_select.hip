// Causal top-k select (DSA resource page: select_topk_causal, index_topk).
// Row t sees scores[t][0 .. position]. It keeps the topk positions of highest score, equal scores
// going to the lower position, and writes them by score descending / position ascending followed
// by -1 entries (a contiguous tail, as ttnn.transformer.sparse_sdpa lays out masked indices).
//
// One workgroup of 1024 threads per row:
//   1. radix select on the 32-bit order key of the score (digits of 11, 11 and 10 bits, LDS
//      histograms) finds the topk-th largest key T and how many keys equal to T are kept;
//   2. one ordered pass collects keys above T and the first such keys equal to T by position;
//   3. a bitonic sort in LDS on (key << 32 | ~position) puts the winners in canonical order.
// Because every composite key is unique, the result is the same for any thread schedule.
#include "dsa_internal.hpp"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

__device__ __forceinline__ uint64_t composite(uint32_t key, int j) {
  return (uint64_t(key) << 32) | uint32_t(~uint32_t(j));
}

// Descending bitonic sort of n (power of two) 64-bit keys in LDS.
__device__ void bitonic_sort_desc(uint64_t* v, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += kThreads) {
        int lo = 2 * i - (i & (j - 1));
        int hi = lo + j;
        bool desc = (lo & k) == 0;
        uint64_t a = v[lo], b = v[hi];
        if ((a < b) == desc) { v[lo] = b; v[hi] = a; }
      }
      __syncthreads();
    }
  }
}

// Exclusive prefix over the block of a per-thread 0/1 flag; returns the thread's offset and
// writes the block total. Uses one LDS slot per wave.
__device__ __forceinline__ int block_excl_scan(bool flag, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t m = __ballot(flag);
  int in_wave = __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wave_sums[wave] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kWaves; ++w) {
    int c = wave_sums[w];
    before += (w < wave) ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

__global__ void __launch_bounds__(kThreads)
select_topk_rows(DevPlan p, const float* __restrict__ scores, int64_t ld, int topk, int sort_n,
                 int32_t* __restrict__ sel) {
  extern __shared__ uint64_t sort_buf[];              // [sort_n]
  __shared__ uint32_t hist[kBins];
  __shared__ int wave_sums[kWaves];
  __shared__ uint32_t scan_buf[kThreads];
  __shared__ int s_digit, s_above, s_gt_count;

  const int t = blockIdx.x;
  const int s = dsa::find_span(p.spans, p.n_spans, t);
  const dsa_span sp = p.spans[s];
  const int pos = sp.ctx_start + (t - sp.q_start);
  const int n = pos + 1;
  const float* row = scores + int64_t(t) * ld;
  int32_t* out = sel + int64_t(t) * topk;

  if (n <= topk) {
    // Every visible key is kept; only the order is computed.
    for (int i = threadIdx.x; i < sort_n; i += kThreads)
      sort_buf[i] = i < n ? composite(dsa::order_key(row[i]), i) : 0ull;
    __syncthreads();
    bitonic_sort_desc(sort_buf, sort_n);
    for (int i = threadIdx.x; i < topk; i += kThreads)
      out[i] = i < n ? int32_t(~uint32_t(sort_buf[i] & 0xFFFFFFFFu)) : -1;
    return;
  }

  // ---- 1. radix select of the topk-th largest order key
  uint32_t prefix = 0, mask = 0;
  int remaining = topk;  // keys still to take at or below the current prefix
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += kThreads) {
      uint32_t k = dsa::order_key(row[j]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> sh) & dmask], 1u);
    }
    __syncthreads();
    // Find the digit where the count from the top reaches `remaining`. Each thread owns two
    // bins counted from the top; a block scan of their sums gives the count above each bin.
    const int nb = int(dmask) + 1;
    const int b_hi = nb - 1 - 2 * int(threadIdx.x);  // this thread's first bin (from the top)
    uint32_t c0 = b_hi >= 0 ? hist[b_hi] : 0u;
    uint32_t c1 = b_hi - 1 >= 0 ? hist[b_hi - 1] : 0u;
    uint32_t mine = c0 + c1;
    // inclusive scan of `mine` over threads, in thread order (= descending bins)
    scan_buf[threadIdx.x] = mine;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
      uint32_t v = threadIdx.x >= unsigned(d) ? scan_buf[threadIdx.x - d] : 0u;
      __syncthreads();
      scan_buf[threadIdx.x] += v;
      __syncthreads();
    }
    uint32_t above = scan_buf[threadIdx.x] - mine;  // keys in bins higher than b_hi
    if (b_hi >= 0) {
      if (above < uint32_t(remaining) && above + c0 >= uint32_t(remaining)) {
        s_digit = b_hi; s_above = int(above);
      } else if (b_hi - 1 >= 0 && above + c0 < uint32_t(remaining) &&
                 above + c0 + c1 >= uint32_t(remaining)) {
        s_digit = b_hi - 1; s_above = int(above + c0);
      }
    }
    __syncthreads();
    remaining -= s_above;
    prefix |= uint32_t(s_digit) << sh;
    mask |= dmask << sh;
    __syncthreads();
  }
  const uint32_t T = prefix;     // the topk-th largest key
  const int need_eq = remaining; // keys equal to T that are kept (the lowest positions)
  const int n_gt = topk - need_eq;

  // ---- 2. ordered collection: every key above T (any slot order) and the first need_eq keys
  // equal to T by position (block scan in position order)
  if (threadIdx.x == 0) s_gt_count = 0;
  __syncthreads();
  int eq_base = 0;  // uniform across the block
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    const int j = j0 + threadIdx.x;
    const uint32_t k = j < n ? dsa::order_key(row[j]) : 0u;
    const bool gt = j < n && k > T;
    const bool eq = j < n && k == T;
    if (gt) sort_buf[atomicAdd(&s_gt_count, 1)] = composite(k, j);
    if (eq_base < need_eq) {
      int total;
      const int off = block_excl_scan(eq, wave_sums, &total);
      if (eq && eq_base + off < need_eq) sort_buf[n_gt + eq_base + off] = composite(k, j);
      eq_base += total;
    }
  }
  for (int i = topk + threadIdx.x; i < sort_n; i += kThreads) sort_buf[i] = 0ull;
  __syncthreads();

  // ---- 3. canonical order
  bitonic_sort_desc(sort_buf, sort_n);
  for (int i = threadIdx.x; i < topk; i += kThreads)
    out[i] = int32_t(~uint32_t(sort_buf[i] & 0xFFFFFFFFu));
}

int pow2_at_least(int n) {
  int v = 1;
  while (v < n) v <<= 1;
  return v;
}

}  // namespace

size_t select_workspace_bytes(const dsa_handle*, const PlanInfo&) { return 0; }

hipError_t launch_select_topk(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                              const float* scores, int64_t ld, int32_t* sel, void*, hipStream_t st) {
  const int topk = h->cfg.topk;
  const int sort_n = pow2_at_least(topk);
  hipLaunchKernelGGL(select_topk_rows, dim3(in.n_rows), dim3(kThreads), size_t(sort_n) * 8, st, p,
                     scores, ld, topk, sort_n, sel);
  return hipGetLastError();
}
