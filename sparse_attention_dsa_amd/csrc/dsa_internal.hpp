// Internal declarations shared by the host API and the kernel translation units of libdsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

struct dsa_handle {
  dsa_config cfg;
  int64_t index_page_bytes;  // bytes of one index-key page
  int64_t latent_row_bytes;  // bytes of one latent token row
};

// Block-sparse MSA: its index side is a DSA handle (the score kernels and plan checks).
struct dsa_msa_handle {
  dsa_msa_config cfg;
  dsa_handle idx;
  int64_t gqa_row_bytes;     // bytes of one token's K and V row
};

// What host validation learns about a plan; handed to the launchers.
struct PlanInfo {
  int32_t n_rows;
  int32_t n_spans;
  int32_t max_visible;     // max over rows of position + 1
  int32_t max_q_len;       // longest span
  int64_t total_visible;   // sum over rows of position + 1
  bool all_decode;         // every span has q_len == 1
  const dsa_span* spans_host;   // the caller's host copy of the spans (valid during the call)
};

// Device view of a plan, passed by value to kernels.
struct DevPlan {
  const dsa_span* spans;
  const int32_t* page_table;
  int32_t n_spans;
  int32_t n_rows;
  int32_t pool_pages;
  int32_t page_size;
};

// Keys per block of the matrix-core score kernel; the select reads one min / max pair per block.
constexpr int kScoreBlock = 2048;

// What the one-row score kernel writes for the select beside the scores: per row and 4096-key
// block, over the fixed bins of the top 16 bits of the order keys (128 bins per octave) in a
// window of at most kWin bins ending at the block's highest bin,
//  - for each bin b, the number of the block's keys in bins >= b (keys below the window are
//    counted in its lowest bin, which is then flagged);
//  - the block's top keys as composites (order key << 32 | ~position), highest bins first (any
//    order inside a bin), from the highest bin down to the bin c where the count reaches
//    list_len(n) (every key when the block has fewer). A row's select reads each block's keys in
//    the bins at or above the row's topk-th bin from these lists, and the scores instead when a
//    block holds more of them than its list.
struct ScoreHist {
  static constexpr int kBlock = 4096;   // keys per block (one score workgroup)
  static constexpr int kWin = 1024;
  uint16_t* counts;     // [n_rows][g_max][kWin]: entry i of a block is its keys in bins >= lowest + i
  uint4* range;         // [n_rows][g_max]: (lowest bin | 1 << 31 if keys were folded into it,
                        //  highest bin, keys in the list, 0)
  uint64_t* lists;      // [n_rows][g_max][kBlock] composites, highest bins first
  int g_max;            // blocks per row
  int topk;
  // keys listed per block of a row of n keys: four times a block's even share of topk, at least
  // 1024, at most the block
  __host__ __device__ int list_len(int n) const {
    const int g = (n + kBlock - 1) / kBlock;
    const int share = 4 * ((topk + g - 1) / g);
    return share < 1024 ? 1024 : (share > kBlock ? kBlock : share);
  }
};

// Split of a plan's rows between the two matrix-core score kernels. Groups of kRows consecutive
// rows of one long span share every key tile (RowGroups); the other rows are scored one per
// workgroup, reached through a map from the launch index to the step row (RowMap). Both travel
// by value in the kernel arguments.
struct RowGroups {
  static constexpr int kMaxSpans = 32;
  static constexpr int kRows = 8;       // rows per group
  static constexpr int kMinQLen = 8;    // shortest span that is grouped
  int32_t n_spans;                      // grouped spans
  int32_t span[kMaxSpans];              // their indices in the plan
  int32_t first[kMaxSpans + 1];         // first group of each; first[n_spans] = total groups
};
struct RowMap {
  static constexpr int kMax = RowGroups::kMaxSpans + 1;
  int32_t n;                            // ranges of consecutive rows
  int32_t start[kMax];                  // first step row of each range
  int32_t first[kMax + 1];              // launch index of each range's first row; first[n] = total
};
// Fills both from the host spans; every row lands in exactly one of them.
void split_rows(const PlanInfo& in, RowGroups* g, RowMap* m);

namespace dsa {

// ---------------------------------------------------------------- device helpers

// Span holding step row t (spans are contiguous and ordered by q_start) and its index: the
// number of spans starting at or before t, minus one. Each lane of the wave loads one whole span,
// so a plan of up to 64 spans costs one memory round trip instead of a search's chain of
// dependent loads; the wave then reads the answer out of the lane that loaded it. Every lane
// gets the result; t must be the same across the wave.
//
// span_chunk loads the lane's span of the 64 starting at base. row_span_from takes the first
// chunk already loaded, so that a kernel can request it together with its other first loads:
// the lookup then waits for that one load, not for every load issued before it (a loop around
// the first load would wait for all of them at its head).
__device__ __forceinline__ dsa_span span_chunk(const dsa_span* spans, int n_spans, int base) {
  const int i = base + (threadIdx.x & 63);
  dsa_span s{};
  if (i < n_spans) s = spans[i];
  return s;
}
__device__ __forceinline__ int row_span_from(const dsa_span& first, const dsa_span* spans,
                                             int n_spans, int t, dsa_span* out) {
  const int lane = threadIdx.x & 63;
  int count = 0;
  dsa_span got{};
  // the spans of one chunk starting at or before t; the answer is the last of them
  auto take = [&](const dsa_span& mine, int base) {
    const int c = __popcll(__ballot(base + lane < n_spans && mine.q_start <= t));
    count += c;
    if (c > 0) {
      got.q_start = __builtin_amdgcn_readlane(mine.q_start, c - 1);
      got.q_len = __builtin_amdgcn_readlane(mine.q_len, c - 1);
      got.ctx_start = __builtin_amdgcn_readlane(mine.ctx_start, c - 1);
      got.page_offset = __builtin_amdgcn_readlane(mine.page_offset, c - 1);
      got.n_pages = __builtin_amdgcn_readlane(mine.n_pages, c - 1);
      got.page_start = __builtin_amdgcn_readlane(mine.page_start, c - 1);
    }
    return c;
  };
  // a full chunk means the answer may lie in a later one
  if (take(first, 0) == 64) {
    for (int base = 64; base < n_spans; base += 64) {
      const dsa_span mine = span_chunk(spans, n_spans, base);
      // every field waited for here, so that no load of this rare path is still counted as
      // outstanding where it joins the common one (that would put a wait for every load there)
      asm volatile("" :: "v"(mine.q_start), "v"(mine.q_len), "v"(mine.ctx_start),
                   "v"(mine.page_offset), "v"(mine.n_pages), "v"(mine.page_start));
      if (take(mine, base) < 64) break;
    }
  }
  *out = got;
  return count - 1;
}
__device__ __forceinline__ int row_span(const dsa_span* spans, int n_spans, int t, dsa_span* out) {
  return row_span_from(span_chunk(spans, n_spans, 0), spans, n_spans, t, out);
}

// Entry of a span's page list holding slot `list`, kept inside the list: a position the host
// did not check (one moved forward on the device after a captured launch) stays in the table.
__device__ __forceinline__ int page_entry(const dsa_span& s, int list) {
  return s.page_offset + min(max(list, 0), s.n_pages - 1);
}

// Pool page of request-local position j; clamped into the span's page list and into the pool,
// so that neither a page id nor a position the host did not check can address memory outside
// them.
__device__ __forceinline__ int page_of(const DevPlan& p, const dsa_span& s, int j, int* off) {
  int slot = s.page_start + j;
  int list = slot / p.page_size;
  *off = slot - list * p.page_size;
  int pg = p.page_table[page_entry(s, list)];
  pg = pg < 0 ? 0 : pg;
  return pg >= p.pool_pages ? p.pool_pages - 1 : pg;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even float -> bf16 bits (finite inputs), with gfx950's converter
// (v_cvt_pk_bf16_f32, which the compiler pairs: two results an instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// OCP e4m3fn byte -> float with the gfx950 converter.
__device__ __forceinline__ float fp8_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(int(byte), 0);
}

// float -> OCP e4m3fn byte, rounded to nearest even and saturated at +-448 (finite inputs).
// Normal results keep the top 3 mantissa bits of the float with its exponent rebiased from 127
// to 7; below 2^-6 the result is the nearest multiple of 2^-9 (the subnormal step).
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  uint32_t code;
  if (a >= 0x1p-6f) {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    code = (u >> 20) - (120u << 3);
    code = code > 0x7Eu ? 0x7Eu : code;
  } else {
    code = uint32_t(__builtin_rintf(a * 512.0f));
  }
  return sign | code;
}

// Wave-wide (64-lane) max, min and inclusive prefix sum on the DPP lane network: shifts by 1, 2,
// 4 and 8 lanes within each 16-lane row, then the broadcasts of lanes 15 and 31 into the rows
// after them (rows 1 and 3, then rows 2 and 3). Six dependent VALU steps instead of a chain of
// LDS permutes. Lanes a step has no source for add 0, which is the identity of both the sum and
// the unsigned max, so the results do not depend on how those lanes are filled.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_zero_fill(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_zero_fill<0x111, 0xF>(x));   // row_shr:1
  x = max(x, dpp_zero_fill<0x112, 0xF>(x));   // row_shr:2
  x = max(x, dpp_zero_fill<0x114, 0xF>(x));   // row_shr:4
  x = max(x, dpp_zero_fill<0x118, 0xF>(x));   // row_shr:8
  x = max(x, dpp_zero_fill<0x142, 0xA>(x));   // row_bcast:15
  x = max(x, dpp_zero_fill<0x143, 0xC>(x));   // row_bcast:31
  return uint32_t(__builtin_amdgcn_readlane(int(x), 63));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }
// lane i gets the sum over lanes 0 .. i
__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t x) {
  x += dpp_zero_fill<0x111, 0xF>(x);
  x += dpp_zero_fill<0x112, 0xF>(x);
  x += dpp_zero_fill<0x114, 0xF>(x);
  x += dpp_zero_fill<0x118, 0xF>(x);
  x += dpp_zero_fill<0x142, 0xA>(x);
  x += dpp_zero_fill<0x143, 0xC>(x);
  return x;
}
// Workgroup barrier for LDS traffic: each wave's LDS operations complete before it, and none
// after it is moved above. Unlike __syncthreads it does not wait for the wave's outstanding
// global loads and stores, which nothing on the other side of such a barrier reads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_readlane(int(wave_incl_sum_u32(x)), 63));
}

// Largest value over each group of G consecutive lanes (G = 8, 16, 32 or 64), left in the
// group's last lane: shifts within 16-lane rows, then the broadcasts across rows.
template <int G>
__device__ __forceinline__ uint32_t group_max_last(uint32_t x) {
  x = max(x, dpp_zero_fill<0x111, 0xF>(x));
  x = max(x, dpp_zero_fill<0x112, 0xF>(x));
  x = max(x, dpp_zero_fill<0x114, 0xF>(x));
  if constexpr (G >= 16) x = max(x, dpp_zero_fill<0x118, 0xF>(x));
  if constexpr (G >= 32) x = max(x, dpp_zero_fill<0x142, 0xA>(x));
  if constexpr (G >= 64) x = max(x, dpp_zero_fill<0x143, 0xC>(x));
  return x;
}

// Score -> unsigned key whose order is the score order; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace dsa

// ---------------------------------------------------------------- launchers (host)

hipError_t launch_store_keys(const dsa_handle* h, const DevPlan& p, const void* keys,
                             const float* scales, void* key_pool, hipStream_t st);

hipError_t launch_index_scores(const dsa_handle* h, const DevPlan& p, const PlanInfo& info,
                               const void* q, const float* w, const void* key_pool, float* scores,
                               int64_t ld, bool fill_masked, hipStream_t st);

hipError_t launch_index_topk(const dsa_handle* h, const DevPlan& p, const PlanInfo& info,
                             const void* q, const float* w, const void* key_pool, int32_t* sel,
                             float* scores, int64_t ld, void* ws_select, hipStream_t st);

// lists: the one-launch select's block lists are part of the workspace (select_lists_used)
size_t select_workspace_bytes(const dsa_handle* h, const PlanInfo& info, bool lists);
bool select_lists_used(const dsa_handle* h, const PlanInfo& info);
// dsa_index_topk's workspace: the score matrix, then the select's buffers
size_t index_topk_workspace_bytes(const dsa_handle* h, const PlanInfo& info, size_t* scores_part);
hipError_t launch_select_topk(const dsa_handle* h, const DevPlan& p, const PlanInfo& info,
                              const float* scores, int64_t ld, int32_t* sel, void* ws,
                              hipStream_t st);

size_t attend_workspace_bytes(const dsa_handle* h, const PlanInfo& info);
// sink: [H] fp32 device array or NULL (no sink)
hipError_t launch_attend(const dsa_handle* h, const DevPlan& p, const PlanInfo& info,
                         const int32_t* sel, const void* q_nope, const void* q_pe,
                         const void* latent_pool, float sm_scale, const float* sink, void* out,
                         void* ws, hipStream_t st);

// once per handle: lets the attention kernel take its dynamic LDS (above 64 KB for large tiles)
hipError_t msa_prepare(const dsa_msa_config& c);
size_t msa_block_keys_ld(const dsa_msa_config& c, const PlanInfo& info);
size_t msa_attend_lds_bytes(const dsa_msa_config& c);
size_t msa_attend_workspace_bytes(const dsa_msa_config& c, const PlanInfo& info);
// keys: [n_rows][msa_block_keys_ld] uint64 scratch for the block keys
hipError_t launch_msa_block_topk(const dsa_msa_handle* h, const DevPlan& p, const PlanInfo& info,
                                 const float* scores, int64_t ld, uint64_t* keys, int32_t* sel,
                                 hipStream_t st);
// 32-key group maxima written by the decode score kernel (every row a decode row, 64 x 128
// matrix-core shapes); runs: [n_rows][msa_runs_ld] uint32
bool index_run_max_supported(const dsa_handle* h, const PlanInfo& info);
hipError_t launch_index_scores_run_max(const dsa_handle* h, const DevPlan& p, const PlanInfo& info,
                                       const void* q, const float* w, const void* key_pool,
                                       float* scores, int64_t ld, uint32_t* run_max, int64_t rm_ld,
                                       hipStream_t st);
int64_t msa_runs_ld(const PlanInfo& info);
hipError_t launch_msa_block_rank_runs(const dsa_msa_handle* h, const DevPlan& p,
                                      const PlanInfo& info, const uint32_t* runs, int32_t* sel,
                                      hipStream_t st);
// ws: msa_attend_workspace_bytes of scratch for the per-block partials
hipError_t launch_msa_attend(const dsa_msa_handle* h, const DevPlan& p, const PlanInfo& info,
                             const int32_t* sel, const void* q, const void* pool, float sm_scale,
                             void* out, void* ws, hipStream_t st);
