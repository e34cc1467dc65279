// C ABI of libdsa: handle, host validation of plans and arguments, workspace sizing, dispatch.
// Nothing here allocates device memory or synchronises; every launch goes to the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>

#include "dsa_internal.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dsa_status fail(dsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dsa_status ok() { return DSA_OK; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(int fmt) { return fmt == DSA_FMT_F32 ? 4 : fmt == DSA_FMT_BF16 ? 2 : 1; }

dsa_status check_config(const dsa_config* c) {
  if (!c) return fail(DSA_ERR_INVALID_ARG, "config is NULL");
  auto fmt_ok = [](int f, bool fp8) {
    return f == DSA_FMT_F32 || f == DSA_FMT_BF16 || (fp8 && f == DSA_FMT_FP8);
  };
  if (c->n_index_heads < 1 || c->n_index_heads > 128)
    return fail(DSA_ERR_INVALID_ARG, "n_index_heads %d outside 1..128", c->n_index_heads);
  if (c->index_dim < 8 || c->index_dim > 512 || c->index_dim % 8)
    return fail(DSA_ERR_INVALID_ARG, "index_dim %d must be a multiple of 8 in 8..512", c->index_dim);
  if (!fmt_ok(c->index_q_fmt, false))
    return fail(DSA_ERR_INVALID_ARG, "index_q_fmt %d must be F32 or BF16", c->index_q_fmt);
  if (!fmt_ok(c->index_key_fmt, true))
    return fail(DSA_ERR_INVALID_ARG, "index_key_fmt %d unknown", c->index_key_fmt);
  if (c->topk < 1 || c->topk > DSA_MAX_TOPK)
    return fail(DSA_ERR_INVALID_ARG, "topk %d outside 1..%d", c->topk, DSA_MAX_TOPK);
  if (c->n_heads < 1 || c->n_heads > 256)
    return fail(DSA_ERR_INVALID_ARG, "n_heads %d outside 1..256", c->n_heads);
  if (c->kv_lora_rank < 8 || c->kv_lora_rank > 1024 || c->kv_lora_rank % 8)
    return fail(DSA_ERR_INVALID_ARG, "kv_lora_rank %d must be a multiple of 8 in 8..1024",
                c->kv_lora_rank);
  if (c->rope_dim < 0 || c->rope_dim > 256 || c->rope_dim % 8)
    return fail(DSA_ERR_INVALID_ARG, "rope_dim %d must be a multiple of 8 in 0..256", c->rope_dim);
  if (!fmt_ok(c->q_fmt, true))
    return fail(DSA_ERR_INVALID_ARG, "q_fmt %d unknown", c->q_fmt);
  if (!fmt_ok(c->latent_fmt, true))
    return fail(DSA_ERR_INVALID_ARG, "latent_fmt %d unknown", c->latent_fmt);
  if (c->latent_fmt == DSA_FMT_FP8 && c->kv_lora_rank % 128)
    return fail(DSA_ERR_UNSUPPORTED, "packed fp8 latents need kv_lora_rank %% 128 == 0 (got %d)",
                c->kv_lora_rank);
  if (c->page_size < 1 || c->page_size > 4096)
    return fail(DSA_ERR_INVALID_ARG, "page_size %d outside 1..4096", c->page_size);
  if (c->index_key_fmt == DSA_FMT_FP8 &&
      ((int64_t(c->page_size) * c->index_dim) % 16 || (int64_t(c->page_size) * 4) % 16))
    return fail(DSA_ERR_UNSUPPORTED,
                "fp8 index pages need page_size*index_dim and page_size*4 to be multiples of 16");
  if (int64_t(c->n_index_heads) * c->index_dim > 16384)
    return fail(DSA_ERR_UNSUPPORTED, "n_index_heads * index_dim must be <= 16384");
  return ok();
}

dsa_status check_plan(const dsa_handle* h, const dsa_plan* p, PlanInfo* info) {
  if (!h) return fail(DSA_ERR_INVALID_ARG, "handle is NULL");
  if (!p) return fail(DSA_ERR_INVALID_ARG, "plan is NULL");
  if (p->n_spans < 1) return fail(DSA_ERR_INVALID_ARG, "plan has %d spans", p->n_spans);
  if (p->n_rows < 1) return fail(DSA_ERR_INVALID_ARG, "plan has %d rows", p->n_rows);
  if (!p->spans_host || !p->spans_dev || !p->page_table_dev)
    return fail(DSA_ERR_INVALID_ARG, "plan arrays must not be NULL");
  if (!aligned(p->spans_dev, 4) || !aligned(p->page_table_dev, 4))
    return fail(DSA_ERR_INVALID_ARG, "plan device arrays must be 4-byte aligned");
  if (p->n_page_ids < 1 || p->pool_pages < 1)
    return fail(DSA_ERR_INVALID_ARG, "plan needs n_page_ids >= 1 and pool_pages >= 1");
  const int ps = h->cfg.page_size;
  int64_t expect_row = 0;
  PlanInfo in{};
  in.n_spans = p->n_spans;
  in.all_decode = true;
  for (int s = 0; s < p->n_spans; ++s) {
    const dsa_span& sp = p->spans_host[s];
    if (sp.q_start != expect_row)
      return fail(DSA_ERR_INVALID_ARG,
                  "span %d starts at row %d; spans must be contiguous in row order (expected %lld)",
                  s, sp.q_start, (long long)expect_row);
    if (sp.q_len < 1) return fail(DSA_ERR_INVALID_ARG, "span %d has q_len %d", s, sp.q_len);
    if (sp.ctx_start < 0 || sp.page_start < 0 || sp.page_offset < 0 || sp.n_pages < 1)
      return fail(DSA_ERR_INVALID_ARG, "span %d has a negative field or no pages", s);
    if (int64_t(sp.page_offset) + sp.n_pages > p->n_page_ids)
      return fail(DSA_ERR_OUT_OF_RANGE, "span %d pages [%d, %lld) run past the page table (%d ids)",
                  s, sp.page_offset, (long long)(int64_t(sp.page_offset) + sp.n_pages), p->n_page_ids);
    int64_t last_pos = int64_t(sp.ctx_start) + sp.q_len - 1;
    int64_t last_slot = int64_t(sp.page_start) + last_pos;
    if (last_slot >= int64_t(sp.n_pages) * ps)
      return fail(DSA_ERR_OUT_OF_RANGE,
                  "span %d: position %lld needs slot %lld but its %d pages hold %lld slots", s,
                  (long long)last_pos, (long long)last_slot, sp.n_pages,
                  (long long)int64_t(sp.n_pages) * ps);
    if (last_pos + 1 > INT32_MAX / 2)
      return fail(DSA_ERR_OUT_OF_RANGE, "span %d: position %lld too large", s, (long long)last_pos);
    int64_t vis = last_pos + 1;
    if (vis > in.max_visible) in.max_visible = int32_t(vis);
    if (sp.q_len > in.max_q_len) in.max_q_len = sp.q_len;
    in.total_visible += int64_t(sp.q_len) * (2 * int64_t(sp.ctx_start) + sp.q_len + 1) / 2;
    if (sp.q_len != 1) in.all_decode = false;
    expect_row += sp.q_len;
  }
  if (expect_row != p->n_rows)
    return fail(DSA_ERR_INVALID_ARG, "spans cover %lld rows but n_rows is %d", (long long)expect_row,
                p->n_rows);
  if (p->max_visible_cap != 0) {
    if (p->max_visible_cap < in.max_visible || p->max_visible_cap > INT32_MAX / 2)
      return fail(DSA_ERR_INVALID_ARG,
                  "max_visible_cap %d must be 0 or cover the longest row (%d visible positions)",
                  p->max_visible_cap, in.max_visible);
    in.max_visible = p->max_visible_cap;   // launch shapes follow the cap
  }
  if (p->page_table_host) {
    for (int i = 0; i < p->n_page_ids; ++i) {
      int32_t pg = p->page_table_host[i];
      if (pg < 0 || pg >= p->pool_pages)
        return fail(DSA_ERR_OUT_OF_RANGE, "page table entry %d is %d, outside the pool of %d pages",
                    i, pg, p->pool_pages);
    }
  }
  in.n_rows = p->n_rows;
  in.spans_host = p->spans_host;
  if (info) *info = in;
  return ok();
}

DevPlan dev_plan(const dsa_handle* h, const dsa_plan* p) {
  DevPlan d;
  d.spans = p->spans_dev;
  d.page_table = p->page_table_dev;
  d.n_spans = p->n_spans;
  d.n_rows = p->n_rows;
  d.pool_pages = p->pool_pages;
  d.page_size = h->cfg.page_size;
  return d;
}

dsa_status check_ptr(const void* ptr, size_t align, const char* name) {
  if (!ptr) return fail(DSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(DSA_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return ok();
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t scores_bytes(const PlanInfo& in) {
  size_t ld = (size_t(in.max_visible) + 63) & ~size_t(63);
  return (size_t(in.n_rows) * ld * 4 + 255) & ~size_t(255);
}


int64_t scores_ld(const PlanInfo& in) { return (int64_t(in.max_visible) + 63) & ~int64_t(63); }

}  // namespace

size_t index_topk_workspace_bytes(const dsa_handle* h, const PlanInfo& in, size_t* scores_part) {
  const size_t sb = scores_bytes(in);
  if (scores_part) *scores_part = sb;
  return sb + select_workspace_bytes(h, in, select_lists_used(h, in));
}

extern "C" {

dsa_status dsa_create(const dsa_config* cfg, dsa_handle** out) {
  if (!out) return fail(DSA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  dsa_status s = check_config(cfg);
  if (s) return s;
  dsa_handle* h = new (std::nothrow) dsa_handle;
  if (!h) return fail(DSA_ERR_INVALID_ARG, "out of host memory");
  h->cfg = *cfg;
  const dsa_config& c = *cfg;
  h->index_page_bytes = c.index_key_fmt == DSA_FMT_FP8
                            ? int64_t(c.page_size) * (c.index_dim + 4)
                            : int64_t(c.page_size) * c.index_dim * elem_bytes(c.index_key_fmt);
  h->latent_row_bytes = c.latent_fmt == DSA_FMT_FP8
                            ? int64_t(c.kv_lora_rank) + 4 * (c.kv_lora_rank / 128) + 2 * c.rope_dim
                            : int64_t(c.kv_lora_rank + c.rope_dim) * elem_bytes(c.latent_fmt);
  *out = h;
  return ok();
}

void dsa_destroy(dsa_handle* h) { delete h; }

dsa_status dsa_plan_check(const dsa_handle* h, const dsa_plan* plan) {
  return check_plan(h, plan, nullptr);
}

dsa_status dsa_workspace_size(const dsa_handle* h, const dsa_plan* plan, int32_t op, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  PlanInfo in;
  dsa_status s = check_plan(h, plan, &in);
  if (s) return s;
  switch (op) {
    case DSA_OP_INDEX_TOPK: *bytes = index_topk_workspace_bytes(h, in, nullptr); break;
    case DSA_OP_SELECT_TOPK: *bytes = select_workspace_bytes(h, in, false); break;
    case DSA_OP_ATTEND: *bytes = attend_workspace_bytes(h, in); break;
    default: return fail(DSA_ERR_INVALID_ARG, "unknown op %d", op);
  }
  return ok();
}

dsa_status dsa_store_keys(const dsa_handle* h, const dsa_plan* plan, const void* keys,
                          const float* scales, void* key_pool, void* stream) {
  PlanInfo in;
  dsa_status s = check_plan(h, plan, &in);
  if (s) return s;
  const int kf = h->cfg.index_key_fmt;
  if ((s = check_ptr(keys, 16, "keys"))) return s;
  if ((s = check_ptr(key_pool, 16, "key_pool"))) return s;
  if (kf == DSA_FMT_FP8) {
    if ((s = check_ptr(scales, 4, "scales"))) return s;
  } else if (scales) {
    return fail(DSA_ERR_INVALID_ARG, "scales must be NULL for non-fp8 index keys");
  }
  return hip_status(launch_store_keys(h, dev_plan(h, plan), keys, scales, key_pool,
                                      (hipStream_t)stream),
                    "store_keys launch");
}

dsa_status dsa_index_scores(const dsa_handle* h, const dsa_plan* plan, const void* q, const float* w,
                            const void* key_pool, float* scores, int64_t ld, void* stream) {
  PlanInfo in;
  dsa_status s = check_plan(h, plan, &in);
  if (s) return s;
  if ((s = check_ptr(q, 16, "q"))) return s;
  if ((s = check_ptr(w, 4, "w"))) return s;
  if ((s = check_ptr(key_pool, 16, "key_pool"))) return s;
  if ((s = check_ptr(scores, 16, "scores"))) return s;
  if (ld < in.max_visible || ld % 4)
    return fail(DSA_ERR_INVALID_ARG, "ld %lld must be a multiple of 4 and >= %d", (long long)ld,
                in.max_visible);
  return hip_status(launch_index_scores(h, dev_plan(h, plan), in, q, w, key_pool, scores, ld, true,
                                        (hipStream_t)stream),
                    "index score launch");
}

dsa_status dsa_select_topk(const dsa_handle* h, const dsa_plan* plan, const float* scores,
                           int64_t ld, int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  PlanInfo in;
  dsa_status s = check_plan(h, plan, &in);
  if (s) return s;
  if ((s = check_ptr(scores, 16, "scores"))) return s;
  if ((s = check_ptr(sel, 16, "sel"))) return s;
  if (ld < in.max_visible || ld % 4)
    return fail(DSA_ERR_INVALID_ARG, "ld %lld must be a multiple of 4 and >= %d", (long long)ld,
                in.max_visible);
  size_t need = select_workspace_bytes(h, in, false);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "select needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (ws && !aligned(ws, 256)) return fail(DSA_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  return hip_status(launch_select_topk(h, dev_plan(h, plan), in, scores, ld, sel, ws,
                                       (hipStream_t)stream),
                    "select launch");
}

dsa_status dsa_index_topk(const dsa_handle* h, const dsa_plan* plan, const void* q, const float* w,
                          const void* key_pool, int32_t* sel, void* ws, size_t ws_bytes,
                          void* stream) {
  PlanInfo in;
  dsa_status s = check_plan(h, plan, &in);
  if (s) return s;
  if ((s = check_ptr(q, 16, "q"))) return s;
  if ((s = check_ptr(w, 4, "w"))) return s;
  if ((s = check_ptr(key_pool, 16, "key_pool"))) return s;
  if ((s = check_ptr(sel, 16, "sel"))) return s;
  size_t sb = 0;
  const size_t need = index_topk_workspace_bytes(h, in, &sb);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "index_topk needs %zu workspace bytes, got %zu", need,
                ws ? ws_bytes : 0);
  if (!aligned(ws, 256)) return fail(DSA_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  float* scores = static_cast<float*>(ws);
  return hip_status(launch_index_topk(h, dev_plan(h, plan), in, q, w, key_pool, sel, scores,
                                      scores_ld(in), static_cast<char*>(ws) + sb,
                                      (hipStream_t)stream),
                    "index_topk launch");
}

}  // extern "C"

// ------------------------------------------------------------------ index_topk without allocation
// Workspace of dsa_index_topk_noalloc: one array per GPU, alive until the process ends. In host
// code `scratch` only names the symbol; its device address on the current GPU comes from
// hipGetSymbolAddress (scratch_ptr), and only that address is handed to kernels.
namespace {

constexpr size_t kScratchBytes = size_t(DSA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch, looked up once per device.
dsa_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "device %d: scratch is kept for devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" {

dsa_status dsa_index_topk_noalloc(const dsa_handle* h, const dsa_plan* plan, const void* q,
                                  const float* w, const void* key_pool, int32_t* sel,
                                  void* stream) {
  PlanInfo in;
  dsa_status s = check_plan(h, plan, &in);
  if (s) return s;
  if ((s = check_ptr(q, 16, "q"))) return s;
  if ((s = check_ptr(w, 4, "w"))) return s;
  if ((s = check_ptr(key_pool, 16, "key_pool"))) return s;
  if ((s = check_ptr(sel, 16, "sel"))) return s;
  size_t sb = 0;
  const size_t need = index_topk_workspace_bytes(h, in, &sb);
  if (need > kScratchBytes)
    return fail(DSA_ERR_WORKSPACE,
                "index_topk_noalloc: this plan needs %zu workspace bytes, over the %zu-byte "
                "static scratch; use dsa_index_topk with a caller workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_ptr(&ws))) return s;
  float* scores = static_cast<float*>(ws);
  return hip_status(launch_index_topk(h, dev_plan(h, plan), in, q, w, key_pool, sel, scores,
                                      scores_ld(in), static_cast<char*>(ws) + sb,
                                      (hipStream_t)stream),
                    "index_topk_noalloc launch");
}

}  // extern "C"

namespace {

dsa_status attend_checked(const dsa_handle* h, const dsa_plan* plan, const int32_t* sel,
                          const void* q_nope, const void* q_pe, const void* latent_pool,
                          float sm_scale, const float* sink, void* out, void* ws, size_t ws_bytes,
                          void* stream) {
  PlanInfo in;
  dsa_status s = check_plan(h, plan, &in);
  if (s) return s;
  if ((s = check_ptr(sel, 16, "sel"))) return s;
  if ((s = check_ptr(q_nope, 16, "q_nope"))) return s;
  if (h->cfg.rope_dim > 0 && (s = check_ptr(q_pe, 16, "q_pe"))) return s;
  if ((s = check_ptr(latent_pool, 16, "latent_pool"))) return s;
  if ((s = check_ptr(out, 16, "out"))) return s;
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(DSA_ERR_INVALID_ARG, "sm_scale must be finite");
  size_t need = attend_workspace_bytes(h, in);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "attend needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (ws && !aligned(ws, 256)) return fail(DSA_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  return hip_status(launch_attend(h, dev_plan(h, plan), in, sel, q_nope, q_pe, latent_pool, sm_scale,
                                  sink, out, ws, (hipStream_t)stream),
                    "attend launch");
}

}  // namespace

extern "C" {

dsa_status dsa_sparse_mla_attend(const dsa_handle* h, const dsa_plan* plan, const int32_t* sel,
                                 const void* q_nope, const void* q_pe, const void* latent_pool,
                                 float sm_scale, void* out, void* ws, size_t ws_bytes, void* stream) {
  return attend_checked(h, plan, sel, q_nope, q_pe, latent_pool, sm_scale, nullptr, out, ws,
                        ws_bytes, stream);
}

dsa_status dsa_sparse_mla_attend_sink(const dsa_handle* h, const dsa_plan* plan, const int32_t* sel,
                                      const void* q_nope, const void* q_pe, const void* latent_pool,
                                      float sm_scale, const float* sink, void* out, void* ws,
                                      size_t ws_bytes, void* stream) {
  dsa_status s = check_ptr(sink, 4, "sink");
  if (s) return s;
  return attend_checked(h, plan, sel, q_nope, q_pe, latent_pool, sm_scale, sink, out, ws, ws_bytes,
                        stream);
}

// ------------------------------------------------------------------ block-sparse MSA

dsa_status dsa_msa_create(const dsa_msa_config* c, dsa_msa_handle** out) {
  if (!out) return fail(DSA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!c) return fail(DSA_ERR_INVALID_ARG, "config is NULL");
  // the index side is checked as a DSA configuration (its attention fields are placeholders)
  dsa_config ic{};
  ic.n_index_heads = c->n_index_heads;
  ic.index_dim = c->index_dim;
  ic.index_q_fmt = c->index_q_fmt;
  ic.index_key_fmt = c->index_key_fmt;
  ic.topk = 1;
  ic.n_heads = 1;
  ic.kv_lora_rank = 8;
  ic.rope_dim = 0;
  ic.q_fmt = DSA_FMT_BF16;
  ic.latent_fmt = DSA_FMT_BF16;
  ic.page_size = c->page_size;
  dsa_status s = check_config(&ic);
  if (s) return s;
  if (c->block_size != 32 && c->block_size != 64 && c->block_size != 128 && c->block_size != 256)
    return fail(DSA_ERR_UNSUPPORTED, "block_size %d must be 32, 64, 128 or 256", c->block_size);
  if (c->topk_blocks < 1 || c->topk_blocks > 64)
    return fail(DSA_ERR_INVALID_ARG, "topk_blocks %d outside 1..64", c->topk_blocks);
  if (c->n_heads < 1 || c->n_heads > 256 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
    return fail(DSA_ERR_INVALID_ARG, "n_heads %d must be 1..256 and a multiple of n_kv_heads %d",
                c->n_heads, c->n_kv_heads);
  if (c->head_dim < 8 || c->head_dim > 256 || c->head_dim % 8)
    return fail(DSA_ERR_INVALID_ARG, "head_dim %d must be a multiple of 8 in 8..256", c->head_dim);
  if (c->q_fmt != DSA_FMT_F32 && c->q_fmt != DSA_FMT_BF16)
    return fail(DSA_ERR_INVALID_ARG, "q_fmt %d must be F32 or BF16", c->q_fmt);
  if (msa_attend_lds_bytes(*c) > 160 * 1024)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d with block_size %d: attention tiles do not fit in LDS",
                c->head_dim, c->block_size);
  // Without a device (a host-only process) the attribute call fails and is of no use; a launch
  // that still lacked the LDS would report its own error.
  if (msa_prepare(*c) != hipSuccess) (void)hipGetLastError();
  dsa_msa_handle* h = new (std::nothrow) dsa_msa_handle;
  if (!h) return fail(DSA_ERR_INVALID_ARG, "out of host memory");
  h->cfg = *c;
  h->idx.cfg = ic;
  h->idx.index_page_bytes = c->index_key_fmt == DSA_FMT_FP8
                                ? int64_t(c->page_size) * (c->index_dim + 4)
                                : int64_t(c->page_size) * c->index_dim * elem_bytes(c->index_key_fmt);
  h->idx.latent_row_bytes = 0;
  h->gqa_row_bytes = int64_t(2) * c->n_kv_heads * c->head_dim * elem_bytes(c->q_fmt);
  *out = h;
  return ok();
}

void dsa_msa_destroy(dsa_msa_handle* h) { delete h; }

namespace {
dsa_status msa_plan(const dsa_msa_handle* h, const dsa_plan* plan, PlanInfo* in) {
  if (!h) return fail(DSA_ERR_INVALID_ARG, "handle is NULL");
  dsa_status s = check_plan(&h->idx, plan, in);
  if (s) return s;
  return ok();
}

// select workspace: the token scores, then the block keys (or the 32-key group maxima)
size_t msa_select_ws_bytes(const dsa_msa_handle* h, const PlanInfo& in) {
  const size_t keys = size_t(in.n_rows) * msa_block_keys_ld(h->cfg, in) * 8;
  const size_t runs = size_t(in.n_rows) * size_t(msa_runs_ld(in)) * 4;
  return scores_bytes(in) + ((std::max(keys, runs) + 255) & ~size_t(255));
}
}  // namespace

dsa_status dsa_msa_workspace_size(const dsa_msa_handle* h, const dsa_plan* plan, int32_t op,
                                  size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  PlanInfo in;
  dsa_status s = msa_plan(h, plan, &in);
  if (s) return s;
  if (op == DSA_OP_SELECT_TOPK) *bytes = msa_select_ws_bytes(h, in);
  else if (op == DSA_OP_ATTEND) *bytes = msa_attend_workspace_bytes(h->cfg, in);
  else return fail(DSA_ERR_INVALID_ARG, "op %d: MSA has select and attend", op);
  return ok();
}

dsa_status dsa_msa_select_blocks(const dsa_msa_handle* h, const dsa_plan* plan, const void* q,
                                 const float* w, const void* key_pool, int32_t* sel, void* ws,
                                 size_t ws_bytes, void* stream) {
  PlanInfo in;
  dsa_status s = msa_plan(h, plan, &in);
  if (s) return s;
  if ((s = check_ptr(q, 16, "q"))) return s;
  if ((s = check_ptr(w, 4, "w"))) return s;
  if ((s = check_ptr(key_pool, 16, "key_pool"))) return s;
  if ((s = check_ptr(sel, 4, "sel"))) return s;
  const size_t need = msa_select_ws_bytes(h, in);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "MSA select needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned(ws, 256)) return fail(DSA_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  const DevPlan dp = dev_plan(&h->idx, plan);
  float* scores = static_cast<float*>(ws);
  const int64_t ld = scores_ld(in);
  char* aux = static_cast<char*>(ws) + scores_bytes(in);
  hipError_t e;
  if (index_run_max_supported(&h->idx, in)) {
    uint32_t* runs = reinterpret_cast<uint32_t*>(aux);
    e = launch_index_scores_run_max(&h->idx, dp, in, q, w, key_pool, scores, ld, runs,
                                    msa_runs_ld(in), (hipStream_t)stream);
    if (e == hipSuccess) e = launch_msa_block_rank_runs(h, dp, in, runs, sel, (hipStream_t)stream);
  } else {
    uint64_t* keys = reinterpret_cast<uint64_t*>(aux);
    e = launch_index_scores(&h->idx, dp, in, q, w, key_pool, scores, ld, false, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_msa_block_topk(h, dp, in, scores, ld, keys, sel, (hipStream_t)stream);
  }
  return hip_status(e, "MSA select launch");
}

dsa_status dsa_msa_attend(const dsa_msa_handle* h, const dsa_plan* plan, const int32_t* sel,
                          const void* q, const void* gqa_pool, float sm_scale, void* out,
                          void* ws, size_t ws_bytes, void* stream) {
  PlanInfo in;
  dsa_status s = msa_plan(h, plan, &in);
  if (s) return s;
  const size_t need = msa_attend_workspace_bytes(h->cfg, in);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "MSA attend needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned(ws, 256)) return fail(DSA_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  if ((s = check_ptr(sel, 4, "sel"))) return s;
  if ((s = check_ptr(q, 16, "q"))) return s;
  if ((s = check_ptr(gqa_pool, 16, "gqa_pool"))) return s;
  if ((s = check_ptr(out, 16, "out"))) return s;
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(DSA_ERR_INVALID_ARG, "sm_scale must be finite");
  return hip_status(launch_msa_attend(h, dev_plan(&h->idx, plan), in, sel, q, gqa_pool, sm_scale,
                                      out, ws, (hipStream_t)stream),
                    "MSA attend launch");
}

const char* dsa_status_str(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_OUT_OF_RANGE: return "out of range";
    case DSA_ERR_UNSUPPORTED: return "unsupported";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "hip error";
  }
  return "unknown status";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
