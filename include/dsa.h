/*
 * dsa.h - C ABI of the DeepSeek Sparse Attention (DSA) select + attend library for MI355X (gfx950).
 *
 * The library computes, on one GPU, the path described by the page
 * "mstar.engine.resources.dsa.manager":
 *   1. store_keys   - each step row's index key goes to its request at its position;
 *   2. index_topk   - each query row scores its request's keys 0..position as
 *                     sum_h w[h] * relu(q[h] . k) in fp32 and keeps the causal top-k positions,
 *                     ties toward the lower position, -1 padded;
 *   3. attend       - absorbed MLA of each row over only its picked latents of a paged MLA cache.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers unless the field name ends in _host.
 *   - The caller owns every buffer. Calls never allocate, free or synchronise; they enqueue work on
 *     the given stream (a hipStream_t passed as void*, NULL = the null stream) and return.
 *   - Every argument is validated on the host before anything is enqueued. On error nothing is
 *     enqueued, a negative dsa_status is returned and dsa_last_error() holds a message for the
 *     calling thread. DSA_ERR_HIP means a launch itself failed.
 *   - A handle is immutable after dsa_create and may be used from several threads at once; calls
 *     that share output or workspace buffers on one stream are ordered by that stream.
 *
 * Storage formats (dsa_format; never inferred from a width, as the page
 * "ttnn.transformer.sparse_sdpa" requires of its kv_format argument):
 *   DSA_FMT_F32   IEEE float32 elements.
 *   DSA_FMT_BF16  bfloat16 elements.
 *   DSA_FMT_FP8   index keys: D OCP e4m3fn codes per token plus one fp32 scale per token, the key
 *                 being e4m3(code) * scale (the 132-byte index record of "Sparse attention (DSA
 *                 and block-sparse MSA)", section "What the KV cache actually holds"); latents:
 *                 the packed row [R e4m3 | R/128 fp32 scales | P bf16], element d < R being
 *                 e4m3(code) * scale[d / 128] (the 656-byte row of ttnn.transformer.sparse_sdpa,
 *                 kv parameter, for R = 512, P = 64). Scales must be finite and >= 0.
 *
 * Pools (one layer each). Pages are numbered 0 .. pool_pages-1 and shared by both pools.
 *   Index-key pool, one page of page_size tokens:
 *     F32/BF16: [page_size][D] elements.
 *     FP8:      [page_size][D] e4m3 codes, then [page_size] fp32 scales (page_size*(D+4) bytes).
 *   Latent pool: [pool_pages][page_size][row], row = R+P elements (F32/BF16) or the packed FP8 row.
 *
 * Plan (DSASpan / DSAPlan of the DSA resource page): span s holds q_len consecutive step rows from
 * row q_start, the first at position ctx_start, so row t has position ctx_start + (t - q_start).
 * Its pages are page_table[page_offset .. page_offset + n_pages) and its position-0 token sits
 * page_start slots into that list: position j lives at slot = page_start + j, in page
 * page_table[page_offset + slot / page_size], offset slot % page_size. A row sees positions
 * 0 .. its own position, itself included.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad span layout, bad value */
  DSA_ERR_OUT_OF_RANGE = -2,  /* a row's position beyond its pages, page id outside the pool */
  DSA_ERR_UNSUPPORTED = -3,   /* a format / shape combination this build does not implement */
  DSA_ERR_WORKSPACE = -4,     /* workspace missing or smaller than dsa_workspace_size */
  DSA_ERR_HIP = -5            /* a kernel launch failed */
} dsa_status;

typedef enum { DSA_FMT_F32 = 0, DSA_FMT_BF16 = 1, DSA_FMT_FP8 = 2 } dsa_format;

/* Operations, for dsa_workspace_size. */
typedef enum { DSA_OP_INDEX_TOPK = 0, DSA_OP_SELECT_TOPK = 1, DSA_OP_ATTEND = 2 } dsa_op;

/* Shapes and formats of one DSA layer pair (indexer + absorbed MLA). */
typedef struct {
  int32_t n_index_heads;  /* H_i: indexer heads (1..128) */
  int32_t index_dim;      /* D: index key / query width (multiple of 8, <= 512) */
  int32_t index_q_fmt;    /* indexer queries q: F32 or BF16 */
  int32_t index_key_fmt;  /* index keys: F32, BF16 or FP8 */
  int32_t topk;           /* positions kept per row (1..DSA_MAX_TOPK) */
  int32_t n_heads;        /* H: MLA heads (1..256) */
  int32_t kv_lora_rank;   /* R: latent width, also the output width (multiple of 8) */
  int32_t rope_dim;       /* P: rope width of the latent (multiple of 8, may be 0) */
  int32_t q_fmt;          /* q_nope, q_pe and the attention output: F32, BF16 or FP8 (plain
                             e4m3fn values without a scale; the output is then e4m3fn too,
                             rounded to nearest even and saturated at +-448, as the q parameter
                             and the Returns line of ttnn.transformer.sparse_sdpa have it) */
  int32_t latent_fmt;     /* latent rows: F32, BF16 or FP8 (FP8 needs R % 128 == 0) */
  int32_t page_size;      /* tokens per page (1..4096) */
} dsa_config;

#define DSA_MAX_TOPK 4096

/* One request's rows in a step (DSASpan). */
typedef struct {
  int32_t q_start;      /* first step row of the span */
  int32_t q_len;        /* number of rows (>= 1) */
  int32_t ctx_start;    /* position of the first row (>= 0) */
  int32_t page_offset;  /* start of the span's list in the page table */
  int32_t n_pages;      /* length of the span's list */
  int32_t page_start;   /* slot of position 0 within the list (>= 0) */
} dsa_span;

/* A step's rows (DSAPlan). Spans are in row order and contiguous: span 0 starts at row 0 and
 * span s+1 starts where span s ends; n_rows is the sum of q_len. spans_dev and page_table_dev
 * are device copies of the host arrays. page_table_host may be NULL, in which case page ids are
 * not checked on the host (out-of-pool ids then give undefined values, never an access outside
 * the pools).
 *
 * Kernels read the plan from the device copies only; the host copy sizes the launches and is
 * checked. With max_visible_cap = 0 launches are sized for the plan's own longest row. With
 * max_visible_cap > 0 (at least that longest row's position + 1) they are sized for rows of up
 * to max_visible_cap visible positions instead (grids, the score matrix, workspace), so a step
 * captured in a graph can be replayed after the caller moves positions forward in spans_dev
 * (ctx_start of a decode span, for example) without capturing again, as long as every row
 * keeps position + 1 <= max_visible_cap and its slot inside its span's pages. Results are then
 * those of the plan that spans_dev holds at replay. A position past its pages reads a page of
 * its own list (undefined values, never an access outside the page table or the pools). */
typedef struct {
  int32_t n_spans;
  int32_t n_rows;
  int32_t n_page_ids;               /* entries in the page table */
  int32_t pool_pages;               /* pages in each pool */
  int32_t max_visible_cap;          /* 0, or the visible positions launches are sized for */
  const dsa_span* spans_host;       /* host, n_spans */
  const int32_t* page_table_host;   /* host, n_page_ids, or NULL */
  const dsa_span* spans_dev;        /* device, n_spans */
  const int32_t* page_table_dev;    /* device, n_page_ids */
} dsa_plan;

typedef struct dsa_handle dsa_handle;

/* Create a handle for one configuration. Fails with DSA_ERR_INVALID_ARG on a bad value and
 * DSA_ERR_UNSUPPORTED on a combination this build does not implement. Touches no GPU state. */
dsa_status dsa_create(const dsa_config* cfg, dsa_handle** out);
void dsa_destroy(dsa_handle* h);

/* Full host check of a plan against the handle (spans, positions vs pages, page ids when
 * page_table_host is given). Every other call runs the same check. */
dsa_status dsa_plan_check(const dsa_handle* h, const dsa_plan* plan);

/* Workspace bytes that op needs for this plan (0 is possible). Workspace is device memory owned
 * by the caller, 256-byte aligned, not shared by calls in flight at the same time. */
dsa_status dsa_workspace_size(const dsa_handle* h, const dsa_plan* plan, int32_t op, size_t* bytes);

/* store_keys (DSA resource page, store_keys; IndexKeyStore.append): write this step's index keys,
 * row t to its request at position ctx_start + t - q_start.
 *   keys      [n_rows][D] in index_key_fmt elements (FP8: e4m3 codes, one byte each)
 *   scales    [n_rows] fp32 for FP8 keys, NULL otherwise
 *   key_pool  the index-key pool (layout above), written in place
 * Keys must be stored before dsa_index_topk reads them: a row scores keys up to its own
 * position, the current chunk included (IndexKeyStore.history). */
dsa_status dsa_store_keys(const dsa_handle* h, const dsa_plan* plan, const void* keys,
                          const float* scales, void* key_pool, void* stream);

/* index_topk (DSA resource page, index_topk, select_topk_causal): for every row t,
 *   s[j] = sum_h w[t][h] * relu(q[t][h] . k_j)   for j = 0 .. position(t), accumulated in fp32,
 * then the top topk positions by score descending, equal scores by position ascending, the
 * first min(topk, position + 1) of them followed by -1 entries.
 *   q    [n_rows][H_i][D] in index_q_fmt;  w [n_rows][H_i] fp32 (any scales folded in)
 *   sel  [n_rows][topk] int32 output
 *   ws   workspace of dsa_workspace_size(DSA_OP_INDEX_TOPK) bytes */
dsa_status dsa_index_topk(const dsa_handle* h, const dsa_plan* plan, const void* q, const float* w,
                          const void* key_pool, int32_t* sel, void* ws, size_t ws_bytes,
                          void* stream);

/* index_topk for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): dsa_index_topk with the library's own workspace
 * instead of a caller buffer. The workspace is one static array of DSA_NOALLOC_SCRATCH_BYTES
 * per GPU, created with the library's code object and held until the process ends; the call
 * allocates and frees nothing. A plan whose workspace (dsa_workspace_size(DSA_OP_INDEX_TOPK))
 * exceeds it is rejected with DSA_ERR_WORKSPACE before anything is enqueued. Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (two streams, two threads) race and
 * must be ordered by the caller. The first call on a device looks up the array's address there
 * (DSA_ERR_HIP if that fails). Results are those of dsa_index_topk; arguments as there. */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
dsa_status dsa_index_topk_noalloc(const dsa_handle* h, const dsa_plan* plan, const void* q,
                                  const float* w, const void* key_pool, int32_t* sel, void* stream);

/* attend (DSA resource page, attend; ttnn.transformer.sparse_sdpa operation line): for every row
 * t and head h over the row's picked positions j (entries < 0 are skipped),
 *   logit_j = sm_scale * (q_nope[t][h] . c_j[0:R] + q_pe[t][h] . c_j[R:R+P]),
 *   out[t][h] = sum_j softmax(logit)_j * c_j[0:R]          (V is the leading R latent columns).
 *   sel     [n_rows][topk] int32 request-local positions, as dsa_index_topk writes them; a
 *           SHARED layer passes the same sel with its own q and latent pool
 *   q_nope  [n_rows][H][R], q_pe [n_rows][H][P] in q_fmt;  out [n_rows][H][R] in q_fmt
 *   A row with no picked position gets a zero output.
 *   ws      workspace of dsa_workspace_size(DSA_OP_ATTEND) bytes */
dsa_status dsa_sparse_mla_attend(const dsa_handle* h, const dsa_plan* plan, const int32_t* sel,
                                 const void* q_nope, const void* q_pe, const void* latent_pool,
                                 float sm_scale, void* out, void* ws, size_t ws_bytes, void* stream);

/* attend with an attention sink (ttnn.transformer.sparse_sdpa, attention_sink parameter): as
 * dsa_sparse_mla_attend, with one more term per head in the softmax denominator only,
 *   out[t][h] = sum_j e^{logit_j} c_j[0:R] / (sum_j e^{logit_j} + e^{sm_scale * sink[h]}).
 *   sink    [H] fp32, DEVICE, one value per head shared by every row, in the units of the unscaled
 *           logits (q . c); -inf adds nothing. Values must be finite or -inf (+inf or NaN give
 *           undefined outputs). A model whose sinks are already scaled logits passes them divided
 *           by sm_scale. Must not be NULL.
 * Workspace, layouts and errors as dsa_sparse_mla_attend. */
dsa_status dsa_sparse_mla_attend_sink(const dsa_handle* h, const dsa_plan* plan, const int32_t* sel,
                                      const void* q_nope, const void* q_pe, const void* latent_pool,
                                      float sm_scale, const float* sink, void* out, void* ws,
                                      size_t ws_bytes, void* stream);

/* The two halves of dsa_index_topk, for tests.
 * dsa_index_scores writes scores[t][j] (fp32, row stride ld >= max position + 1) for
 * j <= position(t) and -inf for position(t) < j < ld.
 * dsa_select_topk selects from such a score matrix exactly as dsa_index_topk does (scores must be
 * finite for j <= position(t)); ws of dsa_workspace_size(DSA_OP_SELECT_TOPK). */
dsa_status dsa_index_scores(const dsa_handle* h, const dsa_plan* plan, const void* q, const float* w,
                            const void* key_pool, float* scores, int64_t ld, void* stream);
dsa_status dsa_select_topk(const dsa_handle* h, const dsa_plan* plan, const float* scores,
                           int64_t ld, int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Block-sparse MSA (page "Sparse attention (DSA and block-sparse MSA)", table "Two shapes, three
 * checkpoints" and section "What the KV cache actually holds"): each row keeps the top blocks of
 * block_size tokens and attends over plain GQA. Index keys are one vector per token in the
 * index-key pool layout above (the page's bf16 index row: 128 dims, 256 B); a token's score is
 * the DSA indexer's, sum_h w[h] * relu(q[h] . k_j) in fp32, and a block scores as its best token
 * the row may see (positions 0 .. its own). The GQA pool holds per token the row
 * [K: n_kv_heads x head_dim | V: n_kv_heads x head_dim] in q_fmt elements (2,048 B for 4 x 128
 * bf16), paged like the latent pool. Plans are dsa_plan, as above. */
typedef struct {
  int32_t n_index_heads;  /* index query heads (1..128) */
  int32_t index_dim;      /* index vector width (multiple of 8, <= 512) */
  int32_t index_q_fmt;    /* F32 or BF16 */
  int32_t index_key_fmt;  /* F32, BF16 or FP8 (as DSA index keys) */
  int32_t block_size;     /* tokens per block: 32, 64, 128 or 256 */
  int32_t topk_blocks;    /* blocks kept per row (1..64) */
  int32_t n_heads;        /* query heads H (1..256) */
  int32_t n_kv_heads;     /* KV heads; n_heads % n_kv_heads == 0 */
  int32_t head_dim;       /* d (multiple of 8, 8..256) */
  int32_t q_fmt;          /* q, the GQA pool and the output: F32 or BF16 */
  int32_t page_size;      /* tokens per page (1..4096) */
} dsa_msa_config;

typedef struct dsa_msa_handle dsa_msa_handle;

dsa_status dsa_msa_create(const dsa_msa_config* cfg, dsa_msa_handle** out);
void dsa_msa_destroy(dsa_msa_handle* h);
/* Workspace bytes for DSA_OP_SELECT_TOPK (dsa_msa_select_blocks: the fp32 token scores and one
 * 8-byte key per block) or DSA_OP_ATTEND (dsa_msa_attend: an fp32 partial output, max and sum
 * per row, query head and picked block). */
dsa_status dsa_msa_workspace_size(const dsa_msa_handle* h, const dsa_plan* plan, int32_t op,
                                  size_t* bytes);

/* Block selection: for every row t, the top topk_blocks blocks 0 .. position(t) / block_size by
 * block score descending, equal scores by block ascending, the first min(topk_blocks, blocks
 * seen) of them followed by -1 entries.
 *   q    [n_rows][n_index_heads][index_dim] in index_q_fmt;  w [n_rows][n_index_heads] fp32
 *   key_pool  the index-key pool (every position the rows see already stored)
 *   sel  [n_rows][topk_blocks] int32 output (request-local block numbers)
 *   ws   256-byte aligned device scratch of dsa_msa_workspace_size(DSA_OP_SELECT_TOPK) bytes
 *        (DSA_ERR_WORKSPACE if missing or short); it holds the token scores afterwards
 * q, key_pool: 16-byte aligned; w, sel: 4-byte aligned (DSA_ERR_INVALID_ARG otherwise). Both MSA
 * calls are asynchronous on `stream`, allocate nothing and may be captured in a HIP graph. */
dsa_status dsa_msa_select_blocks(const dsa_msa_handle* h, const dsa_plan* plan, const void* q,
                                 const float* w, const void* key_pool, int32_t* sel, void* ws,
                                 size_t ws_bytes, void* stream);

/* GQA over the picked blocks: query head h uses KV head h / (n_heads / n_kv_heads) and attends
 * every position of its row's picked blocks up to the row's own,
 *   out[t][h] = sum_j softmax(sm_scale * q[t][h] . K_j)_j V_j ;
 * entries of sel < 0 are skipped, a row with none gets a zero output; a block listed twice
 * counts twice.
 *   sel  [n_rows][topk_blocks] int32 (as dsa_msa_select_blocks writes it)
 *   q    [n_rows][n_heads][head_dim];  out [n_rows][n_heads][head_dim], both in q_fmt
 *   ws   256-byte aligned device scratch of dsa_msa_workspace_size(DSA_OP_ATTEND) bytes;
 *        DSA_ERR_WORKSPACE if missing or short
 *   sm_scale  finite (DSA_ERR_INVALID_ARG otherwise)
 * q, gqa_pool, out: 16-byte aligned. Logits, maxima and sums are fp32; for bf16 caches of
 * head_dim 64, 128 or 256 with blocks of at most 128 tokens the matrix cores take the softmax
 * weights in bf16, other shapes keep them in fp32. */
dsa_status dsa_msa_attend(const dsa_msa_handle* h, const dsa_plan* plan, const int32_t* sel,
                          const void* q, const void* gqa_pool, float sm_scale, void* out,
                          void* ws, size_t ws_bytes, void* stream);

const char* dsa_status_str(dsa_status s);
/* Message of the calling thread's last failed call ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
