"""Plain, slow CPU oracle of DeepSeek Sparse Attention select + attend (numpy, float64).

TEST INFRASTRUCTURE. Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the GPU library and imports nothing from it.

Each function states the definition it writes out. The pages cited:
  * "mstar.engine.resources.dsa.manager" (the DSA resource API page): module description (the
    indexer score, top-k per row, absorbed MLA over picked latents), ``index_topk``,
    ``select_topk_causal``, ``attend``, ``store_keys``, ``DSAPlan``, ``DSASpan``.
  * "ttnn.transformer.sparse_sdpa": the operation line (softmax(Q K^T scale) V with
    V = kv[..., :v_dim], masked entries as a contiguous tail), the ``kv`` parameter (packed
    656-byte fp8 row [512 fp8 | 4 fp32 scales | 64 bf16 rope]), the ``q`` parameter (bf16 or
    e4m3), the ``attention_sink`` parameter and the ``Returns`` line.
  * "Sparse attention (DSA and block-sparse MSA)": the table of what the KV cache holds
    (1,152 B latent, 132 B index row: 128 fp8 keys + fp32 scale).

Readings where the pages leave a step open (listed again in the design notes):
  * scores are defined "in fp32" without an order: computed here in float64 and rounded once to
    float32; the selection then orders those float32 values.
  * ties are IEEE equality of the float32 scores (so -0.0 == +0.0) and go to the lower position.
  * the output order is the stable sort's order: score descending, position ascending, then the
    -1 tail.
  * an fp8 index key is e4m3(byte) * scale; an fp8 latent element d < R is e4m3(byte) *
    scale[d // 128]; the rope part is bf16. e4m3 is the OCP e4m3fn format.
  * the attention output is returned in float64; callers round to the query dtype (for e4m3
    queries the output is e4m3 too, as the Returns line of ttnn.transformer.sparse_sdpa has it).
  * the attention sink is one value per head, taken in the units of the unscaled logits
    (q . c), so it enters the denominator as exp(sm_scale * sink); -inf means no sink.

Parity unpinned: the float32 accumulation order of any GPU implementation (only bounded by the
tolerances of the tests), and the absmax fp8 quantisation used to make inputs (generator only).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "e4m3_to_f64", "bf16_bits_to_f64", "index_page_bytes", "latent_row_bytes", "row_spans",
    "token_pages", "read_index_keys", "read_latents", "store_keys", "index_scores_row",
    "select_topk_causal_row", "index_topk", "sparse_mla_attend", "dense_causal_mla",
]


# ----------------------------------------------------------------------------------------------
# Storage formats
# ----------------------------------------------------------------------------------------------

def e4m3_to_f64(b) -> np.ndarray:
    """OCP e4m3fn byte -> value: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m / 8 * 2^-6); field 15 with mantissa 7 is NaN; there is no
    infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def bf16_bits_to_f64(u) -> np.ndarray:
    """bfloat16 bit pattern -> value: the upper 16 bits of an IEEE float32."""
    u = np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _elems_to_f64(raw: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(raw)
    raise ValueError(fmt)


def index_page_bytes(fmt: str, page_size: int, dim: int) -> int:
    """One index-key page: f32/bf16 rows, or (fp8) page_size*dim e4m3 bytes then page_size fp32
    scales - each token's 132-byte record (128 fp8 keys + its scale) kept in the same page."""
    if fmt == "fp8":
        return page_size * dim + 4 * page_size
    return page_size * dim * (4 if fmt == "f32" else 2)


def latent_row_bytes(fmt: str, rank: int, rope: int) -> int:
    """One latent token: R + P elements, or the packed fp8 row [R e4m3 | R/128 fp32 | P bf16]."""
    if fmt == "fp8":
        return rank * 1 + (rank // 128) * 4 + rope * 2
    return (rank + rope) * (4 if fmt == "f32" else 2)


# ----------------------------------------------------------------------------------------------
# Plan: rows, positions and pages (DSASpan / DSAPlan)
# ----------------------------------------------------------------------------------------------

def row_spans(spans: np.ndarray):
    """For every step row t: (span index, position). A span holds q_len rows from row q_start,
    the first at position ctx_start, so row t sits at ctx_start + (t - q_start) (DSASpan)."""
    out = []
    for s, (q_start, q_len, ctx_start, _po, _np, _pst) in enumerate(np.asarray(spans)):
        for i in range(int(q_len)):
            out.append((s, int(ctx_start) + i))
    return out


def token_pages(span, page_table: np.ndarray, page_size: int, positions: np.ndarray):
    """Pool page and offset of request-local positions: the span's page list starts at
    page_offset in the back-to-back page table and its position-0 token sits page_start slots
    into that list (DSAPlan: row_page_offset, row_start)."""
    page_offset, n_pages, page_start = int(span[3]), int(span[4]), int(span[5])
    slot = page_start + np.asarray(positions, dtype=np.int64)
    idx = slot // page_size
    if np.any(idx >= n_pages) or np.any(slot < 0):
        raise IndexError("position beyond the span's pages")
    return page_table[page_offset + idx].astype(np.int64), slot % page_size


def read_index_keys(key_pool: np.ndarray, fmt: str, span, page_table, page_size: int, dim: int,
                    n: int) -> np.ndarray:
    """The first n stored index keys of a request, decoded to float64 (n, dim)."""
    pages, offs = token_pages(span, page_table, page_size, np.arange(n))
    pb = index_page_bytes(fmt, page_size, dim)
    pool = np.asarray(key_pool, dtype=np.uint8).reshape(-1, pb)
    if fmt == "fp8":
        codes = pool[:, : page_size * dim].reshape(-1, page_size, dim)[pages, offs]
        scale = pool[:, page_size * dim:].copy().view(np.float32).reshape(-1, page_size)[pages, offs]
        return e4m3_to_f64(codes) * scale.astype(np.float64)[:, None]
    dt = np.float32 if fmt == "f32" else np.uint16
    rows = pool.view(dt).reshape(-1, page_size, dim)[pages, offs]
    return _elems_to_f64(rows, fmt)


def read_latents(latent_pool: np.ndarray, fmt: str, span, page_table, page_size: int, rank: int,
                 rope: int, positions) -> np.ndarray:
    """Latent rows of request-local positions decoded to float64 (len, rank + rope).

    Packed fp8 row: element d < rank is e4m3(byte d) * scale[d // 128]; the rope part follows
    the scales as bf16 (ttnn.transformer.sparse_sdpa, kv parameter)."""
    pages, offs = token_pages(span, page_table, page_size, positions)
    rb = latent_row_bytes(fmt, rank, rope)
    rows = np.asarray(latent_pool, dtype=np.uint8).reshape(-1, page_size, rb)[pages, offs]
    if fmt == "fp8":
        ng = rank // 128
        codes = e4m3_to_f64(rows[:, :rank]).reshape(-1, ng, 128)
        scale = rows[:, rank:rank + 4 * ng].copy().view(np.float32).astype(np.float64)
        nope = (codes * scale[:, :, None]).reshape(-1, rank)
        pe = bf16_bits_to_f64(rows[:, rank + 4 * ng:].copy().view(np.uint16))
        return np.concatenate([nope, pe], axis=1)
    dt = np.float32 if fmt == "f32" else np.uint16
    return _elems_to_f64(rows.copy().view(dt), fmt)


def store_keys(key_pool: np.ndarray, fmt: str, spans, page_table, page_size: int, dim: int,
               keys: np.ndarray, scales: np.ndarray | None) -> np.ndarray:
    """store_keys: row t's (dim,) key goes to its request at position ctx_start + t - q_start.
    Returns a new pool (bytes); the stored bytes are the given ones unchanged."""
    pb = index_page_bytes(fmt, page_size, dim)
    pool = np.array(key_pool, dtype=np.uint8, copy=True).reshape(-1, pb)
    spans = np.asarray(spans)
    for t, (s, pos) in enumerate(row_spans(spans)):
        (page,), (off,) = token_pages(spans[s], page_table, page_size, np.array([pos]))
        if fmt == "fp8":
            pool[page, off * dim:(off + 1) * dim] = np.asarray(keys[t], dtype=np.uint8)
            sb = np.asarray([scales[t]], dtype=np.float32).view(np.uint8)
            pool[page, page_size * dim + 4 * off: page_size * dim + 4 * off + 4] = sb
        else:
            dt = np.float32 if fmt == "f32" else np.uint16
            b = np.asarray(keys[t], dtype=dt).view(np.uint8)
            pool[page, off * b.size:(off + 1) * b.size] = b
    return pool.reshape(-1)


# ----------------------------------------------------------------------------------------------
# Indexer score and causal top-k (index_topk, select_topk_causal)
# ----------------------------------------------------------------------------------------------

def index_scores_row(q_t: np.ndarray, w_t: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Score of one query row against its visible keys: s[j] = sum_h w[h] * relu(q[h] . k[j]).

    q_t (H, D), w_t (H,), keys (n, D) - all float64. Evaluated in float64 and rounded once to
    float32 (the module description of the DSA resource defines the score in fp32)."""
    dots = keys @ q_t.T                      # (n, H): q[h] . k[j]
    s = np.maximum(dots, 0.0) @ w_t          # sum over heads of w[h] * relu(.)
    return s.astype(np.float32)


def select_topk_causal_row(scores: np.ndarray, position: int, topk: int) -> np.ndarray:
    """select_topk_causal for one row: keys 0..position are visible (the row sees itself);
    order them by score descending, ties toward the earlier position (one stable sort), keep
    the first min(topk, position + 1) and pad with -1 to topk entries."""
    s = np.asarray(scores[: position + 1], dtype=np.float32)
    if not np.all(np.isfinite(s)):
        raise ValueError("scores must be finite")
    j = np.arange(position + 1)
    order = np.lexsort((j, -s.astype(np.float64)))   # primary: -score ascending; then j ascending
    out = np.full(topk, -1, dtype=np.int32)
    n = min(topk, position + 1)
    out[:n] = order[:n]
    return out


def index_topk(wl_q: np.ndarray, wl_w: np.ndarray, key_pool: np.ndarray, key_fmt: str, spans,
               page_table, page_size: int, topk: int, rows=None, return_scores=False):
    """index_topk over a step: every row scores its request's keys 0..position and keeps its
    causal top-k. q (T, H, D) and w (T, H) float64; returns {row: (topk,) int32} (and scores)."""
    spans = np.asarray(spans)
    rs = row_spans(spans)
    rows = range(len(rs)) if rows is None else rows
    dim = wl_q.shape[2]
    sel, sc = {}, {}
    cache = {}
    for t in rows:
        s, pos = rs[t]
        if s not in cache:
            n = int(spans[s][2]) + int(spans[s][1])
            cache = {s: read_index_keys(key_pool, key_fmt, spans[s], page_table, page_size, dim, n)}
        keys = cache[s][: pos + 1]
        scores = index_scores_row(wl_q[t], wl_w[t], keys)
        sel[t] = select_topk_causal_row(scores, pos, topk)
        sc[t] = scores
    return (sel, sc) if return_scores else sel


# ----------------------------------------------------------------------------------------------
# Absorbed MLA over the picked latents (attend)
# ----------------------------------------------------------------------------------------------

def sparse_mla_attend(sel: dict, q_nope: np.ndarray, q_pe: np.ndarray, latent_pool, latent_fmt: str,
                      spans, page_table, page_size: int, sm_scale: float, return_abs: bool = False,
                      sink=None):
    """attend: for each row and head, logits over the row's selected positions j (-1 = none)
    are sm_scale * (q_nope[h] . c_j[:R] + q_pe[h] . c_j[R:]); the output is the softmax-weighted
    sum of c_j[:R] (V is the leading R columns of the latent). Returns {row: (H, R) float64}.
    A row whose selection is empty yields zeros. With return_abs, also {row: sum_j p_j |c_j[:R]|},
    the scale that rounding the weights p_j (or the values) perturbs the output by.

    sink (H,) adds one term per head to the softmax denominator only: exp(sm_scale * sink[h])
    (ttnn.transformer.sparse_sdpa, attention_sink: the sink is multiplied by the scale and joins
    the denominator, never the numerator). A sink of -inf adds nothing."""
    spans = np.asarray(spans)
    rs = row_spans(spans)
    H, R = q_nope.shape[1], q_nope.shape[2]
    P = q_pe.shape[2]
    if sink is not None:
        sink = np.asarray(sink, dtype=np.float64).reshape(H)
        sink_logit = np.where(np.isneginf(sink), -np.inf, sm_scale * sink)[:, None]   # (H, 1)
    out, mag = {}, {}
    for t, picks in sel.items():
        s, _pos = rs[t]
        j = np.asarray(picks)
        j = j[j >= 0]
        if j.size == 0:
            out[t] = np.zeros((H, R))
            mag[t] = np.zeros((H, R))
            continue
        c = read_latents(latent_pool, latent_fmt, spans[s], page_table, page_size, R, P, j)
        logits = sm_scale * (q_nope[t] @ c[:, :R].T + q_pe[t] @ c[:, R:].T)   # (H, n)
        m = logits.max(axis=1, keepdims=True)
        if sink is not None:
            m = np.maximum(m, sink_logit)
        e = np.exp(logits - m)
        den = e.sum(axis=1, keepdims=True)
        if sink is not None:
            den = den + np.exp(sink_logit - m)
        p = e / den
        out[t] = p @ c[:, :R]
        if return_abs:
            mag[t] = p @ np.abs(c[:, :R])
    return (out, mag) if return_abs else out


def dense_causal_mla(q_nope: np.ndarray, q_pe: np.ndarray, latent_pool, latent_fmt: str, spans,
                     page_table, page_size: int, sm_scale: float, rows) -> dict:
    """Dense causal MLA, kept apart from the sparse path to check it: row t attends every
    position 0..p_t of its request with torch's float64 scaled-dot-product attention."""
    import torch

    spans = np.asarray(spans)
    rs = row_spans(spans)
    R, P = q_nope.shape[2], q_pe.shape[2]
    out = {}
    for t in rows:
        s, pos = rs[t]
        c = read_latents(latent_pool, latent_fmt, spans[s], page_table, page_size, R, P,
                         np.arange(pos + 1))
        q = torch.from_numpy(np.concatenate([q_nope[t], q_pe[t]], axis=1))[None]     # (1, H, R+P)
        k = torch.from_numpy(c)[None, None].expand(1, q.shape[1], -1, -1)
        v = torch.from_numpy(c[:, :R])[None, None].expand(1, q.shape[1], -1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(q[:, :, None], k, v, scale=sm_scale)
        out[t] = o[0, :, 0].numpy()
    return out
