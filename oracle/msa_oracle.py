"""Plain, slow CPU oracle of block-sparse MSA selection and attention (numpy, float64).

TEST INFRASTRUCTURE. Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the GPU library and imports nothing from it; it reuses the DSA oracle's
plan, page and index-score definitions.

The page "Sparse attention (DSA and block-sparse MSA)" (table "Two shapes, three checkpoints" and
section "What the KV cache actually holds") fixes what is selected and over what: the top 16
blocks of 128 tokens, attention over plain GQA, one bf16 index vector per token (256 B), and a
GQA cache of 2 x kv_heads x head_dim bf16 values per token (2,048 B). Readings where it is silent
(listed again in the design notes):
  * a token's score is the DSA indexer's, sum_h w[h] * relu(q[h] . k_j), over the index vectors
    (the same selection machinery at another granularity), rounded once to float32;
  * a block's score is the largest score among its tokens the row may see;
  * a row at position p sees blocks 0 .. p // block and, inside them, positions 0 .. p;
  * picked blocks are ordered by score descending, equal scores by block ascending, the first
    min(topk, visible blocks) of them followed by -1 entries;
  * query head h attends with KV head h // (H / H_kv) over every visible token of its row's
    picked blocks: out = softmax(scale * q . k) v;
  * a token's GQA row is [K: H_kv x d | V: H_kv x d] in bf16 (the page's cache), or in fp32
    where a caller keeps a full-precision cache.
"""
from __future__ import annotations

import numpy as np

from . import dsa_oracle as _dsa

__all__ = ["gqa_row_bytes", "read_gqa", "block_scores_row", "select_blocks_row", "msa_select",
           "block_positions", "msa_attend", "dense_causal_gqa"]


def gqa_row_bytes(n_kv: int, head_dim: int, fmt: str = "bf16") -> int:
    """Bytes of one token's GQA row: K and V for every KV head, bf16 (or fp32)."""
    return 2 * n_kv * head_dim * (4 if fmt == "f32" else 2)


def read_gqa(gqa_pool, span, page_table, page_size: int, n_kv: int, head_dim: int, positions,
             fmt: str = "bf16"):
    """K and V of request-local positions, float64 (n, n_kv, head_dim) each."""
    pages, offs = _dsa.token_pages(span, page_table, page_size, positions)
    rb = gqa_row_bytes(n_kv, head_dim, fmt)
    rows = np.asarray(gqa_pool, dtype=np.uint8).reshape(-1, page_size, rb)[pages, offs].copy()
    flat = (rows.view(np.float32).astype(np.float64) if fmt == "f32"
            else _dsa.bf16_bits_to_f64(rows.view(np.uint16)))
    vals = flat.reshape(-1, 2, n_kv, head_dim)
    return vals[:, 0], vals[:, 1]


def block_scores_row(token_scores: np.ndarray, position: int, block: int) -> np.ndarray:
    """Score of each block the row sees: the largest float32 score among its visible tokens."""
    s = np.asarray(token_scores[: position + 1], dtype=np.float32)
    nb = position // block + 1
    return np.array([s[b * block: min((b + 1) * block, position + 1)].max() for b in range(nb)],
                    dtype=np.float32)


def select_blocks_row(block_scores: np.ndarray, topk: int) -> np.ndarray:
    """Blocks by score descending, ties toward the lower block (one stable sort), the first
    min(topk, blocks) of them, then -1 entries up to topk."""
    s = np.asarray(block_scores, dtype=np.float32)
    b = np.arange(s.size)
    order = np.lexsort((b, -s.astype(np.float64)))
    out = np.full(topk, -1, dtype=np.int32)
    n = min(topk, s.size)
    out[:n] = order[:n]
    return out


def msa_select(q: np.ndarray, w: np.ndarray, key_pool, key_fmt: str, spans, page_table,
               page_size: int, topk: int, block: int, rows=None, return_scores=False):
    """Block selection over a step: token scores as the DSA indexer, block maxima, top blocks.
    q (T, H, D) and w (T, H) float64; returns {row: (topk,) int32} (and block scores)."""
    spans = np.asarray(spans)
    rs = _dsa.row_spans(spans)
    rows = range(len(rs)) if rows is None else rows
    dim = q.shape[2]
    sel, bsc, cache = {}, {}, {}
    for t in rows:
        s, pos = rs[t]
        if s not in cache:
            n = int(spans[s][2]) + int(spans[s][1])
            cache = {s: _dsa.read_index_keys(key_pool, key_fmt, spans[s], page_table, page_size, dim, n)}
        ts = _dsa.index_scores_row(q[t], w[t], cache[s][: pos + 1])
        bs = block_scores_row(ts, pos, block)
        sel[t] = select_blocks_row(bs, topk)
        bsc[t] = bs
    return (sel, bsc) if return_scores else sel


def block_positions(blocks, position: int, block: int) -> np.ndarray:
    """The positions a row attends: every visible position of its picked blocks (-1 = none)."""
    out = []
    for b in np.asarray(blocks):
        if b < 0:
            continue
        out.append(np.arange(b * block, min((b + 1) * block, position + 1)))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def msa_attend(sel: dict, q: np.ndarray, gqa_pool, spans, page_table, page_size: int, n_kv: int,
               head_dim: int, block: int, sm_scale: float, return_abs: bool = False,
               fmt: str = "bf16"):
    """GQA over the picked blocks: head h uses KV head h // (H / n_kv); softmax over the row's
    visible tokens of those blocks. q (T, H, d) float64; returns {row: (H, d) float64} (and, with
    return_abs, sum_j p_j |v_j|, the scale that rounding the weights perturbs the output by)."""
    spans = np.asarray(spans)
    rs = _dsa.row_spans(spans)
    H = q.shape[1]
    group = H // n_kv
    out, mag = {}, {}
    for t, picks in sel.items():
        s, pos = rs[t]
        j = block_positions(picks, pos, block)
        if j.size == 0:
            out[t] = np.zeros((H, head_dim))
            mag[t] = np.zeros((H, head_dim))
            continue
        k, v = read_gqa(gqa_pool, spans[s], page_table, page_size, n_kv, head_dim, j, fmt)
        o = np.empty((H, head_dim))
        m = np.empty((H, head_dim))
        for h in range(H):
            kv = h // group
            logits = sm_scale * (k[:, kv] @ q[t, h])
            e = np.exp(logits - logits.max())
            p = e / e.sum()
            o[h] = p @ v[:, kv]
            m[h] = p @ np.abs(v[:, kv])
        out[t], mag[t] = o, m
    return (out, mag) if return_abs else out


def dense_causal_gqa(q: np.ndarray, gqa_pool, spans, page_table, page_size: int, n_kv: int,
                     head_dim: int, sm_scale: float, rows, fmt: str = "bf16") -> dict:
    """Dense causal GQA, apart from the sparse path to check it: row t attends every position
    0 .. p_t with torch's float64 scaled-dot-product attention, KV heads repeated per group."""
    import torch

    spans = np.asarray(spans)
    rs = _dsa.row_spans(spans)
    H = q.shape[1]
    out = {}
    for t in rows:
        s, pos = rs[t]
        k, v = read_gqa(gqa_pool, spans[s], page_table, page_size, n_kv, head_dim, np.arange(pos + 1), fmt)
        kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(H // n_kv, dim=0)   # (H, n, d)
        vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(H // n_kv, dim=0)
        qq = torch.from_numpy(q[t])[:, None]                                            # (H, 1, d)
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=sm_scale)
        out[t] = o[:, 0].numpy()
    return out
