"""Seeded synthetic block-sparse MSA workloads: index vectors, GQA caches, queries and pages.

Shapes follow the page "Sparse attention (DSA and block-sparse MSA)": top 16 blocks of 128
tokens, plain GQA with a 2,048-byte bf16 cache row per token (here 4 KV heads x 128 dims, K then
V), and one bf16 index vector per token (256 bytes: 128 dims). The index query side is the DSA
indexer's (64 heads x 128 dims, fp32 head weights), so the same score machinery serves both.
No public dataset exists for this path; these draws stand in for the page's shapes.

Nothing here scores, selects or attends. Every key of every position a row may see (its own
included) is written to the index pool, and every token's K and V to the GQA pool.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from .workloads import _absmax_scale, _fp8_bytes, _normal, _slots, _uniform_ints, index_page_bytes


@dataclass
class MsaSpec:
    name: str
    seed: int
    requests: list = field(default_factory=list)    # (q_len, ctx_start) per request
    page_starts: list | None = None
    n_index_heads: int = 64
    index_dim: int = 128
    w_scale: float = 1.0 / 8.0
    block: int = 128
    topk_blocks: int = 16
    n_heads: int = 32
    n_kv_heads: int = 4
    head_dim: int = 128
    page_size: int = 64
    spare_pages: int = 0
    q_fmt: str = "bf16"       # q, the GQA cache and the output: bf16 or f32
    index_key_fmt: str = "bf16"   # index keys: bf16, or fp8 codes with a per-token scale

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass
class MsaWorkload:
    spec: MsaSpec
    spans: np.ndarray          # (n_spans, 6) int32 as the DSA plan
    page_table: np.ndarray
    pool_pages: int
    index_q: torch.Tensor      # (T, H_i, D) bf16
    index_w: torch.Tensor      # (T, H_i) f32
    key_pool: torch.Tensor     # index-key pool bytes (DSA layout), keys of every position
    q: torch.Tensor            # (T, H, d) in q_fmt
    gqa_pool: torch.Tensor     # (pool_pages * page_size * 2 * H_kv * d * elem,) uint8

    @property
    def n_rows(self) -> int:
        return int(self.spans[:, 1].sum())

    @property
    def positions(self) -> np.ndarray:
        out = np.empty(self.n_rows, dtype=np.int64)
        for q_start, q_len, ctx_start, *_ in self.spans:
            out[q_start:q_start + q_len] = ctx_start + np.arange(q_len)
        return out


def make_msa_workload(name_or_spec) -> MsaWorkload:
    spec = MSA_WORKLOADS[name_or_spec]() if isinstance(name_or_spec, str) else name_or_spec
    gen = torch.Generator().manual_seed(spec.seed)
    ps = spec.page_size
    starts = spec.page_starts or [0] * len(spec.requests)
    spans, q_start, page_offset = [], 0, 0
    for (q_len, ctx_start), page_start in zip(spec.requests, starts):
        n_pages = -(-(page_start + ctx_start + q_len) // ps)
        spans.append((q_start, q_len, ctx_start, page_offset, n_pages, page_start))
        q_start += q_len
        page_offset += n_pages
    spans = np.asarray(spans, dtype=np.int32)
    pool_pages = page_offset + spec.spare_pages
    page_table = torch.randperm(pool_pages, generator=gen).numpy().astype(np.int32)[:page_offset].copy()
    T, D, Hi = int(spans[:, 1].sum()), spec.index_dim, spec.n_index_heads
    index_q = _normal(gen, (T, Hi, D)).to(torch.bfloat16)
    index_w = torch.rand(T, Hi, generator=gen, dtype=torch.float32) * spec.w_scale

    H, Hkv, d = spec.n_heads, spec.n_kv_heads, spec.head_dim
    qdt, gdt = (torch.float32, np.float32) if spec.q_fmt == "f32" else (torch.bfloat16, np.uint16)
    q = _normal(gen, (T, H, d)).to(qdt)
    fp8 = spec.index_key_fmt == "fp8"
    key_bytes = np.zeros((pool_pages, index_page_bytes(spec.index_key_fmt, ps, D)), dtype=np.uint8)
    if fp8:                                   # per page: ps x D codes, then ps fp32 scales
        kcodes = key_bytes[:, : ps * D].reshape(pool_pages, ps, D)
        kscale = key_bytes[:, ps * D:].view(np.float32).reshape(pool_pages, ps)
    else:
        keys = key_bytes.view(np.uint16).reshape(pool_pages, ps, D)
    gqa = np.zeros((pool_pages, ps, 2 * Hkv * d), dtype=gdt)
    for span in spans:
        n_tok = int(span[2]) + int(span[1])
        pages, offs = _slots(span, page_table, ps, n_tok)
        for c0 in range(0, n_tok, 1 << 15):
            c1 = min(n_tok, c0 + (1 << 15))
            kx = _normal(gen, (c1 - c0, D))
            kv = _normal(gen, (c1 - c0, 2 * Hkv * d))
            kv = (kv.numpy().astype(np.float32) if spec.q_fmt == "f32"
                  else kv.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
            if fp8:
                sc = _absmax_scale(kx)
                kcodes[pages[c0:c1], offs[c0:c1]] = _fp8_bytes(kx, sc)
                kscale[pages[c0:c1], offs[c0:c1]] = sc[:, 0].numpy()
            else:
                keys[pages[c0:c1], offs[c0:c1]] = kx.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            gqa[pages[c0:c1], offs[c0:c1]] = kv
    return MsaWorkload(spec=spec, spans=spans, page_table=page_table, pool_pages=pool_pages,
                       index_q=index_q, index_w=index_w,
                       key_pool=torch.from_numpy(key_bytes.reshape(-1)),
                       q=q, gqa_pool=torch.from_numpy(gqa.reshape(-1).view(np.uint8)))


def msa_decode_small() -> MsaSpec:
    # decode rows: a spread of contexts, a row at position 0 (one block of one token), one at
    # position 127 (one full block) and one at 128 (a second block of one token)
    ctx = _uniform_ints(3001, 5, 300, 5000)
    reqs = [(1, L - 1) for L in ctx] + [(1, 0), (1, 127), (1, 128)]
    return MsaSpec(name="msa_decode_small", seed=3001, requests=reqs,
                   page_starts=[0, 7, 63, 1, 30, 0, 5, 64], spare_pages=2)


def msa_prefill_small() -> MsaSpec:
    # a chunk crossing block boundaries on a long context, a fresh prompt, a decode row
    return MsaSpec(name="msa_prefill_small", seed=3002, requests=[(150, 1900), (20, 0), (1, 2500)],
                   page_starts=[3, 0, 40])


def msa_generic_f32() -> MsaSpec:
    # fp32 cache, 256-token blocks, 32 query heads per KV head (two head groups), head_dim 256:
    # the attention takes a block in chunks of 32 tokens
    return MsaSpec(name="msa_generic_f32", seed=3004, requests=[(1, 1700), (3, 600), (1, 255), (1, 256)],
                   page_starts=[5, 0, 17, 2], block=256, topk_blocks=4, n_heads=64, n_kv_heads=2,
                   head_dim=256, page_size=32, q_fmt="f32")


def msa_generic_small() -> MsaSpec:
    # 32-token blocks, head_dim 24 (three 16-byte pieces a head row), 2 query heads per KV head,
    # more blocks kept than a short row has, and a row with 2,189 blocks (more than one tile of
    # the block ranking)
    return MsaSpec(name="msa_generic_small", seed=3005,
                   requests=[(1, 700), (5, 95), (1, 40), (1, 0), (1, 70000)],
                   page_starts=[3, 9, 0, 15, 6], block=32, topk_blocks=8, n_heads=6, n_kv_heads=3,
                   head_dim=24, page_size=16, n_index_heads=32, index_dim=64)


def msa_generic_bf16() -> MsaSpec:
    # bf16, head_dim 256 (32 pieces a head row), 16 query heads on one KV head, 64-token blocks
    return MsaSpec(name="msa_generic_bf16", seed=3006, requests=[(2, 900), (1, 63), (1, 64)],
                   page_starts=[1, 0, 30], block=64, topk_blocks=6, n_heads=16, n_kv_heads=1,
                   head_dim=256, page_size=32)


def msa_fp8keys_small() -> MsaSpec:
    # decode rows over fp8 index keys (132 B a token: codes and a per-token scale)
    ctx = _uniform_ints(3007, 6, 200, 6000)
    return MsaSpec(name="msa_fp8keys_small", seed=3007, requests=[(1, L - 1) for L in ctx],
                   page_starts=[0, 9, 33, 2, 63, 1], index_key_fmt="fp8")


def msa_long_decode() -> MsaSpec:
    """8 decode rows at 131072 context (1,024 blocks each)."""
    return MsaSpec(name="msa_long_decode", seed=3003, requests=[(1, 131072 - 1)] * 8)


def msa_pages48_small() -> MsaSpec:
    # 48-token pages (not a power of two): 128-token blocks straddle pages, bf16 index keys
    return MsaSpec(name="msa_pages48_small", seed=3008, requests=[(1, 1000), (3, 300), (1, 47), (1, 48)],
                   page_starts=[0, 47, 5, 1], page_size=48)


def msa_pages48_fp8_small() -> MsaSpec:
    # 48-token pages with fp8 index keys
    ctx = _uniform_ints(3009, 4, 200, 3000)
    return MsaSpec(name="msa_pages48_fp8_small", seed=3009, requests=[(1, L - 1) for L in ctx],
                   page_starts=[0, 9, 47, 2], page_size=48, index_key_fmt="fp8")


MSA_WORKLOADS = {
    "msa_decode_small": msa_decode_small,
    "msa_prefill_small": msa_prefill_small,
    "msa_long_decode": msa_long_decode,
    "msa_generic_f32": msa_generic_f32,
    "msa_generic_small": msa_generic_small,
    "msa_generic_bf16": msa_generic_bf16,
    "msa_fp8keys_small": msa_fp8keys_small,
    "msa_pages48_small": msa_pages48_small,
    "msa_pages48_fp8_small": msa_pages48_fp8_small,
}
