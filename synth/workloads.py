"""Seeded synthetic DSA workloads: shapes, draws, storage encodings and page placement.

Every tensor is drawn on the CPU from one ``torch.Generator`` seeded per workload, so the oracle
and the GPU library see identical bytes. The shapes follow the DSA path described on the page
"mstar.engine.resources.dsa.manager" (index keys per request by position, head weights, a span
plan with pages) and the cache formats of "ttnn.transformer.sparse_sdpa" (kv parameter: the
656-byte packed fp8 row) and "Sparse attention (DSA and block-sparse MSA)" (section "What the KV
cache actually holds": 1,152 B bf16 latent, 132 B fp8 index row). No public dataset exists for
this path; these draws stand in for the pages' workloads.

Nothing here scores, selects or attends. Encodings are torch casts (bf16, OCP e4m3fn) and a
per-token / per-128-group absmax scale used only to produce valid fp8 inputs.

Raw storage conventions handed to both sides:
  * ``f32``  - little-endian IEEE float32
  * ``bf16`` - bfloat16 (torch.bfloat16; numpy views use uint16 bit patterns)
  * ``fp8``  - OCP e4m3fn bytes with fp32 scales (index keys: one scale per token; latents:
               one scale per 128 latent elements, packed in the row)

Index-key pool, one page of ``page_size`` tokens:
  * f32/bf16: ``[page_size][D]`` elements
  * fp8:      ``[page_size][D]`` e4m3 bytes followed by ``[page_size]`` fp32 scales
Latent pool: ``[pages][page_size][row]`` with row = ``R+P`` elements (f32/bf16) or, for fp8,
``[R e4m3 | R/128 fp32 scales | P bf16]`` (656 bytes for R=512, P=64).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

FP8_MAX = 448.0  # largest finite OCP e4m3fn magnitude


def _esize(fmt: str) -> int:
    return {"f32": 4, "bf16": 2}[fmt]


def index_page_bytes(fmt: str, page_size: int, dim: int) -> int:
    """Bytes of one index-key page in the pool."""
    if fmt == "fp8":
        return page_size * (dim + 4)
    return page_size * dim * _esize(fmt)


def latent_row_bytes(fmt: str, rank: int, rope: int) -> int:
    """Bytes of one latent row (one token) in the pool."""
    if fmt == "fp8":
        return rank + 4 * (rank // 128) + 2 * rope
    return (rank + rope) * _esize(fmt)


@dataclass
class Spec:
    name: str
    seed: int
    # indexer
    n_index_heads: int
    index_dim: int
    index_q_fmt: str
    index_key_fmt: str
    topk: int
    w_scale: float
    # absorbed MLA
    n_heads: int
    kv_lora_rank: int
    rope_dim: int
    q_fmt: str
    latent_fmt: str
    page_size: int
    sm_scale: float
    # requests: (q_len, ctx_start) in row order; page_start per request
    requests: list = field(default_factory=list)
    page_starts: list | None = None
    n_attend_layers: int = 1
    shuffle_pages: bool = True
    spare_pages: int = 0
    sink: bool = False          # draw a per-head attention sink for every attend layer


@dataclass
class Workload:
    spec: Spec
    spans: np.ndarray          # (n_spans, 6) int32: q_start, q_len, ctx_start, page_offset, n_pages, page_start
    page_table: np.ndarray     # (n_page_ids,) int32
    pool_pages: int
    index_q: torch.Tensor      # (T, H_i, D) f32 or bf16
    index_w: torch.Tensor      # (T, H_i) f32
    step_keys: torch.Tensor    # (T, D) f32 / bf16, or uint8 e4m3 bytes
    step_key_scales: torch.Tensor | None  # (T,) f32 for fp8 keys
    key_pool: torch.Tensor     # (pool_pages * page_bytes,) uint8, history filled, this step's slots zero
    q_nope: list               # per attend layer: (T, H, R)
    q_pe: list                 # per attend layer: (T, H, P)
    latent_pools: list         # per attend layer: (pool_pages * page_size * row_bytes,) uint8
    sinks: list                # per attend layer: (H,) f32 attention sink, or None

    @property
    def n_rows(self) -> int:
        return int(self.spans[:, 1].sum())

    @property
    def positions(self) -> np.ndarray:
        """Position of every row: ctx_start + (row - q_start)."""
        out = np.empty(self.n_rows, dtype=np.int64)
        for q_start, q_len, ctx_start, *_ in self.spans:
            out[q_start:q_start + q_len] = ctx_start + np.arange(q_len)
        return out


def _normal(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def _to_fmt_elems(x: torch.Tensor, fmt: str) -> torch.Tensor:
    if fmt == "fp8":     # plain e4m3fn values, no scale (the q of ttnn.transformer.sparse_sdpa)
        return torch.clamp(x, -FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return x.to(torch.bfloat16) if fmt == "bf16" else x.to(torch.float32)


def _fp8_bytes(x: torch.Tensor, scale: torch.Tensor) -> np.ndarray:
    """Encode x / scale as e4m3fn bytes (scale broadcast over the last dim group)."""
    y = torch.clamp(x / scale, -FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _absmax_scale(x: torch.Tensor) -> torch.Tensor:
    a = x.abs().amax(dim=-1, keepdim=True) / FP8_MAX
    return torch.where(a > 0, a, torch.ones_like(a))


def _slots(span, page_table, page_size, n_tok):
    """Pool (page, offset) of positions 0..n_tok-1 of one span (paged layout of DSAPlan)."""
    page_offset, page_start = int(span[3]), int(span[5])
    slot = page_start + np.arange(n_tok, dtype=np.int64)
    pages = page_table[page_offset + slot // page_size].astype(np.int64)
    return pages, slot % page_size


def make_workload(name_or_spec, n_attend_layers: int | None = None) -> Workload:
    spec = WORKLOADS[name_or_spec]() if isinstance(name_or_spec, str) else name_or_spec
    if n_attend_layers is not None:
        spec.n_attend_layers = n_attend_layers
    gen = torch.Generator().manual_seed(spec.seed)
    ps = spec.page_size
    starts = spec.page_starts or [0] * len(spec.requests)

    # ---- span plan ----
    spans = []
    q_start = 0
    page_offset = 0
    for (q_len, ctx_start), page_start in zip(spec.requests, starts):
        n_tok = ctx_start + q_len
        n_pages = -(-(page_start + n_tok) // ps)
        spans.append((q_start, q_len, ctx_start, page_offset, n_pages, page_start))
        q_start += q_len
        page_offset += n_pages
    spans = np.asarray(spans, dtype=np.int32)
    pool_pages = page_offset + spec.spare_pages
    if spec.shuffle_pages:
        perm = torch.randperm(pool_pages, generator=gen).numpy().astype(np.int32)
    else:
        perm = np.arange(pool_pages, dtype=np.int32)
    page_table = perm[:page_offset].copy()
    T = int(spans[:, 1].sum())
    D, Hi = spec.index_dim, spec.n_index_heads

    # ---- indexer queries and head weights ----
    index_q = _to_fmt_elems(_normal(gen, (T, Hi, D)), spec.index_q_fmt)
    index_w = torch.rand(T, Hi, generator=gen, dtype=torch.float32) * spec.w_scale

    # ---- index keys: history into the pool, this step's rows returned separately ----
    kfmt = spec.index_key_fmt
    pbytes = index_page_bytes(kfmt, ps, D)
    key_pool = np.zeros((pool_pages, pbytes), dtype=np.uint8)
    if kfmt == "fp8":
        step_keys = np.zeros((T, D), dtype=np.uint8)
        step_scales = np.zeros((T,), dtype=np.float32)
        kdata = key_pool[:, : ps * D].reshape(pool_pages, ps, D)
        kscale = key_pool[:, ps * D:].view(np.float32).reshape(pool_pages, ps)
    else:
        np_dt = np.uint16 if kfmt == "bf16" else np.float32
        step_keys = np.zeros((T, D), dtype=np_dt)
        step_scales = None
        kdata = key_pool.view(np_dt).reshape(pool_pages, ps, D)
    for span in spans:
        qs, ql, cs = int(span[0]), int(span[1]), int(span[2])
        n_tok = cs + ql
        x = _normal(gen, (n_tok, D))
        pages, offs = _slots(span, page_table, ps, cs)  # history only
        if kfmt == "fp8":
            sc = _absmax_scale(x)
            b = _fp8_bytes(x, sc)
            kdata[pages, offs] = b[:cs]
            kscale[pages, offs] = sc[:cs, 0].numpy()
            step_keys[qs:qs + ql] = b[cs:]
            step_scales[qs:qs + ql] = sc[cs:, 0].numpy()
        else:
            e = _to_fmt_elems(x, kfmt)
            raw = e.view(torch.int16).numpy().view(np.uint16) if kfmt == "bf16" else e.numpy()
            kdata[pages, offs] = raw[:cs]
            step_keys[qs:qs + ql] = raw[cs:]
    if kfmt == "bf16":
        step_keys_t = torch.from_numpy(step_keys.view(np.int16)).view(torch.bfloat16)
    else:
        step_keys_t = torch.from_numpy(step_keys)
    step_scales_t = torch.from_numpy(step_scales) if step_scales is not None else None

    # ---- absorbed MLA: per attend layer its own queries and latent cache ----
    H, R, P = spec.n_heads, spec.kv_lora_rank, spec.rope_dim
    lfmt = spec.latent_fmt
    rb = latent_row_bytes(lfmt, R, P)
    q_nope, q_pe, latent_pools, sinks = [], [], [], []
    for _layer in range(spec.n_attend_layers):
        q_nope.append(_to_fmt_elems(_normal(gen, (T, H, R)), spec.q_fmt))
        q_pe.append(_to_fmt_elems(_normal(gen, (T, H, P)), spec.q_fmt))
        sinks.append(_sink(gen, H, spec.sm_scale) if spec.sink else None)
        pool = np.zeros((pool_pages, ps, rb), dtype=np.uint8)
        for span in spans:
            n_tok = int(span[2]) + int(span[1])
            pages, offs = _slots(span, page_table, ps, n_tok)
            # draw in chunks to bound temporary memory
            for c0 in range(0, n_tok, 1 << 16):
                c1 = min(n_tok, c0 + (1 << 16))
                x = _normal(gen, (c1 - c0, R + P))
                if lfmt == "fp8":
                    lat = x[:, :R].reshape(c1 - c0, R // 128, 128)
                    sc = _absmax_scale(lat)
                    b = _fp8_bytes(lat, sc).reshape(c1 - c0, R)
                    row = np.empty((c1 - c0, rb), dtype=np.uint8)
                    row[:, :R] = b
                    row[:, R:R + 4 * (R // 128)] = sc[..., 0].numpy().view(np.uint8).reshape(c1 - c0, -1)
                    rope = x[:, R:].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
                    row[:, R + 4 * (R // 128):] = rope.reshape(c1 - c0, 2 * P)
                else:
                    e = _to_fmt_elems(x, lfmt)
                    raw = e.view(torch.int16) if lfmt == "bf16" else e
                    row = raw.numpy().view(np.uint8).reshape(c1 - c0, rb)
                pool[pages[c0:c1], offs[c0:c1]] = row
        latent_pools.append(torch.from_numpy(pool.reshape(-1)))

    return Workload(spec=spec, spans=spans, page_table=page_table, pool_pages=pool_pages,
                    index_q=index_q, index_w=index_w, step_keys=step_keys_t,
                    step_key_scales=step_scales_t, key_pool=torch.from_numpy(key_pool.reshape(-1)),
                    q_nope=q_nope, q_pe=q_pe, latent_pools=latent_pools, sinks=sinks)


def _sink(gen: torch.Generator, H: int, sm_scale: float) -> torch.Tensor:
    """Per-head sinks in the units of the unscaled logits (the denominator gains
    exp(sm_scale * sink)). Scaled values ~U(-2, 12) span a negligible sink up to one that outweighs
    thousands of keys (log-sum-exp of 2048 such logits is about 9); head 0 has none (-inf), head 1
    one that dominates every key (scaled 60), head 2 a negligible finite one (scaled -60)."""
    scaled = torch.rand(H, generator=gen, dtype=torch.float64) * 14.0 - 2.0
    if H > 2:
        scaled[1], scaled[2] = 60.0, -60.0
    sink = (scaled / sm_scale).to(torch.float32)
    sink[0] = -math.inf
    return sink


# --------------------------------------------------------------------------------------------
# The workloads. Seeds are 1000 + workload index for the five named shapes.
# --------------------------------------------------------------------------------------------

def _big_dims(**kw) -> dict:
    d = dict(n_index_heads=64, index_dim=128, index_q_fmt="bf16", index_key_fmt="bf16", topk=2048,
             w_scale=1.0 / 8.0, n_heads=128, kv_lora_rank=512, rope_dim=64, q_fmt="bf16",
             latent_fmt="bf16", page_size=64, sm_scale=1.0 / math.sqrt(192.0))
    d.update(kw)
    return d


def _uniform_ints(seed: int, n: int, lo: int, hi: int) -> list:
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


def tiny_prefill() -> Spec:
    """1 request, 64 rows at positions 0..63, 4x32 fp32 indexer, topk 16, 8-head fp32 MLA 64+16."""
    return Spec(name="tiny_prefill", seed=1000, n_index_heads=4, index_dim=32, index_q_fmt="f32",
                index_key_fmt="f32", topk=16, w_scale=1.0, n_heads=8, kv_lora_rank=64, rope_dim=16,
                q_fmt="f32", latent_fmt="f32", page_size=16, sm_scale=1.0 / math.sqrt(80.0),
                requests=[(64, 0)])


def decode_batch() -> Spec:
    """32 decode rows, contexts ~U[4096, 32768], bf16 keys and latents, topk 2048."""
    ctx = _uniform_ints(1001 * 7, 32, 4096, 32768)
    return Spec(name="decode_batch", seed=1001, requests=[(1, L - 1) for L in ctx], **_big_dims())


def causal_prefill() -> Spec:
    """1 request, 8192 new rows from position 0, bf16, topk 2048."""
    return Spec(name="causal_prefill", seed=1002, requests=[(8192, 0)], **_big_dims())


def long_decode() -> Spec:
    """8 decode rows at 131072 context, fp8 132-byte index keys, 656-byte packed fp8 latents."""
    return Spec(name="long_decode", seed=1003, requests=[(1, 131072 - 1)] * 8,
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8"))


def chunked_mix() -> Spec:
    """4 x 2048-row prefill chunks on contexts ~U[16384, 65536] plus 16 decode rows at
    ~U[8192, 65536]; one indexer layer whose selection 3 more attend layers reuse."""
    pre = _uniform_ints(1004 * 7, 4, 16384, 65536)
    dec = _uniform_ints(1004 * 11, 16, 8192, 65536)
    reqs = [(2048, c) for c in pre] + [(1, L - 1) for L in dec]
    return Spec(name="chunked_mix", seed=1004, requests=reqs, n_attend_layers=4, **_big_dims())


# Reduced shapes of the same structure for tests the oracle finishes in seconds.

def decode_small() -> Spec:
    ctx = _uniform_ints(2001, 6, 700, 5000)
    return Spec(name="decode_small", seed=2001, requests=[(1, L - 1) for L in ctx],
                page_starts=[0, 5, 63, 0, 17, 1], spare_pages=3, **_big_dims())


def long_decode_small() -> Spec:
    ctx = _uniform_ints(2003, 4, 1500, 9000)
    return Spec(name="long_decode_small", seed=2003, requests=[(1, L - 1) for L in ctx],
                page_starts=[3, 0, 40, 0],
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8"))


def prefill_small() -> Spec:
    return Spec(name="prefill_small", seed=2002, requests=[(700, 37)], page_starts=[9],
                **_big_dims(topk=256))


def mix_small() -> Spec:
    reqs = [(300, 1100), (157, 2900), (1, 2500), (1, 90), (1, 4000)]
    return Spec(name="mix_small", seed=2004, requests=reqs, n_attend_layers=3,
                page_starts=[0, 11, 0, 60, 2], **_big_dims(topk=512))


def prefill_fp8_small() -> Spec:
    # fp8 index keys and packed fp8 latents under multi-row spans: a chunk over two key blocks, a
    # span of 9 rows (one group of 8 and one left over), a decode row, a fresh 16-row prompt
    reqs = [(203, 2100), (9, 50), (1, 300), (16, 0)]
    return Spec(name="prefill_fp8_small", seed=2005, requests=reqs, page_starts=[5, 0, 31, 2],
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8", topk=384, page_size=32))


def pages1_small() -> Spec:
    # one token per page (a 2048-key block spans 2048 pages) with bf16 keys, a prefill chunk and
    # two decode rows
    reqs = [(37, 2500), (1, 1800), (1, 40)]
    return Spec(name="pages1_small", seed=2006, requests=reqs,
                **_big_dims(topk=300, page_size=1))


def pages128_small() -> Spec:
    # 128-token pages with fp8 keys and packed fp8 latents, spans starting mid-page
    reqs = [(64, 3000), (1, 4500), (12, 130)]
    return Spec(name="pages128_small", seed=2007, requests=reqs, page_starts=[100, 3, 127],
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8", topk=512, page_size=128))


def many_spans_small() -> Spec:
    # 40 requests of 9 rows, more than the 32 spans the grouped score kernel takes at once, then
    # decode rows: groups, one leftover row per grouped span, whole spans scored row by row
    reqs = [(9, 60 + 37 * i) for i in range(40)] + [(1, 900), (1, 3)]
    return Spec(name="many_spans_small", seed=2008, requests=reqs, **_big_dims(topk=128))


def sink_decode_small() -> Spec:
    # per-head attention sinks over decode rows (picks split across workgroups and merged), a row
    # at position 0 with a single pick, and a SHARED layer with its own sinks
    ctx = _uniform_ints(2009, 5, 300, 6000)
    return Spec(name="sink_decode_small", seed=2009, requests=[(1, L - 1) for L in ctx] + [(1, 0)],
                page_starts=[7, 0, 63, 12, 1, 40], n_attend_layers=2, sink=True, **_big_dims())


def fp8q_sink_small() -> Spec:
    # e4m3 queries (and so e4m3 outputs) over fp8 keys and packed fp8 latents, with sinks: a
    # prefill chunk, decode rows and a fresh prompt
    reqs = [(40, 1500), (1, 2200), (1, 700), (1, 3900), (5, 0)]
    return Spec(name="fp8q_sink_small", seed=2010, requests=reqs, page_starts=[0, 9, 33, 2, 60],
                n_attend_layers=2, sink=True,
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8", q_fmt="fp8", topk=512))


def fp8q_small() -> Spec:
    # e4m3 queries over bf16 latents without a sink, decode rows only (merged splits)
    ctx = _uniform_ints(2011, 4, 900, 5000)
    return Spec(name="fp8q_small", seed=2011, requests=[(1, L - 1) for L in ctx],
                **_big_dims(q_fmt="fp8"))


def tiny_fp8q_sink() -> Spec:
    """The tiny shapes (no matrix-core kernel) with e4m3 queries and sinks over fp32 latents."""
    return Spec(name="tiny_fp8q_sink", seed=2012, n_index_heads=4, index_dim=32, index_q_fmt="f32",
                index_key_fmt="f32", topk=16, w_scale=1.0, n_heads=8, kv_lora_rank=64, rope_dim=16,
                q_fmt="fp8", latent_fmt="f32", page_size=16, sm_scale=1.0 / math.sqrt(80.0),
                requests=[(40, 0), (3, 50)], sink=True)


def sink_fp8_decode_small() -> Spec:
    # packed fp8 latents with bf16 queries and sinks over decode rows: the 32-head split kernel
    # with 16 pick-splits merged by the combine (which adds the sink), a row at position 0 and a
    # row of 41 picks, and a SHARED layer with its own sinks
    ctx = _uniform_ints(2013, 5, 300, 6000)
    return Spec(name="sink_fp8_decode_small", seed=2013,
                requests=[(1, L - 1) for L in ctx] + [(1, 0), (1, 40)],
                page_starts=[7, 0, 63, 12, 1, 40, 33], n_attend_layers=2, sink=True,
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8"))


def sink_fp8_rows_small() -> Spec:
    # enough rows (66) for the 32-head split kernel to run unsplit, so that it applies the sink
    # itself: a prefill chunk and decode rows, one at position 0
    reqs = [(60, 1000), (1, 2500), (1, 0), (1, 300), (1, 4000), (1, 50), (1, 1500)]
    return Spec(name="sink_fp8_rows_small", seed=2014, requests=reqs,
                page_starts=[3, 0, 20, 63, 1, 0, 9], n_attend_layers=2, sink=True,
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8", topk=256))


def steps_fp8_small() -> Spec:
    # 70 decode rows over fp8 keys and packed fp8 latents, top 400: the 32-head split kernel runs
    # unsplit with 400 picks a workgroup, 13 tiles of 32 in 4 steps (the last holding one tile),
    # applying the sink itself; rows at positions 0, 50 and 390 end their picks early
    ctx = _uniform_ints(2015, 67, 600, 4000)
    reqs = [(1, L - 1) for L in ctx] + [(1, 0), (1, 50), (1, 390)]
    return Spec(name="steps_fp8_small", seed=2015, requests=reqs, n_attend_layers=1, sink=True,
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8", topk=400))


def pages48_small() -> Spec:
    # 48-token pages (not a power of two) with bf16 keys and latents: a prefill chunk, decode rows
    # at the last slot of a page and the first of the next, spans starting mid-page
    reqs = [(37, 1000), (1, 2200), (1, 47), (1, 48)]
    return Spec(name="pages48_small", seed=2015, requests=reqs, page_starts=[5, 0, 47, 0],
                **_big_dims(topk=256, page_size=48))


def pages48_fp8_small() -> Spec:
    # 48-token pages with fp8 keys (6,336-byte pages) and packed fp8 latents
    reqs = [(20, 600), (1, 3000), (1, 0), (1, 95)]
    return Spec(name="pages48_fp8_small", seed=2016, requests=reqs, page_starts=[0, 13, 47, 1],
                **_big_dims(index_key_fmt="fp8", latent_fmt="fp8", topk=384, page_size=48))


def spans70_bf16_small() -> Spec:
    # 70 decode rows over bf16 keys and latents, top 128: more than the 64 spans one wave looks up
    # at once, so the rows past the first 64 spans take the lookup's second chunk in the score,
    # select and 128-head attention kernels
    ctx = _uniform_ints(2017, 70, 200, 3000)
    return Spec(name="spans70_bf16_small", seed=2017, requests=[(1, L - 1) for L in ctx],
                **_big_dims(topk=128))


WORKLOADS = {
    "tiny_prefill": tiny_prefill,
    "decode_batch": decode_batch,
    "causal_prefill": causal_prefill,
    "long_decode": long_decode,
    "chunked_mix": chunked_mix,
    "decode_small": decode_small,
    "long_decode_small": long_decode_small,
    "prefill_small": prefill_small,
    "mix_small": mix_small,
    "prefill_fp8_small": prefill_fp8_small,
    "pages1_small": pages1_small,
    "pages128_small": pages128_small,
    "many_spans_small": many_spans_small,
    "sink_decode_small": sink_decode_small,
    "fp8q_sink_small": fp8q_sink_small,
    "fp8q_small": fp8q_small,
    "tiny_fp8q_sink": tiny_fp8q_sink,
    "sink_fp8_decode_small": sink_fp8_decode_small,
    "sink_fp8_rows_small": sink_fp8_rows_small,
    "steps_fp8_small": steps_fp8_small,
    "pages48_small": pages48_small,
    "pages48_fp8_small": pages48_fp8_small,
    "spans70_bf16_small": spans70_bf16_small,
}
