"""Device state of one DSA step and the calls that run it (marshalling over the C ABI only).

A step is: store this step's index keys, index_topk (scores + causal top-k) once, then attend for
the FULL layer and for every SHARED layer that reuses the same selection.
"""
from __future__ import annotations

import torch

from . import dsa


def _dev(x, device):
    return None if x is None else x.to(device).contiguous()


class DSAStep:
    def __init__(self, *, n_index_heads, index_dim, index_q_fmt, index_key_fmt, topk, n_heads,
                 kv_lora_rank, rope_dim, q_fmt, latent_fmt, page_size, sm_scale, spans, page_table,
                 pool_pages, index_q, index_w, step_keys, step_key_scales, key_pool, q_nope, q_pe,
                 latent_pools, sinks=None, device="cuda", check_pages=True):
        self.cfg = dsa.make_config(n_index_heads, index_dim, index_q_fmt, index_key_fmt, topk,
                                   n_heads, kv_lora_rank, rope_dim, q_fmt, latent_fmt, page_size)
        self.h = dsa.dsa_create(self.cfg)
        self.plan = dsa.Plan.on_device(spans, page_table, pool_pages, device, check_pages)
        self.sm_scale = float(sm_scale)
        self.topk = int(topk)
        T = self.plan.n_rows
        self.index_q = _dev(index_q, device)
        self.index_w = _dev(index_w, device)
        self.step_keys = _dev(step_keys, device)
        self.step_key_scales = _dev(step_key_scales, device)
        self.key_pool = _dev(key_pool, device)
        self.q_nope = [_dev(x, device) for x in q_nope]
        self.q_pe = [_dev(x, device) for x in q_pe]
        self.latent_pools = [_dev(x, device) for x in latent_pools]
        # per attend layer: (H,) fp32 attention sink or None
        self.sinks = [_dev(x, device) for x in (sinks or [None] * len(self.q_nope))]
        qdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[q_fmt]
        self.sel = torch.empty(T, self.topk, dtype=torch.int32, device=device)
        self.out = [torch.empty(T, n_heads, kv_lora_rank, dtype=qdt, device=device)
                    for _ in self.q_nope]
        self.ws_index = self._ws(dsa.DSA_OP_INDEX_TOPK, device)
        self.ws_attend = self._ws(dsa.DSA_OP_ATTEND, device)

    def _ws(self, op, device):
        n = dsa.dsa_workspace_size(self.h, self.plan, op)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    @classmethod
    def from_workload(cls, wl, device="cuda", n_layers=None, check_pages=True):
        s = wl.spec
        n = len(wl.q_nope) if n_layers is None else n_layers
        return cls(n_index_heads=s.n_index_heads, index_dim=s.index_dim, index_q_fmt=s.index_q_fmt,
                   index_key_fmt=s.index_key_fmt, topk=s.topk, n_heads=s.n_heads,
                   kv_lora_rank=s.kv_lora_rank, rope_dim=s.rope_dim, q_fmt=s.q_fmt,
                   latent_fmt=s.latent_fmt, page_size=s.page_size, sm_scale=s.sm_scale,
                   spans=wl.spans, page_table=wl.page_table, pool_pages=wl.pool_pages,
                   index_q=wl.index_q, index_w=wl.index_w, step_keys=wl.step_keys,
                   step_key_scales=wl.step_key_scales, key_pool=wl.key_pool,
                   q_nope=wl.q_nope[:n], q_pe=wl.q_pe[:n], latent_pools=wl.latent_pools[:n],
                   sinks=wl.sinks[:n], device=device, check_pages=check_pages)

    # ---- the calls
    def store_keys(self, key_pool=None, stream=None):
        dsa.dsa_store_keys(self.h, self.plan, self.step_keys, self.step_key_scales,
                           self.key_pool if key_pool is None else key_pool, stream)

    def index_topk(self, key_pool=None, stream=None):
        dsa.dsa_index_topk(self.h, self.plan, self.index_q, self.index_w,
                           self.key_pool if key_pool is None else key_pool, self.sel,
                           self.ws_index, stream=stream)

    def attend(self, layer=0, latent_pool=None, stream=None):
        pool = self.latent_pools[layer] if latent_pool is None else latent_pool
        if self.sinks[layer] is None:
            dsa.dsa_sparse_mla_attend(self.h, self.plan, self.sel, self.q_nope[layer], self.q_pe[layer],
                                      pool, self.sm_scale, self.out[layer], self.ws_attend, stream=stream)
        else:
            dsa.dsa_sparse_mla_attend_sink(self.h, self.plan, self.sel, self.q_nope[layer],
                                           self.q_pe[layer], pool, self.sm_scale, self.sinks[layer],
                                           self.out[layer], self.ws_attend, stream=stream)

    def run(self, stream=None):
        """One whole step: store, select, then every attend layer (FULL + SHARED reuse)."""
        self.store_keys(stream=stream)
        self.index_topk(stream=stream)
        for layer in range(len(self.q_nope)):
            self.attend(layer, stream=stream)


class MSAStep:
    """Device state of one block-sparse MSA step: select the top blocks, then GQA over them."""

    def __init__(self, wl, device="cuda"):
        s = wl.spec
        self.cfg = dsa.make_msa_config(s.n_index_heads, s.index_dim, "bf16", s.index_key_fmt, s.block,
                                       s.topk_blocks, s.n_heads, s.n_kv_heads, s.head_dim, s.q_fmt,
                                       s.page_size)
        self.h = dsa.dsa_msa_create(self.cfg)
        self.plan = dsa.Plan.on_device(wl.spans, wl.page_table, wl.pool_pages, device)
        self.sm_scale = float(s.sm_scale)
        self.index_q = _dev(wl.index_q, device)
        self.index_w = _dev(wl.index_w, device)
        self.key_pool = _dev(wl.key_pool, device)
        self.q = _dev(wl.q, device)
        self.gqa_pool = _dev(wl.gqa_pool, device)
        T = self.plan.n_rows
        self.sel = torch.empty(T, s.topk_blocks, dtype=torch.int32, device=device)
        odt = torch.float32 if s.q_fmt == "f32" else torch.bfloat16
        self.out = torch.empty(T, s.n_heads, s.head_dim, dtype=odt, device=device)
        n = dsa.dsa_msa_workspace_size(self.h, self.plan, dsa.DSA_OP_SELECT_TOPK)
        self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
        n = dsa.dsa_msa_workspace_size(self.h, self.plan, dsa.DSA_OP_ATTEND)
        self.attend_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def select(self, key_pool=None, stream=None):
        dsa.dsa_msa_select_blocks(self.h, self.plan, self.index_q, self.index_w,
                                  self.key_pool if key_pool is None else key_pool, self.sel, self.ws,
                                  stream=stream)

    def attend(self, gqa_pool=None, stream=None):
        dsa.dsa_msa_attend(self.h, self.plan, self.sel, self.q,
                           self.gqa_pool if gqa_pool is None else gqa_pool, self.sm_scale, self.out,
                           self.attend_ws, stream=stream)
