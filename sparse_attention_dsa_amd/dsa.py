"""Python binding of libdsa (ctypes). Argument marshalling only: every step runs in the library.

Functions carry the C names. Tensor arguments may be torch tensors (their data pointer is passed)
or plain integers (device addresses, taken as they are). A tensor must be contiguous, live on the
GPU and hold at least the bytes its argument needs for the plan and configuration (the layouts of
include/dsa.h); otherwise ``DSAError`` (DSA_ERR_INVALID_ARG) is raised before the library is
called, since the library itself can check only null and alignment. A ``stream`` of None means
torch's current stream. A negative status raises ``DSAError`` with the library's message.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_FMT_F32, DSA_FMT_BF16, DSA_FMT_FP8 = 0, 1, 2
DSA_ERR_INVALID_ARG = -1
_ESIZE = {DSA_FMT_F32: 4, DSA_FMT_BF16: 2, DSA_FMT_FP8: 1}
DSA_OP_INDEX_TOPK, DSA_OP_SELECT_TOPK, DSA_OP_ATTEND = 0, 1, 2
DSA_MAX_TOPK = 4096
FORMATS = {"f32": DSA_FMT_F32, "bf16": DSA_FMT_BF16, "fp8": DSA_FMT_FP8}

EXPORTS = (
    "dsa_create", "dsa_destroy", "dsa_plan_check", "dsa_workspace_size", "dsa_store_keys",
    "dsa_index_topk", "dsa_index_topk_noalloc", "dsa_sparse_mla_attend",
    "dsa_sparse_mla_attend_sink", "dsa_index_scores", "dsa_select_topk", "dsa_msa_create", "dsa_msa_destroy", "dsa_msa_workspace_size",
    "dsa_msa_select_blocks", "dsa_msa_attend",
    "dsa_status_str", "dsa_last_error",
)


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class dsa_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_index_heads", "index_dim", "index_q_fmt", "index_key_fmt", "topk", "n_heads",
        "kv_lora_rank", "rope_dim", "q_fmt", "latent_fmt", "page_size")]


class dsa_msa_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_index_heads", "index_dim", "index_q_fmt", "index_key_fmt", "block_size", "topk_blocks",
        "n_heads", "n_kv_heads", "head_dim", "q_fmt", "page_size")]


class dsa_span(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "q_start", "q_len", "ctx_start", "page_offset", "n_pages", "page_start")]


class dsa_plan(ctypes.Structure):
    _fields_ = [
        ("n_spans", ctypes.c_int32), ("n_rows", ctypes.c_int32), ("n_page_ids", ctypes.c_int32),
        ("pool_pages", ctypes.c_int32), ("max_visible_cap", ctypes.c_int32),
        ("spans_host", ctypes.c_void_p), ("page_table_host", ctypes.c_void_p),
        ("spans_dev", ctypes.c_void_p), ("page_table_dev", ctypes.c_void_p),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load libdsa.so (built in-tree). Raises if it is missing: there is no other path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m sparse_attention_dsa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "dsa_create": ([ctypes.POINTER(dsa_config), ctypes.POINTER(P)], I32),
        "dsa_destroy": ([P], None),
        "dsa_plan_check": ([P, ctypes.POINTER(dsa_plan)], I32),
        "dsa_workspace_size": ([P, ctypes.POINTER(dsa_plan), I32, ctypes.POINTER(SZ)], I32),
        "dsa_store_keys": ([P, ctypes.POINTER(dsa_plan), P, P, P, P], I32),
        "dsa_index_topk": ([P, ctypes.POINTER(dsa_plan), P, P, P, P, P, SZ, P], I32),
        "dsa_index_topk_noalloc": ([P, ctypes.POINTER(dsa_plan), P, P, P, P, P], I32),
        "dsa_sparse_mla_attend": ([P, ctypes.POINTER(dsa_plan), P, P, P, P, ctypes.c_float, P, P, SZ, P], I32),
        "dsa_sparse_mla_attend_sink": ([P, ctypes.POINTER(dsa_plan), P, P, P, P, ctypes.c_float, P, P, P,
                                        SZ, P], I32),
        "dsa_index_scores": ([P, ctypes.POINTER(dsa_plan), P, P, P, P, ctypes.c_int64, P], I32),
        "dsa_select_topk": ([P, ctypes.POINTER(dsa_plan), P, ctypes.c_int64, P, P, SZ, P], I32),
        "dsa_msa_create": ([ctypes.POINTER(dsa_msa_config), ctypes.POINTER(P)], I32),
        "dsa_msa_destroy": ([P], None),
        "dsa_msa_workspace_size": ([P, ctypes.POINTER(dsa_plan), I32, ctypes.POINTER(SZ)], I32),
        "dsa_msa_select_blocks": ([P, ctypes.POINTER(dsa_plan), P, P, P, P, P, SZ, P], I32),
        "dsa_msa_attend": ([P, ctypes.POINTER(dsa_plan), P, P, P, ctypes.c_float, P, P, SZ, P], I32),
        "dsa_status_str": ([I32], ctypes.c_char_p),
        "dsa_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _ptr(x, name: str = "tensor", need: int = 0) -> int | None:
    """Device address of x. A torch tensor must be contiguous, hold >= need bytes and be on the
    GPU (checked in that order); None and integers pass through unchecked."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise DSAError(DSA_ERR_INVALID_ARG, f"{name}: not contiguous (strides {tuple(x.stride())})")
    nbytes = x.numel() * x.element_size()
    if nbytes < need:
        raise DSAError(DSA_ERR_INVALID_ARG, f"{name}: {nbytes} bytes, the call needs {need}")
    if not x.is_cuda:
        raise DSAError(DSA_ERR_INVALID_ARG, f"{name}: on {x.device}, not on the GPU")
    return x.data_ptr()


def _ws_bytes(ws, ws_bytes):
    if ws_bytes is not None:
        return int(ws_bytes)
    return ws.numel() * ws.element_size() if ws is not None and not isinstance(ws, int) else 0


def index_page_bytes(cfg) -> int:
    """Bytes of one index-key page (include/dsa.h, pool layouts)."""
    ps, d, f = cfg.page_size, cfg.index_dim, cfg.index_key_fmt
    return ps * (d + 4) if f == DSA_FMT_FP8 else ps * d * _ESIZE[f]


def latent_row_bytes(cfg) -> int:
    """Bytes of one latent row: R + P elements, or the packed fp8 row."""
    r, p = cfg.kv_lora_rank, cfg.rope_dim
    if cfg.latent_fmt == DSA_FMT_FP8:
        return r + 4 * (r // 128) + 2 * p
    return (r + p) * _ESIZE[cfg.latent_fmt]


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        lib = load()
        raise DSAError(status, lib.dsa_last_error().decode())


def dsa_status_str(status: int) -> str:
    return load().dsa_status_str(status).decode()


def dsa_last_error() -> str:
    return load().dsa_last_error().decode()


def make_config(n_index_heads, index_dim, index_q_fmt, index_key_fmt, topk, n_heads, kv_lora_rank,
                rope_dim, q_fmt, latent_fmt, page_size) -> dsa_config:
    f = lambda v: FORMATS[v] if isinstance(v, str) else int(v)  # noqa: E731
    return dsa_config(int(n_index_heads), int(index_dim), f(index_q_fmt), f(index_key_fmt), int(topk),
                      int(n_heads), int(kv_lora_rank), int(rope_dim), f(q_fmt), f(latent_fmt),
                      int(page_size))


class Handle:
    """Owns a dsa_handle*."""

    def __init__(self, cfg: dsa_config):
        lib = load()
        h = ctypes.c_void_p()
        _check(lib.dsa_create(ctypes.byref(cfg), ctypes.byref(h)))
        self.ptr = h.value
        self.cfg = cfg

    def __del__(self):
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.dsa_destroy(self.ptr)
            self.ptr = None


def dsa_create(cfg: dsa_config) -> Handle:
    return Handle(cfg)


def dsa_destroy(h: Handle):
    if h.ptr:
        load().dsa_destroy(h.ptr)
        h.ptr = None


class Plan:
    """A dsa_plan with its host arrays kept alive. spans: (n, 6) int32 array-like;
    spans_dev / page_table_dev: device tensors holding the same values."""

    def __init__(self, spans, page_table, pool_pages: int, spans_dev, page_table_dev,
                 check_pages: bool = True, max_visible_cap: int = 0):
        self.spans_host = np.ascontiguousarray(np.asarray(spans, dtype=np.int32).reshape(-1, 6))
        self.page_table_host = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
        self.spans_dev, self.page_table_dev = spans_dev, page_table_dev
        n_rows = int(self.spans_host[:, 1].sum())
        self.c = dsa_plan(
            len(self.spans_host), n_rows, len(self.page_table_host), int(pool_pages),
            int(max_visible_cap), self.spans_host.ctypes.data,
            self.page_table_host.ctypes.data if check_pages else None,
            _ptr(spans_dev, "spans_dev", self.spans_host.nbytes),
            _ptr(page_table_dev, "page_table_dev", self.page_table_host.nbytes))

    @property
    def n_rows(self) -> int:
        return int(self.c.n_rows)

    @staticmethod
    def on_device(spans, page_table, pool_pages: int, device="cuda", check_pages: bool = True,
                  max_visible_cap: int = 0):
        import torch
        s = torch.as_tensor(np.asarray(spans, dtype=np.int32).reshape(-1)).to(device)
        p = torch.as_tensor(np.asarray(page_table, dtype=np.int32)).to(device)
        return Plan(spans, page_table, pool_pages, s, p, check_pages, max_visible_cap)


def dsa_plan_check(h: Handle, plan: Plan):
    _check(load().dsa_plan_check(h.ptr, ctypes.byref(plan.c)))


def dsa_workspace_size(h: Handle, plan: Plan, op: int) -> int:
    n = ctypes.c_size_t()
    _check(load().dsa_workspace_size(h.ptr, ctypes.byref(plan.c), int(op), ctypes.byref(n)))
    return int(n.value)


def _rows(plan: Plan) -> int:
    return int(plan.c.n_rows)


def dsa_store_keys(h: Handle, plan: Plan, keys, scales, key_pool, stream=None):
    c, T = h.cfg, _rows(plan)
    args = (_ptr(keys, "keys", T * c.index_dim * _ESIZE[c.index_key_fmt]),
            _ptr(scales, "scales", 4 * T if c.index_key_fmt == DSA_FMT_FP8 else 0),
            _ptr(key_pool, "key_pool", plan.c.pool_pages * index_page_bytes(c)))
    _check(load().dsa_store_keys(h.ptr, ctypes.byref(plan.c), *args, _stream(stream)))


def _index_args(h: Handle, plan: Plan, q, w, key_pool, sel):
    c, T = h.cfg, _rows(plan)
    return (_ptr(q, "q", T * c.n_index_heads * c.index_dim * _ESIZE[c.index_q_fmt]),
            _ptr(w, "w", 4 * T * c.n_index_heads),
            _ptr(key_pool, "key_pool", plan.c.pool_pages * index_page_bytes(c)),
            _ptr(sel, "sel", 4 * T * c.topk))


def dsa_index_topk(h: Handle, plan: Plan, q, w, key_pool, sel, ws, ws_bytes=None, stream=None):
    nb = _ws_bytes(ws, ws_bytes)
    args = _index_args(h, plan, q, w, key_pool, sel)
    _check(load().dsa_index_topk(h.ptr, ctypes.byref(plan.c), *args, _ptr(ws, "ws", nb), nb,
                                 _stream(stream)))


def dsa_index_topk_noalloc(h: Handle, plan: Plan, q, w, key_pool, sel, stream=None):
    args = _index_args(h, plan, q, w, key_pool, sel)
    _check(load().dsa_index_topk_noalloc(h.ptr, ctypes.byref(plan.c), *args, _stream(stream)))


def _attend_args(h: Handle, plan: Plan, sel, q_nope, q_pe, latent_pool, out):
    c, T = h.cfg, _rows(plan)
    e = _ESIZE[c.q_fmt]
    return (_ptr(sel, "sel", 4 * T * c.topk),
            _ptr(q_nope, "q_nope", T * c.n_heads * c.kv_lora_rank * e),
            _ptr(q_pe, "q_pe", T * c.n_heads * c.rope_dim * e),
            _ptr(latent_pool, "latent_pool", plan.c.pool_pages * c.page_size * latent_row_bytes(c)),
            _ptr(out, "out", T * c.n_heads * c.kv_lora_rank * e))


def dsa_sparse_mla_attend(h: Handle, plan: Plan, sel, q_nope, q_pe, latent_pool, sm_scale, out, ws,
                          ws_bytes=None, stream=None):
    nb = _ws_bytes(ws, ws_bytes)
    s_, qn, qp, pool, o = _attend_args(h, plan, sel, q_nope, q_pe, latent_pool, out)
    _check(load().dsa_sparse_mla_attend(h.ptr, ctypes.byref(plan.c), s_, qn, qp, pool,
                                        float(sm_scale), o, _ptr(ws, "ws", nb), nb, _stream(stream)))


def dsa_sparse_mla_attend_sink(h: Handle, plan: Plan, sel, q_nope, q_pe, latent_pool, sm_scale, sink,
                               out, ws, ws_bytes=None, stream=None):
    nb = _ws_bytes(ws, ws_bytes)
    s_, qn, qp, pool, o = _attend_args(h, plan, sel, q_nope, q_pe, latent_pool, out)
    sk = _ptr(sink, "sink", 4 * h.cfg.n_heads)
    _check(load().dsa_sparse_mla_attend_sink(h.ptr, ctypes.byref(plan.c), s_, qn, qp, pool,
                                             float(sm_scale), sk, o, _ptr(ws, "ws", nb), nb,
                                             _stream(stream)))


def dsa_index_scores(h: Handle, plan: Plan, q, w, key_pool, scores, ld: int, stream=None):
    c, T = h.cfg, _rows(plan)
    qp = _ptr(q, "q", T * c.n_index_heads * c.index_dim * _ESIZE[c.index_q_fmt])
    wp = _ptr(w, "w", 4 * T * c.n_index_heads)
    kp = _ptr(key_pool, "key_pool", plan.c.pool_pages * index_page_bytes(c))
    sp = _ptr(scores, "scores", 4 * T * max(int(ld), 0))
    _check(load().dsa_index_scores(h.ptr, ctypes.byref(plan.c), qp, wp, kp, sp, int(ld),
                                   _stream(stream)))


def dsa_select_topk(h: Handle, plan: Plan, scores, ld: int, sel, ws, ws_bytes=None, stream=None):
    nb = _ws_bytes(ws, ws_bytes)
    T = _rows(plan)
    sp = _ptr(scores, "scores", 4 * T * max(int(ld), 0))
    sl = _ptr(sel, "sel", 4 * T * h.cfg.topk)
    _check(load().dsa_select_topk(h.ptr, ctypes.byref(plan.c), sp, int(ld), sl, _ptr(ws, "ws", nb),
                                  nb, _stream(stream)))


# ---------------------------------------------------------------------------- block-sparse MSA

def make_msa_config(n_index_heads, index_dim, index_q_fmt, index_key_fmt, block_size, topk_blocks,
                    n_heads, n_kv_heads, head_dim, q_fmt, page_size) -> dsa_msa_config:
    f = lambda v: FORMATS[v] if isinstance(v, str) else int(v)  # noqa: E731
    return dsa_msa_config(int(n_index_heads), int(index_dim), f(index_q_fmt), f(index_key_fmt),
                          int(block_size), int(topk_blocks), int(n_heads), int(n_kv_heads),
                          int(head_dim), f(q_fmt), int(page_size))


class MsaHandle:
    """Owns a dsa_msa_handle*."""

    def __init__(self, cfg: dsa_msa_config):
        self.cfg = cfg
        ptr = ctypes.c_void_p()
        _check(load().dsa_msa_create(ctypes.byref(cfg), ctypes.byref(ptr)))
        self.ptr = ptr.value

    def __del__(self):
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.dsa_msa_destroy(self.ptr)
            self.ptr = None


def dsa_msa_create(cfg: dsa_msa_config) -> MsaHandle:
    return MsaHandle(cfg)


def dsa_msa_workspace_size(h: MsaHandle, plan: Plan, op: int) -> int:
    n = ctypes.c_size_t()
    _check(load().dsa_msa_workspace_size(h.ptr, ctypes.byref(plan.c), int(op), ctypes.byref(n)))
    return int(n.value)


def dsa_msa_select_blocks(h: MsaHandle, plan: Plan, q, w, key_pool, sel, ws, ws_bytes=None, stream=None):
    c, T = h.cfg, _rows(plan)
    nb = _ws_bytes(ws, ws_bytes)
    kpb = (c.page_size * (c.index_dim + 4) if c.index_key_fmt == DSA_FMT_FP8
           else c.page_size * c.index_dim * _ESIZE[c.index_key_fmt])
    args = (_ptr(q, "q", T * c.n_index_heads * c.index_dim * _ESIZE[c.index_q_fmt]),
            _ptr(w, "w", 4 * T * c.n_index_heads),
            _ptr(key_pool, "key_pool", plan.c.pool_pages * kpb),
            _ptr(sel, "sel", 4 * T * c.topk_blocks))
    _check(load().dsa_msa_select_blocks(h.ptr, ctypes.byref(plan.c), *args, _ptr(ws, "ws", nb), nb,
                                        _stream(stream)))


def dsa_msa_attend(h: MsaHandle, plan: Plan, sel, q, gqa_pool, sm_scale, out, ws=None, ws_bytes=None,
                   stream=None):
    c, T = h.cfg, _rows(plan)
    nb = _ws_bytes(ws, ws_bytes)
    e = _ESIZE[c.q_fmt]
    row = 2 * c.n_kv_heads * c.head_dim * e
    args = (_ptr(sel, "sel", 4 * T * c.topk_blocks),
            _ptr(q, "q", T * c.n_heads * c.head_dim * e),
            _ptr(gqa_pool, "gqa_pool", plan.c.pool_pages * c.page_size * row))
    o = _ptr(out, "out", T * c.n_heads * c.head_dim * e)
    _check(load().dsa_msa_attend(h.ptr, ctypes.byref(plan.c), *args, float(sm_scale), o,
                                 _ptr(ws, "ws", nb), nb, _stream(stream)))
