"""Test helpers: hand workload tensors to the oracle as numpy, and compare results."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.float64).numpy()


def raw_keys(wl):
    """This step's index keys as the oracle's store_keys takes them (raw storage elements)."""
    k = wl.step_keys
    if k.dtype == torch.bfloat16:
        return k.view(torch.int16).numpy().view(np.uint16)
    return k.numpy()


def oracle_key_pool(wl) -> np.ndarray:
    """The index-key pool after the oracle stores this step's keys."""
    s = wl.spec
    scales = None if wl.step_key_scales is None else wl.step_key_scales.numpy()
    return oracle.store_keys(wl.key_pool.numpy(), s.index_key_fmt, wl.spans, wl.page_table,
                             s.page_size, s.index_dim, raw_keys(wl), scales)


def oracle_index_topk(wl, rows=None, pool=None, return_scores=False):
    s = wl.spec
    pool = oracle_key_pool(wl) if pool is None else pool
    return oracle.index_topk(to_f64(wl.index_q), to_f64(wl.index_w), pool, s.index_key_fmt,
                             wl.spans, wl.page_table, s.page_size, s.topk, rows=rows,
                             return_scores=return_scores)


def oracle_attend(wl, sel: dict, layer: int = 0, return_abs: bool = False):
    s = wl.spec
    sink = None if wl.sinks[layer] is None else wl.sinks[layer].numpy()
    return oracle.sparse_mla_attend(sel, to_f64(wl.q_nope[layer]), to_f64(wl.q_pe[layer]),
                                    wl.latent_pools[layer].numpy(), s.latent_fmt, wl.spans,
                                    wl.page_table, s.page_size, s.sm_scale, return_abs=return_abs,
                                    sink=sink)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest OCP e4m3fn value (ties to even, saturated at +-448), by torch's
    cast; float64 in and out."""
    y = torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float32)
    return y.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_interval_ok(g: np.ndarray, o: np.ndarray, tol) -> np.ndarray:
    """Whether each e4m3 value g can be the rounding of some v with |v - o| <= tol: rounding is
    monotone, so g must lie between the roundings of o - tol and o + tol."""
    return (g >= e4m3_round(o - tol)) & (g <= e4m3_round(o + tol))


def sample_rows(wl, n_max: int, seed: int = 0) -> list:
    """A deterministic row sample: first and last rows of every span plus a seeded spread."""
    T = wl.n_rows
    rows = set()
    for q_start, q_len, *_ in wl.spans:
        rows.add(int(q_start))
        rows.add(int(q_start + q_len - 1))
    rng = np.random.default_rng(seed)
    extra = rng.choice(T, size=min(T, max(0, n_max - len(rows))), replace=False)
    rows.update(int(r) for r in extra)
    return sorted(rows)[: max(n_max, 1)] if len(rows) > n_max else sorted(rows)


def score_close(gpu: np.ndarray, ref: np.ndarray, rtol: float = 1e-5) -> tuple:
    """Score tolerance: |g - o| <= rtol * max(|o|, mean|o| of the row)."""
    floor = np.mean(np.abs(ref)) if ref.size else 0.0
    bound = rtol * np.maximum(np.abs(ref), floor)
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    return bool(np.all(err <= bound)), float(np.max(err / np.maximum(bound, 1e-300)) if ref.size else 0.0)


def selection_band_ok(sel_gpu: np.ndarray, scores_ref: np.ndarray, pos: int, topk: int,
                      rel_band: float = 2e-5) -> tuple:
    """Set agreement outside the score-margin band around the oracle's k-th score.

    Keys scoring clearly above the band must be picked, keys clearly below must not, the count
    must be min(topk, pos + 1) and the -1 entries must form a tail."""
    n = min(topk, pos + 1)
    picked = sel_gpu[:n]
    if np.any(picked < 0) or np.any(sel_gpu[n:] != -1):
        return False, "bad -1 tail"
    if np.any(picked > pos):
        return False, "non-causal pick"
    if len(set(picked.tolist())) != n:
        return False, "duplicate picks"
    s = scores_ref[: pos + 1].astype(np.float64)
    if n == pos + 1:
        return True, "all"
    tau = np.sort(s)[::-1][n - 1]
    delta = rel_band * max(abs(tau), float(np.mean(np.abs(s))))
    must = np.nonzero(s > tau + delta)[0]
    never = np.nonzero(s < tau - delta)[0]
    ps = set(picked.tolist())
    if not set(must.tolist()) <= ps:
        return False, "missed a key above the band"
    if ps & set(never.tolist()):
        return False, "picked a key below the band"
    return True, "ok"
