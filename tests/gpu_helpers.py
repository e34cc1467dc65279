"""Shared pieces of the GPU parity tests: run the library on a workload and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from sparse_attention_dsa_amd import dsa
from sparse_attention_dsa_amd.step import DSAStep
from tests import helpers

# bf16 attention outputs. The product stores P (the softmax weights, with an fp8 group scale
# folded in) as bf16 for the matrix cores and rounds the output to bf16; each rounding moves a
# value by at most 2^-8 of itself. So |g - o| <= 2^-8 * sum_j p_j |c_j| + 2^-8 |o| up to fp32
# noise; the tripwire allows 1.5x the first term plus 1e-4. The hard bound is the 2e-2 absolute
# contract, widened by the output's own bf16 rounding where outputs are O(1) (rows of few keys).
BF16_CONTRACT = 2e-2
BF16_P, BF16_OUT, BF16_FLOOR, BF16_RMS = 1.5 * 2.0 ** -8, 2.0 ** -8, 1e-4, 1e-2
# f32 attention outputs: fp32 accumulation over at most a few thousand terms of O(1) values.
F32_ATOL, F32_RTOL = 1e-4, 1e-4
# e4m3 outputs (e4m3 queries): the product rounds an fp32 value v once to e4m3. v differs from the
# exact output o by the bf16 weights (and, where picks are split, the bf16 partial outputs) of the
# matrix-core kernel, or by fp32 noise in the plain kernel; rounding is monotone, so the code must
# lie between the roundings of o - tol and o + tol.


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def scores_on_gpu(step: DSAStep):
    ld = (step.plan.c.n_rows and int(max(step.plan.spans_host[:, 2] + step.plan.spans_host[:, 1])))
    ld = (ld + 3) // 4 * 4
    sc = torch.empty(step.plan.n_rows, ld, dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(step.h, step.plan, step.index_q, step.index_w, step.key_pool, sc, ld)
    return sc, ld


def select_on_gpu(step: DSAStep, scores, ld):
    sel = torch.empty(step.plan.n_rows, step.topk, dtype=torch.int32, device="cuda")
    n = dsa.dsa_workspace_size(step.h, step.plan, dsa.DSA_OP_SELECT_TOPK)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    dsa.dsa_select_topk(step.h, step.plan, scores, ld, sel, ws)
    return sel


def check_attend(wl, step: DSAStep, rows, sel_dict, layer=0, label=""):
    """GPU attend output at `rows` against the oracle attend on the same selection."""
    ref, mag = helpers.oracle_attend(wl, {t: sel_dict[t] for t in rows}, layer, return_abs=True)
    o_dev = step.out[layer]
    if wl.spec.q_fmt == "fp8":
        codes = o_dev.view(torch.uint8)[rows].cpu()
        out = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    else:
        out = o_dev[rows].float().cpu().numpy().astype(np.float64)
    matrix_core = wl.spec.kv_lora_rank == 512 and wl.spec.rope_dim == 64
    worst = 0.0
    for i, t in enumerate(rows):
        g, o = out[i], ref[t]
        if wl.spec.q_fmt == "fp8":
            if matrix_core:
                tol = (BF16_P + BF16_OUT) * mag[t] + BF16_FLOOR
            else:
                tol = F32_ATOL + F32_RTOL * np.abs(o)
            ok = helpers.e4m3_interval_ok(g, o, tol)
            assert ok.all(), f"{label} row {t}: {int((~ok).sum())} e4m3 outputs outside the rounding " \
                             f"interval (max abs {np.abs(g - o).max():.3g})"
            worst = max(worst, np.abs(g - o).max())
        elif wl.spec.q_fmt == "bf16":
            err = np.abs(g - o)
            rms = np.sqrt(np.mean((g - o) ** 2)) / max(np.sqrt(np.mean(o ** 2)), 1e-30)
            trip = err <= BF16_P * mag[t] + BF16_OUT * np.abs(o) + BF16_FLOOR
            hard = err <= BF16_CONTRACT + BF16_OUT * np.abs(o)
            assert hard.all() and trip.all() and rms <= BF16_RMS, \
                f"{label} row {t}: max abs {err.max():.3g} rel rms {rms:.3g} " \
                f"(tripwire {int((~trip).sum())} elems, contract {int((~hard).sum())} elems)"
            worst = max(worst, err.max())
        else:
            ok = np.abs(g - o) <= F32_ATOL + F32_RTOL * np.abs(o)
            assert ok.all(), f"{label} row {t}: max abs {np.abs(g - o).max():.3g}"
            worst = max(worst, np.abs(g - o).max())
    return worst


def full_parity(wl, rows=None, check_scores=True, layers=None):
    """The whole path on the GPU against the oracle at `rows` (all rows if None)."""
    step = DSAStep.from_workload(wl)
    T = step.plan.n_rows
    rows = list(range(T)) if rows is None else list(rows)
    pos = wl.positions

    # a2: store_keys writes exactly the oracle's bytes
    step.store_keys()
    pool_ref = helpers.oracle_key_pool(wl)
    pool_gpu = step.key_pool.cpu().numpy()
    assert np.array_equal(pool_gpu, pool_ref), "store_keys bytes differ from the oracle"

    # a3 + a4: the fused call, and its two halves
    step.index_topk()
    sel_fused = step.sel.cpu().numpy()
    sc, ld = scores_on_gpu(step)
    sel_split = select_on_gpu(step, sc, ld).cpu().numpy()
    assert np.array_equal(sel_fused, sel_split), "index_topk differs from index_scores + select_topk"
    sc_gpu = sc.cpu().numpy()

    sel_ref, sc_ref = helpers.oracle_index_topk(wl, rows=rows, pool=pool_ref, return_scores=True)
    worst_score = 0.0
    for t in rows:
        p = int(pos[t])
        # scores within the tolerance; -inf past the position
        if check_scores:
            ok, w = helpers.score_close(sc_gpu[t, : p + 1], sc_ref[t])
            worst_score = max(worst_score, w)
            assert ok, f"row {t}: score error {w:.3g} x tolerance"
        assert np.all(np.isneginf(sc_gpu[t, p + 1:])), f"row {t}: masked scores not -inf"
        # selection bit-exact given the GPU's own fp32 scores
        exact = oracle.select_topk_causal_row(sc_gpu[t], p, step.topk)
        assert np.array_equal(sel_fused[t], exact), f"row {t}: selection not bit-exact on GPU scores"
        # and in agreement with the oracle's scores outside the margin band
        ok, why = helpers.selection_band_ok(sel_fused[t], sc_ref[t], p, step.topk)
        assert ok, f"row {t}: {why}"

    # a5 (+ a7): attend, with the GPU selection and with the oracle selection
    n_layers = len(step.q_nope) if layers is None else layers
    worst_att = 0.0
    gpu_sel = {t: sel_fused[t] for t in rows}
    for layer in range(n_layers):
        step.attend(layer)
        worst_att = max(worst_att, check_attend(wl, step, rows, gpu_sel, layer, f"layer {layer} gpu-sel"))
    ref_sel_full = sel_fused.copy()
    for t in rows:
        ref_sel_full[t] = sel_ref[t]
    step.sel.copy_(torch.from_numpy(ref_sel_full))
    step.attend(0)
    worst_att = max(worst_att, check_attend(wl, step, rows, sel_ref, 0, "oracle-sel"))
    torch.cuda.synchronize()
    return dict(worst_score=worst_score, worst_attend=worst_att, step=step)
