"""Block-sparse MSA on the GPU against the oracle: token scores, block selection and GQA
attention over the picked blocks."""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as msa
from synth import make_msa_workload
from sparse_attention_dsa_amd import dsa
from sparse_attention_dsa_amd.step import MSAStep
from tests import helpers
from tests.gpu_helpers import note

pytestmark = pytest.mark.gpu

# |g - o| <= a * sum_j p_j |v_j| + r * |o| + floor.
# bf16: the matrix-core kernel rounds each weight p_j to bf16 (at most 2^-9 of itself, 1.5 x
# that as margin for the fp32 sums) and the output to bf16 (2^-9 of |o|, 2^-8 as margin).
# fp32 (the VALU kernel, fp32 weights): accumulation over head_dim products and a few
# thousand weights (2^-24 a step), far below these.
TOL = {"bf16": (1.5 * 2.0 ** -8, 2.0 ** -8, 1e-5), "f32": (1e-5, 1e-4, 1e-6)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()


def _gpu_scores(st, wl):
    T = st.plan.n_rows
    ld = (int(wl.positions.max()) + 1 + 63) // 64 * 64
    return st.ws[: T * ld * 4].view(torch.float32).view(T, ld).cpu().numpy()


def _check(wl, rows):
    s = wl.spec
    st = MSAStep(wl)
    st.select()
    torch.cuda.synchronize()
    sel = st.sel.cpu().numpy()
    sc_gpu = _gpu_scores(st, wl)
    q_idx, w = helpers.to_f64(wl.index_q), helpers.to_f64(wl.index_w)
    sel_ref, bs_ref = msa.msa_select(q_idx, w, wl.key_pool.numpy(), s.index_key_fmt, wl.spans, wl.page_table,
                                     s.page_size, s.topk_blocks, s.block, rows=rows, return_scores=True)
    from oracle import dsa_oracle
    keys_cache = {}
    for t in rows:
        p = int(wl.positions[t])
        # selection bit-exact given the GPU's own token scores
        exact = msa.select_blocks_row(msa.block_scores_row(sc_gpu[t], p, s.block), s.topk_blocks)
        assert np.array_equal(sel[t], exact), f"row {t}: selection not bit-exact on GPU scores"
        # and in agreement with the oracle's block scores outside the margin band
        ok, why = helpers.selection_band_ok(sel[t], bs_ref[t], p // s.block, s.topk_blocks)
        assert ok, f"row {t}: {why}"
        # token scores within the score tolerance
        span = wl.spans[[i for i, sp in enumerate(wl.spans) if sp[0] <= t < sp[0] + sp[1]][0]]
        key = int(span[0])
        if key not in keys_cache:
            keys_cache = {key: dsa_oracle.read_index_keys(wl.key_pool.numpy(), s.index_key_fmt, span, wl.page_table,
                                                          s.page_size, s.index_dim, int(span[2] + span[1]))}
        ref = dsa_oracle.index_scores_row(q_idx[t], w[t], keys_cache[key][: p + 1])
        okc, worst = helpers.score_close(sc_gpu[t, : p + 1], ref)
        assert okc, f"row {t}: token score error {worst:.3g} x tolerance"

    def check_out(picks, label):
        st.sel.copy_(torch.from_numpy(picks))
        st.attend()
        torch.cuda.synchronize()
        out = st.out.float().cpu().numpy().astype(np.float64)
        ref, mag = msa.msa_attend({t: picks[t] for t in rows}, helpers.to_f64(wl.q), wl.gqa_pool.numpy(),
                                  wl.spans, wl.page_table, s.page_size, s.n_kv_heads, s.head_dim,
                                  s.block, s.sm_scale, return_abs=True, fmt=s.q_fmt)
        a, rel, floor = TOL[s.q_fmt]
        worst = 0.0
        for t in rows:
            err = np.abs(out[t] - ref[t])
            ok = err <= a * mag[t] + rel * np.abs(ref[t]) + floor
            assert ok.all(), f"{label} row {t}: max abs {err.max():.3g} ({int((~ok).sum())} elements)"
            worst = max(worst, float(err.max()))
        return worst

    w1 = check_out(sel.copy(), "gpu-sel")
    ref_sel = sel.copy()
    for t in rows:
        ref_sel[t] = sel_ref[t]
    w2 = check_out(ref_sel, "oracle-sel")
    # edited lists: a block listed twice counts twice, -1 entries and blocks past the row's
    # position add nothing
    edit = sel.copy()
    for t in rows:
        nb = int(wl.positions[t]) // s.block + 1
        if s.topk_blocks >= 3:
            edit[t, 1] = edit[t, 0]
            edit[t, 2] = nb + 3
        edit[t, -1] = -1
    w3 = check_out(edit, "edited-sel")
    return max(w1, w2, w3)


@pytest.mark.parametrize("name", ["msa_decode_small", "msa_prefill_small", "msa_generic_f32",
                                  "msa_generic_small", "msa_generic_bf16", "msa_fp8keys_small",
                                  "msa_pages48_small", "msa_pages48_fp8_small"])
def test_msa_small_workloads_all_rows(name):
    wl = make_msa_workload(name)
    worst = _check(wl, list(range(wl.n_rows)))
    note(f"[msa] {name}: all {wl.n_rows} rows, worst attention error {worst:.3g}")


def test_msa_long_decode_sampled_rows():
    wl = make_msa_workload("msa_long_decode")
    worst = _check(wl, [0, 5])
    note(f"[msa] msa_long_decode: rows 0 and 5 of 8 at 131072 positions, worst attention error {worst:.3g}")


@pytest.mark.parametrize("name", ["msa_decode_small", "msa_generic_small"])
def test_msa_captured_step_replays_match_eager(name):
    # select + attend captured in a HIP graph: every replay, after eager work that overwrites
    # the outputs and the workspaces, equals the eager step bit for bit
    wl = make_msa_workload(name)
    st = MSAStep(wl)
    st.select()
    st.attend()
    torch.cuda.synchronize()
    ref_sel, ref_out = st.sel.clone(), st.out.clone()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            st.select(stream=cap)
            st.attend(stream=cap)
    torch.cuda.synchronize()
    for rep in range(3):
        st.sel.fill_(-7)
        st.out.zero_()
        st.ws.fill_(0xA5)
        st.attend_ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.sel, ref_sel), f"replay {rep}: selection differs"
        assert torch.equal(st.out, ref_out), f"replay {rep}: output differs"
    note(f"[msa graph] {name}: 3 replays identical to the eager step")


def test_msa_captured_decode_step_replays_as_positions_grow():
    # captured once with launches sized by max_visible_cap, replayed while the decode rows move
    # forward in the device copy of the plan; the rows at positions 126..130 cross a block
    # boundary (127 -> 128) and so gain a block between replays. Each replay equals the eager
    # step on an exact plan, bit for bit.
    back = 3
    wl = make_msa_workload("msa_decode_small")
    st = MSAStep(wl)
    base = wl.spans.copy()
    base[:, 2] -= np.minimum(back, base[:, 2])      # a row at position 0 stays there
    cap = int((wl.spans[:, 2] + wl.spans[:, 1]).max())
    plan = dsa.Plan.on_device(base, wl.page_table, wl.pool_pages, max_visible_cap=cap)

    def workspaces(p):
        return [torch.empty(max(dsa.dsa_msa_workspace_size(st.h, p, op), 256), dtype=torch.uint8,
                            device="cuda") for op in (dsa.DSA_OP_SELECT_TOPK, dsa.DSA_OP_ATTEND)]

    def run(p, ws, sel, out, stream=None):
        dsa.dsa_msa_select_blocks(st.h, p, st.index_q, st.index_w, st.key_pool, sel, ws[0], stream=stream)
        dsa.dsa_msa_attend(st.h, p, sel, st.q, st.gqa_pool, st.sm_scale, out, ws[1], stream=stream)

    ws = workspaces(plan)
    sel, out = torch.empty_like(st.sel), torch.empty_like(st.out)
    run(plan, ws, sel, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(g, stream=cap_stream):
            run(plan, ws, sel, out, stream=cap_stream)
    torch.cuda.synchronize()
    for k in range(back + 1):
        spans_k = base.copy()
        spans_k[:, 2] = np.minimum(base[:, 2] + k, wl.spans[:, 2])
        plan.spans_dev.copy_(torch.from_numpy(spans_k.reshape(-1)))
        sel.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_plan = dsa.Plan.on_device(spans_k, wl.page_table, wl.pool_pages)
        sel_ref, out_ref = torch.empty_like(sel), torch.empty_like(out)
        run(ref_plan, workspaces(ref_plan), sel_ref, out_ref)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_ref), f"position step {k}: selection differs"
        assert torch.equal(out, out_ref), f"position step {k}: attention output differs"
    note(f"[msa graph] msa_decode_small: {back + 1} replays at advancing positions equal the eager steps")
