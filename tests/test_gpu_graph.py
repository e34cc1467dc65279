"""A select + attend step captured in a HIP graph and replayed gives the eager step's results.

The library allocates nothing and clears no memory inside a call (every kernel writes its whole
output), so a step captures as it is. Each replay follows eager work that overwrites the outputs,
and every replay is compared with the eager result bit for bit (the kernels are deterministic)."""
import pytest
import torch

from synth import make_workload
from sparse_attention_dsa_amd import dsa
from sparse_attention_dsa_amd.step import DSAStep
from tests.gpu_helpers import note
from tests.test_gpu_random_plans import random_spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()


@pytest.mark.parametrize("name", ["decode_small", "mix_small", "sink_decode_small"])
def test_captured_step_replays_match_eager(name):
    note(f"[graph] {name}")
    _capture_and_replay(make_workload(name), name)


@pytest.mark.parametrize("seed", [0, 1, 2, 5, 9, 13])
def test_captured_random_plan_replays_match_eager(seed):
    """The same on seeded random plans (formats, page sizes, top-k, sinks; see the random-plan
    parity tests)."""
    note(f"[graph] random plan {seed}")
    _capture_and_replay(make_workload(random_spec(seed)), f"random plan {seed}")


def _capture_and_replay(wl, name):
    st = DSAStep.from_workload(wl)
    st.store_keys()
    n_layers = len(st.q_nope)
    st.index_topk()
    for layer in range(n_layers):
        st.attend(layer)
    torch.cuda.synchronize()
    ref_sel = st.sel.clone()
    ref_out = [o.clone() for o in st.out]

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            st.index_topk(stream=cap)
            for layer in range(n_layers):
                st.attend(layer, stream=cap)
    torch.cuda.synchronize()

    for rep in range(3):
        st.sel.fill_(-7)                      # eager work between replays
        for o in st.out:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.sel, ref_sel), f"replay {rep}: selection differs"
        for layer in range(n_layers):
            assert torch.equal(st.out[layer], ref_out[layer]), f"replay {rep}: layer {layer} output differs"
    note(f"[graph] {name}: 3 replays identical to the eager step")


def test_captured_decode_step_replays_as_positions_grow():
    """A select + attend step captured once with launches sized by max_visible_cap, replayed
    while the decode rows' positions move forward in the device copy of the plan (as a decode
    loop would), equals the eager step run on an exact plan at each position, bit for bit."""
    name, back = "decode_small", 3
    note(f"[graph] {name}: replays over {back + 1} positions")
    wl = make_workload(name, n_attend_layers=1)
    st = DSAStep.from_workload(wl)
    st.store_keys()                      # every row's own key at its final position
    base = wl.spans.copy()
    base[:, 2] -= back                   # start `back` positions earlier
    cap = int((wl.spans[:, 2] + wl.spans[:, 1]).max())
    plan = dsa.Plan.on_device(base, wl.page_table, wl.pool_pages, max_visible_cap=cap)

    def workspaces(p):
        return [torch.empty(max(dsa.dsa_workspace_size(st.h, p, op), 256), dtype=torch.uint8,
                            device="cuda") for op in (dsa.DSA_OP_INDEX_TOPK, dsa.DSA_OP_ATTEND)]

    def run(p, ws, sel, out, stream=None):
        dsa.dsa_index_topk(st.h, p, st.index_q, st.index_w, st.key_pool, sel, ws[0], stream=stream)
        dsa.dsa_sparse_mla_attend(st.h, p, sel, st.q_nope[0], st.q_pe[0], st.latent_pools[0],
                                  st.sm_scale, out, ws[1], stream=stream)

    ws = workspaces(plan)
    sel, out = torch.empty_like(st.sel), torch.empty_like(st.out[0])
    run(plan, ws, sel, out)              # warm up outside the capture
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
        spans_k[:, 2] += k
        plan.spans_dev.copy_(torch.from_numpy(spans_k.reshape(-1)))   # the plan moves on
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
    note(f"[graph] {name}: {back + 1} replays at advancing positions equal the eager steps")
