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

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()


@pytest.mark.parametrize("name", ["decode_small", "mix_small", "sink_decode_small"])
def test_captured_step_replays_match_eager(name):
    note(f"[graph] {name}")
    wl = make_workload(name)
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
