"""dsa_index_topk_noalloc (the library's static per-GPU scratch) against dsa_index_topk (a caller
workspace) on the same inputs: two calls in a row, the second on a smaller plan, each bit-equal
(the outputs are indices); then a run of calls on seeded random plans. Also: a plan whose
workspace exceeds the scratch is refused on the host."""
import numpy as np
import pytest
import torch

from synth import make_workload
from sparse_attention_dsa_amd import dsa
from sparse_attention_dsa_amd.step import DSAStep


def _both(wl):
    st = DSAStep.from_workload(wl, n_layers=1)
    st.store_keys()
    st.index_topk()                              # caller workspace
    ref = st.sel.cpu().numpy()
    got = torch.full_like(st.sel, -7)
    dsa.dsa_index_topk_noalloc(st.h, st.plan, st.index_q, st.index_w, st.key_pool, got)
    torch.cuda.synchronize()
    return ref, got.cpu().numpy(), dsa.dsa_workspace_size(st.h, st.plan, dsa.DSA_OP_INDEX_TOPK)


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()
    ref1, got1, ws1 = _both(make_workload("long_decode"))     # 8 rows x 131072 positions
    print(f"[noalloc] long_decode: workspace {ws1} bytes", flush=True)
    assert np.array_equal(ref1, got1)
    ref2, got2, ws2 = _both(make_workload("decode_small"))    # a smaller plan on the same scratch
    print(f"[noalloc] decode_small: workspace {ws2} bytes", flush=True)
    assert ws2 < ws1
    assert np.array_equal(ref2, got2)


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_on_random_plans():
    """Calls in a row on the shared scratch, each on a different seeded random plan (formats, page
    sizes, top-k, prefill chunks and decode rows), each bit-equal to the workspace call."""
    from tests.test_gpu_random_plans import random_generic_spec, random_spec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()
    specs = [random_spec(s) for s in range(6)] + [random_generic_spec(s) for s in range(3)]
    for spec in specs:
        ref, got, ws = _both(make_workload(spec))
        print(f"[noalloc] {spec.name}: workspace {ws} bytes", flush=True)
        assert np.array_equal(ref, got), spec.name


def test_noalloc_refuses_plans_beyond_the_scratch():
    # 512 decode rows at 131072 positions need 256 MiB of scores: refused before any launch
    cfg = dsa.make_config(64, 128, "bf16", "fp8", 2048, 128, 512, 64, "bf16", "fp8", 64)
    h = dsa.dsa_create(cfg)
    rows = 512
    spans = np.array([[r, 1, 131071, 0, 2048, 0] for r in range(rows)], np.int32)
    fake = 1 << 40
    plan = dsa.Plan(spans, np.zeros(2048, np.int32), 2048, fake, fake + 4096, check_pages=False)
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_index_topk_noalloc(h, plan, fake, fake, fake, fake, stream=0)
    assert e.value.status == -4 and "static scratch" in str(e.value)
