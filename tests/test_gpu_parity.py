"""GPU parity: every step of the path through the C ABI against the CPU oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_workload
from sparse_attention_dsa_amd import dsa
from sparse_attention_dsa_amd.step import DSAStep
from tests import helpers
from tests.gpu_helpers import full_parity, note, scores_on_gpu, select_on_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()


@pytest.mark.parametrize("name", ["tiny_prefill", "decode_small", "long_decode_small",
                                  "prefill_small", "mix_small", "prefill_fp8_small",
                                  "pages1_small", "pages128_small", "many_spans_small",
                                  "sink_decode_small", "fp8q_sink_small", "fp8q_small",
                                  "tiny_fp8q_sink", "sink_fp8_decode_small",
                                  "sink_fp8_rows_small", "steps_fp8_small", "pages48_small",
                                  "pages48_fp8_small", "spans70_bf16_small"])
def test_small_workloads_all_rows(name):
    note(f"[parity] {name} all rows")
    wl = make_workload(name)
    r = full_parity(wl)
    note(f"[parity] {name}: worst score err {r['worst_score']:.3g}x tol, attend {r['worst_attend']:.3g}")


def test_determinism_two_runs_identical():
    wl = make_workload("decode_small")
    a = DSAStep.from_workload(wl)
    a.run()
    s1, o1 = a.sel.clone(), a.out[0].clone()
    a.index_topk()
    a.attend(0)
    assert torch.equal(a.sel, s1) and torch.equal(a.out[0], o1)


def test_selection_independent_of_batch_packing():
    wl = make_workload("mix_small")
    st = DSAStep.from_workload(wl, n_layers=1)
    st.store_keys()
    st.index_topk()
    full = st.sel.cpu().numpy()
    # each span alone, at row 0 of its own plan, over the same (already stored) pool
    for s_idx, span in enumerate(wl.spans):
        q0, ql = int(span[0]), int(span[1])
        one = span.copy()[None]
        one[0, 0] = 0
        plan = dsa.Plan.on_device(one, wl.page_table, wl.pool_pages)
        sel = torch.empty(ql, st.topk, dtype=torch.int32, device="cuda")
        ws = torch.empty(dsa.dsa_workspace_size(st.h, plan, dsa.DSA_OP_INDEX_TOPK), dtype=torch.uint8,
                         device="cuda")
        dsa.dsa_index_topk(st.h, plan, st.index_q[q0:q0 + ql].contiguous(),
                           st.index_w[q0:q0 + ql].contiguous(), st.key_pool, sel, ws)
        assert np.array_equal(sel.cpu().numpy(), full[q0:q0 + ql]), f"span {s_idx}"


def test_zero_queries_tie_to_lowest_positions():
    wl = make_workload("decode_small")
    wl.index_q.zero_()
    st = DSAStep.from_workload(wl, n_layers=1)
    st.store_keys()
    st.index_topk()
    sel = st.sel.cpu().numpy()
    for t, p in enumerate(wl.positions):
        n = min(st.topk, int(p) + 1)
        assert sel[t, :n].tolist() == list(range(n)) and np.all(sel[t, n:] == -1)


def test_ties_at_the_threshold_take_lower_positions():
    # Scores drawn from a few integer values so that the k-th score is shared by many keys.
    wl = make_workload("decode_small")
    st = DSAStep.from_workload(wl, n_layers=1)
    T = st.plan.n_rows
    ld = int((wl.positions.max() + 1 + 3) // 4 * 4)
    g = torch.Generator().manual_seed(9)
    sc = torch.randint(0, 5, (T, ld), generator=g).float()
    sc[sc == 0] = -0.0
    sel = select_on_gpu(st, sc.cuda(), ld).cpu().numpy()
    for t, p in enumerate(wl.positions):
        assert np.array_equal(sel[t], oracle.select_topk_causal_row(sc[t].numpy(), int(p), st.topk)), t


@pytest.mark.parametrize("topk", [1, 7, 64, 4096])
def test_topk_edge_values(topk):
    wl = make_workload("long_decode_small")
    wl.spec.topk = topk
    st = DSAStep.from_workload(wl, n_layers=1)
    st.store_keys()
    st.index_topk()
    st.attend(0)
    sc, ld = scores_on_gpu(st)
    sc = sc.cpu().numpy()
    sel = st.sel.cpu().numpy()
    rows = list(range(st.plan.n_rows))
    for t in rows:
        assert np.array_equal(sel[t], oracle.select_topk_causal_row(sc[t], int(wl.positions[t]), topk))
    from tests.gpu_helpers import check_attend
    check_attend(wl, st, rows, {t: sel[t] for t in rows}, 0, f"topk={topk}")
    if topk == 1:   # out = the picked latent's leading R columns
        # up to two bf16 roundings (the fp8 group scale folded into P, then the output), each at
        # most 2^-8 of the value
        R, P = wl.spec.kv_lora_rank, wl.spec.rope_dim
        for t in rows:
            c = oracle.read_latents(wl.latent_pools[0].numpy(), "fp8", wl.spans[t], wl.page_table,
                                    wl.spec.page_size, R, P, [int(sel[t, 0])])[0, :R]
            got = st.out[0][t].float().cpu().numpy()
            assert np.all(np.abs(got - c[None]) <= 2.0 ** -7 * np.abs(c[None]) + 1e-6)


def test_single_key_rows_and_page_start():
    # rows at position 0 see only themselves; spans start mid-page
    wl = make_workload("prefill_small")
    r = full_parity(wl, rows=[0, 1, 2, 255, 256, 699])
    note(f"[parity] prefill_small edges: {r['worst_attend']:.3g}")


@pytest.mark.parametrize("name,n_rows", [("decode_batch", 32), ("long_decode", 8)])
def test_full_size_decode(name, n_rows):
    note(f"[parity] {name} full size, all {n_rows} rows")
    wl = make_workload(name)
    r = full_parity(wl)
    note(f"[parity] {name}: worst score err {r['worst_score']:.3g}x tol, attend {r['worst_attend']:.3g}")


@pytest.mark.parametrize("name", ["causal_prefill", "chunked_mix"])
def test_full_size_prefill_sampled(name):
    note(f"[parity] {name} full size, sampled rows")
    wl = make_workload(name)
    rows = helpers.sample_rows(wl, 24, seed=3)
    if name == "causal_prefill":
        rows = sorted(set(rows) | {0, 1, 2046, 2047, 2048, 8191})
    r = full_parity(wl, rows=rows)
    # exact -1 count over every row (a closed form of positions and topk)
    sel = r["step"].sel  # the oracle selection was copied over the sampled rows; recompute
    r["step"].index_topk()
    n_pad = int((r["step"].sel == -1).sum().item())
    expect = int(sum(max(0, wl.spec.topk - int(p) - 1) for p in wl.positions))
    assert n_pad == expect
    note(f"[parity] {name}: pads {n_pad}, worst score err {r['worst_score']:.3g}x tol, attend {r['worst_attend']:.3g}")


@pytest.mark.parametrize("name", ["long_decode_small", "prefill_fp8_small"])
def test_pools_past_4gib(name):
    # Pools of more than 4 GiB of index keys make the score kernels address pages with 64-bit
    # offsets. The workload's pages are moved past the 4 GiB mark of both pools (page p -> p +
    # shift); every result must be that of the same workload in its own small pools, bit for bit,
    # and the attention must match the oracle.
    wl = make_workload(name)
    s = wl.spec
    kpb = oracle.index_page_bytes(s.index_key_fmt, s.page_size, s.index_dim)
    lpb = s.page_size * oracle.latent_row_bytes(s.latent_fmt, s.kv_lora_rank, s.rope_dim)
    shift = (1 << 32) // kpb + 1
    big_pages = wl.pool_pages + shift
    note(f"[parity] {name}: pools of {big_pages} pages ({big_pages * kpb / 2**30:.2f} GiB of keys, "
         f"{big_pages * lpb / 2**30:.2f} GiB of latents), pages moved up by {shift}")
    small = DSAStep.from_workload(wl, n_layers=1)
    small.run()

    key_big = torch.empty(big_pages * kpb, dtype=torch.uint8, device="cuda")
    lat_big = torch.empty(big_pages * lpb, dtype=torch.uint8, device="cuda")
    key_big[shift * kpb:].copy_(wl.key_pool)
    lat_big[shift * lpb:].copy_(wl.latent_pools[0])
    table = wl.page_table.astype(np.int64) + shift
    assert table.max() < 2**31
    big = DSAStep(n_index_heads=s.n_index_heads, index_dim=s.index_dim, index_q_fmt=s.index_q_fmt,
                  index_key_fmt=s.index_key_fmt, topk=s.topk, n_heads=s.n_heads,
                  kv_lora_rank=s.kv_lora_rank, rope_dim=s.rope_dim, q_fmt=s.q_fmt,
                  latent_fmt=s.latent_fmt, page_size=s.page_size, sm_scale=s.sm_scale,
                  spans=wl.spans, page_table=table.astype(np.int32), pool_pages=big_pages,
                  index_q=wl.index_q, index_w=wl.index_w, step_keys=wl.step_keys,
                  step_key_scales=wl.step_key_scales, key_pool=key_big, q_nope=wl.q_nope[:1],
                  q_pe=wl.q_pe[:1], latent_pools=[lat_big], sinks=wl.sinks[:1])
    big.run()
    torch.cuda.synchronize()
    assert np.array_equal(key_big[shift * kpb:].cpu().numpy(), helpers.oracle_key_pool(wl))
    assert torch.equal(big.sel, small.sel), "selection differs past 4 GiB"
    assert torch.equal(big.out[0].view(torch.uint8), small.out[0].view(torch.uint8)), \
        "attention differs past 4 GiB"
    from tests.gpu_helpers import check_attend
    rows = list(range(big.plan.n_rows))
    sel = big.sel.cpu().numpy()
    check_attend(wl, big, rows, {t: sel[t] for t in rows}, 0, f"{name} past 4 GiB")
    del big, key_big, lat_big
    torch.cuda.empty_cache()
