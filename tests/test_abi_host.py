"""The C-ABI library loads, exports every symbol its header declares, and rejects bad arguments on
the host before anything is enqueued. CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import torch
import pytest

from sparse_attention_dsa_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

FAKE = 1 << 40   # a 256-aligned address the host only compares, never dereferences


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_header_functions_are_all_exported():
    lib = dsa.load()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsa.EXPORTS)


def big_cfg(**kw):
    d = dict(n_index_heads=64, index_dim=128, index_q_fmt="bf16", index_key_fmt="bf16", topk=2048,
             n_heads=128, kv_lora_rank=512, rope_dim=64, q_fmt="bf16", latent_fmt="bf16",
             page_size=64)
    d.update(kw)
    return dsa.make_config(**d)


def fake_plan(spans, table, pool_pages, host_table=True, cap=0):
    spans = np.asarray(spans, np.int32).reshape(-1, 6)
    return dsa.Plan(spans, table, pool_pages, FAKE, FAKE + 4096, check_pages=host_table,
                    max_visible_cap=cap)


def expect(status, fn, *a):
    with pytest.raises(dsa.DSAError) as e:
        fn(*a)
    assert e.value.status == status, str(e.value)
    return str(e.value)


@pytest.mark.parametrize("field,value", [
    ("n_index_heads", 0), ("index_dim", 12), ("topk", 0), ("topk", dsa.DSA_MAX_TOPK + 1),
    ("n_heads", 0), ("kv_lora_rank", 7), ("rope_dim", -8), ("page_size", 0), ("q_fmt", 5),
    ("index_q_fmt", 7), ("index_q_fmt", 2), ("latent_fmt", 9),
])
def test_create_rejects_bad_config(field, value):
    cfg = big_cfg()
    setattr(cfg, field, value)
    expect(-1, dsa.dsa_create, cfg)


def test_create_rejects_unsupported_combinations():
    expect(-3, dsa.dsa_create, big_cfg(latent_fmt="fp8", kv_lora_rank=64))


def test_workspace_and_plan_errors():
    h = dsa.dsa_create(big_cfg())
    good = fake_plan([[0, 1, 100, 0, 2, 0], [1, 3, 0, 2, 1, 5]], [3, 1, 0], 4)
    dsa.dsa_plan_check(h, good)
    assert dsa.dsa_workspace_size(h, good, dsa.DSA_OP_INDEX_TOPK) > 0
    # spans must be contiguous in row order
    expect(-1, dsa.dsa_plan_check, h, fake_plan([[0, 1, 100, 0, 2, 0], [2, 1, 0, 2, 1, 0]], [3, 1, 0], 4))
    # a row's position beyond its pages (the analogue of IndexKeyStore.history raising)
    msg = expect(-2, dsa.dsa_plan_check, h, fake_plan([[0, 1, 128, 0, 2, 0]], [3, 1], 4))
    assert "position 128" in msg
    # page_start pushes the last slot past the list
    expect(-2, dsa.dsa_plan_check, h, fake_plan([[0, 1, 100, 0, 2, 28]], [3, 1], 4))
    # page ids outside the pool are caught when the host table is given, not otherwise
    bad = fake_plan([[0, 1, 100, 0, 2, 0]], [3, 9], 4)
    expect(-2, dsa.dsa_plan_check, h, bad)
    dsa.dsa_plan_check(h, fake_plan([[0, 1, 100, 0, 2, 0]], [3, 9], 4, host_table=False))
    # page list past the page table
    expect(-2, dsa.dsa_plan_check, h, fake_plan([[0, 1, 100, 1, 2, 0]], [3, 1], 4))
    # zero-length span and negative position
    expect(-1, dsa.dsa_plan_check, h, fake_plan([[0, 0, 100, 0, 2, 0]], [3, 1], 4))
    expect(-1, dsa.dsa_plan_check, h, fake_plan([[0, 1, -1, 0, 2, 0]], [3, 1], 4))
    # unknown op
    expect(-1, dsa.dsa_workspace_size, h, good, 17)
    # a launch-size cap must cover the longest row (position 100: 101 visible) and sizes the
    # workspace in its place
    expect(-1, dsa.dsa_plan_check, h, fake_plan([[0, 1, 100, 0, 2, 0]], [3, 1], 4, cap=100))
    sp = [[0, 1, 100, 0, 2, 0], [1, 3, 0, 2, 1, 5]]
    dsa.dsa_plan_check(h, fake_plan(sp, [3, 1, 0], 4, cap=101))
    small = dsa.dsa_workspace_size(h, fake_plan(sp, [3, 1, 0], 4, cap=101), dsa.DSA_OP_INDEX_TOPK)
    assert small == dsa.dsa_workspace_size(h, good, dsa.DSA_OP_INDEX_TOPK)
    big = dsa.dsa_workspace_size(h, fake_plan(sp, [3, 1, 0], 4, cap=50000), dsa.DSA_OP_INDEX_TOPK)
    assert big > small


def test_call_argument_errors_before_launch():
    h = dsa.dsa_create(big_cfg())
    plan = fake_plan([[0, 2, 100, 0, 2, 0]], [3, 1], 4)
    need = dsa.dsa_workspace_size(h, plan, dsa.DSA_OP_INDEX_TOPK)
    # null / misaligned pointers
    expect(-1, dsa.dsa_index_topk, h, plan, 0, FAKE, FAKE, FAKE, FAKE, need, 0)
    expect(-1, dsa.dsa_index_topk, h, plan, FAKE + 2, FAKE, FAKE, FAKE, FAKE, need, 0)
    # too small or misaligned workspace
    expect(-4, dsa.dsa_index_topk, h, plan, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0)
    expect(-1, dsa.dsa_index_topk, h, plan, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need, 0)
    # store_keys: bf16 keys take no scales; fp8 keys need them
    expect(-1, dsa.dsa_store_keys, h, plan, FAKE, FAKE, FAKE, 0)
    h8 = dsa.dsa_create(big_cfg(index_key_fmt="fp8"))
    expect(-1, dsa.dsa_store_keys, h8, plan, FAKE, None, FAKE, 0)
    # scores leading dimension must cover every visible key
    expect(-1, dsa.dsa_index_scores, h, plan, FAKE, FAKE, FAKE, FAKE, 100, 0)
    expect(-1, dsa.dsa_select_topk, h, plan, FAKE, 102, FAKE, FAKE, 1 << 20, 0)
    # attend: non-finite scale, null output
    expect(-1, dsa.dsa_sparse_mla_attend, h, plan, FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, FAKE, 1 << 30, 0)
    expect(-1, dsa.dsa_sparse_mla_attend, h, plan, FAKE, FAKE, FAKE, FAKE, 0.1, 0, FAKE, 1 << 30, 0)
    # attend with a sink: the sink array is required and 4-byte aligned
    msg = expect(-1, dsa.dsa_sparse_mla_attend_sink, h, plan, FAKE, FAKE, FAKE, FAKE, 0.1, 0, FAKE,
                 FAKE, 1 << 30, 0)
    assert "sink" in msg
    expect(-1, dsa.dsa_sparse_mla_attend_sink, h, plan, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE + 2, FAKE,
           FAKE, 1 << 30, 0)
    # e4m3 queries are accepted for the attention
    dsa.dsa_create(big_cfg(q_fmt="fp8", latent_fmt="fp8"))
    assert dsa.dsa_last_error() != ""


def test_status_strings():
    assert dsa.dsa_status_str(0) == "ok"
    assert dsa.dsa_status_str(-4) == "workspace too small"


def test_e4m3_output_check_tells_rounding_from_truncation():
    # The parity check of e4m3 outputs accepts the nearest-even rounding of any value within the
    # tolerance, and rejects outputs truncated toward zero (a plausible wrong conversion).
    from tests import helpers
    rng = np.random.default_rng(3)
    o = rng.normal(0.0, 0.3, 20000)
    tol = 2e-3
    v = o + rng.uniform(-tol, tol, o.size)
    assert helpers.e4m3_interval_ok(helpers.e4m3_round(v), o, tol).all()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    mags = np.unique(np.abs(codes.to(torch.float64).numpy()))
    mags = mags[np.isfinite(mags)]                                     # 0 .. 448, ascending
    trunc = np.sign(v) * mags[np.searchsorted(mags, np.abs(v), side="right") - 1]
    bad = ~helpers.e4m3_interval_ok(trunc, o, tol)
    assert bad.mean() > 0.2, bad.mean()


def msa_cfg(**kw):
    d = dict(n_index_heads=64, index_dim=128, index_q_fmt="bf16", index_key_fmt="bf16", block_size=128,
             topk_blocks=16, n_heads=32, n_kv_heads=4, head_dim=128, q_fmt="bf16", page_size=64)
    d.update(kw)
    return dsa.make_msa_config(**d)


@pytest.mark.parametrize("field,value,status", [
    ("block_size", 100, -3), ("topk_blocks", 0, -1), ("topk_blocks", 65, -1), ("n_kv_heads", 3, -1),
    ("head_dim", 12, -1), ("q_fmt", 2, -1), ("index_dim", 12, -1), ("page_size", 0, -1),
])
def test_msa_create_rejects_bad_config(field, value, status):
    cfg = msa_cfg()
    setattr(cfg, field, value)
    expect(status, dsa.dsa_msa_create, cfg)


def test_msa_plan_and_argument_errors():
    h = dsa.dsa_msa_create(msa_cfg())
    plan = fake_plan([[0, 2, 300, 0, 5, 0]], [3, 1, 0, 2, 4], 5)
    need = dsa.dsa_msa_workspace_size(h, plan, dsa.DSA_OP_SELECT_TOPK)
    # two rows of 320 scores, then one key per block (3 blocks of 128 at position 301)
    assert need >= 2 * 320 * 4 + 2 * 3 * 8
    att = dsa.dsa_msa_workspace_size(h, plan, dsa.DSA_OP_ATTEND)
    assert att >= 2 * 32 * 16 * (128 + 2) * 4            # rows x heads x blocks x (d + max, sum)
    expect(-2, dsa.dsa_msa_workspace_size, h, fake_plan([[0, 1, 400, 0, 5, 0]], [3, 1, 0, 2, 4], 5),
           dsa.DSA_OP_SELECT_TOPK)
    expect(-4, dsa.dsa_msa_select_blocks, h, plan, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0)
    expect(-1, dsa.dsa_msa_select_blocks, h, plan, 0, FAKE, FAKE, FAKE, FAKE, need, 0)
    expect(-1, dsa.dsa_msa_attend, h, plan, FAKE, FAKE, FAKE, float("inf"), FAKE, FAKE, att, 0)
    expect(-1, dsa.dsa_msa_attend, h, plan, FAKE, FAKE, 0, 0.1, FAKE, FAKE, att, 0)
    expect(-4, dsa.dsa_msa_attend, h, plan, FAKE, FAKE, FAKE, 0.1, FAKE, None, 0, 0)
    expect(-4, dsa.dsa_msa_attend, h, plan, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, att - 1, 0)


def test_binding_rejects_host_strided_and_short_tensors():
    # The library can check only null and alignment, so the binding checks every torch tensor:
    # contiguous, at least the bytes its argument needs, and on the GPU. Each failure raises
    # before anything reaches the library (no GPU here: a call that got through would fail later
    # with another status and message).
    cfg = big_cfg(n_index_heads=4, index_dim=16, topk=8, n_heads=2, kv_lora_rank=16, rope_dim=8,
                  page_size=4)
    h = dsa.dsa_create(cfg)
    plan = fake_plan([[0, 3, 5, 0, 2, 0]], [1, 0], 2)          # 3 rows at positions 5..7
    T, need = 3, dsa.dsa_workspace_size(h, plan, dsa.DSA_OP_INDEX_TOPK)
    q = torch.zeros(T, 4, 16, dtype=torch.bfloat16)
    w = torch.zeros(T, 4, dtype=torch.float32)
    pool = torch.zeros(2 * 4 * 16 * 2, dtype=torch.uint8)
    sel = torch.zeros(T, 8, dtype=torch.int32)
    # right sizes, but host memory
    msg = expect(-1, dsa.dsa_index_topk, h, plan, q, FAKE, FAKE, FAKE, FAKE, need, 0)
    assert "q:" in msg and "not on the GPU" in msg
    for bad in (w, pool, sel):
        args = [FAKE, FAKE, FAKE, FAKE]
        args[[w is bad, pool is bad, sel is bad].index(True) + 1] = bad
        assert "not on the GPU" in expect(-1, dsa.dsa_index_topk, h, plan, *args, FAKE, need, 0)
    # a strided view of the right size: the q slice of a wider tensor
    wide = torch.zeros(T, 4, 32, dtype=torch.bfloat16)
    assert "not contiguous" in expect(-1, dsa.dsa_index_topk, h, plan, wide[:, :, :16], FAKE, FAKE,
                                      FAKE, FAKE, need, 0)
    # one element short, and a workspace tensor smaller than the byte count passed with it
    assert "bytes, the call needs" in expect(-1, dsa.dsa_index_topk, h, plan, FAKE, FAKE, FAKE,
                                             sel.view(-1)[:-1], FAKE, need, 0)
    ws = torch.zeros(need - 1, dtype=torch.uint8)
    assert "ws:" in expect(-1, dsa.dsa_index_topk, h, plan, FAKE, FAKE, FAKE, FAKE, ws, need, 0)
    # attend: q_pe and out sized from n_heads, the rope and latent widths and q_fmt
    qpe_short = torch.zeros(T * 2 * 8 - 1, dtype=torch.bfloat16)
    assert "q_pe:" in expect(-1, dsa.dsa_sparse_mla_attend, h, plan, FAKE, FAKE, qpe_short, FAKE,
                             0.1, FAKE, FAKE, 1 << 20, 0)
    lat_short = torch.zeros(2 * 4 * (16 + 8) * 2 - 2, dtype=torch.uint8)
    assert "latent_pool:" in expect(-1, dsa.dsa_sparse_mla_attend, h, plan, FAKE, FAKE, FAKE,
                                    lat_short, 0.1, FAKE, FAKE, 1 << 20, 0)
    sink = torch.zeros(1, dtype=torch.float32)
    assert "sink:" in expect(-1, dsa.dsa_sparse_mla_attend_sink, h, plan, FAKE, FAKE, FAKE, FAKE,
                             0.1, sink, FAKE, FAKE, 1 << 20, 0)
    # store_keys: fp8 keys need T fp32 scales, and the pool's fp8 page is page_size * (D + 4)
    h8 = dsa.dsa_create(big_cfg(index_dim=16, topk=8, n_heads=2, kv_lora_rank=16, rope_dim=8,
                                page_size=4, index_key_fmt="fp8"))
    pool8 = torch.zeros(2 * 4 * 16, dtype=torch.uint8)          # bf16-sized for fp8: too short
    assert "key_pool:" in expect(-1, dsa.dsa_store_keys, h8, plan, FAKE, FAKE, pool8, 0)
    # plan device copies
    with pytest.raises(dsa.DSAError, match="spans_dev"):
        dsa.Plan([[0, 3, 5, 0, 2, 0]], [1, 0], 2, torch.zeros(6, dtype=torch.int32), FAKE)
    with pytest.raises(dsa.DSAError, match="page_table_dev"):
        dsa.Plan([[0, 3, 5, 0, 2, 0]], [1, 0], 2, FAKE, torch.zeros(1, dtype=torch.int32))
