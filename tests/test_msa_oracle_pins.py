"""Pins of the block-sparse MSA oracle to facts fixed outside it: brute force on small inputs,
the byte sizes the sparse-attention page prints, and dense causal GQA attention through torch.
CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import msa_oracle as msa
from synth import make_msa_workload
from tests import helpers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_cache_row_bytes_match_page_numbers():
    # "Sparse attention (DSA and block-sparse MSA)", section "What the KV cache actually holds":
    # M3 GQA 2,048 B and M3 indexer cache 256 B per token per layer
    pages = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))
    assert msa.gqa_row_bytes(4, 128) == pages["m3_gqa_bytes_per_token"]["value"] == 2048
    assert oracle.index_page_bytes("bf16", 1, 128) == pages["m3_index_bytes_per_token"]["value"] == 256
    assert (pages["msa_blocks"]["value"], pages["msa_blocks"]["block"]) == (16, 128)


def test_block_scores_are_brute_force_maxima():
    rng = np.random.default_rng(1)
    for pos in (0, 5, 127, 128, 129, 300, 511):
        s = rng.normal(size=pos + 1 + 40).astype(np.float32)
        got = msa.block_scores_row(s, pos, 128)
        want = [max(float(s[j]) for j in range(pos + 1) if j // 128 == b) for b in range(pos // 128 + 1)]
        assert got.dtype == np.float32 and got.tolist() == want


def test_select_blocks_matches_sorted_with_forced_ties():
    rng = np.random.default_rng(2)
    for trial in range(200):
        nb = int(rng.integers(1, 40))
        k = int(rng.integers(1, 20))
        s = rng.integers(0, 6, size=nb).astype(np.float32)      # many equal scores
        order = sorted(range(nb), key=lambda b: (-float(s[b]), b))
        want = (order[:k] + [-1] * k)[:k]
        assert msa.select_blocks_row(s, k).tolist() == want


def _wl_and_sel(name, topk=None):
    wl = make_msa_workload(name)
    s = wl.spec
    sel, bs = msa.msa_select(helpers.to_f64(wl.index_q), helpers.to_f64(wl.index_w), wl.key_pool.numpy(),
                             "bf16", wl.spans, wl.page_table, s.page_size, topk or s.topk_blocks, s.block,
                             return_scores=True)
    return wl, sel, bs


def test_select_pad_counts_and_visibility():
    wl, sel, _ = _wl_and_sel("msa_decode_small")
    for t, p in enumerate(wl.positions):
        nb = int(p) // 128 + 1
        assert int((sel[t] >= 0).sum()) == min(16, nb)
        assert np.all(sel[t][sel[t] >= 0] < nb)
    # a row at position 128 sees two blocks, the second holding only itself
    t128 = int(np.nonzero(wl.positions == 128)[0][0])
    assert sorted(sel[t128][:2].tolist()) == [0, 1] and np.all(sel[t128][2:] == -1)


def test_all_blocks_equals_dense_causal_gqa():
    wl, sel, _ = _wl_and_sel("msa_prefill_small", topk=64)   # 64 blocks cover every position here
    s = wl.spec
    q = helpers.to_f64(wl.q)
    rows = [0, 75, 149, 150, 160, 170]
    sparse = msa.msa_attend({t: sel[t] for t in rows}, q, wl.gqa_pool.numpy(), wl.spans, wl.page_table,
                            s.page_size, s.n_kv_heads, s.head_dim, s.block, s.sm_scale)
    dense = msa.dense_causal_gqa(q, wl.gqa_pool.numpy(), wl.spans, wl.page_table, s.page_size,
                                 s.n_kv_heads, s.head_dim, s.sm_scale, rows)
    for t in rows:
        np.testing.assert_allclose(sparse[t], dense[t], rtol=0, atol=1e-12)


def test_attend_special_cases():
    wl, sel, _ = _wl_and_sel("msa_decode_small")
    s = wl.spec
    q = helpers.to_f64(wl.q)
    pool = wl.gqa_pool.numpy()
    t0 = int(np.nonzero(wl.positions == 0)[0][0])
    out = msa.msa_attend({t0: sel[t0]}, q, pool, wl.spans, wl.page_table, s.page_size, s.n_kv_heads,
                         s.head_dim, s.block, s.sm_scale)
    _, v = msa.read_gqa(pool, wl.spans[t0], wl.page_table, s.page_size, s.n_kv_heads, s.head_dim, [0])
    for h in range(s.n_heads):          # one visible token: its V row for every head of the group
        np.testing.assert_array_equal(out[t0][h], v[0, h // (s.n_heads // s.n_kv_heads)])
    # q = 0: uniform weights over the visible tokens of the picked blocks
    t = 0
    zero = np.zeros_like(q)
    out0 = msa.msa_attend({t: sel[t]}, zero, pool, wl.spans, wl.page_table, s.page_size, s.n_kv_heads,
                          s.head_dim, s.block, s.sm_scale)
    j = msa.block_positions(sel[t], int(wl.positions[t]), s.block)
    _, vv = msa.read_gqa(pool, wl.spans[t], wl.page_table, s.page_size, s.n_kv_heads, s.head_dim, j)
    for h in range(s.n_heads):
        np.testing.assert_allclose(out0[t][h], vv[:, h // 8].mean(0), rtol=0, atol=1e-13)
    # heads of one group with equal queries give equal outputs
    q2 = q.copy()
    q2[t, 1] = q2[t, 0]
    o2 = msa.msa_attend({t: sel[t]}, q2, pool, wl.spans, wl.page_table, s.page_size, s.n_kv_heads,
                        s.head_dim, s.block, s.sm_scale)
    np.testing.assert_array_equal(o2[t][0], o2[t][1])


def test_empty_selection_gives_zeros():
    wl = make_msa_workload("msa_decode_small")
    s = wl.spec
    out = msa.msa_attend({0: np.full(16, -1, np.int32)}, helpers.to_f64(wl.q), wl.gqa_pool.numpy(),
                         wl.spans, wl.page_table, s.page_size, s.n_kv_heads, s.head_dim, s.block, s.sm_scale)
    assert np.all(out[0] == 0) and out[0].shape == (s.n_heads, s.head_dim)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_gqa_row_layout_read_back(fmt):
    # a hand-built pool: slot (page, off), K (part 0) or V (part 1), KV head kv holds
    # 8 page + 4 off + 2 part + kv + e / 8 at element e: distinct, and exact in bf16 (below 24
    # with three fraction bits: 8 significant bits)
    n_kv, d, ps, n_pages = 2, 8, 2, 3
    vals = np.zeros((n_pages, ps, 2, n_kv, d))
    for pg in range(n_pages):
        for off in range(ps):
            for part in range(2):
                for kv in range(n_kv):
                    vals[pg, off, part, kv] = 8 * pg + 4 * off + 2 * part + kv + np.arange(d) / 8
    flat = vals.reshape(n_pages, ps, -1)
    if fmt == "f32":
        pool = flat.astype(np.float32).view(np.uint8).reshape(-1)
    else:
        pool = torch.from_numpy(flat).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8).reshape(-1)
    assert pool.size == n_pages * ps * msa.gqa_row_bytes(n_kv, d, fmt)
    # one request over pages [2, 0], starting at slot 1 of its first page: position j sits at
    # page list entry (1 + j) // 2, offset (1 + j) % 2
    span = np.array([0, 1, 2, 0, 2, 1], dtype=np.int32)
    k, v = msa.read_gqa(pool, span, np.array([2, 0], np.int32), ps, n_kv, d, [0, 1, 2], fmt)
    for j, (pg, off) in enumerate([(2, 1), (0, 0), (0, 1)]):
        for kv in range(n_kv):
            want_k = 8 * pg + 4 * off + kv + np.arange(d) / 8
            assert np.array_equal(k[j, kv], want_k), (fmt, j, kv)
            assert np.array_equal(v[j, kv], want_k + 2)
