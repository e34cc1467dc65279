"""Pins of the CPU oracle to facts fixed outside it: numbers the pages print, closed forms,
brute force on tiny inputs, library routines and invariants. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import make_workload
from tests import helpers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- storage formats

def test_e4m3_decode_matches_torch_for_every_byte():
    b = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3_decode_spec_values():
    # OCP 8-bit floating point spec, E4M3: bias 7, max normal 448, min subnormal 2^-9, NaN S.1111.111
    cases = {0x00: 0.0, 0x38: 1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0xC6: -3.5,
             0x3C: 1.5, 0x80: -0.0}
    for byte, val in cases.items():
        assert oracle.e4m3_to_f64([byte])[0] == val, hex(byte)
    assert np.isnan(oracle.e4m3_to_f64([0x7F])[0]) and np.isnan(oracle.e4m3_to_f64([0xFF])[0])


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(4096, generator=g) * 100).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x.to(torch.float64).numpy())


def test_layout_bytes_match_page_numbers():
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        g = json.load(f)
    R, P, D = g["kv_lora_rank"]["value"], g["rope_dim"]["value"], g["index_head_dim"]["value"]
    assert oracle.latent_row_bytes("bf16", R, P) == g["latent_row_bf16_bytes"]["value"]
    assert oracle.latent_row_bytes("fp8", R, P) == g["packed_fp8_latent_row_bytes"]["value"]
    assert oracle.index_page_bytes("fp8", 64, D) // 64 == g["index_row_bytes"]["value"]
    per_layer = oracle.latent_row_bytes("bf16", R, P) + oracle.index_page_bytes("fp8", 1, D)
    t = g["deepseek_v32_bytes_per_token_all_layers"]
    assert t["layers"] * per_layer == t["value"]


# ---------------------------------------------------------------- paging (DSASpan / DSAPlan)

def _place_keys(keys_raw, fmt, page_size, dim, page_table, page_start, pool_pages, scales=None):
    """Independent placement used only by these pins: token j -> list slot page_start + j."""
    pb = oracle.index_page_bytes(fmt, page_size, dim)
    pool = np.zeros((pool_pages, pb), dtype=np.uint8)
    for j in range(len(keys_raw)):
        slot = page_start + j
        page, off = page_table[slot // page_size], slot % page_size
        if fmt == "fp8":
            pool[page, off * dim:(off + 1) * dim] = keys_raw[j]
            pool[page, page_size * dim + 4 * off: page_size * dim + 4 * off + 4] = \
                np.array([scales[j]], np.float32).view(np.uint8)
        else:
            b = np.ascontiguousarray(keys_raw[j]).view(np.uint8)
            pool[page, off * b.size:(off + 1) * b.size] = b
    return pool.reshape(-1)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8"])
def test_read_index_keys_follows_the_page_table(fmt):
    rng = np.random.default_rng(1)
    ps, dim, n, pool_pages = 16, 32, 70, 9
    page_start = 13
    table = rng.permutation(pool_pages).astype(np.int32)
    n_pages = -(-(page_start + n) // ps)
    span = np.array([0, 1, n - 1, 2, n_pages, page_start])
    full_table = np.concatenate([np.array([7, 7], np.int32), table[:n_pages]])
    x = rng.standard_normal((n, dim)).astype(np.float32)
    if fmt == "fp8":
        codes = rng.integers(0, 0x7E, size=(n, dim), dtype=np.uint8)
        codes[:, 1] |= 0x80
        scales = rng.uniform(0.1, 2, n).astype(np.float32)
        pool = _place_keys(codes, fmt, ps, dim, full_table[2:], page_start, pool_pages, scales)
        expect = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * scales[:, None]
    elif fmt == "bf16":
        t = torch.from_numpy(x).to(torch.bfloat16)
        pool = _place_keys(t.view(torch.int16).numpy(), fmt, ps, dim, full_table[2:], page_start, pool_pages)
        expect = t.double().numpy()
    else:
        pool = _place_keys(x, fmt, ps, dim, full_table[2:], page_start, pool_pages)
        expect = x.astype(np.float64)
    got = oracle.read_index_keys(pool, fmt, span, full_table, ps, dim, n)
    assert np.array_equal(got, expect)


def test_read_latents_packed_fp8_row_by_hand():
    # One 656-byte row [512 e4m3 | 4 fp32 scales | 64 bf16 rope] built byte by byte.
    R, P, ps = 512, 64, 4
    rb = oracle.latent_row_bytes("fp8", R, P)
    row = np.zeros(rb, np.uint8)
    row[0] = 0x38          # 1.0 in group 0
    row[130] = 0xC6        # -3.5 in group 1
    row[511] = 0x7E        # 448 in group 3
    row[512:528] = np.array([0.5, 2.0, 4.0, 0.25], np.float32).view(np.uint8)
    rope = np.zeros(P, np.uint16)
    rope[0] = 0x3FC0       # bf16 1.5
    rope[63] = 0xC040      # bf16 -3.0
    row[528:] = rope.view(np.uint8)
    pool = np.zeros((3, ps, rb), np.uint8)
    pool[2, 1] = row
    span = np.array([0, 1, 0, 0, 1, 1])
    got = oracle.read_latents(pool.reshape(-1), "fp8", span, np.array([2], np.int32), ps, R, P, [0])[0]
    expect = np.zeros(R + P)
    expect[0], expect[130], expect[511] = 0.5, -7.0, 112.0
    expect[R], expect[R + 63] = 1.5, -3.0
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_read_latents_plain_rows_by_hand(fmt):
    # A bf16 or f32 latent row [R elements | P elements] written byte by byte (little-endian), in
    # page 2 at offset 3 of a pool whose other rows hold garbage.
    import struct
    R, P, ps = 16, 8, 4
    width = 2 if fmt == "bf16" else 4
    rb = oracle.latent_row_bytes(fmt, R, P)
    assert rb == (R + P) * width
    vals = {0: 1.0, 5: -5.0, 15: 200.0, R: 1.5, R + 7: -0.375}
    row = bytearray(rb)
    for i, v in vals.items():
        if fmt == "bf16":
            bits = struct.unpack("<I", struct.pack("<f", v))[0] >> 16   # exact in bf16
            row[2 * i:2 * i + 2] = struct.pack("<H", bits)
        else:
            row[4 * i:4 * i + 4] = struct.pack("<f", v)
    rng = np.random.default_rng(5)
    pool = rng.integers(0, 255, (3, ps, rb), dtype=np.uint8)
    pool[:, :, width - 1::width] &= 0x3F       # keep the garbage finite
    pool[2, 3] = np.frombuffer(bytes(row), np.uint8)
    # position 2 of a span whose list is [0, 2] starting at slot 5: slot 7 -> list entry 1 -> page
    # 2, offset 3
    span = np.array([0, 1, 2, 0, 2, 5])
    got = oracle.read_latents(pool.reshape(-1), fmt, span, np.array([0, 2], np.int32), ps, R, P, [2])
    expect = np.zeros(R + P)
    for i, v in vals.items():
        expect[i] = v
    assert got.shape == (1, R + P) and np.array_equal(got[0], expect)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_store_keys_plain_rows_write_only_their_slots(fmt):
    import struct
    ps, dim = 4, 8
    width = 2 if fmt == "bf16" else 4
    pb = oracle.index_page_bytes(fmt, ps, dim)
    assert pb == ps * dim * width
    spans = np.array([[0, 2, 3, 0, 2, 0], [2, 1, 6, 2, 2, 1]], np.int32)
    table = np.array([2, 0, 1, 3], np.int32)
    rng = np.random.default_rng(6)
    pool = rng.integers(0, 255, 4 * pb, dtype=np.uint8)
    if fmt == "bf16":
        keys = rng.integers(0, 0x7F7F, (3, dim), dtype=np.uint16)
        enc = lambda x: struct.pack("<H", int(x))          # noqa: E731
    else:
        keys = rng.normal(size=(3, dim)).astype(np.float32)
        enc = lambda x: struct.pack("<f", float(x))        # noqa: E731
    new = oracle.store_keys(pool, fmt, spans, table, ps, dim, keys, None)
    # row 0: request 0 position 3 -> slot 3 -> table[0] = 2, offset 3; row 1: position 4 -> slot
    # 4 -> table[1] = 0, offset 0; row 2: request 1 position 6 -> slot 7 -> table[2 + 1] = 3,
    # offset 3
    where = [(2, 3), (0, 0), (3, 3)]
    expect = bytearray(pool.tobytes())
    for t, (page, off) in enumerate(where):
        at = page * pb + off * dim * width
        expect[at:at + dim * width] = b"".join(enc(x) for x in keys[t])
    assert new.tobytes() == bytes(expect)


def test_store_keys_writes_only_the_rows_slots():
    rng = np.random.default_rng(2)
    ps, dim = 8, 16
    spans = np.array([[0, 3, 5, 0, 2, 2], [3, 1, 0, 2, 1, 0]], np.int32)
    table = np.array([4, 1, 3], np.int32)
    pool = rng.integers(0, 255, 5 * oracle.index_page_bytes("fp8", ps, dim), dtype=np.uint8)
    keys = rng.integers(0, 0x70, (4, dim), dtype=np.uint8)
    scales = np.array([1.5, 2.5, 3.5, 4.5], np.float32)
    new = oracle.store_keys(pool, "fp8", spans, table, ps, dim, keys, scales)
    pb = oracle.index_page_bytes("fp8", ps, dim)
    # row 0 -> request 0 position 5 -> slot 7 -> page table[0] = 4, offset 7, and so on
    where = [(4, 7), (1, 0), (1, 1), (3, 0)]
    expect = pool.reshape(-1, pb).copy()
    for t, (page, off) in enumerate(where):
        expect[page, off * dim:(off + 1) * dim] = keys[t]
        expect[page, ps * dim + 4 * off: ps * dim + 4 * off + 4] = scales[t:t + 1].view(np.uint8)
    assert np.array_equal(new.reshape(-1, pb), expect)


# ---------------------------------------------------------------- indexer score

def test_score_small_example_by_hand():
    # Two heads, three dims; every value below is worked out from sum_h w[h]*relu(q[h].k).
    q = np.array([[1.0, 2.0, 0.0], [0.0, -1.0, 1.0]])
    w = np.array([0.5, 2.0])
    k = np.array([[1.0, 1.0, 1.0],     # h0: 3 -> 1.5 ; h1: 0 -> 0   => 1.5
                  [2.0, 0.0, -1.0],    # h0: 2 -> 1.0 ; h1: -1 -> 0  => 1.0
                  [-1.0, -1.0, -1.0],  # h0: -3 -> 0  ; h1: 0 -> 0   => 0.0
                  [0.0, -3.0, 2.0],    # h0: -6 -> 0  ; h1: 5 -> 10  => 10.0
                  [2.0, 0.0, -1.0]])   # same key as row 1                => 1.0
    s = oracle.index_scores_row(q, w, k)
    assert s.dtype == np.float32
    assert s.tolist() == [1.5, 1.0, 0.0, 10.0, 1.0]
    # ordering: 10 (j3), 1.5 (j0), 1.0 tie j1 < j4, 0 (j2)
    assert oracle.select_topk_causal_row(s, 4, 6).tolist() == [3, 0, 1, 4, 2, -1]
    assert oracle.select_topk_causal_row(s, 4, 3).tolist() == [3, 0, 1]
    # a row at position 2 sees keys 0..2 only
    assert oracle.select_topk_causal_row(s, 2, 4).tolist() == [0, 1, 2, -1]


def test_score_one_hot_queries_closed_form():
    # q[h] = a_h * e_{d_h}: q[h].k = a_h * k[d_h], so s = sum_h w_h * max(0, a_h * k[d_h]).
    rng = np.random.default_rng(3)
    H, D, n = 5, 16, 40
    d = np.array([0, 3, 3, 15, 7])
    a = np.array([1.0, -2.0, 0.5, 3.0, 1.0])
    q = np.zeros((H, D))
    q[np.arange(H), d] = a
    w = rng.uniform(0, 1, H)
    k = rng.standard_normal((n, D))
    s = oracle.index_scores_row(q, w, k)
    for j in range(n):
        ref = math.fsum(w[h] * max(0.0, a[h] * k[j, d[h]]) for h in range(H))
        assert s[j] == np.float32(ref)


def test_score_single_head_reduces_to_matvec():
    rng = np.random.default_rng(4)
    D, n = 64, 200
    q = rng.uniform(0, 1, (1, D))
    k = rng.uniform(0, 1, (n, D))
    s = oracle.index_scores_row(q, np.ones(1), k)
    ref = np.array([math.fsum(q[0] * k[j]) for j in range(n)])
    assert np.array_equal(s, ref.astype(np.float32))


def test_fp8_index_key_closed_form():
    # 132-byte record: 128 e4m3 codes then the fp32 scale; the key is e4m3(code) * scale.
    ps, dim = 4, 128
    codes = np.zeros((1, dim), np.uint8)
    codes[0, 2] = 0x7E          # 448
    codes[0, 5] = 0xC6          # -3.5
    pool = _place_keys(codes, "fp8", ps, dim, np.array([0], np.int32), 0, 1, np.array([0.5], np.float32))
    span = np.array([0, 1, 0, 0, 1, 0])
    k = oracle.read_index_keys(pool, "fp8", span, np.array([0], np.int32), ps, dim, 1)
    q = np.zeros((2, dim))
    q[0, 2] = 1.0
    q[1, 5] = 1.0
    s = oracle.index_scores_row(q, np.array([0.25, 1.0]), k)
    assert s[0] == np.float32(0.25 * 224.0)      # head 1 sees -1.75 -> relu 0


# ---------------------------------------------------------------- causal top-k select

def test_select_matches_brute_force_with_forced_ties():
    rng = np.random.default_rng(5)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        s = rng.integers(0, 4, n).astype(np.float32)          # many exact ties
        if trial % 3 == 0:
            s[rng.random(n) < 0.3] = -0.0                    # -0 ties +0
        pos = int(rng.integers(0, n))
        k = int(rng.integers(1, 50))
        ref = sorted(range(pos + 1), key=lambda j: (-float(s[j]), j))[:k]
        ref = ref + [-1] * (k - len(ref))
        assert oracle.select_topk_causal_row(s, pos, k).tolist() == ref


def test_select_all_equal_scores_takes_lowest_positions():
    s = np.zeros(100, np.float32)
    assert oracle.select_topk_causal_row(s, 99, 10).tolist() == list(range(10))


def test_select_pad_count_closed_form_prefill_from_zero():
    # Rows at positions 0..N-1 with topk k: row p keeps min(k, p+1) keys and k - that pads.
    # 8192 rows from 0 with k = 2048 give sum_{p<2047} (2047 - p) = 2047*2048/2 = 2,096,128;
    # rows at p >= 2047 pad nothing, so the rows below 2100 decide the count.
    rng = np.random.default_rng(6)
    k = 2048
    pads = 0
    for p in range(2100):
        pads += int(np.sum(oracle.select_topk_causal_row(rng.standard_normal(p + 1).astype(np.float32), p, k) == -1))
    assert pads == 2047 * 2048 // 2 == 2_096_128


def test_tiny_prefill_pad_count_and_ties():
    wl = make_workload("tiny_prefill")
    sel = helpers.oracle_index_topk(wl)
    arr = np.stack([sel[t] for t in range(wl.n_rows)])
    # 64 rows at 0..63, topk 16: rows 0..14 pad 15 - p entries -> 120
    assert int(np.sum(arr == -1)) == 120
    for t in range(wl.n_rows):
        n = min(16, t + 1)
        assert np.all(arr[t, :n] >= 0) and np.all(arr[t, n:] == -1)


def test_zero_queries_give_position_order():
    wl = make_workload("tiny_prefill")
    q = np.zeros_like(helpers.to_f64(wl.index_q))
    sel = oracle.index_topk(q, helpers.to_f64(wl.index_w), helpers.oracle_key_pool(wl), "f32",
                            wl.spans, wl.page_table, wl.spec.page_size, 16)
    for t in range(wl.n_rows):
        n = min(16, t + 1)
        assert sel[t][:n].tolist() == list(range(n))


# ---------------------------------------------------------------- absorbed sparse MLA

def _tiny_attend_inputs(topk):
    wl = make_workload("tiny_prefill")
    s = wl.spec
    pool = helpers.oracle_key_pool(wl)
    sel = oracle.index_topk(helpers.to_f64(wl.index_q), helpers.to_f64(wl.index_w), pool, "f32",
                            wl.spans, wl.page_table, s.page_size, topk)
    return wl, sel


def test_topk_at_least_context_equals_dense_causal_mla():
    wl, sel = _tiny_attend_inputs(64)
    s = wl.spec
    sparse = helpers.oracle_attend(wl, sel)
    dense = oracle.dense_causal_mla(helpers.to_f64(wl.q_nope[0]), helpers.to_f64(wl.q_pe[0]),
                                    wl.latent_pools[0].numpy(), s.latent_fmt, wl.spans, wl.page_table,
                                    s.page_size, s.sm_scale, rows=range(wl.n_rows))
    for t in range(wl.n_rows):
        np.testing.assert_allclose(sparse[t], dense[t], rtol=0, atol=1e-12)


def test_sparse_attend_matches_sdpa_on_gathered_rows():
    wl, sel = _tiny_attend_inputs(16)
    s = wl.spec
    out = helpers.oracle_attend(wl, sel)
    qn, qp = helpers.to_f64(wl.q_nope[0]), helpers.to_f64(wl.q_pe[0])
    R, P = s.kv_lora_rank, s.rope_dim
    for t in range(wl.n_rows):
        j = sel[t][sel[t] >= 0]
        c = oracle.read_latents(wl.latent_pools[0].numpy(), "f32", wl.spans[0], wl.page_table,
                                s.page_size, R, P, j)
        q = torch.from_numpy(np.concatenate([qn[t], qp[t]], 1))[:, None]      # (H, 1, R+P)
        k = torch.from_numpy(c)[None].expand(q.shape[0], -1, -1)
        v = torch.from_numpy(c[:, :R])[None].expand(q.shape[0], -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=s.sm_scale)[:, 0]
        np.testing.assert_allclose(out[t], ref.numpy(), rtol=0, atol=1e-12)


def test_attend_special_cases():
    wl, sel1 = _tiny_attend_inputs(1)
    s = wl.spec
    R, P = s.kv_lora_rank, s.rope_dim
    lat = oracle.read_latents(wl.latent_pools[0].numpy(), "f32", wl.spans[0], wl.page_table,
                              s.page_size, R, P, np.arange(64))
    out = helpers.oracle_attend(wl, sel1)
    for t in range(wl.n_rows):   # topk = 1: the output is the picked latent's first R columns
        assert np.array_equal(out[t], np.broadcast_to(lat[sel1[t][0], :R], out[t].shape))
    # row 0 sees only itself
    _, sel = _tiny_attend_inputs(16)
    out = helpers.oracle_attend(wl, sel)
    np.testing.assert_allclose(out[0], np.broadcast_to(lat[0, :R], out[0].shape), atol=0)
    # q = 0: uniform weights, the mean of the picked latents
    zero = np.zeros_like(helpers.to_f64(wl.q_nope[0]))
    zp = np.zeros_like(helpers.to_f64(wl.q_pe[0]))
    out0 = oracle.sparse_mla_attend(sel, zero, zp, wl.latent_pools[0].numpy(), "f32", wl.spans,
                                    wl.page_table, s.page_size, s.sm_scale)
    for t in range(wl.n_rows):
        j = sel[t][sel[t] >= 0]
        np.testing.assert_allclose(out0[t], np.broadcast_to(lat[j, :R].mean(0), out0[t].shape), atol=1e-14)


def test_empty_selection_gives_zeros():
    wl = make_workload("tiny_prefill")
    s = wl.spec
    sel = {0: np.full(16, -1, np.int32)}
    out = helpers.oracle_attend(wl, sel)
    assert np.all(out[0] == 0) and out[0].shape == (s.n_heads, s.kv_lora_rank)


def test_selection_does_not_depend_on_batch_packing():
    # The same request alone and packed behind another request picks the same positions.
    wl = make_workload("decode_small")
    sel = helpers.oracle_index_topk(wl, rows=[3])
    s = wl.spec
    one = wl.spans[3:4].copy()
    one[0, 0] = 0
    alone = oracle.index_topk(helpers.to_f64(wl.index_q[3:4]), helpers.to_f64(wl.index_w[3:4]),
                              helpers.oracle_key_pool(wl), s.index_key_fmt, one, wl.page_table,
                              s.page_size, s.topk)
    assert np.array_equal(alone[0], sel[3])


# ---------------------------------------------------------------- attention sink

def _tiny_sink(wl, seed=7):
    """Per-head sinks of the tiny workload: scaled values spread over the logits' range, one head
    without a sink, one whose sink dominates."""
    s = wl.spec
    rng = np.random.default_rng(seed)
    scaled = rng.uniform(-2.0, 4.0, size=s.n_heads)
    scaled[1] = 60.0
    sink = scaled / s.sm_scale
    sink[0] = -np.inf
    return sink


def _logits(wl, t, j):
    s = wl.spec
    R, P = s.kv_lora_rank, s.rope_dim
    c = oracle.read_latents(wl.latent_pools[0].numpy(), s.latent_fmt, wl.spans[0], wl.page_table,
                            s.page_size, R, P, j)
    qn, qp = helpers.to_f64(wl.q_nope[0])[t], helpers.to_f64(wl.q_pe[0])[t]
    return s.sm_scale * (qn @ c[:, :R].T + qp @ c[:, R:].T), c


def test_sink_is_a_key_with_zero_value_in_sdpa():
    # The sink behaves as one more key whose logit is sm_scale * sink and whose value is zero.
    # Built per head as a key k* with q_h . k* = sink_h and run through torch's attention.
    wl, sel = _tiny_attend_inputs(16)
    s = wl.spec
    R = s.kv_lora_rank
    sink = _tiny_sink(wl)
    out = oracle.sparse_mla_attend(sel, helpers.to_f64(wl.q_nope[0]), helpers.to_f64(wl.q_pe[0]),
                                   wl.latent_pools[0].numpy(), s.latent_fmt, wl.spans, wl.page_table,
                                   s.page_size, s.sm_scale, sink=sink)
    qn, qp = helpers.to_f64(wl.q_nope[0]), helpers.to_f64(wl.q_pe[0])
    for t in range(wl.n_rows):
        j = sel[t][sel[t] >= 0]
        _, c = _logits(wl, t, j)
        q = np.concatenate([qn[t], qp[t]], 1)                                   # (H, R+P)
        k = np.broadcast_to(c, (q.shape[0],) + c.shape).copy()                  # (H, n, R+P)
        v = np.broadcast_to(c[:, :R], (q.shape[0], c.shape[0], R)).copy()
        finite = np.isfinite(sink)
        kstar = q * (np.where(finite, sink, 0.0) / np.sum(q * q, 1))[:, None]   # q_h . k* = sink_h
        k = np.concatenate([k, kstar[:, None]], 1)
        v = np.concatenate([v, np.zeros((q.shape[0], 1, R))], 1)
        mask = np.ones((q.shape[0], 1, k.shape[1]), bool)
        mask[~finite, 0, -1] = False                                            # head without a sink
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, None], torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=torch.from_numpy(mask), scale=s.sm_scale)[:, 0].numpy()
        np.testing.assert_allclose(out[t], ref, rtol=0, atol=1e-12)


def test_sink_closed_forms():
    from scipy.special import expit, logsumexp
    wl, sel = _tiny_attend_inputs(16)
    s = wl.spec
    sink = _tiny_sink(wl)
    args = (helpers.to_f64(wl.q_nope[0]), helpers.to_f64(wl.q_pe[0]), wl.latent_pools[0].numpy(),
            s.latent_fmt, wl.spans, wl.page_table, s.page_size, s.sm_scale)
    plain = oracle.sparse_mla_attend(sel, *args)
    with_sink = oracle.sparse_mla_attend(sel, *args, sink=sink)
    none = oracle.sparse_mla_attend(sel, *args, sink=np.full(s.n_heads, -np.inf))
    for t in range(wl.n_rows):
        # every head's output shrinks by Z / (Z + e^{scaled sink}), Z = sum_j e^{logit_j}
        j = sel[t][sel[t] >= 0]
        lg, _ = _logits(wl, t, j)
        ratio = expit(logsumexp(lg, axis=1) - s.sm_scale * sink)        # sink -inf: ratio 1
        np.testing.assert_allclose(with_sink[t], plain[t] * ratio[:, None], rtol=1e-12, atol=1e-14)
        assert np.array_equal(none[t], plain[t])                         # -inf everywhere: no sink
        assert np.all(np.abs(with_sink[t][1]) < 1e-20)                   # a dominant sink
    # one pick: out = c_j * sigmoid(logit_j - scaled sink)
    _, sel1 = _tiny_attend_inputs(1)
    one = oracle.sparse_mla_attend(sel1, *args, sink=sink)
    for t in range(wl.n_rows):
        lg, c = _logits(wl, t, sel1[t][:1])
        w = expit(lg[:, 0] - s.sm_scale * sink)
        np.testing.assert_allclose(one[t], w[:, None] * c[0, : s.kv_lora_rank][None], rtol=1e-12,
                                   atol=1e-14)
    # nothing picked: zeros, whatever the sink
    empty = oracle.sparse_mla_attend({0: np.full(16, -1, np.int32)}, *args, sink=sink)
    assert np.all(empty[0] == 0)
