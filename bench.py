"""Benchmark of the DSA select + attend hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_decode]

A step is one pass of the whole path over one batch: store this step's index keys, index_topk
(scores + causal top-k), then attend for every attend layer of the workload. Inputs are resident
in HBM before the timed region; the step rotates over several copies of the pools so that no pool
is still in the 256 MB Infinity Cache from the previous step. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6    # MI355X dense bf16 matrix peak (256 CUs x 2.4 GHz x 4096 flop/clk)
# the sources of each measured kernel: a counter file is stale once any of them changed
KERNEL_SOURCES = {
    "score": ("k_index_mfma.hip", "k_index_rows.hip", "k_index_generic.hip", "dsa_internal.hpp"),
    "select": ("k_select.hip", "k_index_mfma.hip", "dsa_internal.hpp"),
    "attend": ("k_attend_split.hip", "k_attend_mfma.hip", "dsa_internal.hpp"),
}
# kernel-name patterns (as rocprofv3 stores the demangled names) of each measured part: a part's
# kernels, one launch each per step (template arguments: key format 1 bf16 / 2 fp8, 32-bit
# offsets, mode 0 plain / 1 block maxima / 2 block lists)
COUNTER_KERNELS = {
    "score": ("index_scores_mfma<2, true, 0>",),       # dsa_index_scores: the kernel timed alone
    "score_step": ("index_scores_mfma<2, true, 2>",),  # the same kernel inside dsa_index_topk
    "select": ("select_lists",),
    "attend": ("attend_f8_split", "attend_combine"),
}
MSA_COUNTER_KERNELS = {
    "score": ("index_scores_mfma<1, true, 0>",),       # dsa_index_scores: the kernel timed alone
    "score_step": ("index_scores_mfma<1, true, 1>",),  # inside dsa_msa_select_blocks
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_decode")
    ap.add_argument("--copies", type=int, default=4, help="pool copies rotated over the steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the decode_batch, causal_prefill and chunked_mix steps reported "
                         "beside the long_decode line")
    ap.add_argument("--prefill-steps", type=int, default=10,
                    help="timed steps of causal_prefill (decode_batch: at least 50, chunked_mix: half)")
    ap.add_argument("--no-graph", action="store_true", help="skip the captured-graph timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="about this much CPU work for the oracle baseline")
    ap.add_argument("--profile-only", action="store_true",
                    help="a short run for rocprofv3 counters: a few steps, a known-size copy, no JSON")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write the score kernel's measured HBM traffic from two --profile-only "
                         "counter runs into profiles/, then exit")
    return ap.parse_args()


def algorithmic(wl):
    """What the method itself must move and compute per step (bytes, flops), per part."""
    s = wl.spec
    T = wl.n_rows
    pos = wl.positions
    key_b = s.index_dim + 4 if s.index_key_fmt == "fp8" else s.index_dim * (2 if s.index_key_fmt == "bf16" else 4)
    qb = 2 if s.index_q_fmt == "bf16" else 4
    # index keys: each request's keys are read once per step (all its rows share them)
    req_keys = sum(int(sp[2]) + int(sp[1]) for sp in wl.spans)
    idx_bytes = req_keys * key_b + T * (s.n_index_heads * s.index_dim * qb + s.n_index_heads * 4)
    pairs = int(sum(int(p) + 1 for p in pos))
    idx_flops = pairs * (2 * s.n_index_heads * s.index_dim + 3 * s.n_index_heads)
    sel_bytes = T * s.topk * 4
    picked = int(sum(min(s.topk, int(p) + 1) for p in pos))
    row_b = (s.kv_lora_rank + 4 * (s.kv_lora_rank // 128) + 2 * s.rope_dim if s.latent_fmt == "fp8"
             else (s.kv_lora_rank + s.rope_dim) * (2 if s.latent_fmt == "bf16" else 4))
    q_b = 2 if s.q_fmt == "bf16" else 4
    att_bytes_layer = (picked * row_b + T * s.n_heads * (s.kv_lora_rank + s.rope_dim) * q_b
                       + T * s.n_heads * s.kv_lora_rank * q_b + sel_bytes)
    att_flops_layer = picked * s.n_heads * (2 * (s.kv_lora_rank + s.rope_dim) + 2 * s.kv_lora_rank)
    L = len(wl.q_nope)
    return dict(index_bytes=idx_bytes, index_flops=idx_flops, select_bytes=sel_bytes,
                attend_bytes=att_bytes_layer * L, attend_flops=att_flops_layer * L,
                total_bytes=idx_bytes + sel_bytes + att_bytes_layer * L,
                total_flops=idx_flops + att_flops_layer * L, rows=T, pairs=pairs, picked=picked)


def kernel_source_hash(part: str = "score") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES["score" if part == "score_step" else part]:
        p = os.path.join(ROOT, "sparse_attention_dsa_amd", "csrc", name)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, part: str = "score"):
    """HBM bytes (read + written) per step of one measured part from committed rocprofv3 counter
    runs, or None when there are none for this workload or the part's sources changed since."""
    p = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p)).get("parts", {}).get(part)
    if not d or d.get("source_hash") != kernel_source_hash(part):
        return None
    return d.get("traffic_bytes_per_step")


def copy_rate() -> float:
    """A plain 1 GiB device-to-device copy, read + write bytes per second (GB/s): the streaming
    rate this chip reaches outside the library, reported beside the 8 TB/s peak."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a, b
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(wl, target_s: float):
    """The oracle as it stands, on the host cores: whole passes over a bounded row sample (every
    row of a decode batch, an even spread of a prefill's rows) until about target_s seconds of
    CPU work are done. Each pass stores the step's keys, then runs index_topk and every attend
    layer for the sampled rows."""
    import threadpoolctl

    from tests import helpers
    T = wl.n_rows
    rows = list(range(T)) if T <= 32 else sorted(set(range(0, T, max(1, T // 8))) | {T - 1})
    passes = 0
    t0 = time.perf_counter()
    while True:
        pool = helpers.oracle_key_pool(wl)
        sel = helpers.oracle_index_topk(wl, rows=rows, pool=pool)
        for layer in range(len(wl.q_nope)):
            helpers.oracle_attend(wl, sel, layer)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    threads = max([i["num_threads"] for i in threadpoolctl.threadpool_info()] + [1])
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    done = passes * len(rows)
    which = "all" if len(rows) == T else f"an even spread of {len(rows)}"
    return dict(value=done / dt, unit="rows/s", cores=threads, kind="oracle",
                sample=f"{passes} passes over {which} of the {T} rows of {wl.spec.name} "
                       f"(store_keys for the step, then index_topk and every attend layer for "
                       f"those rows), float64 numpy, {threads} BLAS threads of {os.cpu_count()} "
                       f"host cores ({cpu}); {dt:.1f} s",
                seconds=dt)


def summarize_counters(workload: str, fetch_db: str, write_db: str):
    """HBM traffic of each measured part (COUNTER_KERNELS) from two rocprofv3 counter runs of
    --profile-only (one with FETCH_SIZE, one with WRITE_SIZE). Each counter is scaled by what it
    reads for the run's plain device copy of 1 GiB; a part's launches within one step are added,
    and the median over the run's steps is kept. The result goes to profiles/ with a hash of each
    part's sources, so that a later change to them makes that part's figures stale."""
    import sqlite3
    import statistics

    def rows(db, counter):
        con = sqlite3.connect(db)
        r = con.execute("select kernel_name, value from counters_collection where counter_name=? "
                        "order by dispatch_id", (counter,)).fetchall()
        con.close()
        return r

    out = {"workload": workload, "copy_bytes": 1 << 30, "parts": {}}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        r = rows(db, counter)
        # the calibration copy is the run's last copy dispatch (earlier ones clone the pools)
        copy_kib = [v for n, v in r if "copy" in n.lower()][-1]
        scale = (1 << 30) / (copy_kib * 1024.0)
        out[counter + "_copy_kib"] = copy_kib
        parts = MSA_COUNTER_KERNELS if workload.startswith("msa_") else COUNTER_KERNELS
        for part, pats in parts.items():
            # launches in order; a step holds one launch of each of the part's kernels
            seq = [v for n, v in r if any(pt in n for pt in pats)]
            k = len(pats)
            per_step = [sum(seq[i:i + k]) for i in range(0, len(seq) - k + 1, k)]
            if not per_step:
                continue
            med = statistics.median(per_step)
            d = out["parts"].setdefault(part, {"kernels": list(pats),
                                               "source_hash": kernel_source_hash(part)})
            d[counter] = {"kib_per_step_median": med, "steps": len(per_step), "scale": scale,
                          "bytes_per_step": med * 1024.0 * scale}
    for d in out["parts"].values():
        if "FETCH_SIZE" in d and "WRITE_SIZE" in d:
            d["traffic_bytes_per_step"] = (d["FETCH_SIZE"]["bytes_per_step"]
                                           + d["WRITE_SIZE"]["bytes_per_step"])
    p = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.json")
    with open(p, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def msa_algorithmic(wl):
    """Bytes and flops a block-sparse MSA step must move and compute: the index keys of every
    request once, the index queries and weights, and the K/V rows of every picked token."""
    s = wl.spec
    T = wl.n_rows
    pos = wl.positions
    req_keys = sum(int(sp[2]) + int(sp[1]) for sp in wl.spans)
    score_bytes = req_keys * s.index_dim * 2 + T * s.n_index_heads * (s.index_dim * 2 + 4)
    score_flops = int(sum(int(p) + 1 for p in pos)) * (2 * s.n_index_heads * s.index_dim
                                                       + 3 * s.n_index_heads)
    # The attention's K/V bytes depend on which blocks win (a row's own block may be partial):
    # they are counted from the picked block ids by msa_picked_tokens.
    row_bytes = 2 * s.n_kv_heads * s.head_dim * 2
    qo_bytes = T * s.n_heads * s.head_dim * 2 * 2
    return dict(score_bytes=score_bytes, score_flops=score_flops, row_bytes=row_bytes,
                qo_bytes=qo_bytes, sel_bytes=T * s.topk_blocks * 4)


def msa_picked_tokens(sel, positions, block: int) -> int:
    """Visible tokens of the picked blocks over a step (the attention's K/V rows)."""
    n = 0
    for t, p in enumerate(positions):
        for b in sel[t]:
            if b >= 0:
                n += min((int(b) + 1) * block, int(p) + 1) - int(b) * block
    return n


def msa_cpu_baseline(wl, target_s: float):
    """The block-sparse MSA oracle on the host cores: whole passes (block selection, then GQA
    over the picked blocks) over every row of the step until about target_s seconds are done."""
    import threadpoolctl

    from oracle import msa_oracle
    from tests import helpers
    s = wl.spec
    T = wl.n_rows
    rows = list(range(T)) if T <= 32 else sorted(set(range(0, T, max(1, T // 8))) | {T - 1})
    q_idx, w, q = helpers.to_f64(wl.index_q), helpers.to_f64(wl.index_w), helpers.to_f64(wl.q)
    kp, gp = wl.key_pool.numpy(), wl.gqa_pool.numpy()
    passes = 0
    t0 = time.perf_counter()
    while True:
        sel = msa_oracle.msa_select(q_idx, w, kp, "bf16", wl.spans, wl.page_table, s.page_size,
                                    s.topk_blocks, s.block, rows=rows)
        msa_oracle.msa_attend(sel, q, gp, wl.spans, wl.page_table, s.page_size, s.n_kv_heads,
                              s.head_dim, s.block, s.sm_scale)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    threads = max([i["num_threads"] for i in threadpoolctl.threadpool_info()] + [1])
    which = "all" if len(rows) == T else f"an even spread of {len(rows)}"
    return dict(value=round(passes * len(rows) / dt, 4), unit="rows/s", cores=threads,
                kind="oracle",
                sample=f"{passes} passes over {which} of the {T} rows of {s.name} (block "
                       f"selection, then GQA over the picked blocks), float64 numpy, {threads} "
                       f"BLAS threads of {os.cpu_count()} host cores; {dt:.1f} s")


def main_msa(args):
    """Block-sparse MSA step: dsa_msa_select_blocks (token scores, block maxima, top blocks),
    then dsa_msa_attend (GQA over the picked blocks). Same timing discipline as the DSA step."""
    import torch

    from synth import make_msa_workload
    from sparse_attention_dsa_amd import dsa
    from sparse_attention_dsa_amd.step import MSAStep

    torch.cuda.set_device(0)
    dsa.load()
    t_gen = time.perf_counter()
    wl = make_msa_workload(args.workload)
    t_gen = time.perf_counter() - t_gen
    s = wl.spec
    st = MSAStep(wl)
    copies = max(1, args.copies)
    key_pools = [st.key_pool] + [st.key_pool.clone() for _ in range(copies - 1)]
    gqa_pools = [st.gqa_pool] + [st.gqa_pool.clone() for _ in range(copies - 1)]
    stream = torch.cuda.current_stream()

    def run(i, strm=stream):
        c = i % copies
        st.select(key_pool=key_pools[c], stream=strm)
        st.attend(gqa_pool=gqa_pools[c], stream=strm)

    alg = msa_algorithmic(wl)
    if args.profile_only:
        for i in range(5):
            run(i)
        torch.cuda.synchronize()
        # the score kernel alone, as the bench times it (dsa_index_scores on an index handle)
        dcfg = dsa.make_config(s.n_index_heads, s.index_dim, "bf16", "bf16", 2048, 128, 512, 64,
                               "bf16", "bf16", s.page_size)
        dh = dsa.dsa_create(dcfg)
        ld = (int(wl.positions.max()) + 1 + 3) // 4 * 4
        scores = torch.empty(st.plan.n_rows, ld, dtype=torch.float32, device="cuda")
        for i in range(5):
            dsa.dsa_index_scores(dh, st.plan, st.index_q, st.index_w, key_pools[i % copies], scores,
                                 ld, stream)
        torch.cuda.synchronize()
        del scores
        nbytes = 1 << 30                     # a plain copy of known size for scaling the counters
        a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(f"profile run done: copy of {nbytes} bytes; score bytes per launch {alg['score_bytes']}")
        return

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms = timed(lambda i: run(args.warmup + i), args.steps)
    wall = time.perf_counter() - wall0

    n_d = min(args.steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_d + 1)]
    evs[0].record(stream)
    for i in range(n_d):
        run(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n_d))
    pct = lambda q: per_step[min(n_d - 1, int(q * n_d))]  # noqa: E731

    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for c in range(copies):
                    run(c, strm=cap)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        n_g = max(1, args.steps // copies)
        cs = torch.cuda.current_stream()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(cs)
        for _ in range(n_g):
            g.replay()
        g1.record(cs)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (n_g * copies)

    # The score kernel alone, at the same launch shape: the MSA select's first launch is the DSA
    # indexer's score kernel, reached here through dsa_index_scores on a handle with the same index
    # configuration (the attention fields of that handle play no part in scoring).
    dcfg = dsa.make_config(s.n_index_heads, s.index_dim, "bf16", "bf16", 2048, 128, 512, 64,
                           "bf16", "bf16", s.page_size)
    dh = dsa.dsa_create(dcfg)
    ld = (int(wl.positions.max()) + 1 + 3) // 4 * 4
    scores = torch.empty(st.plan.n_rows, ld, dtype=torch.float32, device="cuda")
    score = lambda i: dsa.dsa_index_scores(dh, st.plan, st.index_q, st.index_w,  # noqa: E731
                                           key_pools[i % copies], scores, ld, stream)
    for i in range(5):
        score(i)
    torch.cuda.synchronize()
    k_ms = timed(score, max(20, args.steps // 2))
    achieved = alg["score_bytes"] / (k_ms * 1e-3) / 1e9

    # Select (score + block top-k) and attend, each alone.
    sel_ms = timed(lambda i: st.select(key_pool=key_pools[i % copies], stream=stream),
                   max(20, args.steps // 2))
    att_ms = timed(lambda i: st.attend(gqa_pool=gqa_pools[i % copies], stream=stream),
                   max(20, args.steps // 2))
    picked = msa_picked_tokens(st.sel.cpu().numpy(), wl.positions, s.block)
    att_bytes = picked * alg["row_bytes"] + alg["qo_bytes"] + alg["sel_bytes"]
    att_gbs = att_bytes / (att_ms * 1e-3) / 1e9

    rows = wl.n_rows
    out = {
        "metric": f"MSA decode tokens/s (block select + GQA attend) at {int(wl.positions.max()) + 1} "
                  f"ctx, top {s.topk_blocks} blocks of {s.block}; % HBM peak",
        "value": round(rows / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "step_ms_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5), round(pct(0.9), 5)],
        "select_ms": round(sel_ms, 5),
        "attend_ms": round(att_ms, 5),
        "graph": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 5), "value": round(rows / (graph_ms * 1e-3), 1),
            "note": "the same select + attend steps replayed from one captured HIP graph"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "formats": "bf16 index keys and queries, bf16 GQA cache, queries and output; fp32 "
                   "accumulation",
        "data": "synthetic (seeded; N(0,1) draws in bf16)",
        "config": {
            "workload": f"{s.name}: {rows} decode rows, positions up to {int(wl.positions.max())}, "
                        f"{s.n_index_heads}x{s.index_dim} bf16 index keys, top {s.topk_blocks} "
                        f"blocks of {s.block} tokens, {s.n_heads}-head GQA over {s.n_kv_heads} KV "
                        f"heads of {s.head_dim}, {s.page_size}-token pages",
            "rows_per_step": rows, "pool_copies_rotated": copies,
        },
        "step_bytes_algorithmic": alg["score_bytes"] + att_bytes,
        "step_hbm_frac": round((alg["score_bytes"] + att_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": "index score (first launch of dsa_msa_select_blocks)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(s.name, "score"),
            "kernel_ms": round(k_ms, 5), "algorithmic_bytes_per_launch": alg["score_bytes"],
        },
        "hbm_copy_measured_gbs": copy_rate(),
        "other_kernel": {
            "kernel": "GQA attend over the picked blocks (dsa_msa_attend)",
            "bound": "hbm", "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(att_gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel_ms": round(att_ms, 5), "algorithmic_bytes_per_launch": att_bytes,
            "picked_tokens": picked,
        },
        "wall_s_timed": round(wall, 3),
        "gen_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = msa_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def workload_line(name: str, steps: int, warmup: int = 2):
    """One more workload's step timed beside the headline line: index_topk + every attend layer
    over two rotated pool copies, `steps` timed steps after `warmup`, then the attention (layer 0)
    and the score kernel alone. A decode workload (one row per request) reports the score kernel
    against HBM and the step's HBM fraction; a workload with prefill rows reports the attention and
    the score kernel against the bf16 matrix peak."""
    import torch

    from synth import make_workload
    from sparse_attention_dsa_amd import dsa
    from sparse_attention_dsa_amd.step import DSAStep

    t_gen = time.perf_counter()
    wl = make_workload(name)
    t_gen = time.perf_counter() - t_gen
    step = DSAStep.from_workload(wl, check_pages=True)
    dsa.dsa_plan_check(step.h, step.plan)
    step.plan = dsa.Plan(wl.spans, wl.page_table, wl.pool_pages, step.plan.spans_dev,
                         step.plan.page_table_dev, check_pages=False)
    n_layers = len(step.q_nope)
    copies = 2
    key_pools = [step.key_pool] + [step.key_pool.clone() for _ in range(copies - 1)]
    lat_pools = [[p] + [p.clone() for _ in range(copies - 1)] for p in step.latent_pools]
    st = torch.cuda.current_stream()
    for c in range(copies):
        step.store_keys(key_pool=key_pools[c], stream=st)
    alg = algorithmic(wl)

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(n):
            fn(i)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def run(i):
        c = i % copies
        step.index_topk(key_pool=key_pools[c], stream=st)
        for layer in range(n_layers):
            step.attend(layer, latent_pool=lat_pools[layer][c], stream=st)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ms = timed(run, steps)
    a_ms = timed(lambda i: step.attend(0, latent_pool=lat_pools[0][i % copies], stream=st), steps)
    ld = int((wl.positions.max() + 1 + 3) // 4 * 4)
    scores = torch.empty(step.plan.n_rows, ld, dtype=torch.float32, device="cuda")
    sc = lambda i: dsa.dsa_index_scores(step.h, step.plan, step.index_q, step.index_w,  # noqa: E731
                                        key_pools[i % copies], scores, ld, st)
    sc(0)
    torch.cuda.synchronize()
    s_ms = timed(sc, steps)
    a_flops = alg["attend_flops"] / n_layers
    a_tf = a_flops / (a_ms * 1e-3) / 1e12
    s_tf = alg["index_flops"] / (s_ms * 1e-3) / 1e12
    s_gbs = alg["index_bytes"] / (s_ms * 1e-3) / 1e9
    spec = wl.spec
    prefill = int(max(wl.spans[:, 1])) > 1
    line = {
        "workload": f"{spec.name}: {wl.n_rows} rows in {len(wl.spans)} requests (longest "
                    f"{int(max(wl.spans[:, 1]))} rows), positions up to {int(wl.positions.max())}, "
                    f"{spec.n_index_heads}x{spec.index_dim} {spec.index_key_fmt} index keys, topk "
                    f"{spec.topk}, {n_layers} attend layer(s) of {spec.n_heads}-head absorbed MLA over "
                    f"{spec.kv_lora_rank}+{spec.rope_dim} {spec.latent_fmt} latents",
        "steps": steps, "warmup": warmup, "pool_copies_rotated": copies,
        "ms_per_step": round(ms, 5), "tokens_per_s": round(wl.n_rows / (ms * 1e-3), 1),
        "step_hbm_frac": round(alg["total_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "attend": {"kernel": "sparse MLA attend, one layer (dsa_sparse_mla_attend)",
                   "ms": round(a_ms, 5), "achieved": round(a_tf, 1), "peak": MFMA_BF16_PEAK_TFS,
                   "unit": "TFLOP/s", "frac": round(a_tf / MFMA_BF16_PEAK_TFS, 4),
                   "algorithmic_flops_per_launch": a_flops},
        "gen_s": round(t_gen, 1),
    }
    if prefill:
        line["score"] = {"kernel": "index score (dsa_index_scores)", "ms": round(s_ms, 5),
                         "achieved": round(s_tf, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(s_tf / MFMA_BF16_PEAK_TFS, 4),
                         "algorithmic_flops_per_launch": alg["index_flops"]}
    else:
        line["score"] = {"kernel": "index score (dsa_index_scores)", "ms": round(s_ms, 5),
                         "achieved": round(s_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(s_gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": alg["index_bytes"]}
    del key_pools, lat_pools, scores, step
    torch.cuda.empty_cache()
    return line


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.workload, *args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build "
              f"(the multi-GPU sharding is a design note, not code).", file=sys.stderr)
        sys.exit(2)
    if args.workload.startswith("msa_"):
        main_msa(args)
        return

    import numpy as np
    import torch

    from synth import make_workload
    from sparse_attention_dsa_amd import dsa
    from sparse_attention_dsa_amd.step import DSAStep

    torch.cuda.set_device(0)
    dsa.load()
    t_gen = time.perf_counter()
    wl = make_workload(args.workload)
    t_gen = time.perf_counter() - t_gen
    step = DSAStep.from_workload(wl, check_pages=True)
    dsa.dsa_plan_check(step.h, step.plan)          # page ids checked once on the host ...
    step.plan = dsa.Plan(wl.spans, wl.page_table, wl.pool_pages, step.plan.spans_dev,
                         step.plan.page_table_dev, check_pages=False)   # ... not on every call
    n_layers = len(step.q_nope)
    copies = max(1, args.copies)
    key_pools = [step.key_pool] + [step.key_pool.clone() for _ in range(copies - 1)]
    lat_pools = [[p] + [p.clone() for _ in range(copies - 1)] for p in step.latent_pools]
    st = torch.cuda.current_stream()

    # This step's keys go into every pool copy once, up front: the timed step is select + attend
    # (index_topk, then every attend layer); store_keys is timed on its own below.
    for c in range(copies):
        step.store_keys(key_pool=key_pools[c], stream=st)

    def run(i, stream=st):
        c = i % copies
        step.index_topk(key_pool=key_pools[c], stream=stream)
        for layer in range(n_layers):
            step.attend(layer, latent_pool=lat_pools[layer][c], stream=stream)

    alg = algorithmic(wl)

    if args.profile_only:
        for i in range(5):
            run(i)
        torch.cuda.synchronize()
        # the score kernel alone, as the bench times it (dsa_index_scores)
        ld = int((wl.positions.max() + 1 + 3) // 4 * 4)
        scores = torch.empty(step.plan.n_rows, ld, dtype=torch.float32, device="cuda")
        for i in range(5):
            dsa.dsa_index_scores(step.h, step.plan, step.index_q, step.index_w, key_pools[i % copies],
                                 scores, ld, st)
        torch.cuda.synchronize()
        del scores
        # a plain copy of known size for scaling the HBM counters
        nbytes = 1 << 30
        a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(f"profile run done: copy of {nbytes} bytes; index bytes per launch {alg['index_bytes']}")
        return

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(st)
    for i in range(args.steps):
        run(args.warmup + i)
    t1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps

    # Per-step times (events around each step) for the spread.
    n_d = min(args.steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_d + 1)]
    evs[0].record(st)
    for i in range(n_d):
        run(i)
        evs[i + 1].record(st)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n_d))
    pct = lambda q: per_step[min(n_d - 1, int(q * n_d))]

    # store_keys alone (not part of the select + attend step)
    for i in range(3):
        step.store_keys(key_pool=key_pools[i % copies], stream=st)
    torch.cuda.synchronize()
    n_s = 50
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record(st)
    for i in range(n_s):
        step.store_keys(key_pool=key_pools[i % copies], stream=st)
    s1.record(st)
    torch.cuda.synchronize()
    store_ms = s0.elapsed_time(s1) / n_s

    # With several attend layers (one FULL layer whose selection the SHARED layers reuse), the
    # same step without the FULL layer's own attend: select + the SHARED attends only.
    shared_ms = None
    if n_layers > 1:
        def run_shared(i):
            c = i % copies
            step.index_topk(key_pool=key_pools[c], stream=st)
            for layer in range(1, n_layers):
                step.attend(layer, latent_pool=lat_pools[layer][c], stream=st)
        for i in range(3):
            run_shared(i)
        torch.cuda.synchronize()
        n_sh = max(5, args.steps // 4)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(n_sh):
            run_shared(i)
        e1.record(st)
        torch.cuda.synchronize()
        shared_ms = e0.elapsed_time(e1) / n_sh

    # The same steps captured once in a HIP graph (one step per pool copy) and replayed: no launch
    # work on the host. The library neither allocates nor clears memory inside a call, so a step
    # captures as it is.
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(st)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for c in range(copies):
                    run(c, stream=cap)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        n_g = max(1, args.steps // copies)
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        cs = torch.cuda.current_stream()
        g0.record(cs)
        for _ in range(n_g):
            g.replay()
        g1.record(cs)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (n_g * copies)

    # The dominant kernel alone (the index score kernel behind dsa_index_scores), same launch shape,
    # timed with events on the stream it runs on.
    ld = int((wl.positions.max() + 1 + 3) // 4 * 4)
    scores = torch.empty(step.plan.n_rows, ld, dtype=torch.float32, device="cuda")
    for i in range(5):
        dsa.dsa_index_scores(step.h, step.plan, step.index_q, step.index_w, key_pools[i % copies], scores, ld, st)
    torch.cuda.synchronize()
    n_k = max(20, args.steps // 2)
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record(st)
    for i in range(n_k):
        dsa.dsa_index_scores(step.h, step.plan, step.index_q, step.index_w, key_pools[i % copies], scores, ld, st)
    k1.record(st)
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / n_k
    k_bytes = alg["index_bytes"]
    achieved = k_bytes / (k_ms * 1e-3) / 1e9

    # The attention kernel of one layer (dsa_sparse_mla_attend), timed the same way.
    for i in range(3):
        step.attend(0, latent_pool=lat_pools[0][i % copies], stream=st)
    torch.cuda.synchronize()
    n_a = max(10, n_k // 2)
    k0.record(st)
    for i in range(n_a):
        step.attend(0, latent_pool=lat_pools[0][i % copies], stream=st)
    k1.record(st)
    torch.cuda.synchronize()
    a_ms = k0.elapsed_time(k1) / n_a
    a_flops = alg["attend_flops"] / n_layers
    a_tflops = a_flops / (a_ms * 1e-3) / 1e12

    # index_topk alone: the score kernel (its dsa_index_topk form, which also lists each block's
    # top keys) and the select
    for i in range(3):
        step.index_topk(key_pool=key_pools[i % copies], stream=st)
    torch.cuda.synchronize()
    k0.record(st)
    for i in range(n_a):
        step.index_topk(key_pool=key_pools[i % copies], stream=st)
    k1.record(st)
    torch.cuda.synchronize()
    t_ms = k0.elapsed_time(k1) / n_a
    index_line = {
        "kernel": "index score (dsa_index_scores / first launch of dsa_index_topk)",
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(wl.spec.name, "score"),
        "kernel_ms": round(k_ms, 5), "algorithmic_bytes_per_launch": k_bytes,
        "mfma_tflops": round(alg["index_flops"] / (k_ms * 1e-3) / 1e12, 1),
    }
    attend_line = {
        "kernel": "sparse MLA attend, one layer (dsa_sparse_mla_attend)",
        "bound": "mfma", "achieved": round(a_tflops, 1), "peak": MFMA_BF16_PEAK_TFS,
        "unit": "TFLOP/s", "frac": round(a_tflops / MFMA_BF16_PEAK_TFS, 4),
        "traffic": measured_traffic(wl.spec.name, "attend"),
        "kernel_ms": round(a_ms, 5), "algorithmic_flops_per_launch": a_flops,
        "algorithmic_bytes_per_launch": alg["attend_bytes"] // n_layers,
    }
    # A decode step is bound by the index scan over each request's whole context (HBM); a step
    # with prefill rows by the attention contractions (MFMA). The roofline line is that kernel;
    # the other is reported beside it.
    prefill = int(max(wl.spans[:, 1])) > 1
    dominant, other = (attend_line, index_line) if prefill else (index_line, attend_line)

    rows = wl.n_rows
    value = rows / (ms * 1e-3)
    s = wl.spec
    out = {
        "metric": "DSA decode tokens/s (select+attend) at 128K ctx topk=2048; % HBM peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "step_ms_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5), round(pct(0.9), 5)],
        "store_keys_ms": round(store_ms, 5),
        "graph": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 5), "value": round(rows / (graph_ms * 1e-3), 1),
            "note": "the same select + attend steps replayed from one captured HIP graph"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "formats": f"{s.index_key_fmt} index keys, {s.latent_fmt} latents, {s.q_fmt} queries and "
                   f"output; bf16 MFMA operands with f32 accumulation",
        "data": "synthetic (seeded; N(0,1) draws encoded to the cache formats)",
        "config": {
            "workload": f"{s.name}: {rows} rows in {len(wl.spans)} requests (longest {int(max(wl.spans[:, 1]))} "
                        f"rows), positions up to {int(wl.positions.max())}, "
                        f"{s.n_index_heads}x{s.index_dim} {s.index_key_fmt} index keys, topk {s.topk}, "
                        f"{s.n_heads}-head absorbed MLA over {s.kv_lora_rank}+{s.rope_dim} "
                        f"{s.latent_fmt} latents, {s.page_size}-token pages",
            "rows_per_step": rows, "attend_layers": n_layers, "pool_copies_rotated": copies,
        },
        "step_bytes_algorithmic": alg["total_bytes"],
        "step_hbm_frac": round(alg["total_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "shared_layers_only": None if shared_ms is None else {
            "attend_layers": n_layers - 1, "ms_per_step": round(shared_ms, 5),
            "value": round(rows / (shared_ms * 1e-3), 1),
            "note": "select + the SHARED layers' attends (the FULL layer's own attend left out)"},
        "roofline": dominant,
        "other_kernel": other,
        "index_topk": {
            "ms": round(t_ms, 5),
            "select_ms": round(t_ms - k_ms, 5),
            "note": "dsa_index_topk alone; select_ms is that minus the score kernel timed alone "
                    "(so it also holds the block lists the score kernel writes inside index_topk)",
            "select_traffic": measured_traffic(wl.spec.name, "select"),
            "score_kernel_traffic": measured_traffic(wl.spec.name, "score_step")},
        "hbm_copy_measured_gbs": copy_rate(),
        "wall_s_timed": round(wall, 3),
        "gen_s": round(t_gen, 1),
    }
    if not args.no_prefill and args.workload == "long_decode":
        # the other named workloads, each its own step, timed after the headline line
        del key_pools, lat_pools, scores
        torch.cuda.empty_cache()
        out["decode_batch"] = workload_line("decode_batch", max(50, args.prefill_steps))
        out["causal_prefill"] = workload_line("causal_prefill", args.prefill_steps)
        out["chunked_mix"] = workload_line("chunked_mix", max(3, args.prefill_steps // 2))
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_seconds)
        cb["value"] = round(cb["value"], 4)
        cb.pop("seconds")
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
