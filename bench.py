"""Benchmark of the paged Top-K decode step on one MI355X.

Workload: Llama-3.1-8B-shaped GQA decode of one layer at 128k context (batch 1,
32 query / 8 KV heads, head_dim 128, bf16 KV in 16-token pages, shuffled page
table, 5% planted blocks, Top-K 256 blocks), synthetic seeded data.

One step = one pass over every stage of the path on that input:
  block meta build over all 8192 pages -> append of the newest token + Quest scores + Top-K 256
  (one call) ->
  sparse split-K attention -> merge -> dense split-K attention -> merge.
The metric is KV GB/s (algorithmic bytes of the step / step time, and the same
per stage) and decode steps/s; the dominant kernel (dense attention) is also
reported against the 8 TB/s HBM peak.  Inputs are resident in HBM before the
timed region.  Twelve copies of the workload are rotated, and every HIP graph
steps through each copy once, so no step is served from the 256 MB last-level
cache by the steps before it (a sparse decode step reads ~53 MB at 128k: twelve
copies hold ~640 MB).

Also in the same run: the zero-copy variant (K/V pools in mapped pinned host
memory; its roofline is the measured host-to-device copy bandwidth), and the
fp64 oracle timed on the host cores on every named workload (cpu_baseline; its
value is the 128k workload's).

The dominant kernel is also reported against two read ceilings measured in the
same run by kernels that compute nothing: a plain stream read of 1 GiB, and
the dense attention's own gather of K/V tiles (roofline.read_ceilings).

Beside the step, kernel-level timings of the selection variants: the mean-key
index (build and select) and either index with the first 4 / last 64 tokens
forced in (selection_variants).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
       [--no-variants | --only-variants] [--no-zero-copy] [--no-other-workloads]
       python bench.py --copy-calibration    (a plain 1 GiB device copy, for counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
GRAPH_STEPS = 8          # fewest decode steps captured per HIP graph (each graph steps
                         # through every workload copy once, so len(copies) when larger)
GRAPH_MIN_REPLAYS = 25   # decode-step figures: median over >= 25 replays (>= 200 timed steps)
GRAPH_WARM_REPLAYS = 3   # ... after >= 24 untimed ones
STREAM_PROBE_BYTES = 1 << 30
WORKLOAD = "llama3.1_8b_gqa_b1_128k_bf16"
HOSTKV_WORKLOAD = "llama3.1_8b_gqa_b1_128k_bf16_hostkv"
# measured beside the headline step at kernel level (not part of `value`)
OTHER_WORKLOADS = ("llama3.1_8b_gqa_b4_32k_bf16", "opt6.7b_mha_b32_544_f16")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "paged_attn_dense_gqa128k_pmc.md")
# sources that define the dense attention kernel: the counter-derived traffic
# is only reported while they are unchanged since the counters were taken
ATTN_SOURCES = [os.path.join(ROOT, "kv_cache_decode_amd", "csrc", f)
                for f in ("kvd_attn.hip", "kvd_device.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic bytes
#
# Per (block, KV head) unit: K and V tiles of bs x D elements, meta rows of 2 x D.

def stage_bytes(spec, topk: int, s_sparse: int, s_dense: int) -> dict:
    eb = spec.elem_bytes
    bs, D, B, Hq, Hkv = spec.block_size, spec.head_dim, spec.num_seqs, spec.num_q_heads, spec.num_kv_heads
    blocks = spec.used_pages                       # sum_b N_b
    maxN = spec.max_blocks
    tile = bs * D * eb                             # one K (or V) tile
    meta_row = 2 * D * eb
    q_bytes = B * Hq * D * eb
    keff = sum(min(topk, spec.blocks(b)) for b in range(B))
    part = lambda S: B * Hq * S * (D + 2) * 4
    out = B * Hq * (D + 1) * 4
    return {
        "meta_build": blocks * Hkv * (tile + meta_row) + blocks * 8,
        # new K and V rows in and out, the meta rows of their pages read and written
        "append": B * Hkv * (4 * D * eb + 2 * meta_row) + 2 * B * 4,
        "score_topk": blocks * Hkv * meta_row + q_bytes + blocks * Hkv * 4      # meta + q + table
                      + 2 * B * Hkv * maxN * 4                                   # scores out + in
                      + B * Hkv * (topk + 1) * 4,                                # selection
        "sparse_attn": keff * Hkv * 2 * tile + q_bytes + keff * Hkv * 8 + part(s_sparse),
        "sparse_combine": part(s_sparse) + out,
        "dense_attn": blocks * Hkv * 2 * tile + q_bytes + blocks * Hkv * 4 + part(s_dense),
        "dense_combine": part(s_dense) + out,
    }


def tiered_bytes(spec, block_table, tier, fmt: str, splits: int):
    """Algorithmic bytes of one dense attention over tiered pools: per (page, KV
    head) unit a hot page gives 2 * 16 * D 16-bit values, a cold one its codes
    (D bytes per row in FP8, D / 2 in INT4) and two fp32 scales; every unit adds
    its 4-byte table entry and its tier byte; q in, the split partials out.
    Returns (bytes, fraction of the listed pages that are cold)."""
    used = np.concatenate([block_table[b, :spec.blocks(b)] for b in range(spec.num_seqs)])
    n_cold = int((tier[used] != 0).sum())
    n_hot = len(used) - n_cold
    D, Hkv, B, Hq = spec.head_dim, spec.num_kv_heads, spec.num_seqs, spec.num_q_heads
    tile = spec.block_size * D
    code_tile = tile if fmt == "fp8" else tile // 2
    units = Hkv * (n_hot * 2 * tile * spec.elem_bytes + n_cold * (2 * code_tile + 8)) \
        + len(used) * Hkv * (4 + 1)
    return units + B * Hq * D * spec.elem_bytes + B * Hq * splits * (D + 2) * 4, n_cold / len(used)


def variant_bytes(spec, topk: int) -> dict:
    """Algorithmic bytes of the selection variants: the mean-key index holds one
    fp32 row of D per (page, KV head)."""
    eb = spec.elem_bytes
    bs, D, B, Hq, Hkv = spec.block_size, spec.head_dim, spec.num_seqs, spec.num_q_heads, spec.num_kv_heads
    blocks, maxN = spec.used_pages, spec.max_blocks
    mean_row, meta_row = 4 * D, 2 * D * eb
    rest = B * Hq * D * eb + blocks * Hkv * 4 + 2 * B * Hkv * maxN * 4 + B * Hkv * (topk + 1) * 4
    return {
        "mean_build": blocks * Hkv * (bs * D * eb + mean_row) + blocks * 8,
        "meta_build": blocks * Hkv * (bs * D * eb + meta_row) + blocks * 8,
        "mean_select_forced": blocks * Hkv * mean_row + rest,
        "minmax_select_forced": blocks * Hkv * meta_row + rest,
        "minmax_select": blocks * Hkv * meta_row + rest,
    }


# ---------------------------------------------------------------- HBM traffic from counters

def source_digest() -> str:
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Counter-derived HBM bytes per dense-attention launch, if the committed
    profile was taken on the current kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b) or m_sha.group(1) != source_digest():
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------- GPU part

def graph_step_us(fn, copies, args):
    """Time per step of fn, replayed from one HIP graph that holds one step per
    workload copy (at least GRAPH_STEPS; one host launch per graph, so a short
    step is not timed at the host's graph launch rate): the
    median over at least GRAPH_MIN_REPLAYS replays, each bracketed by its own
    events.  Raises RuntimeError where a call cannot be captured."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in copies:
            fn(c)
    torch.cuda.current_stream().wait_stream(side)
    steps = max(GRAPH_STEPS, len(copies))
    g_ = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_):
        for i in range(steps):
            fn(copies[i % len(copies)])
    reps = max(GRAPH_MIN_REPLAYS, args.steps // steps)
    for _ in range(max(GRAPH_WARM_REPLAYS, args.warmup // steps)):
        g_.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        g_.replay()
        b.record()
    torch.cuda.synchronize()
    del g_
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3 / steps


def run_gpu(args, spec, data):
    import torch
    from kv_cache_decode_amd.step import DeviceWorkload

    dev = torch.device("cuda:0")
    k = spec.topk_blocks
    copies = [DeviceWorkload(data, device=dev) for _ in range(args.copies)]
    for c in copies:                       # the index exists before decoding starts
        c.meta_build()
    torch.cuda.synchronize()
    from kv_cache_decode_amd import kvdecode as kd
    s_sparse = kd.kv_auto_num_splits(copies[0].shape, k)
    s_sel = kd.kv_auto_select_splits(copies[0].shape, k)
    s_dense = kd.kv_auto_num_splits(copies[0].shape, spec.max_blocks)
    stages = ["meta_build", "append_select", "sparse_attn", "sparse_combine", "dense_attn",
              "dense_combine"]
    actions = [
        lambda c: c.meta_build(),
        # append of the newest token again (state is unchanged) + score + Top-K
        lambda c: c.decode_select(k),
        lambda c: c.attention(sparse=True, num_splits=s_sparse),
        lambda c: c.combine(s_sparse),
        lambda c: c.attention(sparse=False, num_splits=s_dense),
        lambda c: c.combine(s_dense),
    ]

    def step(c, ev=None):
        for i, act in enumerate(actions):
            if ev is not None:
                ev[i].record()
            act(c)
        if ev is not None:
            ev[len(actions)].record()

    def time_loop(run_one, calls=None):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record()
        for i in range(args.steps if calls is None else calls):
            run_one(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1), time.perf_counter() - wall0

    def graph_us(fn):
        try:
            return graph_step_us(fn, copies, args)
        except RuntimeError:
            ms_, _ = time_loop(lambda i: fn(copies[i % len(copies)]))
            return ms_ * 1e3 / args.steps

    res = {"s_sparse": s_sparse, "s_sel": s_sel, "s_dense": s_dense}
    if not args.only_variants:
        for i in range(args.warmup):
            step(copies[i % len(copies)])
        torch.cuda.synchronize()

        # per-stage timing: eager launches bracketed by events on the launch stream
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(copies[i % len(copies)], evs[i])
        torch.cuda.synchronize()
        per_stage_ms = {s: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                        for i, s in enumerate(stages)}

        # whole-step timing, eager launches without stage events
        eager_ms, _ = time_loop(lambda i: step(copies[i % len(copies)]))

        # the dominant kernel alone: back-to-back dense launches over the rotated
        # copies, so per-launch event overhead does not enter its average
        dense_loop_ms, _ = time_loop(
            lambda i: copies[i % len(copies)].attention(sparse=False, num_splits=s_dense))

        ceilings = time_read_ceilings(copies, s_dense, time_loop, args.steps)

        # whole-step timing: HIP graphs of one step per copy (>= GRAPH_STEPS) cycling
        # over the workload copies (so each graph launch's fixed cost of a few us
        # is spread over several steps, as a decode loop that captures its
        # layers would), replayed args.steps // per times, plus one graph
        # of the remaining steps: exactly args.steps steps between the events
        launch = "hip_graph"
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for c in copies:
                    step(c)
            torch.cuda.current_stream().wait_stream(side)

            def capture(n):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(n):
                        step(copies[i % len(copies)])
                return g

            per = max(GRAPH_STEPS, len(copies))
            full_g = capture(per)
            tail = args.steps % per
            tail_g = capture(tail) if tail else None
            for _ in range(max(1, args.warmup // per)):
                full_g.replay()

            def replay(i):
                if i < args.steps // per:
                    full_g.replay()
                elif tail_g is not None:
                    tail_g.replay()

            total_ms, wall = time_loop(replay, args.steps // per + (1 if tail else 0))
            del full_g, tail_g
        except RuntimeError as e:          # capture unavailable: report eager launches
            log(f"[bench] graph capture failed ({e}); timing eager launches")
            launch = "eager"
            total_ms, wall = time_loop(lambda i: step(copies[i % len(copies)]))
        # the per-token decode steps on their own, each one HIP graph per copy:
        # sparse = append + score (one call), Top-K + sparse attention (one
        #          call: one launch for rows of <= 2048 blocks, else two) + merge,
        # dense  = append + dense attention + merge; and for comparison the
        # sparse step as append + score + Top-K (one call), sparse attention,
        # merge, and with the append, score and Top-K as three separate calls
        def decode_sparse(c):
            c.decode_score()
            c.select_attention(k, s_sel)
            c.combine(s_sel)

        def decode_sparse_select(c):
            c.decode_select(k)
            c.attention(sparse=True, num_splits=s_sparse)
            c.combine(s_sparse)

        def decode_sparse_unfused(c):
            c.append()
            c.score_topk(k)
            c.attention(sparse=True, num_splits=s_sparse)
            c.combine(s_sparse)

        def decode_dense(c):
            c.append()
            c.attention(sparse=False, num_splits=s_dense)
            c.combine(s_dense)

        decode_us = {"sparse": graph_us(decode_sparse), "dense": graph_us(decode_dense),
                     "sparse_decode_select": graph_us(decode_sparse_select),
                     "sparse_unfused": graph_us(decode_sparse_unfused)}
        dense_graph_us = graph_us(lambda c: c.attention(sparse=False, num_splits=s_dense))
        res.update({
            "total_ms": total_ms, "wall_s": wall, "stage_ms": per_stage_ms,
            "decode_us": decode_us, "launch": launch,
            "dense_attn_loop_us": dense_loop_ms * 1e3 / args.steps,
            "dense_attn_graph_us": dense_graph_us,
            "ceilings": ceilings,
            "eager_ms_per_step": eager_ms / args.steps,
        })

    # selection variants, kernel level (not part of the step): the mean-key
    # index, and either index with the first 4 / last 64 tokens forced in
    variants = None if args.no_variants else time_variants(args, copies, k, s_sparse,
                                                            time_loop, graph_us)
    # cold pages in HBM: the same attention over FP8 E4M3 (1 byte) and INT4
    # (half a byte per channel) codes
    fp8 = None if args.no_variants else time_codes(args, copies, k, time_loop, graph_us, "fp8")
    int4 = None if args.no_variants else time_codes(args, copies, k, time_loop, graph_us, "int4")
    for c in copies:
        c.close()
    del copies
    torch.cuda.empty_cache()
    res["variants"] = variants
    res["fp8"] = fp8
    res["int4"] = int4
    return res


def time_read_ceilings(copies, s_dense, time_loop, steps):
    """What the memory system delivers to kernels that compute nothing, on this
    GPU in this run: a plain front-to-back stream read (two 1 GiB buffers
    alternated, together beyond the last-level cache), and the dense decode
    attention's own gather of K/V tiles (same pages, order, splits, lane layout
    and prefetch depth, rotated over the same workload copies)."""
    import torch
    from kv_cache_decode_amd import kvdecode as kd

    dev = copies[0].device
    n = STREAM_PROBE_BYTES
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(2)]
    for b_ in bufs:
        b_.fill_(5)
    sink = torch.empty(kd.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    for i in range(4):
        kd.kv_probe_stream_read(bufs[i % 2], n, sink)
    stream_ms, _ = time_loop(lambda i: kd.kv_probe_stream_read(bufs[i % 2], n, sink))
    stream_us = stream_ms * 1e3 / steps
    del bufs
    spec = copies[0].spec
    B, Hkv = spec.num_seqs, spec.num_kv_heads
    gsink = torch.empty(B * Hkv * s_dense, dtype=torch.int32, device=dev)

    def gather(c):
        kd.kv_probe_gather_read(c.shape, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                s_dense, gsink)
    for c in copies:
        gather(c)
    gather_ms, _ = time_loop(lambda i: gather(copies[i % len(copies)]))
    gather_us = gather_ms * 1e3 / steps
    kv_bytes = spec.used_pages * Hkv * 2 * spec.block_size * spec.head_dim * spec.elem_bytes
    torch.cuda.empty_cache()
    return {"stream_read": {"bytes": n, "us": stream_us, "gbps": n / (stream_us * 1e-6) / 1e9},
            "dense_gather_read": {"bytes": kv_bytes, "us": gather_us, "splits": s_dense,
                                  "gbps": kv_bytes / (gather_us * 1e-6) / 1e9}}


def time_codes(args, copies, k, time_loop, graph_us, fmt: str):
    """Code pages in HBM (fmt "fp8" or "int4"): quantiser, dense and sparse
    attention kernels (back-to-back launches), and the decode graphs."""
    import torch
    from kv_cache_decode_amd import kvdecode as kd
    # the code-page paths share their own split heuristic
    s_sparse = kd.kv_auto_num_splits_fp8(copies[0].shape, k)
    s_dense = kd.kv_auto_num_splits_fp8(copies[0].shape, copies[0].spec.max_blocks)
    # the quantizer call alone, into code pools allocated once per copy
    qcall = kd.kv_quantize_pages_fp8 if fmt == "fp8" else kd.kv_quantize_pages_int4
    qbufs = {}

    def quantize(c):
        if id(c) not in qbufs:
            P, Hkv, bs, D = c.data.k_raw.shape
            row = D if fmt == "fp8" else D // 2
            kq = torch.zeros((P, Hkv, bs, row), dtype=torch.uint8, device=c.device)
            qbufs[id(c)] = (kq, torch.zeros_like(kq),
                            torch.zeros((P, Hkv, 2), dtype=torch.float32, device=c.device))
        kq, vq, sq = qbufs[id(c)]
        qcall(c.shape, c.k_cache, c.v_cache, c.page_ids, c.page_valid, int(c.page_ids.numel()),
              kq, vq, sq)
    attn = (lambda c, sp, S: c.attention_fp8(sparse=sp, num_splits=S)) if fmt == "fp8" else \
        (lambda c, sp, S: c.attention_int4(sparse=sp, num_splits=S))

    def kernel_us(fn):
        for i in range(args.warmup):
            fn(copies[i % len(copies)])
        ms_, _ = time_loop(lambda i: fn(copies[i % len(copies)]))
        return ms_ * 1e3 / args.steps

    for c in copies:
        (c.quantize_fp8 if fmt == "fp8" else c.quantize_int4)(host=False)   # the pools attention reads
        quantize(c)
        c.score_topk(k)
    torch.cuda.synchronize()
    res = {
        "quantize_us": kernel_us(quantize),
        "dense_attn_us": kernel_us(lambda c: attn(c, False, s_dense)),
        "sparse_attn_us": kernel_us(lambda c: attn(c, True, s_sparse)),
    }

    def decode_sparse(c):
        c.score_topk(k)
        attn(c, True, s_sparse)
        c.combine(s_sparse)

    def decode_dense(c):
        attn(c, False, s_dense)
        c.combine(s_dense)

    res["decode_sparse_us"] = graph_us(decode_sparse)
    res["decode_dense_us"] = graph_us(decode_dense)
    res["s_sparse"], res["s_dense"] = s_sparse, s_dense
    # tiered pools: the most recent quarter of each sequence hot (16-bit), the
    # rest cold code pages, dense attention over both in one call
    spec = copies[0].spec
    data = copies[0].data
    tier_np = np.ones(spec.num_pages, np.uint8)
    for b in range(spec.num_seqs):
        nb = spec.blocks(b)
        tier_np[data.block_table[b, nb - nb // 4:nb]] = 0
    tier = torch.from_numpy(tier_np).to(copies[0].device)
    s_tier = kd.kv_auto_num_splits_tiered(copies[0].shape, spec.max_blocks)
    res["tiered_dense_us"] = kernel_us(lambda c: c.attention_tiered(False, fmt, tier, s_tier))
    # the same as two launches over the block lists split by tier
    nb = spec.max_blocks
    s_hot = kd.kv_auto_num_splits(copies[0].shape, nb // 4)
    s_cold = kd.kv_auto_num_splits_fp8(copies[0].shape, nb - nb // 4)
    res["tiered_split_dense_us"] = kernel_us(
        lambda c: c.attention_tiered_split(False, fmt, tier, s_hot, s_cold))
    res["tiered_split_splits"] = [s_hot, s_cold]
    res["tiered_dense_bytes"], res["tiered_cold_fraction"] = tiered_bytes(spec, data.block_table,
                                                                          tier_np, fmt, s_tier)
    res["tiered_splits"] = s_tier
    if fmt == "int4":
        res["tier_policy"] = time_tier_policy(args, copies[0], k)
    return res


TIER_POLICY = {"decay": 0.875, "hot_above": 0.5, "cold_below": 0.125, "recent_tokens": 64,
               "cooldown_steps": 8}


def time_tier_policy(args, dw, k):
    """The hot/cold tier policy over a CACHE_STEPS-step decode trajectory (the
    AR(1) queries of the block cache's trajectory), INT4 cold pages in HBM.  A
    step is: score + Top-K, kv_tier_plan (page heat from the step's selection,
    demotions and promotions), the INT4 codes of the demoted pages, tiered
    sparse attention and the merge.  Every page starts hot with heat 0, so the
    first step demotes every page outside the selection and the recent tokens.
    The trajectory runs twice more from that state, counting the pages that
    move, once more on a side stream, and is then captured as one HIP graph
    with the next step numbers.  Each timed replay starts from the state the
    capture followed (heat, tier and stamp restored outside the events), so
    every replay runs the same continuation of the trajectory; the median
    replay gives the step time.  kv_tier_plan alone is timed as a graph of
    GRAPH_STEPS calls (it keeps updating the state it reads)."""
    import torch
    from kv_cache_decode_amd import kvdecode as kd
    from kv_cache_decode_amd import workload as wl
    from kv_cache_decode_amd.step import storage_tensor

    spec, data = dw.spec, dw.data
    q0 = dw.q
    qs = [storage_tensor(q, spec.dtype).to(dw.device)
          for q in wl.query_trajectory(data, CACHE_STEPS, CACHE_RHO, seed=21)]
    S = kd.kv_auto_num_splits_tiered(dw.shape, k)
    dw.tier_init()
    step_no = [0]

    def step(q, counts=None):
        dw.q = q
        dw.score_topk(k)
        dw.tier_step(step_no[0], cold="int4", **TIER_POLICY)
        dw.attention_tiered(True, "int4", dw.page_tier, S)
        dw.combine(S)
        step_no[0] += 1
        if counts is not None:
            counts.append(torch.stack([dw.demote_count.sum(), dw.promote_count.sum()]))

    first, moved = [], []
    for q in qs:                                 # from all hot: the first step demotes
        step(q, first)
    for _ in range(2):                           # the same trajectory again, counted
        for q in qs:
            step(q, moved)
    torch.cuda.synchronize()
    moved = torch.stack(moved).cpu().numpy().astype(np.int64)
    first = torch.stack(first).cpu().numpy().astype(np.int64)
    hot = float((dw.page_tier[:spec.used_pages] == 0).float().mean())

    res = {"steps": CACHE_STEPS, "rho": CACHE_RHO, "topk_blocks": k, "splits": S,
           "cold": "int4", "policy": dict(TIER_POLICY),
           "first_step_demoted_pages": int(first[0, 0]),
           "demoted_pages_per_step": float(moved[:, 0].mean()),
           "promoted_pages_per_step": float(moved[:, 1].mean()),
           "hot_page_fraction_after": hot}
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for q in qs:
                step(q)
        torch.cuda.current_stream().wait_stream(side)
        # the step numbers are launch arguments, fixed at capture: every replay
        # starts from the policy state the capture followed (restored, untimed),
        # so each one runs the same continuation of the counted trajectory
        state = [t.clone() for t in (dw.page_heat, dw.page_tier, dw.page_stamp)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for q in qs:
                step(q)
        times = []
        for rep in range(GRAPH_WARM_REPLAYS + GRAPH_MIN_REPLAYS):
            for t, s0 in zip((dw.page_heat, dw.page_tier, dw.page_stamp), state):
                t.copy_(s0)
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            g.replay()
            b_.record()
            torch.cuda.synchronize()
            if rep >= GRAPH_WARM_REPLAYS:
                times.append(a.elapsed_time(b_))
        del g
        res["step_us"] = float(np.median(times)) * 1e3 / len(qs)
        res["timing"] = ("HIP graph of the trajectory, each replay from the same policy state, "
                         "median of replays")
        res["tier_plan_us"] = graph_step_us(
            lambda c: c.tier_step(step_no[0], cold=None, **TIER_POLICY), [dw], args)
    except RuntimeError as e:
        log(f"[bench] tier policy graph capture failed ({e}); timing eager launches")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for q in qs:
            step(q)
        torch.cuda.synchronize()
        res["step_us"] = (time.perf_counter() - t0) * 1e6 / len(qs)
        res["timing"] = "eager launches (host time included)"
    dw.q = q0
    return res


LONG_SELECT = dict(num_kv_heads=8, num_q_heads=32, head_dim=128, blocks=65536, topk=256,
                   seed=6100)


def time_long_select(args):
    """Score + Top-K over a 1M-token layer (one sequence of 65536 blocks, 8 KV
    heads, G = 4, D = 128, a bf16 min/max index of normal values behind a
    shuffled block table, Top-K 256): kv_block_score_topk without candidate
    storage (one workgroup selects each row) and with a workspace that holds
    it (the two-level select), each graph-timed; the two lists must be equal."""
    import torch
    from kv_cache_decode_amd import kvdecode as kd
    c = LONG_SELECT
    Hkv, Hq, D, N, K = c["num_kv_heads"], c["num_q_heads"], c["head_dim"], c["blocks"], c["topk"]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(c["seed"])
    shape = kd.make_shape(1, Hq, Hkv, D, N, N, "bf16")
    q = torch.randn(1, Hq, D, device=dev, generator=g).to(torch.bfloat16)
    kmeta = torch.randn(N, Hkv, 2, D, device=dev, generator=g).to(torch.bfloat16)
    table = torch.randperm(N, device=dev, generator=g).to(torch.int32).view(1, N)
    lens = torch.full((1,), N * 16, device=dev, dtype=torch.int32)
    scores = torch.empty(1, Hkv, N, device=dev)
    need = kd.kv_score_topk_workspace_size(shape, K)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = {}
    for name, w, nw in (("one_level", None, 0), ("two_level", ws, need)):
        sel = torch.empty(1, Hkv, K, device=dev, dtype=torch.int32)
        cnt = torch.empty(1, Hkv, device=dev, dtype=torch.int32)
        call = (lambda _, w=w, nw=nw, sel=sel, cnt=cnt:
                kd.kv_block_score_topk(shape, q, kmeta, table, lens, K, scores, sel, cnt, w, nw,
                                       torch.cuda.current_stream()))
        us = graph_step_us(call, [None], args)
        torch.cuda.synchronize()
        out[name] = (us, sel.cpu(), cnt.cpu())
    same = bool(torch.equal(out["one_level"][1], out["two_level"][1]) and
                torch.equal(out["one_level"][2], out["two_level"][2]))
    if not same:
        raise RuntimeError("two-level and one-level Top-K lists differ")
    return {"workload": f"1M-token layer: 1 sequence x {N} blocks of 16 tokens, {Hkv} KV heads, "
                        f"G={Hq // Hkv}, D={D}, bf16 min/max index, Top-K {K}",
            "score_topk_one_level_us": out["one_level"][0],
            "score_topk_two_level_us": out["two_level"][0],
            "workspace_bytes": need, "lists_equal": same,
            "timing": "kv_block_score_topk per call, median over HIP graph replays"}


def time_variants(args, copies, k, s_sparse, time_loop, graph_us):
    import torch

    def kernel_us(fn):
        for i in range(args.warmup):
            fn(copies[i % len(copies)])
        ms_, _ = time_loop(lambda i: fn(copies[i % len(copies)]))
        return ms_ * 1e3 / args.steps

    for c in copies:
        c.mean_build()            # from here on append() refreshes the mean rows too
    torch.cuda.synchronize()
    variants = {
        "mean_build_us": kernel_us(lambda c: c.mean_build()),
        "meta_build_us": kernel_us(lambda c: c.meta_build()),
        "mean_select_forced_us": kernel_us(lambda c: c.select(k, "mean", 4, 64)),
        "minmax_select_forced_us": kernel_us(lambda c: c.select(k, "minmax", 4, 64)),
        "minmax_select_us": kernel_us(lambda c: c.select(k, "minmax", 0, 0)),
    }

    def decode_sparse_mean(c):
        c.decode_select(k, "mean", 4, 64)
        c.attention(sparse=True, num_splits=s_sparse)
        c.combine(s_sparse)

    variants["decode_sparse_mean_forced_us"] = graph_us(decode_sparse_mean)
    return variants


def run_other_workload(args, name, cpu_out=None):
    """Kernel-level figures of another named workload (steps replayed from HIP
    graphs over rotated copies): dense attention GB/s, and the sparse decode
    path."""
    import torch
    from kv_cache_decode_amd import kvdecode as kd
    from kv_cache_decode_amd import workload as wl
    from kv_cache_decode_amd.step import DeviceWorkload

    spec = wl.WORKLOADS[name]
    data = wl.generate(spec)
    copies = [DeviceWorkload(data) for _ in range(args.copies)]
    reps = max(20, args.steps // 2)

    def loop(fn):
        try:
            return graph_step_us(fn, copies, args)
        except RuntimeError:       # eager back-to-back launches
            for i in range(4):
                fn(copies[i % len(copies)])
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for i in range(reps):
                fn(copies[i % len(copies)])
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) * 1e3 / reps

    def eager(fn):
        """Back-to-back launches between two events on the launch stream: the
        timer of the headline roofline, so every workload's dense figure is
        taken the same way."""
        for i in range(4):
            fn(copies[i % len(copies)])
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(args.steps):
            fn(copies[i % len(copies)])
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / args.steps

    s_dense = kd.kv_auto_num_splits(copies[0].shape, spec.max_blocks)
    dense_us = eager(lambda c: c.attention(sparse=False, num_splits=s_dense))
    dense_graph_us = loop(lambda c: c.attention(sparse=False, num_splits=s_dense))
    k = spec.topk_blocks
    s_sp = kd.kv_auto_num_splits(copies[0].shape, k) if k else 1
    sb = stage_bytes(spec, k or 1, s_sp, s_dense)
    gbps = lambda name, us: sb[name] / (us * 1e-6) / 1e9
    dense_comb_us = loop(lambda c: c.combine(s_dense))
    res = {"dense_attn_us": dense_us, "dense_attn_gbps": gbps("dense_attn", dense_us),
           "dense_frac_of_hbm_peak": gbps("dense_attn", dense_us) / HBM_PEAK_GBPS,
           "dense_attn_timing": f"{args.steps} back-to-back launches between two HIP events "
                                f"over {len(copies)} rotated copies",
           "dense_attn_graph_us": dense_graph_us,
           "dense_combine_us": dense_comb_us,
           "dense_combine_gbps": gbps("dense_combine", dense_comb_us),
           "splits_dense": s_dense, "dtype": spec.dtype, "group": spec.group}
    if k:
        for c in copies:
            c.meta_build()
            c.score_topk(k)
        res["meta_build_us"] = loop(lambda c: c.meta_build())
        res["score_topk_us"] = loop(lambda c: c.score_topk(k))
        res["sparse_attn_us"] = loop(lambda c: c.attention(sparse=True, num_splits=s_sp))
        res["sparse_combine_us"] = loop(lambda c: c.combine(s_sp))
        s_sel = kd.kv_auto_select_splits(copies[0].shape, k)
        # the sparse decode step as in the headline record: append + score, Top-K
        # + sparse attention, merge; and as append + score + Top-K, attention, merge
        res["sparse_decode_us"] = loop(lambda c: (c.decode_score(), c.select_attention(k, s_sel),
                                                  c.combine(s_sel)))
        res["sparse_decode_steps_per_s"] = 1e6 / res["sparse_decode_us"]
        res["sparse_decode_select_us"] = loop(lambda c: (c.decode_select(k),
                                                         c.decode(sparse=True, num_splits=s_sp)))
        res["splits_sparse"] = s_sp
        res["splits_select"] = s_sel
        res["stage_gbps"] = {name: gbps(name, res[f"{name}_us"])
                             for name in ("meta_build", "score_topk", "sparse_attn",
                                          "sparse_combine")}
    res.setdefault("stage_gbps", {})
    res["stage_gbps"]["dense_attn"] = res["dense_attn_gbps"]
    res["stage_gbps"]["dense_combine"] = res["dense_combine_gbps"]
    for c in copies:
        c.close()
    del copies
    torch.cuda.empty_cache()
    if cpu_out is not None:            # the oracle on the same arrays
        log(f"[bench] oracle on {name}")
        cpu_out[name] = oracle_steps(spec, data, CPU_STAGES[name], 3, args.cpu_seconds_other)
    return res


def run_zero_copy(args):
    """Sparse decode with K/V read directly from mapped pinned host memory."""
    import torch
    from kv_cache_decode_amd import kvdecode as kd
    from kv_cache_decode_amd import workload as wl
    from kv_cache_decode_amd.step import DeviceWorkload

    spec = wl.WORKLOADS[HOSTKV_WORKLOAD]
    data = wl.generate(spec)
    dev = torch.device("cuda:0")
    dw = DeviceWorkload(data, device=dev, host_kv=True)
    dw.meta_build()                  # the index (kmeta) is built once and lives in HBM
    k = spec.topk_blocks
    dw.score_topk(k)
    S = dw.auto_splits(sparse=True)
    for _ in range(3):
        dw.decode(sparse=True, num_splits=S)
    torch.cuda.synchronize()
    reps = args.zc_reps
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    attn_ms, comb_ms = [], []
    for _ in range(reps):
        e[0].record()
        dw.attention(sparse=True, num_splits=S)
        e[1].record()
        dw.combine(S)
        e[2].record()
        torch.cuda.synchronize()
        attn_ms.append(e[0].elapsed_time(e[1]))
        comb_ms.append(e[1].elapsed_time(e[2]))
    # dense over the host link once, for scale
    e[0].record()
    S_d = dw.attention(sparse=False)
    e[1].record()
    torch.cuda.synchronize()
    dense_ms = e[0].elapsed_time(e[1])
    # decode trajectories through the GPU block cache (delta fetch of the missing
    # blocks only) against the plain zero-copy step, on the same queries
    cache = None if args.no_variants else time_cache_trajectory(args, dw, data, k, S)
    # the same sparse step over FP8 E4M3 code pages in host memory: half the bytes
    fp8_ms = []
    if not args.no_variants:
        dw.quantize_fp8(host=True)
        for _ in range(3):
            dw.attention_fp8(sparse=True, num_splits=S)
        for _ in range(reps):
            e[0].record()
            dw.attention_fp8(sparse=True, num_splits=S)
            e[1].record()
            torch.cuda.synchronize()
            fp8_ms.append(e[0].elapsed_time(e[1]))
    # and over INT4 code pages in host memory: a quarter of the bytes
    int4_ms = []
    cache4 = None
    if not args.no_variants:
        dw.quantize_int4(host=True)
        for _ in range(3):
            dw.attention_int4(sparse=True, num_splits=S)
        for _ in range(reps):
            e[0].record()
            dw.attention_int4(sparse=True, num_splits=S)
            e[1].record()
            torch.cuda.synchronize()
            int4_ms.append(e[0].elapsed_time(e[1]))
        # the block cache over the INT4 host pages: codes and scales in the cache
        cache4 = time_cache_trajectory(args, dw, data, k, S, codes="int4")
    # KVDrive's tiering: the most recent quarter of each sequence hot in HBM (16-bit
    # pages), the rest cold INT4 pages in host memory; each selected block is read
    # from its own tier, so only the cold ones cross the link
    tier_ms, tier_split_ms, tier_link = [], [], 0
    if not args.no_variants:
        from kv_cache_decode_amd.step import storage_tensor
        tier_np = np.ones(spec.num_pages, np.uint8)
        for b in range(spec.num_seqs):
            nb = spec.blocks(b)
            tier_np[data.block_table[b, nb - nb // 4:nb]] = 0
        tier = torch.from_numpy(tier_np).to(dev)
        k_host, v_host = dw.k_cache, dw.v_cache
        dw.k_cache = storage_tensor(data.k_raw, spec.dtype).to(dev)
        dw.v_cache = storage_tensor(data.v_raw, spec.dtype).to(dev)
        for _ in range(3):
            dw.attention_tiered(True, "int4", tier, num_splits=S)
        for _ in range(reps):
            e[0].record()
            dw.attention_tiered(True, "int4", tier, num_splits=S)
            e[1].record()
            torch.cuda.synchronize()
            tier_ms.append(e[0].elapsed_time(e[1]))
        # the same as a hot launch (HBM) and a cold launch (host link) over the
        # lists split by tier
        s_hot = kd.kv_auto_num_splits(dw.shape, k // 4)
        s_cold = kd.kv_auto_num_splits(dw.shape, k - k // 4)
        for _ in range(3):
            dw.attention_tiered_split(True, "int4", tier, s_hot, s_cold)
        for _ in range(reps):
            e[0].record()
            dw.attention_tiered_split(True, "int4", tier, s_hot, s_cold)
            e[1].record()
            torch.cuda.synchronize()
            tier_split_ms.append(e[0].elapsed_time(e[1]))
        sel_np, cnt_np = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
        cold_blocks = sum(int(tier_np[data.block_table[b, n]])
                          for b in range(spec.num_seqs) for j in range(spec.num_kv_heads)
                          for n in sel_np[b, j, :cnt_np[b, j]])
        tier_link = cold_blocks * 2 * spec.block_size * spec.head_dim // 2
        del dw.k_cache, dw.v_cache
        dw.k_cache, dw.v_cache = k_host, v_host
    dw.close()

    # measured host-to-device copy bandwidth: 256 MiB from pinned memory, best of 10,
    # and a stream-read kernel over 256 MiB of mapped pinned memory, best of 10
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    best = float("inf")
    for _ in range(10):
        e[0].record()
        dst.copy_(src, non_blocking=True)
        e[1].record()
        torch.cuda.synchronize()
        best = min(best, e[0].elapsed_time(e[1]))
    h2d_gbps = n / (best * 1e-3) / 1e9
    del src, dst
    # the same bytes read by a kernel straight from mapped pinned memory
    hp, dp = kd.kv_host_alloc(n)
    try:
        sink = torch.empty(kd.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
        kd.kv_probe_stream_read(dp, n, sink)
        rd = []
        for _ in range(10):
            e[0].record()
            kd.kv_probe_stream_read(dp, n, sink)
            e[1].record()
            torch.cuda.synchronize()
            rd.append(e[0].elapsed_time(e[1]))
    finally:
        torch.cuda.synchronize()
        kd.kv_host_free(hp)
    host_read_gbps = n / (min(rd) * 1e-3) / 1e9

    eb = spec.elem_bytes
    keff = sum(min(k, spec.blocks(b)) for b in range(spec.num_seqs))
    link_bytes = keff * spec.num_kv_heads * 2 * spec.block_size * spec.head_dim * eb
    dense_link_bytes = spec.used_pages * spec.num_kv_heads * 2 * spec.block_size * spec.head_dim * eb
    attn = float(np.median(attn_ms))
    host_gbps = link_bytes / (attn * 1e-3) / 1e9
    fp8 = None
    if fp8_ms:
        f8 = float(np.median(fp8_ms))
        f8_bytes = link_bytes // eb
        fp8 = {"sparse_attn_us": f8 * 1e3, "host_link_bytes": f8_bytes,
               "host_link_gbps": f8_bytes / (f8 * 1e-3) / 1e9,
               "frac_of_h2d": f8_bytes / (f8 * 1e-3) / 1e9 / h2d_gbps,
               "speedup_vs_bf16": attn / f8}
    tiered = None
    if tier_ms:
        tm = float(np.median(tier_ms))
        tiered = {"sparse_attn_us": tm * 1e3, "hot": "most recent quarter of each sequence, 16-bit "
                  "pages in HBM", "cold": "INT4 pages in mapped host memory",
                  "host_link_bytes": tier_link,
                  "host_link_gbps": tier_link / (tm * 1e-3) / 1e9,
                  "speedup_vs_bf16": attn / tm,
                  "split_launches_us": float(np.median(tier_split_ms)) * 1e3}
    int4 = None
    if int4_ms:
        f4 = float(np.median(int4_ms))
        f4_bytes = link_bytes // (2 * eb)
        int4 = {"sparse_attn_us": f4 * 1e3, "host_link_bytes": f4_bytes,
                "host_link_gbps": f4_bytes / (f4 * 1e-3) / 1e9,
                "frac_of_h2d": f4_bytes / (f4 * 1e-3) / 1e9 / h2d_gbps,
                "speedup_vs_bf16": attn / f4}
    return {
        "block_cache": cache,
        "block_cache_int4": cache4,
        "fp8_pages": fp8,
        "int4_pages": int4,
        "tiered_int4": tiered,
        "workload": HOSTKV_WORKLOAD,
        "sparse_attn_us": attn * 1e3,
        "sparse_combine_us": float(np.median(comb_ms)) * 1e3,
        "host_link_bytes": link_bytes,
        "host_link_gbps": host_gbps,
        "dense_attn_us": dense_ms * 1e3,
        "dense_host_link_gbps": dense_link_bytes / (dense_ms * 1e-3) / 1e9,
        "h2d_memcpy_gbps": h2d_gbps,
        "frac_of_h2d": host_gbps / h2d_gbps,
        "kernel_host_read_gbps": host_read_gbps,
        "frac_of_kernel_host_read": host_gbps / host_read_gbps,
        "splits": S,
    }


CACHE_STEPS = 32
CACHE_RHO = 0.95


def time_cache_trajectory(args, dw, data, k, S, codes=None):
    """Per-step time of a CACHE_STEPS-step decode trajectory (queries: the seeded
    AR(1) walk of workload.query_trajectory, rho = CACHE_RHO), plain zero-copy
    against the GPU block cache at several capacities.  The trajectory runs once
    untimed to fill the cache (and to count the fetched blocks), then once timed.
    With ``codes`` ("fp8" / "int4", after the matching quantize_* call) both the
    plain step and the cache read the code pages in host memory."""
    import torch
    from kv_cache_decode_amd import workload as wl
    from kv_cache_decode_amd.step import storage_tensor

    spec = data.spec
    q0 = dw.q
    qs = [storage_tensor(q, spec.dtype).to(dw.device)
          for q in wl.query_trajectory(data, CACHE_STEPS, CACHE_RHO, seed=21)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(step_fn, record=None):
        torch.cuda.synchronize()
        e0.record()
        for t, q in enumerate(qs):
            dw.q = q
            step_fn()
            if record is not None:
                record.append(dw.fetch_count.clone())
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / len(qs)

    attend = {None: dw.attention, "fp8": dw.attention_fp8, "int4": dw.attention_int4}[codes]

    def plain():
        dw.score_topk(k)
        attend(sparse=True, num_splits=S)
        dw.combine(S)

    run(plain)
    res = {"steps": CACHE_STEPS, "rho": CACHE_RHO, "topk_blocks": k,
           "pages": codes or spec.dtype, "plain_zero_copy_step_us": run(plain)}
    rows = spec.block_size * spec.head_dim                              # elements of one tile
    tile = {None: 2 * rows * spec.elem_bytes, "fp8": 2 * rows + 8,       # K + V (+ scales)
            "int4": rows + 8}[codes]
    for C in (256, 512, 1024):
        dw.cache_init(C, k, codes=codes)
        counts = []
        run(lambda: dw.cache_step(k, S), counts)                        # cold start, counted
        cold = int(sum(int(c.sum()) for c in counts))
        counts = []
        run(lambda: dw.cache_step(k, S), counts)                        # warm, counted
        warm = [int(c.sum()) for c in counts]
        us = run(lambda: dw.cache_step(k, S))                           # warm, timed
        # the same warm trajectory with the fetch fused into the attention
        dw.cache_init(C, k, codes=codes)
        run(lambda: dw.cache_step(k, S, fused=True))
        run(lambda: dw.cache_step(k, S, fused=True))
        us_fused = run(lambda: dw.cache_step(k, S, fused=True))
        selected = k * spec.num_seqs * spec.num_kv_heads
        res[f"slots_{C}"] = {
            "step_us": us,
            "step_us_fused_fetch": us_fused,
            "fetched_blocks_per_step": float(np.mean(warm)),
            "hit_rate": 1.0 - float(np.mean(warm)) / selected,
            "host_link_bytes_per_step": float(np.mean(warm)) * tile,
            "cold_fetched_blocks_first_pass": cold,
        }
        del dw.cache_k, dw.cache_v, dw.cache_scales
    dw.q = q0
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- CPU baseline (oracle)

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# the stages of each named workload's oracle step (its configuration's list:
# the OPT-shaped batch is a dense configuration, the host-KV one a sparse step)
CPU_STAGES = {
    "tiny_mha_d64_1k_f32": ("meta_build", "score_topk", "sparse_attn", "dense_attn"),
    "opt6.7b_mha_b32_544_f16": ("dense_attn",),
    "llama3.1_8b_gqa_b4_32k_bf16": ("meta_build", "score_topk", "sparse_attn", "dense_attn"),
    WORKLOAD: ("meta_build", "score_topk", "sparse_attn", "dense_attn"),
    HOSTKV_WORKLOAD: ("meta_build", "score_topk", "sparse_attn"),
}


def oracle_steps(spec, data, stages, min_reps: int, budget_s: float) -> dict:
    """The fp64 oracle on the host cores: whole steps of one workload (the given
    stages in order), at least min_reps of them and more until about budget_s
    seconds have been spent; each stage timed on its own, medians reported."""
    import oracle

    q, kp, vp = data.q64(), data.k64(), data.v64()
    bt, sl = data.block_table, data.seq_lens
    bs, k = spec.block_size, spec.topk_blocks or 1
    ids, val = [], []
    for b in range(spec.num_seqs):
        for n in range(spec.blocks(b)):
            ids.append(int(bt[b, n]))
            val.append(min(bs, spec.seq_lens[b] - n * bs))
    ids, val = np.array(ids, np.int32), np.array(val, np.int32)
    scale = 1.0 / np.sqrt(spec.head_dim)
    times = {st: [] for st in stages}
    steps = []
    start = time.perf_counter()
    while len(steps) < min_reps or (time.perf_counter() - start < budget_s and len(steps) < 200):
        km = sel = cnt = None
        t_step = 0.0
        for st in stages:
            t0 = time.perf_counter()
            if st == "meta_build":
                km = oracle.block_meta(kp, ids, val)
            elif st == "score_topk":
                hs = oracle.head_scores(q, km, bt, sl, bs)
                sel, cnt = oracle.topk(oracle.group_scores(hs, spec.num_kv_heads), sl, bs, k)
            elif st == "sparse_attn":
                oracle.attention(q, kp, vp, bt, sl, scale, sel, cnt)
            else:
                oracle.attention(q, kp, vp, bt, sl, scale)
            dt = time.perf_counter() - t0
            times[st].append(dt)
            t_step += dt
        steps.append(t_step)
    t = float(np.median(steps))
    sb = stage_bytes(spec, k, 1, 1)
    step_bytes = sum(sb[st] for st in stages)
    stage_s = {st: float(np.median(v)) for st, v in times.items()}
    return {
        "stages": list(stages),
        "step_s": t,
        "steps_per_s": 1.0 / t,
        "gbps": step_bytes / t / 1e9,
        "step_bytes": step_bytes,
        "steps_timed": len(steps),
        "seconds": float(sum(steps)),
        "stage_s": stage_s,
        "stage_gbps": {st: sb[st] / v / 1e9 for st, v in stage_s.items()},
    }


def run_cpu_baseline(args, spec, data, other_cpu=None) -> dict:
    """The oracle timed on every named workload; `value` is the 128k step's GB/s
    on the same algorithmic-byte definition as the GPU figures.  other_cpu:
    figures already taken on workloads generated for the GPU legs."""
    import oracle
    from kv_cache_decode_amd import workload as wl

    per = dict(other_cpu or {})
    for name, stages in CPU_STAGES.items():
        if name in per:
            continue
        log(f"[bench] oracle on {name}")
        if name == WORKLOAD:
            per[name] = oracle_steps(spec, data, stages, args.cpu_reps, args.cpu_seconds)
        elif name == HOSTKV_WORKLOAD:
            # the same shapes as the 128k workload (only the seed differs) and the
            # oracle reads host memory either way: its step over the 128k arrays
            per[name] = oracle_steps(spec, data, stages, 3, args.cpu_seconds_other)
            per[name]["arrays"] = f"{spec.name} (same shapes)"
        else:
            other = wl.WORKLOADS[name]
            per[name] = oracle_steps(other, wl.generate(other), stages, 3, args.cpu_seconds_other)
    main = per[WORKLOAD]
    return {
        "value": main["gbps"],
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{main['steps_timed']} full steps of {spec.name} (meta build, scores, Top-K, "
                  f"sparse and dense attention; the append and the merges are not part of the "
                  f"oracle step) in fp64, {main['seconds']:.1f} s in all; median step "
                  f"{main['step_s']:.3f} s; the other workloads' steps in per_config",
        "step_s": main["step_s"],
        "steps_per_s": main["steps_per_s"],
        "stage_s": main["stage_s"],
        "stage_gbps": main["stage_gbps"],
        "per_config": per,
        "host": {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
                 "affinity": len(os.sched_getaffinity(0))},
    }


# ---------------------------------------------------------------- main

def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(3)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}), flush=True)


def codes_record(spec, f: dict, fmt: str) -> dict:
    """Code pages in HBM: per (page, KV head) unit the attention reads 2 * 16 * D
    code bytes (FP8; half that for INT4) and 8 bytes of scales instead of
    2 * 16 * D * eb."""
    D, Hkv, B, Hq = spec.head_dim, spec.num_kv_heads, spec.num_seqs, spec.num_q_heads
    k = spec.topk_blocks
    s_sparse, s_dense = f["s_sparse"], f["s_dense"]
    code_bytes = 2 * spec.block_size * D // (1 if fmt == "fp8" else 2)
    unit = code_bytes + 8
    keff = sum(min(k, spec.blocks(b)) for b in range(B))
    part = lambda S: B * Hq * S * (D + 2) * 4
    q_bytes = B * Hq * D * spec.elem_bytes
    dense_b = spec.used_pages * Hkv * (unit + 4) + q_bytes + part(s_dense)
    sparse_b = keff * Hkv * (unit + 8) + q_bytes + part(s_sparse)
    quant_b = spec.used_pages * Hkv * (2 * spec.block_size * D * spec.elem_bytes + code_bytes + 8) \
        + spec.used_pages * 8
    dense_gbps = dense_b / (f["dense_attn_us"] * 1e-6) / 1e9
    fmt_text = ("OCP FP8 E4M3, one fp32 scale per (page, KV head) and tensor" if fmt == "fp8" else
                "symmetric INT4 (scale amax/7, codes in [-7, 7], two per byte), one fp32 scale "
                "per (page, KV head) and tensor")
    return {
        "splits": {"sparse": s_sparse, "dense": s_dense},
        "format": fmt_text,
        "quantize": {"us": f["quantize_us"], "bytes": quant_b,
                     "gbps": quant_b / (f["quantize_us"] * 1e-6) / 1e9},
        "dense_attn": {"us": f["dense_attn_us"], "bytes": dense_b, "gbps": dense_gbps,
                       "frac_of_hbm_peak": dense_gbps / HBM_PEAK_GBPS},
        "sparse_attn": {"us": f["sparse_attn_us"], "bytes": sparse_b,
                        "gbps": sparse_b / (f["sparse_attn_us"] * 1e-6) / 1e9},
        "decode_step_us": {"sparse": f["decode_sparse_us"], "dense": f["decode_dense_us"]},
        "decode_steps_per_s": {"sparse": 1e6 / f["decode_sparse_us"],
                               "dense": 1e6 / f["decode_dense_us"]},
        "tiered_dense_attn": {
            "hot": "most recent quarter of each sequence, 16-bit pages",
            "cold_fraction": f["tiered_cold_fraction"], "us": f["tiered_dense_us"],
            "splits": f["tiered_splits"],
            "bytes": f["tiered_dense_bytes"],
            "gbps": f["tiered_dense_bytes"] / (f["tiered_dense_us"] * 1e-6) / 1e9,
            "split_launches_us": f["tiered_split_dense_us"],
            "split_launches_splits": f["tiered_split_splits"],
            "split_launches_gbps": f["tiered_dense_bytes"] / (f["tiered_split_dense_us"] * 1e-6)
            / 1e9},
        **({"tier_policy": f["tier_policy"]} if "tier_policy" in f else {}),
    }


def variants_record(spec, v: dict) -> dict:
    vb = variant_bytes(spec, spec.topk_blocks)
    rec = {"forced_tokens": {"sink": 4, "local": 64}}
    for name, b in vb.items():
        us = v[f"{name}_us"]
        rec[name] = {"us": us, "gbps": b / (us * 1e-6) / 1e9, "bytes": b}
    rec["decode_sparse_mean_forced"] = {"us": v["decode_sparse_mean_forced_us"],
                                        "steps_per_s": 1e6 / v["decode_sparse_mean_forced_us"]}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=12,
                    help="workload copies rotated by the timed loops and graphs")
    ap.add_argument("--zc-reps", type=int, default=5)
    ap.add_argument("--cpu-reps", type=int, default=5, help="fewest oracle steps timed")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle steps of the 128k workload are added until about this much "
                         "host time is spent")
    ap.add_argument("--cpu-seconds-other", type=float, default=4.0,
                    help="the same for each other named workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-zero-copy", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only-other-workloads", action="store_true",
                    help="run only the other named workloads (for profiling them)")
    ap.add_argument("--only-zero-copy", action="store_true",
                    help="run only the host-KV variant (for profiling it)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the variant timings (mean-key index, forced tokens, FP8 pages)")
    ap.add_argument("--only-variants", action="store_true",
                    help="run only the variant timings (for profiling them)")
    ap.add_argument("--no-long-select", action="store_true",
                    help="skip the score + Top-K timing over a 1M-token layer")
    ap.add_argument("--only-long-select", action="store_true",
                    help="run only the score + Top-K timing over a 1M-token layer")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from kv_cache_decode_amd import workload as wl

    if args.only_other_workloads:
        print(json.dumps({"other_workloads": {n: run_other_workload(args, n)
                                              for n in OTHER_WORKLOADS}}), flush=True)
        return
    if args.only_zero_copy:
        print(json.dumps({"zero_copy": run_zero_copy(args)}), flush=True)
        return
    if args.only_long_select:
        print(json.dumps({"long_select": time_long_select(args)}), flush=True)
        return
    spec = wl.WORKLOADS[WORKLOAD]
    log(f"[bench] generating {spec.name}")
    data = wl.generate(spec)
    if args.only_variants:
        args.no_variants = False
        g = run_gpu(args, spec, data)
        print(json.dumps({"selection_variants": variants_record(spec, g["variants"]),
                          "fp8_pages": codes_record(spec, g["fp8"], "fp8"),
                          "int4_pages": codes_record(spec, g["int4"], "int4")}),
              flush=True)
        return
    log("[bench] timing GPU steps")
    g = run_gpu(args, spec, data)
    sb_all = stage_bytes(spec, spec.topk_blocks, g["s_sparse"], g["s_dense"])
    sb = {s_: sb_all[s_] for s_ in ("meta_build", "sparse_attn", "sparse_combine", "dense_attn",
                                    "dense_combine")}
    sb["append_select"] = sb_all["append"] + sb_all["score_topk"]
    sb_sel = stage_bytes(spec, spec.topk_blocks, g["s_sel"], g["s_dense"])
    step_bytes = int(sum(sb.values()))
    ms = g["total_ms"] / args.steps
    st = g["stage_ms"]
    stage_us = {s: st[s] * 1e3 for s in st}
    stage_gbps = {s: sb[s] / (st[s] * 1e-3) / 1e9 for s in st}
    dense_us = g["dense_attn_loop_us"]
    dense_gbps = sb["dense_attn"] / (dense_us * 1e-6) / 1e9
    traffic = measured_traffic()

    others, other_cpu = {}, ({} if not args.no_cpu_baseline else None)
    if not args.no_other_workloads:
        for name in OTHER_WORKLOADS:
            log(f"[bench] {name}")
            others[name] = run_other_workload(args, name, other_cpu)

    long_sel = None
    if not args.no_long_select:
        log("[bench] score + Top-K over a 1M-token layer")
        long_sel = time_long_select(args)
    zc = None
    if not args.no_zero_copy:
        log("[bench] zero-copy host-KV variant")
        zc = run_zero_copy(args)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        cpu = run_cpu_baseline(args, spec, data, other_cpu)

    rec = {
        "metric": "KV GB/s streamed by decode attention (% of HBM peak) + decode steps/sec",
        "value": step_bytes / (ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "arithmetic": "K/V and q in their bf16 storage type as matrix-core operands (products "
                      "exact in fp32); fp32 sums, softmax, Quest scores and merge",
        "data": "synthetic",
        "config": {
            "workload": spec.name, "batch": spec.num_seqs, "context": spec.seq_lens[0],
            "q_heads": spec.num_q_heads, "kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim, "block_size": spec.block_size,
            "kv_storage": spec.dtype, "topk_blocks": spec.topk_blocks,
            "splits_sparse": g["s_sparse"], "splits_dense": g["s_dense"],
            "step": "meta_build(all pages) + append_select (append + score + Top-K) + sparse "
                    "attn + combine + dense attn + combine",
            "launch": g["launch"],
            "step_timing": f"all timed steps between two events, as replays of HIP graphs of "
                           f"{max(GRAPH_STEPS, args.copies)} steps cycling over the "
                           f"{args.copies} workload copies",
        },
        "eager_ms_per_step": g["eager_ms_per_step"],
        "frac_of_hbm_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        # one decode step of this layer, timed on its own as a HIP graph replay
        "decode_steps_per_s": {"sparse": 1e6 / g["decode_us"]["sparse"],
                               "dense": 1e6 / g["decode_us"]["dense"],
                               "sparse_decode_select": 1e6 / g["decode_us"]["sparse_decode_select"],
                               "sparse_unfused": 1e6 / g["decode_us"]["sparse_unfused"],
                               "full_step": 1e3 / ms},
        "decode_step_us": g["decode_us"],
        "decode_step_calls": {
            "sparse": "kv_decode_score + kv_select_decode_attn + kv_decode_combine "
                      f"({g['s_sel']} splits)",
            "sparse_decode_select": "kv_decode_select + kv_paged_decode_attn + kv_decode_combine "
                                    f"({g['s_sparse']} splits)",
            "sparse_unfused": "kv_append_token + kv_block_score_topk + kv_paged_decode_attn + "
                              "kv_decode_combine",
            "dense": "kv_append_token + kv_paged_decode_attn + kv_decode_combine"},
        "decode_step_timing": f"median per step over >= {GRAPH_MIN_REPLAYS} replays of a "
                              f"{max(GRAPH_STEPS, args.copies)}-step HIP graph over "
                              f"{args.copies} workload copies, each between its own events",
        "decode_step_gbps": {
            "sparse": (sb["append_select"] + sb_sel["sparse_attn"] + sb_sel["sparse_combine"])
                      / (g["decode_us"]["sparse"] * 1e-6) / 1e9,
            "dense": (sb_all["append"] + sb["dense_attn"] + sb["dense_combine"])
                     / (g["decode_us"]["dense"] * 1e-6) / 1e9},
        "step_bytes": step_bytes,
        "stage_bytes": sb,
        "stage_us": stage_us,
        "stage_gbps": stage_gbps,
        "roofline": {
            "kernel": "paged_attn_mfma_kernel (dense)",
            "bound": "hbm",
            "achieved": dense_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": dense_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": sb["dense_attn"],
            "avg_launch_us": dense_us,
            "timing": f"{args.steps} back-to-back launches between two HIP events",
            "avg_launch_us_graph": g["dense_attn_graph_us"],
            # measured in the same run by kernels that read and compute nothing
            "read_ceilings": g["ceilings"],
            "frac_of_stream_read": dense_gbps / g["ceilings"]["stream_read"]["gbps"],
            "frac_of_gather_read": g["ceilings"]["dense_gather_read"]["us"] / dense_us,
        },
        "selection_variants": variants_record(spec, g["variants"]) if g["variants"] else None,
        "fp8_pages": codes_record(spec, g["fp8"], "fp8") if g.get("fp8") else None,
        "int4_pages": codes_record(spec, g["int4"], "int4") if g.get("int4") else None,
        "other_workloads": others,
        "long_select": long_sel,
        "zero_copy": zc,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
