"""A decode step captured in a HIP graph replays to the eager result (GPU).

The step is captured once, then replayed several times with eager work and
synchronisations between the replays; every replay must reproduce the eager
outputs bit for bit (the kernels are deterministic and record no memset).
"""
import numpy as np
import pytest
import torch

from kv_cache_decode_amd import workload as wl

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu):
    from kv_cache_decode_amd.step import DeviceWorkload
    spec = wl.Workload(name="graph", num_seqs=2, num_q_heads=16, num_kv_heads=4, head_dim=128,
                       seq_lens=(3000, 1111), dtype="bf16", seed=31, planted_frac=0.05)
    data = wl.generate(spec)
    dw = DeviceWorkload(data, device=gpu)
    k = 24
    S_sp = 16
    S_de = 12

    def step():
        dw.meta_build()
        dw.score_topk(k)
        dw.attention(sparse=True, num_splits=S_sp)
        dw.combine(S_sp)
        sparse_out.copy_(dw.out)
        dw.attention(sparse=False, num_splits=S_de)
        dw.combine(S_de)

    sparse_out = torch.empty_like(dw.out)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (dw.kmeta, dw.scores, dw.sel, dw.sel_count, sparse_out, dw.out,
                                 dw.lse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (dw.kmeta, dw.scores, dw.out, dw.lse, sparse_out):
            t.zero_()                       # eager work between replays
        dw.sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (dw.kmeta, dw.scores, dw.sel, dw.sel_count, sparse_out, dw.out, dw.lse)
        for a, b in zip(got, eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"replay {rep}"


def test_cache_steps_in_a_graph_match_eager(gpu):
    """A decode trajectory through the GPU block cache (select, plan, fetch,
    attention over the cache, merge, slot masses), one graph per step's query:
    replaying the graphs from the same starting directory reproduces the eager
    trajectory bit for bit (outputs, directory, masses, cache pools)."""
    from kv_cache_decode_amd.step import DeviceWorkload, storage_tensor
    spec = wl.Workload(name="graph_cache", num_seqs=2, num_q_heads=16, num_kv_heads=4,
                       head_dim=128, seq_lens=(3000, 1111), dtype="bf16", seed=32,
                       planted_frac=0.05)
    data = wl.generate(spec)
    dw = DeviceWorkload(data, device=gpu)
    dw.meta_build()
    k, C, S = 16, 24, 4
    dw.cache_init(C, k)
    qs = [storage_tensor(q, "bf16").to(gpu) for q in wl.query_trajectory(data, 5, 0.9, seed=3)]
    q_buf = torch.empty_like(qs[0])
    dw.q = q_buf

    def reset():
        dw.slot_block.fill_(-1)
        dw.block_slot.fill_(-1)
        dw.slot_mass.zero_()
        dw.cache_k.zero_()
        dw.cache_v.zero_()

    def snapshot():
        return [t.clone() for t in (dw.out, dw.lse, dw.sel, dw.slot_block, dw.block_slot,
                                    dw.slot_mass, dw.fetch_count, dw.cache_k.view(torch.int16))]

    reset()
    eager = []
    for q in qs:
        q_buf.copy_(q)
        dw.cache_step(k, S)
        torch.cuda.synchronize()
        eager.append(snapshot())
    # warm up on a side stream, then capture one step reading q_buf
    reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dw.cache_step(k, S)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dw.cache_step(k, S)
    for rep in range(2):
        reset()
        torch.cuda.synchronize()
        for t, q in enumerate(qs):
            q_buf.copy_(q)
            g.replay()
            torch.cuda.synchronize()
            for a, b in zip(snapshot(), eager[t]):
                assert torch.equal(a, b), f"replay pass {rep} step {t}"
