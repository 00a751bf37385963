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
