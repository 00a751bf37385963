"""kv_block_select_no_alloc (scores in the library's own device memory) against
kv_block_select (scores in a caller buffer), through the C ABI (GPU).

Two calls in a row on one GPU, the second with a smaller input: the second
must not see the first call's scores, which stay in the shared scratch.  The
selected lists are integers, so they must be identical; the first case is
also checked against the oracle's selection.
"""
import numpy as np
import pytest
import torch

from kv_cache_decode_amd import kvdecode as kd
from kv_cache_decode_amd import workload as wl
from parity import OracleRun, check_selection_vs_oracle, forced_blocks

pytestmark = pytest.mark.gpu


def device(B, G, lens, seed, dtype="bf16", D=128, gpu=None):
    from kv_cache_decode_amd.step import DeviceWorkload
    spec = wl.Workload(name=f"noalloc{seed}", num_seqs=B, num_q_heads=2 * G, num_kv_heads=2,
                       head_dim=D, seq_lens=tuple(lens), dtype=dtype, seed=seed,
                       planted_frac=0.05)
    data = wl.generate(spec)
    dw = DeviceWorkload(data, device=gpu)
    dw.meta_build()
    dw.mean_build()
    return data, dw


def no_alloc_select(dw, k, index, sink, local):
    kind, idx = ((kd.KV_INDEX_MEAN, dw.kmean) if index == "mean" else (kd.KV_INDEX_MINMAX, dw.kmeta))
    sel = torch.full((dw.shape.num_seqs, dw.shape.num_kv_heads, k), -7, dtype=torch.int32,
                     device=dw.q.device)
    cnt = torch.full((dw.shape.num_seqs, dw.shape.num_kv_heads), -7, dtype=torch.int32,
                     device=dw.q.device)
    kd.kv_block_select_no_alloc(dw.shape, kind, dw.q, idx, dw.block_table, dw.seq_lens, k, sink,
                                local, sel, cnt)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("index,sink,local", [("minmax", 0, 0), ("minmax", 4, 64),
                                              ("mean", 4, 64)])
def test_no_alloc_select_equals_select_twice_then_smaller(gpu, index, sink, local):
    k = 40
    # a larger call first: 3 sequences of up to 9000 tokens
    data, dw = device(3, 4, (9000, 4095, 777), seed=501, gpu=gpu)
    got_sel, got_cnt = no_alloc_select(dw, k, index, sink, local)
    dw.select(k, index, sink, local)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got_cnt, dw.sel_count.cpu().numpy())
    np.testing.assert_array_equal(got_sel, dw.sel.cpu().numpy())
    o = OracleRun(data)
    import oracle
    gs = o.mean_scores() if index == "mean" else o.scores()
    rsel, rcnt = oracle.select(gs, data.seq_lens, 16, k, sink, local)
    check_selection_vs_oracle(got_sel, got_cnt, rsel, rcnt, gs, data.num_blocks(),
                              bound=o.mean_score_bound() if index == "mean" else None,
                              forced=lambda b: forced_blocks(int(data.seq_lens[b]), 16, sink, local))
    # then a smaller one (fewer sequences, a shorter table): the scratch still
    # holds the first call's scores beyond this call's rows
    data2, dw2 = device(1, 2, (1500,), seed=502, gpu=gpu)
    got2, cnt2 = no_alloc_select(dw2, 12, index, sink, local)
    dw2.select(12, index, sink, local)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cnt2, dw2.sel_count.cpu().numpy())
    np.testing.assert_array_equal(got2, dw2.sel.cpu().numpy())
    dw.close()
    dw2.close()


def test_no_alloc_select_at_the_128k_workload(gpu):
    """The 128k GQA shape (8 KV heads x 8192 blocks = 65536 scores) with Top-K 256."""
    from kv_cache_decode_amd.step import DeviceWorkload
    spec = wl.WORKLOADS["llama3.1_8b_gqa_b1_128k_bf16"]
    dw = DeviceWorkload(wl.generate(spec), device=gpu)
    dw.meta_build()
    got_sel, got_cnt = no_alloc_select(dw, spec.topk_blocks, "minmax", 0, 0)
    dw.score_topk(spec.topk_blocks)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got_cnt, dw.sel_count.cpu().numpy())
    np.testing.assert_array_equal(got_sel, dw.sel.cpu().numpy())
    dw.close()
