"""The two-level select of long rows (more than 16384 blocks) vs the one-level
select and the oracle (GPU), through the C ABI.

With a workspace of kv_score_topk_workspace_size bytes a long row's Top-K runs
in two launches (each 4096-block chunk's forced blocks and best K competing
blocks, then the select among them); without it, one workgroup per row
selects.  Both must give the same lists bit for bit, equal to the oracle's
rank count: exact scores with heavy ties across chunk boundaries, random
scores, forced sink and local tokens, ragged lengths (the last chunk partly
past the sequence), K from 1 to the largest the two-level path takes, through
kv_block_select, kv_block_score_topk, kv_decode_select and
kv_block_select_no_alloc.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import kvdecode as kd
from kv_cache_decode_amd import workload as wl
from test_gpu_topk import scored_workload

pytestmark = pytest.mark.gpu


def lists(dw):
    torch.cuda.synchronize()
    return dw.sel.cpu().numpy().copy(), dw.sel_count.cpu().numpy().copy()


def check_oracle(dw, data, sel, cnt, k, sink, local):
    gs = dw.scores.cpu().numpy().astype(np.float64)
    rsel, rcnt = oracle.select(gs, data.seq_lens, 16, k, sink, local)
    np.testing.assert_array_equal(cnt, rcnt)
    np.testing.assert_array_equal(sel[:, :, :k], rsel)


@pytest.mark.parametrize("nblocks,ragged,kind", [(65536, 7, "ties"), (65536, 0, "spread"),
                                                 (32768, 1000, "ties"), (20000, 9, "spread")],
                         ids=["1M-ties", "1M-spread", "512k-ragged-ties", "20000-blocks"])
def test_two_level_equals_one_level_and_oracle(gpu, nblocks, ragged, kind):
    from kv_cache_decode_amd.step import DeviceWorkload
    rng = np.random.default_rng(nblocks + ragged)
    if kind == "ties":      # small integers: long runs of equal scores in every chunk
        rows = [rng.integers(-3, 4, size=(1, nblocks)).astype(np.float32)]
    else:
        rows = [rng.standard_normal((1, nblocks)).astype(np.float32)]
    data = scored_workload(rows, Hkv=1, G=2, ragged=[ragged * 16 + 5])
    dw = DeviceWorkload(data, device=gpu)
    dw.meta_build()
    maxn = int(data.num_blocks().max())
    nch = -(-maxn // 4096)
    kmax = 16384 // (2 * nch)
    for k in sorted({1, 37, 256, kmax}):
        assert kd.kv_score_topk_workspace_size(dw.shape, k) > 4 * maxn   # candidates included
        for sink, local in ((0, 0), (4, 64), (20, 1)):
            if kd.kv_max_forced_blocks(dw.shape, sink, local) > k:
                continue
            dw.select(k, "minmax", sink, local)
            one = lists(dw)
            dw.select(k, "minmax", sink, local, workspace=True)
            two = lists(dw)
            np.testing.assert_array_equal(two[0], one[0], err_msg=f"K={k} sink={sink} local={local}")
            np.testing.assert_array_equal(two[1], one[1])
            if k == 256 or (k == kmax and kmax < 256):   # the rank count is O(N^2): one K
                check_oracle(dw, data, *two, k, sink, local)
    # the same through kv_block_score_topk with the scores in the workspace only
    k = 256 if kmax >= 256 else kmax
    dw.select(k, "minmax")
    one = lists(dw)
    need = kd.kv_score_topk_workspace_size(dw.shape, k)
    ws = torch.empty(need, dtype=torch.uint8, device=gpu)
    kd.kv_block_score_topk(dw.shape, dw.q, dw.kmeta, dw.block_table, dw.seq_lens, k, None, dw.sel,
                           dw.sel_count, ws, need)
    two = lists(dw)
    np.testing.assert_array_equal(two[0], one[0])
    np.testing.assert_array_equal(two[1], one[1])
    dw.close()


def test_two_level_decode_select_and_no_alloc(gpu):
    """kv_decode_select (append + select) and kv_block_select_no_alloc take the
    two-level path too (the no-alloc call keeps its candidates after its
    scores in the library's array); lists as the one-level select's."""
    from kv_cache_decode_amd.step import DeviceWorkload
    rng = np.random.default_rng(4242)
    rows = [rng.integers(-2, 3, size=(2, 32768)).astype(np.float32),
            rng.standard_normal((2, 32768)).astype(np.float32)]
    data = scored_workload(rows, Hkv=2, G=1, ragged=[3, 4000])
    dw = DeviceWorkload(data, device=gpu)
    dw.meta_build()
    for k, (sink, local) in ((128, (0, 0)), (256, (4, 64))):
        dw.select(k, "minmax", sink, local)
        one = lists(dw)
        dw.decode_select(k, "minmax", sink, local, workspace=True)
        two = lists(dw)
        np.testing.assert_array_equal(two[0], one[0])
        np.testing.assert_array_equal(two[1], one[1])
        kd.kv_block_select_no_alloc(dw.shape, kd.KV_INDEX_MINMAX, dw.q, dw.kmeta, dw.block_table,
                                    dw.seq_lens, k, sink, local, dw.sel, dw.sel_count)
        three = lists(dw)
        np.testing.assert_array_equal(three[0], one[0])
        np.testing.assert_array_equal(three[1], one[1])
        check_oracle(dw, data, *three, k, sink, local)
    dw.close()
