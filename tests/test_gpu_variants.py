"""Selection variants vs the oracle (GPU): the mean-key block index (KVDrive
§2.3, §4) and forced sink / local tokens (KVDrive §9.1), through the C ABI.

Mean rows are compared bit for bit with the oracle's fp64 mean rounded to fp32;
scores and selections with the tolerances stated in tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import (ROW_TOL, OracleRun, assert_rows_close, check_scores,
                    check_selection_valid_forced, check_selection_vs_oracle, forced_blocks,
                    page_lists, to_f64)

pytestmark = pytest.mark.gpu

FORCING = ((0, 0), (4, 64), (20, 1), (0, 40))


def mk(B, Hq, Hkv, D, lens, dtype, seed, **kw):
    spec = wl.Workload(name=f"var{seed}", num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, seq_lens=tuple(lens), dtype=dtype, seed=seed, **kw)
    return wl.generate(spec)


def device(data, gpu):
    from kv_cache_decode_amd.step import DeviceWorkload
    return DeviceWorkload(data, device=gpu)


def check_select(dw, data, index, k, sink, local, ref_gs, bound):
    from kv_cache_decode_amd import kvdecode as kd
    if kd.kv_max_forced_blocks(dw.shape, sink, local) > k:
        return None
    dw.select(k, index, sink, local)
    torch.cuda.synchronize()
    nb = data.num_blocks()
    check_scores(to_f64(dw.scores), ref_gs, nb, bound)
    sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    check_selection_valid_forced(sel, cnt, dw.scores.cpu().numpy(), data.seq_lens, k, sink, local)
    rsel, rcnt = oracle.select(ref_gs, data.seq_lens, 16, k, sink, local)
    check_selection_vs_oracle(sel, cnt, rsel, rcnt, ref_gs, nb,
                              bound=bound if index == "mean" else None,
                              forced=lambda b: forced_blocks(int(data.seq_lens[b]), 16, sink,
                                                             local))
    return sel, cnt


GRID = []
_seed = 3000
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        for G in (1, 4, 8):
            _seed += 1
            GRID.append((dtype, D, G, _seed))


@pytest.mark.parametrize("dtype,D,G,seed", GRID, ids=[f"{d}-D{D}-G{G}" for d, D, G, _ in GRID])
def test_mean_index_and_forced_selection_grid(gpu, dtype, D, G, seed):
    """Ragged lengths (543, 1, 15, 16, 17 tokens), shuffled pages, unused pages."""
    Hkv = 2
    data = mk(5, Hkv * G, Hkv, D, (543, 1, 15, 16, 17), dtype, seed, extra_pages=3,
              planted_frac=0.1)
    o = OracleRun(data)
    dw = device(data, gpu)
    dw.mean_build()
    dw.meta_build()
    torch.cuda.synchronize()
    ids, _ = page_lists(data)
    got = dw.kmean.cpu().numpy()
    np.testing.assert_array_equal(got[ids], o.mean()[ids].astype(np.float32))
    unused = np.setdiff1d(np.arange(data.spec.num_pages), ids)
    assert unused.size >= 3 and np.all(got[unused] == 0), "unlisted pages must stay untouched"

    ref_mean, bound_mean = o.mean_scores(), o.mean_score_bound()
    ref_mm, bound_mm = o.scores(), o.score_bound()
    for k in (1, 6, 8, 34, 40):
        for sink, local in FORCING:
            check_select(dw, data, "mean", k, sink, local, ref_mean, bound_mean)
            check_select(dw, data, "minmax", k, sink, local, ref_mm, bound_mm)

    # sparse attention over a mean-index selection with forcing
    sel, cnt = check_select(dw, data, "mean", 8, 4, 64, ref_mean, bound_mean)
    ref_sp, _ = o.attention(sel, cnt)
    for S in (1, 3):
        dw.decode(sparse=True, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_sp, ROW_TOL[dtype], f"sparse (mean) S={S}")


def test_select_minmax_unforced_is_score_topk(gpu):
    data = mk(3, 32, 8, 128, (4000, 1200, 33), "bf16", seed=3100, planted_frac=0.05)
    dw = device(data, gpu)
    dw.meta_build()
    dw.score_topk(64)
    torch.cuda.synchronize()
    a = (dw.scores.clone(), dw.sel.clone(), dw.sel_count.clone())
    dw.scores.fill_(7.0)
    dw.sel.fill_(-5)
    dw.select(64, "minmax", 0, 0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], dw.scores) and torch.equal(a[1], dw.sel)
    assert torch.equal(a[2], dw.sel_count)


@pytest.mark.parametrize("index", ["mean", "minmax"])
def test_forced_with_all_scores_equal(gpu, index):
    """q = 0 makes every score 0: the selection is the forced blocks plus the
    lowest-index others, fixed exactly by the oracle."""
    data = mk(3, 8, 2, 128, (1000, 100, 5), "bf16", seed=3200)
    data.q_raw[:] = 0
    dw = device(data, gpu)
    dw.mean_build()
    dw.meta_build()
    for k, sink, local in ((6, 4, 64), (10, 4, 64), (3, 20, 1), (40, 4, 64)):
        dw.select(k, index, sink, local)
        torch.cuda.synchronize()
        gs = np.zeros((3, 2, data.spec.max_blocks))
        rsel, rcnt = oracle.select(gs, data.seq_lens, 16, k, sink, local)
        assert np.array_equal(dw.sel.cpu().numpy(), rsel)
        assert np.array_equal(dw.sel_count.cpu().numpy(), rcnt)


def test_forced_blocks_win_against_higher_scores(gpu):
    """Blocks far above every forced block's score still cannot push a forced one out."""
    data = mk(2, 4, 1, 64, (640, 300), "f32", seed=3300, planted_frac=0.3)
    o = OracleRun(data)
    dw = device(data, gpu)
    dw.mean_build()
    k = 7
    sel, cnt = check_select(dw, data, "mean", k, 4, 64, o.mean_scores(), o.mean_score_bound())
    for b in range(2):
        fb = forced_blocks(int(data.seq_lens[b]), 16, 4, 64)
        assert fb <= set(sel[b, 0, :cnt[b, 0]].tolist())
