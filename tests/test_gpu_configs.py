"""The five named workloads at full size vs the oracle (GPU).

Same launch configuration as the benchmark (automatic split count).  The oracle
computes every output of these sizes in seconds on the host cores, so every
row is compared, not a sample.
"""
import numpy as np
import pytest
import torch

from kv_cache_decode_amd import workload as wl
from parity import (ROW_TOL, OracleRun, assert_lse_close, assert_rows_close, check_scores,
                    check_selection_valid, check_selection_vs_oracle, to_f64)

pytestmark = pytest.mark.gpu


def _dw(data, gpu):
    from kv_cache_decode_amd.step import DeviceWorkload
    return DeviceWorkload(data, device=gpu)


@pytest.mark.parametrize("name", wl.WORKLOAD_ORDER)
def test_named_workload_full_size(gpu, name):
    spec = wl.WORKLOADS[name]
    print(f"\n[{name}] generating", flush=True)
    data = wl.generate(spec)
    o = OracleRun(data)
    dw = _dw(data, gpu)
    tol = ROW_TOL[spec.dtype]
    nb = data.num_blocks()
    try:
        print(f"[{name}] dense", flush=True)
        S = dw.decode(sparse=False)
        ref, ref_lse = o.attention()
        rel = assert_rows_close(to_f64(dw.out), ref, tol, f"{name} dense S={S}")
        assert_lse_close(to_f64(dw.lse), ref_lse, tol)
        print(f"[{name}] dense ok, S={S}, worst row rel-err {rel:.2e}", flush=True)
        if spec.topk_blocks is None:
            return
        k = spec.topk_blocks
        dw.meta_build()
        dw.score_topk(k)
        torch.cuda.synchronize()
        pages = np.concatenate([data.block_table[b, :nb[b]] for b in range(spec.num_seqs)])
        np.testing.assert_array_equal(to_f64(dw.kmeta)[pages], o.meta()[pages])
        ref_gs = o.scores()
        check_scores(to_f64(dw.scores), ref_gs, nb, o.score_bound())
        sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
        check_selection_valid(sel, cnt, dw.scores.cpu().numpy(), nb, k)
        rsel, rcnt = o.topk(k, ref_gs)
        ndiff = check_selection_vs_oracle(sel, cnt, rsel, rcnt, ref_gs, nb)
        print(f"[{name}] selection ok ({ndiff} rows differ inside the tie band)", flush=True)
        # sparse attention over the GPU's own selection vs the oracle over the same list
        S = dw.decode(sparse=True)
        ref_sp, _ = o.attention(sel, cnt)
        rel = assert_rows_close(to_f64(dw.out), ref_sp, tol, f"{name} sparse S={S}")
        print(f"[{name}] sparse ok, S={S}, worst row rel-err {rel:.2e}", flush=True)
        if ndiff == 0:
            ref_full, _ = o.attention(rsel, rcnt)
            assert_rows_close(to_f64(dw.out), ref_full, tol, f"{name} sparse vs oracle step")
    finally:
        torch.cuda.synchronize()
        dw.close()


VARIANT_WORKLOADS = [n for n in wl.WORKLOAD_ORDER
                     if wl.WORKLOADS[n].topk_blocks is not None and not wl.WORKLOADS[n].host_kv]


@pytest.mark.parametrize("name", VARIANT_WORKLOADS)
def test_named_workload_mean_index_forced(gpu, name):
    """Mean-key index with the first 4 and last 64 tokens forced in, full size."""
    import oracle
    from parity import check_selection_valid_forced, forced_blocks
    spec = wl.WORKLOADS[name]
    print(f"\n[{name}] generating", flush=True)
    data = wl.generate(spec)
    o = OracleRun(data)
    dw = _dw(data, gpu)
    nb = data.num_blocks()
    k = spec.topk_blocks
    try:
        dw.mean_build()
        dw.select(k, "mean", 4, 64)
        torch.cuda.synchronize()
        pages = np.concatenate([data.block_table[b, :nb[b]] for b in range(spec.num_seqs)])
        np.testing.assert_array_equal(dw.kmean.cpu().numpy()[pages],
                                      o.mean()[pages].astype(np.float32))
        ref_gs, bound = o.mean_scores(), o.mean_score_bound()
        check_scores(to_f64(dw.scores), ref_gs, nb, bound)
        sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
        check_selection_valid_forced(sel, cnt, dw.scores.cpu().numpy(), data.seq_lens, k, 4, 64)
        rsel, rcnt = oracle.select(ref_gs, data.seq_lens, 16, k, 4, 64)
        ndiff = check_selection_vs_oracle(
            sel, cnt, rsel, rcnt, ref_gs, nb, bound=bound,
            forced=lambda b: forced_blocks(int(data.seq_lens[b]), 16, 4, 64))
        print(f"[{name}] mean selection ok ({ndiff} rows differ inside the band)", flush=True)
        S = dw.decode(sparse=True)
        ref_sp, _ = o.attention(sel, cnt)
        rel = assert_rows_close(to_f64(dw.out), ref_sp, ROW_TOL[spec.dtype], f"{name} mean sparse")
        print(f"[{name}] mean sparse ok, S={S}, worst row rel-err {rel:.2e}", flush=True)
    finally:
        torch.cuda.synchronize()
        dw.close()
