"""Seeded random shapes through the whole step vs the oracle (GPU).

Twenty cases drawn from a fixed seed, away from the hand-picked grids: odd KV
head counts, one to six sequences of random lengths (1 to 3000 tokens, so
partial last pages and one-page sequences occur), unused pages, random Top-K
budgets (including budgets above a sequence's block count), random split
counts (including more splits than blocks), both indexes and random forced
sink / local tokens.  Each case checks the meta (bit for bit), the scores,
the selection (against the oracle's, inside the tie band, and as a valid
Top-K of the GPU's own scores), dense attention and sparse attention over the
GPU's selection.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import (ROW_TOL, OracleRun, assert_lse_close, assert_rows_close, check_scores,
                    check_selection_valid_forced, check_selection_vs_oracle, forced_blocks,
                    to_f64)

pytestmark = pytest.mark.gpu


def draw_cases(n=20, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["f32", "f16", "bf16"][rng.integers(3)]
        D = [64, 128][rng.integers(2)]
        G = [1, 2, 4, 8][rng.integers(4)]
        Hkv = int(rng.integers(1, 4))
        B = int(rng.integers(1, 7))
        lens = tuple(int(x) for x in rng.integers(1, 3001, size=B))
        k = int(rng.integers(1, 70))
        S = int(rng.integers(1, 41))
        mean = bool(rng.integers(2))
        sink = int(rng.choice([0, 4, 20]))
        local = int(rng.choice([0, 1, 64]))
        extra = int(rng.integers(0, 5))
        cases.append((i, dtype, D, G, Hkv, lens, k, S, mean, sink, local, extra))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_shape(gpu, case):
    from kv_cache_decode_amd import kvdecode as kd
    from kv_cache_decode_amd.step import DeviceWorkload
    i, dtype, D, G, Hkv, lens, k, S, mean, sink, local, extra = case
    spec = wl.Workload(name=f"rand{i}", num_seqs=len(lens), num_q_heads=G * Hkv,
                       num_kv_heads=Hkv, head_dim=D, seq_lens=lens, dtype=dtype,
                       seed=7000 + i, planted_frac=0.05, extra_pages=extra)
    data = wl.generate(spec)
    o = OracleRun(data)
    dw = DeviceWorkload(data, device=gpu)
    try:
        nb = data.num_blocks()
        tol = ROW_TOL[dtype]
        dw.meta_build()
        ref_meta = o.meta()
        got_meta = to_f64(dw.kmeta)
        for b in range(spec.num_seqs):
            pages = data.block_table[b, :nb[b]]
            np.testing.assert_array_equal(got_meta[pages], ref_meta[pages])

        if kd.kv_max_forced_blocks(dw.shape, sink, local) > k:
            sink = local = 0                        # the budget cannot hold the forced blocks
        index = "mean" if mean else "minmax"
        if mean:
            dw.mean_build()
            ref_gs, bound = o.mean_scores(), o.mean_score_bound()
        else:
            ref_gs, bound = o.scores(), o.score_bound()
        if not mean and sink == 0 and local == 0:
            dw.score_topk(k)
        else:
            dw.select(k, index, sink, local)
        torch.cuda.synchronize()
        check_scores(to_f64(dw.scores), ref_gs, nb, bound)
        sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
        check_selection_valid_forced(sel, cnt, dw.scores.cpu().numpy(), data.seq_lens, k, sink,
                                     local)
        rsel, rcnt = oracle.select(ref_gs, data.seq_lens, 16, k, sink, local)
        check_selection_vs_oracle(sel, cnt, rsel, rcnt, ref_gs, nb,
                                  bound=bound if mean else None,
                                  forced=lambda b: forced_blocks(int(data.seq_lens[b]), 16, sink,
                                                                 local))

        ref_dense, ref_lse = o.attention()
        dw.decode(sparse=False, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_dense, tol, f"dense S={S}")
        assert_lse_close(to_f64(dw.lse), ref_lse, tol)
        ref_sparse, _ = o.attention(sel, cnt)
        dw.decode(sparse=True, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_sparse, tol, f"sparse S={S}")
    finally:
        torch.cuda.synchronize()
        dw.close()
