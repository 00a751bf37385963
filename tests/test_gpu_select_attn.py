"""kv_select_decode_attn (Top-K + sparse attention in one launch) and
kv_decode_score (append + scores in one launch), through the C ABI (GPU).

kv_select_decode_attn must equal, bit for bit, the Top-K of kv_block_select
over the same scores followed by kv_paged_decode_attn over that list with the
same split count: the list, its count and all three partial arrays.  The merged
output is also checked against the oracle's attention over the selection.
kv_decode_score must leave the pools, the index and the scores exactly as
kv_decode_select does.
"""
import numpy as np
import pytest
import torch

from kv_cache_decode_amd import kvdecode as kd
from kv_cache_decode_amd import workload as wl
from parity import ROW_TOL, OracleRun, assert_rows_close, to_f64

pytestmark = pytest.mark.gpu


def mk(B, Hq, Hkv, D, lens, dtype, seed, **kw):
    spec = wl.Workload(name=f"sa{seed}", num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, seq_lens=tuple(lens), dtype=dtype, seed=seed, **kw)
    return wl.generate(spec)


def device(data, gpu):
    from kv_cache_decode_amd.step import DeviceWorkload
    return DeviceWorkload(data, device=gpu)


def fused_vs_separate(dw, data, k, S, sink=0, local=0, oracle_check=True):
    """Run both paths on the same scores; compare bit for bit; return the fused list."""
    dw.select(k, "minmax", sink, local)          # scores (and the reference list)
    dw.attention(sparse=True, num_splits=S)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dw.sel, dw.sel_count, *dw.partials(S))]
    dw.sel.fill_(-7)
    dw.sel_count.fill_(-7)
    for t in dw.partials(S):
        t.fill_(float("nan"))
    dw.select_attention(k, S, sink, local)
    torch.cuda.synchronize()
    got = (dw.sel, dw.sel_count, *dw.partials(S))
    for name, a, b in zip(("sel", "sel_count", "part_o", "part_m", "part_l"), got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name} differs (K={k}, S={S})"
    if oracle_check:
        dw.combine(S)
        sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
        ref_out, _ = OracleRun(data).attention(sel, cnt)
        assert_rows_close(to_f64(dw.out), ref_out, ROW_TOL[data.spec.dtype], "select+attention")


GRID = []
_seed = 7000
for dtype in ("bf16", "f16"):
    for D in (64, 128):
        for G in (2, 4, 8):
            _seed += 1
            GRID.append((dtype, D, G, _seed))


@pytest.mark.parametrize("dtype,D,G,seed", GRID, ids=[f"{d}-D{D}-G{G}" for d, D, G, _ in GRID])
def test_fused_equals_topk_then_attention(gpu, dtype, D, G, seed):
    """Ragged lengths (1, 15, 17, 543, 1300 tokens), K below and above N_b, split
    counts that are not multiples of the workgroup's four and exceed the list,
    with and without 4 + 64 forced tokens."""
    data = mk(5, 2 * G, 2, D, (1300, 1, 15, 17, 543), dtype, seed, extra_pages=2,
              planted_frac=0.1)
    dw = device(data, gpu)
    dw.meta_build()
    for k in (1, 5, 34, 90):
        for S in (1, 3, 8, 9, 17):
            fused_vs_separate(dw, data, k, S, oracle_check=(S == 9))
        if kd.kv_max_forced_blocks(dw.shape, 4, 64) <= k:
            fused_vs_separate(dw, data, k, 7, 4, 64)
    dw.close()


@pytest.mark.parametrize("dtype,G", [("f32", 2), ("bf16", 1), ("f16", 1)])
def test_shapes_outside_the_fused_kernel_run_two_launches(gpu, dtype, G):
    """fp32 keys and G = 1 are not fused: the call still equals the two launches."""
    data = mk(3, 2 * G, 2, 128, (700, 33, 1), dtype, seed=7100 + G, planted_frac=0.1)
    dw = device(data, gpu)
    dw.meta_build()
    for k, S in ((6, 2), (50, 5)):
        fused_vs_separate(dw, data, k, S)
    dw.close()


@pytest.mark.parametrize("name", ["llama3.1_8b_gqa_b4_32k_bf16", "llama3.1_8b_gqa_b1_128k_bf16"])
def test_fused_at_full_size(gpu, name):
    """The 32k workload (2048-block rows, one launch) and the 128k one (8192-block
    rows, two launches) with their Top-K, at the split counts of both auto
    rules, plain and with 4 + 64 forced tokens."""
    spec = wl.WORKLOADS[name]
    data = wl.generate(spec)
    dw = device(data, gpu)
    dw.meta_build()
    k = spec.topk_blocks
    for S in sorted({kd.kv_auto_num_splits(dw.shape, k), kd.kv_auto_select_splits(dw.shape, k)}):
        fused_vs_separate(dw, data, k, S)
        fused_vs_separate(dw, data, k, S, 4, 64, oracle_check=False)
    dw.close()


@pytest.mark.parametrize("dtype,G,index", [("bf16", 4, "minmax"), ("f16", 8, "mean"),
                                           ("f32", 2, "minmax")])
def test_decode_score_equals_decode_select(gpu, dtype, G, index):
    """Two copies append 20 tokens one by one over a prefix whose future slots
    hold NaN: one with kv_decode_select, the other with kv_decode_score; after
    every token the pools, both indexes and the scores are equal bit for bit."""
    from kv_cache_decode_amd.step import DeviceWorkload, storage_tensor
    from test_gpu_decode_select import bits, prefix_start
    final = wl.generate(wl.Workload(name="dscore", num_seqs=3, num_q_heads=2 * G, num_kv_heads=2,
                                    head_dim=128, seq_lens=(530, 47, 256), dtype=dtype,
                                    seed=7200 + G, planted_frac=0.1))
    start, new_k, new_v = prefix_start(final, 20)
    A, B = DeviceWorkload(start, device=gpu), DeviceWorkload(start, device=gpu)
    for dw in (A, B):
        dw.meta_build()
        dw.mean_build()
    for i in range(20):
        kn, vn = storage_tensor(new_k[i], dtype).to(gpu), storage_tensor(new_v[i], dtype).to(gpu)
        for dw in (A, B):
            dw.seq_lens += 1
        A.decode_select(8, index, k_new=kn, v_new=vn)
        B.scores.fill_(3.0)
        B.decode_score(index, k_new=kn, v_new=vn)
        torch.cuda.synchronize()
        for name in ("k_cache", "v_cache", "kmeta"):
            assert torch.equal(bits(getattr(A, name)), bits(getattr(B, name))), (name, i)
        assert torch.equal(A.kmean.view(torch.int32), B.kmean.view(torch.int32)), ("kmean", i)
        assert torch.equal(A.scores, B.scores), ("scores", i)
    A.close()
    B.close()


def test_fused_select_with_many_tied_candidates(gpu):
    """Exact scores where hundreds of blocks share the K-th score, so more than
    64 keys reach the rank count, which then spreads over the workgroup's waves
    (in the fused kernel's 256-thread select, more candidate blocks than
    waves).  The fused list and partials equal kv_block_select + attention bit
    for bit, and the list equals the oracle's rank count."""
    import oracle
    from kv_cache_decode_amd.step import DeviceWorkload
    from test_gpu_topk import scored_workload
    rng = np.random.default_rng(7777)
    n = 1800
    rows = []
    for h, n_tied in enumerate((300, 420)):
        r = rng.uniform(-4.0, 4.0, size=n)
        tied = rng.choice(n, n_tied, replace=False)
        r[tied] = 4.5
        rest = np.setdiff1d(np.arange(n), tied)
        r[rng.choice(rest, 200, replace=False)] = rng.uniform(5.0, 9.0, size=200)
        rows.append(r.astype(np.float32))
    data = scored_workload([np.stack(rows)], G=2, Hkv=2, seed=7778)
    dw = DeviceWorkload(data, device=gpu)
    dw.meta_build()
    for k in (256, 300, 450, 650):
        for S in (4, 8):
            fused_vs_separate(dw, data, k, S)
            gs = dw.scores.cpu().numpy().astype(np.float64)
            rsel, rcnt = oracle.select(gs, data.seq_lens, 16, k)
            np.testing.assert_array_equal(dw.sel_count.cpu().numpy(), rcnt)
            np.testing.assert_array_equal(dw.sel.cpu().numpy()[:, :, :k], rsel)
    dw.close()
