"""Top-K selection under adversarial score distributions (GPU).

With q one-hot on channel 0 and every key of logical block n equal to s_n on
channel 0, the Quest score of block n is exactly s_n (one nonzero product, the
other channels add exact zeros), so arbitrary score distributions reach the
selection kernel through the public call.  Scores are exact on both sides, so
the GPU list must equal the oracle's rank-count selection exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import check_selection_valid

pytestmark = pytest.mark.gpu


def scored_workload(rows, G=1, Hkv=2, seed=0, ragged=None):
    """rows: list over sequences of arrays [Hkv, N_b] of bf16-representable scores."""
    B = len(rows)
    D = 64
    lens = []
    for b, r in enumerate(rows):
        L = r.shape[1] * 16
        if ragged is not None:
            L -= ragged[b]
        lens.append(L)
    spec = wl.Workload(name="topk", num_seqs=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D,
                       seq_lens=tuple(lens), dtype="bf16", seed=seed)
    data = wl.generate(spec)
    q = np.zeros((B, Hkv * G, D), np.float32)
    q[:, :, 0] = 1.0
    data.q_raw[:] = wl.to_storage(q, "bf16")
    k32 = wl.bf16_bits_to_f32(data.k_raw).copy()
    nb = data.num_blocks()
    for b, r in enumerate(rows):
        for n in range(min(r.shape[1], nb[b])):      # blocks past the sequence have no page
            p = data.block_table[b, n]
            k32[p, :, :, 0] = r[:, n][:, None]
    data.k_raw[:] = wl.to_storage(k32, "bf16")
    return data


def run_case(gpu, rows, k, **kw):
    from kv_cache_decode_amd.step import DeviceWorkload
    data = scored_workload(rows, **kw)
    dw = DeviceWorkload(data, device=gpu)
    dw.meta_build()
    dw.score_topk(k)
    torch.cuda.synchronize()
    sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    scores = dw.scores.cpu().numpy()
    nb = data.num_blocks()
    # the scores are exact: compare them to the intended values
    for b, r in enumerate(rows):
        exp = wl.bf16_bits_to_f32(wl.to_storage(r.astype(np.float32), "bf16"))
        np.testing.assert_array_equal(scores[b, :, :nb[b]], exp[:, :nb[b]] + 0.0)
    check_selection_valid(sel, cnt, scores, nb, k)
    q64, k64 = data.q64(), data.k64()
    _, _, gs, rsel, rcnt = oracle.sparse_step(q64, k64, data.block_table, data.seq_lens, 16, k)
    np.testing.assert_array_equal(cnt, rcnt)
    np.testing.assert_array_equal(sel, rsel)
    dw.close()


@pytest.mark.parametrize("k", [1, 7, 256, 1000])
def test_heavy_ties_small_integers(gpu, k):
    rng = np.random.default_rng(k)
    rows = [rng.integers(-3, 4, size=(2, 3000)).astype(np.float32),
            rng.integers(0, 2, size=(2, 777)).astype(np.float32)]
    run_case(gpu, rows, k)


def test_all_scores_equal_and_signed_zero(gpu):
    rows = [np.full((2, 500), 5.0, np.float32),
            np.where(np.arange(1000) % 2 == 0, 0.0, -0.0).astype(np.float32).reshape(2, 500)]
    for k in (1, 33, 499, 500, 600):
        run_case(gpu, rows, k)


def test_many_binades_negatives_and_outliers(gpu):
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((2, 4096)) * np.exp(rng.uniform(-20, 20, (2, 4096)))).astype(np.float32)
    a[0, :5] = [3e38, -3e38, 1.5e-38, -1.5e-38, 0.0]
    b = rng.standard_normal((2, 2048)).astype(np.float32) * 100 + 100
    b[:, ::97] = 1e6                                       # a few planted outliers
    for k in (1, 64, 256, 2047):
        run_case(gpu, [a, b], k, ragged=[0, 5])


def test_largest_table_32768_blocks(gpu):
    rng = np.random.default_rng(4)
    rows = [rng.standard_normal((1, 32768)).astype(np.float32)]
    for k in (1, 1024, 32768):
        run_case(gpu, rows, k, Hkv=1, G=2)


@pytest.mark.parametrize("n_eq", [511, 512, 513, 1700])
def test_boundary_digit_holding_many_equal_keys(gpu, n_eq):
    """n_eq equal top scores: after the wide first pass the boundary digit holds
    n_eq keys, which the rank count resolves (up to 512) or the 8-bit passes do
    (above); with a few larger keys in front of them and a spread of smaller ones."""
    rng = np.random.default_rng(n_eq)
    n = 4000
    r = np.empty(n, np.float32)
    r[:] = rng.uniform(-4.0, 0.5, n).astype(np.float32)
    pos = rng.permutation(n)
    r[pos[:n_eq]] = 1.0
    r[pos[n_eq:n_eq + 3]] = [2.0, 3.0, 5.0]
    rows = [np.stack([r, r[::-1].copy()])]
    for k in (1, 4, 256, n_eq + 2, n_eq + 4):
        run_case(gpu, rows, k)


def test_table_65536_blocks_ties_and_forced_tokens(gpu):
    """A 1M-token context (65536 blocks of 16, one KV head; KVDrive evaluates
    1M-token windows): exact integer scores with heavy ties and random scores,
    plain Top-K and Top-K with 4 sink + 64 local tokens forced, against the
    oracle's rank count."""
    from kv_cache_decode_amd.step import DeviceWorkload
    rng = np.random.default_rng(65536)
    ties = rng.integers(-3, 4, size=(1, 65536)).astype(np.float32)
    spread = rng.standard_normal((1, 65536)).astype(np.float32)
    for rows, ks in (([ties], (2048, 65536)), ([spread], (256,))):
        data = scored_workload(rows, Hkv=1, G=2, ragged=[7])
        dw = DeviceWorkload(data, device=gpu)
        dw.meta_build()
        nb = data.num_blocks()
        gs = None
        for k in ks:
            for sink, local in ((0, 0), (4, 64)):
                dw.select(k, "minmax", sink, local)
                torch.cuda.synchronize()
                sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
                scores = dw.scores.cpu().numpy()
                exp = wl.bf16_bits_to_f32(wl.to_storage(rows[0], "bf16"))
                np.testing.assert_array_equal(scores[0, :, :nb[0]], exp[:, :nb[0]] + 0.0)
                if gs is None:
                    gs = scores.astype(np.float64)
                rsel, rcnt = oracle.select(gs, data.seq_lens, 16, k, sink, local)
                np.testing.assert_array_equal(cnt, rcnt)
                np.testing.assert_array_equal(sel[:, :, :k], rsel)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(10):
            dw.select(256, "minmax")
        t1.record()
        torch.cuda.synchronize()
        print(f"\n65536-block score + Top-K 256: {t0.elapsed_time(t1) * 100:.1f} us per call",
              flush=True)
        dw.close()
