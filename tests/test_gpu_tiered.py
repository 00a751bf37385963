"""Tiered pools: hot 16-bit pages and cold FP8 / INT4 code pages in one
attention call (GPU), against the oracle's attention over pools whose cold
pages hold their decoded values (code * scale)."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import kvdecode as kd
from kv_cache_decode_amd import workload as wl
from parity import (ROW_TOL, OracleRun, assert_lse_close, assert_rows_close, page_lists,
                    to_f64)

pytestmark = pytest.mark.gpu


def mk(B, Hq, Hkv, D, lens, dtype, seed, **kw):
    spec = wl.Workload(name=f"tier_{seed}", num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, seq_lens=tuple(lens), dtype=dtype, seed=seed, **kw)
    return wl.generate(spec)


class TieredRun(OracleRun):
    """Oracle attention over pools whose cold pages are the decoded codes."""

    def __init__(self, data, cold, tier):
        super().__init__(data)
        ids, val = page_lists(data)
        quant = oracle.fp8_quantize if cold == "fp8" else oracle.int4_quantize
        deq = oracle.fp8_dequantize if cold == "fp8" else oracle.int4_dequantize
        k, v = data.k64().copy(), data.v64().copy()
        kc, ks = quant(data.k64(), ids, val)
        vc, vs = quant(data.v64(), ids, val)
        cold_pages = np.nonzero(tier)[0]
        k[cold_pages] = deq(kc, ks)[cold_pages]
        v[cold_pages] = deq(vc, vs)[cold_pages]
        self._k, self._v = k, v


GRID = []
_seed = 6000
for dtype in ("f16", "bf16"):
    for D in (64, 128):
        for G in (2, 8):
            for cold in ("fp8", "int4"):
                _seed += 1
                GRID.append((dtype, D, G, cold, _seed))


@pytest.mark.parametrize("dtype,D,G,cold,seed", GRID,
                         ids=[f"{d}-D{D}-G{G}-{c}" for d, D, G, c, _ in GRID])
def test_tiered_attention_grid(gpu, dtype, D, G, cold, seed):
    from kv_cache_decode_amd.step import DeviceWorkload
    Hkv = 2
    data = mk(5, Hkv * G, Hkv, D, (543, 1, 15, 16, 17), dtype, seed, extra_pages=3,
              planted_frac=0.1)
    dw = DeviceWorkload(data, device=gpu)
    dw.quantize_fp8(host=False) if cold == "fp8" else dw.quantize_int4(host=False)
    rng = np.random.default_rng(seed)
    tier = (rng.random(data.spec.num_pages) < 0.5).astype(np.uint8)
    tier_dev = torch.from_numpy(tier).to(gpu)
    o = TieredRun(data, cold, tier)
    tol = ROW_TOL[dtype]
    ref_dense, ref_lse = o.attention()
    for S in (1, 3, 7):
        dw.decode_tiered(False, cold, tier_dev, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_dense, tol, f"tiered dense S={S}")
        assert_lse_close(to_f64(dw.lse), ref_lse, tol)
    sel, cnt = wl.random_selection(data, 6, seed=seed)
    dw.set_selection(sel, cnt)
    ref_sparse, _ = o.attention(sel, cnt)
    for S in (1, 2, 5):
        dw.decode_tiered(True, cold, tier_dev, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_sparse, tol, f"tiered sparse S={S}")
    dw.close()


@pytest.mark.parametrize("cold", ["fp8", "int4"])
def test_all_hot_equals_the_plain_call_and_all_cold_the_oracle(gpu, cold):
    from kv_cache_decode_amd.step import DeviceWorkload
    data = mk(2, 32, 8, 128, (3000, 777), "bf16", seed=6100, planted_frac=0.05)
    dw = DeviceWorkload(data, device=gpu)
    dw.quantize_fp8(host=False) if cold == "fp8" else dw.quantize_int4(host=False)
    P = data.spec.num_pages
    hot = torch.zeros(P, dtype=torch.uint8, device=gpu)
    dw.decode(sparse=False, num_splits=24)
    plain = dw.out.clone()
    dw.decode_tiered(False, cold, hot, num_splits=24)
    assert torch.equal(dw.out, plain), "all-hot tiered call differs from the plain call"
    all_cold = np.ones(P, np.uint8)
    dw.decode_tiered(False, cold, torch.from_numpy(all_cold).to(gpu), num_splits=24)
    ref, _ = TieredRun(data, cold, all_cold).attention()
    assert_rows_close(to_f64(dw.out), ref, ROW_TOL["bf16"], "all cold")
    dw.close()


def test_tiered_cold_pages_in_host_memory(gpu):
    """The 128k host-KV shape at reduced length: cold INT4 pages read over the host link."""
    from kv_cache_decode_amd.step import DeviceWorkload
    data = mk(1, 32, 8, 128, (16384,), "bf16", seed=6200, planted_frac=0.05)
    dw = DeviceWorkload(data, device=gpu)
    dw.quantize_int4(host=True)
    rng = np.random.default_rng(1)
    tier = (rng.random(data.spec.num_pages) < 0.9).astype(np.uint8)
    o = TieredRun(data, "int4", tier)
    sel, cnt = wl.random_selection(data, 64, seed=2)
    dw.set_selection(sel, cnt)
    dw.decode_tiered(True, "int4", torch.from_numpy(tier).to(gpu))
    assert_rows_close(to_f64(dw.out), o.attention(sel, cnt)[0], ROW_TOL["bf16"], "host cold")
    dw.close()


def test_tiered_rejects_unsupported_shapes(gpu):
    from kv_cache_decode_amd.step import DeviceWorkload
    for dtype, G in (("f32", 4), ("bf16", 1)):
        data = mk(1, 2 * G, 2, 64, (64,), dtype, seed=6300)
        dw = DeviceWorkload(data, device=gpu)
        tier = torch.zeros(data.spec.num_pages, dtype=torch.uint8, device=gpu)
        with pytest.raises(kd.KVError) as e:
            kd.kv_paged_decode_attn_tiered(dw.shape, dw.q, dw.k_cache, dw.v_cache, dw.k_cache,
                                           dw.v_cache, dw.kmeta, kd.KV_COLD_INT4, tier,
                                           dw.block_table, dw.seq_lens, None, None, 0, 0.1, 1,
                                           *dw.partials(1))
        assert e.value.status == kd.KV_ERR_UNSUPPORTED
        dw.close()


SPLIT_GRID = [("bf16", 128, 4, "int4", 6401), ("f16", 64, 2, "fp8", 6402),
              ("bf16", 64, 8, "fp8", 6403), ("f16", 128, 1, "int4", 6404),
              ("f32", 128, 2, "fp8", 6405), ("f32", 64, 1, "fp8", 6406)]


@pytest.mark.parametrize("dtype,D,G,cold,seed", SPLIT_GRID,
                         ids=[f"{d}-D{D}-G{G}-{c}" for d, D, G, c, _ in SPLIT_GRID])
def test_tiered_split_launches(gpu, dtype, D, G, cold, seed):
    """kv_paged_decode_attn_tiered_split: hot and cold lists as two launches,
    merged over hot + cold splits, against the oracle over the decoded pools;
    both kernels (G = 1 and fp32 run the VALU kernel), dense and selected
    lists, split counts from 1 to more than a list holds, all-hot and
    all-cold tiers (one launch then has only empty splits)."""
    from kv_cache_decode_amd.step import DeviceWorkload
    Hkv = 2
    data = mk(5, Hkv * G, Hkv, D, (543, 1, 15, 16, 17), dtype, seed, extra_pages=3,
              planted_frac=0.1)
    dw = DeviceWorkload(data, device=gpu)
    try:
        dw.quantize_fp8(host=False) if cold == "fp8" else dw.quantize_int4(host=False)
        rng = np.random.default_rng(seed)
        P = data.spec.num_pages
        tol = ROW_TOL[dtype]
        sel, cnt = wl.random_selection(data, 6, seed=seed)
        for tier in ((rng.random(P) < 0.5).astype(np.uint8), np.zeros(P, np.uint8),
                     np.ones(P, np.uint8)):
            tier_dev = torch.from_numpy(tier).to(gpu)
            o = TieredRun(data, cold, tier)
            ref_dense, ref_lse = o.attention()
            for sh, sc in ((1, 1), (2, 5), (7, 3)):
                S = dw.attention_tiered_split(False, cold, tier_dev, sh, sc)
                dw.combine(S)
                assert_rows_close(to_f64(dw.out), ref_dense, tol, f"split dense {sh}+{sc}")
                assert_lse_close(to_f64(dw.lse), ref_lse, tol)
            dw.set_selection(sel, cnt)
            ref_sparse, _ = o.attention(sel, cnt)
            for sh, sc in ((1, 1), (3, 2)):
                S = dw.attention_tiered_split(True, cold, tier_dev, sh, sc)
                dw.combine(S)
                assert_rows_close(to_f64(dw.out), ref_sparse, tol, f"split sparse {sh}+{sc}")
    finally:
        torch.cuda.synchronize()
        dw.close()


def test_tiered_split_full_size_128k(gpu):
    """The 128k GQA shape, a quarter hot, INT4 cold pages: split launches against
    the oracle (dense, automatic split counts)."""
    from kv_cache_decode_amd.step import DeviceWorkload
    spec = wl.WORKLOADS["llama3.1_8b_gqa_b1_128k_bf16"]
    print("\n[tiered split 128k] generating", flush=True)
    data = wl.generate(spec)
    dw = DeviceWorkload(data, device=gpu)
    try:
        dw.quantize_int4(host=False)
        tier = np.ones(spec.num_pages, np.uint8)
        nb = spec.blocks(0)
        tier[data.block_table[0, nb - nb // 4:nb]] = 0
        sh = kd.kv_auto_num_splits(dw.shape, nb // 4)
        sc = kd.kv_auto_num_splits_fp8(dw.shape, nb - nb // 4)
        S = dw.attention_tiered_split(False, "int4", torch.from_numpy(tier).to(gpu), sh, sc)
        dw.combine(S)
        rel = assert_rows_close(to_f64(dw.out), TieredRun(data, "int4", tier).attention()[0],
                                ROW_TOL["bf16"], "tiered split 128k")
        print(f"[tiered split 128k] {sh} + {sc} splits, worst row rel-err {rel:.2e}", flush=True)
    finally:
        torch.cuda.synchronize()
        dw.close()
