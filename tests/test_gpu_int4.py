"""INT4 cold pages vs the oracle (GPU), through the C ABI.

Codes and scales are compared bit for bit with the oracle's quantiser (same
fp32 decisions).  Attention over the code pages is compared with the oracle's
fp64 attention over n * scale, with the tolerances of tests/parity.py for the
query dtype.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import (ROW_TOL, OracleRun, assert_lse_close, assert_rows_close, page_lists,
                    to_f64)

pytestmark = pytest.mark.gpu


def mk(B, Hq, Hkv, D, lens, dtype, seed, **kw):
    spec = wl.Workload(name=f"int4_{seed}", num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, seq_lens=tuple(lens), dtype=dtype, seed=seed, **kw)
    return wl.generate(spec)


def device(data, gpu, **kw):
    from kv_cache_decode_amd.step import DeviceWorkload
    return DeviceWorkload(data, device=gpu, **kw)


def oracle_int4(data):
    ids, val = page_lists(data)
    kc, ks = oracle.int4_quantize(data.k64(), ids, val)
    vc, vs = oracle.int4_quantize(data.v64(), ids, val)
    return kc, ks, vc, vs


def check_codes(dw, data, ref):
    kc, ks, vc, vs = ref
    torch.cuda.synchronize()
    ids, _ = page_lists(data)
    gk, gv = dw.k4_dev.cpu().numpy(), dw.v4_dev.cpu().numpy()
    gs = dw.kv_scales4.cpu().numpy()
    np.testing.assert_array_equal(gk[ids], kc[ids])
    np.testing.assert_array_equal(gv[ids], vc[ids])
    np.testing.assert_array_equal(gs[ids, :, 0], ks[ids])
    np.testing.assert_array_equal(gs[ids, :, 1], vs[ids])
    return ids


class DequantRun(OracleRun):
    """Oracle attention over the dequantised pools."""

    def __init__(self, data, ref):
        super().__init__(data)
        kc, ks, vc, vs = ref
        self._k = oracle.int4_dequantize(kc, ks)
        self._v = oracle.int4_dequantize(vc, vs)


GRID = []
_seed = 5500
for dtype in ("f16", "bf16"):
    for D in (64, 128):
        for G in (1, 2, 4, 8):
            _seed += 1
            GRID.append((dtype, D, G, _seed))


@pytest.mark.parametrize("dtype,D,G,seed", GRID, ids=[f"{d}-D{D}-G{G}" for d, D, G, _ in GRID])
def test_int4_quantize_and_attention_grid(gpu, dtype, D, G, seed):
    """Ragged lengths (543, 1, 15, 16, 17), shuffled pages, unused pages, NaN in
    every slot past the sequence end of the source pools."""
    Hkv = 2
    data = mk(5, Hkv * G, Hkv, D, (543, 1, 15, 16, 17), dtype, seed, extra_pages=3,
              planted_frac=0.1)
    nan = {"f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]
    for b in range(5):
        L = int(data.seq_lens[b])
        last = data.block_table[b, (L - 1) // 16]
        data.k_raw[last, :, L % 16 or 16:] = nan
        data.v_raw[last, :, L % 16 or 16:] = nan
    ref = oracle_int4(data)
    dw = device(data, gpu)
    dw.quantize_int4()
    ids = check_codes(dw, data, ref)
    unused = np.setdiff1d(np.arange(data.spec.num_pages), ids)
    assert unused.size >= 3
    assert np.all(dw.k4_dev.cpu().numpy()[unused] == 0)
    assert np.all(dw.kv_scales4.cpu().numpy()[unused] == 0)

    o = DequantRun(data, ref)
    tol = ROW_TOL[dtype]
    ref_dense, ref_lse = o.attention()
    for S in (1, 3, 7):
        dw.decode_int4(sparse=False, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_dense, tol, f"int4 dense S={S}")
        assert_lse_close(to_f64(dw.lse), ref_lse, tol)
    sel, cnt = wl.random_selection(data, 6, seed=seed)
    dw.set_selection(sel, cnt)
    ref_sparse, _ = o.attention(sel, cnt)
    for S in (1, 2, 5):
        dw.decode_int4(sparse=True, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_sparse, tol, f"int4 sparse S={S}")
    dw.close()


def test_int4_tail_codes_are_ignored(gpu):
    """Code pages written by another producer may hold anything past the
    sequence end (here the largest codes); the attention must not read them."""
    data = mk(2, 8, 2, 128, (40, 17), "bf16", seed=5600)
    ref = oracle_int4(data)
    dw = device(data, gpu)
    dw.quantize_int4()
    check_codes(dw, data, ref)
    for b, L in enumerate((40, 17)):
        last = int(data.block_table[b, (L - 1) // 16])
        dw.k4_dev[last, :, L % 16:] = 0x77
        dw.v4_dev[last, :, L % 16:] = 0x77
    o = DequantRun(data, ref)
    ref_dense, _ = o.attention()
    dw.decode_int4(sparse=False, num_splits=2)
    assert_rows_close(to_f64(dw.out), ref_dense, ROW_TOL["bf16"], "int4 with junk tails")
    dw.close()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("q_scale", [0.0, 1.0, 6.0])
def test_int4_one_split_long_context(gpu, dtype, q_scale):
    """32768 tokens in one split: the longest accumulation the kernel runs.
    q = 0 gives every token the same weight, so the output is the mean of V,
    a small number from a long cancelling sum (the case the bf16 offset
    bookkeeping is most exposed to); larger q spreads the logits."""
    data = mk(1, 8, 2, 128, (32768,), dtype, seed=5800 + int(q_scale), planted_frac=0.05)
    data.q_raw = wl.to_storage((data.q64() * q_scale).astype(np.float32), dtype)
    ref = oracle_int4(data)
    dw = device(data, gpu)
    try:
        dw.quantize_int4()
        check_codes(dw, data, ref)
        o = DequantRun(data, ref)
        ref_out, ref_lse = o.attention()
        worst = 0.0
        for S in (1, 3):
            dw.decode_int4(sparse=False, num_splits=S)
            rel = assert_rows_close(to_f64(dw.out), ref_out, ROW_TOL[dtype], f"int4 S={S}")
            np.testing.assert_allclose(to_f64(dw.lse), ref_lse, rtol=0, atol=1e-4)
            worst = max(worst, rel)
        print(f"\n[int4 one split {dtype} q*{q_scale}] worst row rel-err {worst:.2e}")
    finally:
        torch.cuda.synchronize()
        dw.close()


def test_int4_rejects_fp32(gpu):
    from kv_cache_decode_amd import kvdecode as kd
    data = mk(1, 2, 1, 64, (32,), "f32", seed=5650)
    dw = device(data, gpu)
    with pytest.raises(kd.KVError) as e:
        dw.quantize_int4()
    assert e.value.status == kd.KV_ERR_UNSUPPORTED
    dw.close()


def test_int4_error_against_the_unquantised_attention(gpu):
    """Quantisation error itself, as a sanity bound (15 levels per tile): the
    output of the 32k GQA shape moves by a few tens of percent at most, and
    more than FP8's."""
    data = mk(1, 32, 8, 128, (4096,), "bf16", seed=5700, planted_frac=0.05)
    dw = device(data, gpu)
    ref, _ = OracleRun(data).attention()
    dw.quantize_int4()
    dw.decode_int4(sparse=False)
    rel4 = np.linalg.norm(to_f64(dw.out) - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    dw.quantize_fp8()
    dw.decode_fp8(sparse=False)
    rel8 = np.linalg.norm(to_f64(dw.out) - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    print(f"\nworst row rel-err vs unquantised: int4 {rel4.max():.3f}, fp8 {rel8.max():.3f}")
    assert rel4.max() < 0.5 and rel8.max() < rel4.max()
    dw.close()


@pytest.mark.parametrize("name", ["llama3.1_8b_gqa_b4_32k_bf16", "llama3.1_8b_gqa_b1_128k_bf16",
                                  "llama3.1_8b_gqa_b1_128k_bf16_hostkv",
                                  "opt6.7b_mha_b32_544_f16"])
def test_int4_named_workload_full_size(gpu, name):
    """Full size, the benchmark's launch configuration (automatic splits); the
    host-KV workload reads its code pages from mapped pinned host memory."""
    spec = wl.WORKLOADS[name]
    print(f"\n[{name}] generating", flush=True)
    data = wl.generate(spec)
    ref = oracle_int4(data)
    dw = device(data, gpu)
    try:
        dw.quantize_int4()
        check_codes(dw, data, ref)
        print(f"[{name}] codes ok", flush=True)
        o = DequantRun(data, ref)
        tol = ROW_TOL[spec.dtype]
        if not spec.host_kv:
            S = dw.decode_int4(sparse=False)
            rel = assert_rows_close(to_f64(dw.out), o.attention()[0], tol, f"{name} int4 dense")
            print(f"[{name}] int4 dense ok, S={S}, worst row rel-err {rel:.2e}", flush=True)
        k = spec.topk_blocks or 8
        sel, cnt = wl.random_selection(data, k, seed=7)
        dw.set_selection(sel, cnt)
        S = dw.decode_int4(sparse=True)
        rel = assert_rows_close(to_f64(dw.out), o.attention(sel, cnt)[0], tol,
                                f"{name} int4 sparse")
        print(f"[{name}] int4 sparse ok, S={S}, worst row rel-err {rel:.2e}", flush=True)
    finally:
        torch.cuda.synchronize()
        dw.close()
