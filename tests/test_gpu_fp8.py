"""FP8 E4M3 cold pages vs the oracle (GPU), through the C ABI.

Codes and scales are compared bit for bit with the oracle's quantiser (same
fp32 decisions).  Attention over the code pages is compared with the oracle's
fp64 attention over decode(code) * scale, with the tolerances of
tests/parity.py for the query dtype.
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
    spec = wl.Workload(name=f"fp8_{seed}", num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, seq_lens=tuple(lens), dtype=dtype, seed=seed, **kw)
    return wl.generate(spec)


def device(data, gpu, **kw):
    from kv_cache_decode_amd.step import DeviceWorkload
    return DeviceWorkload(data, device=gpu, **kw)


def oracle_fp8(data):
    ids, val = page_lists(data)
    kc, ks = oracle.fp8_quantize(data.k64(), ids, val)
    vc, vs = oracle.fp8_quantize(data.v64(), ids, val)
    return kc, ks, vc, vs


def check_codes(dw, data, ref):
    kc, ks, vc, vs = ref
    torch.cuda.synchronize()
    ids, _ = page_lists(data)
    gk, gv = dw.k8_dev.cpu().numpy(), dw.v8_dev.cpu().numpy()
    gs = dw.kv_scales.cpu().numpy()
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
        self._k = oracle.fp8_dequantize(kc, ks)
        self._v = oracle.fp8_dequantize(vc, vs)


GRID = []
_seed = 5000
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        for G in (1, 2, 4, 8):
            _seed += 1
            GRID.append((dtype, D, G, _seed))


@pytest.mark.parametrize("dtype,D,G,seed", GRID, ids=[f"{d}-D{D}-G{G}" for d, D, G, _ in GRID])
def test_fp8_quantize_and_attention_grid(gpu, dtype, D, G, seed):
    """Ragged lengths (543, 1, 15, 16, 17), shuffled pages, unused pages, NaN in
    every slot past the sequence end of the source pools."""
    Hkv = 2
    data = mk(5, Hkv * G, Hkv, D, (543, 1, 15, 16, 17), dtype, seed, extra_pages=3,
              planted_frac=0.1)
    nan = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]
    for b in range(5):
        L = int(data.seq_lens[b])
        last = data.block_table[b, (L - 1) // 16]
        data.k_raw[last, :, L % 16 or 16:] = nan
        data.v_raw[last, :, L % 16 or 16:] = nan
    ref = oracle_fp8(data)
    dw = device(data, gpu)
    dw.quantize_fp8()
    ids = check_codes(dw, data, ref)
    unused = np.setdiff1d(np.arange(data.spec.num_pages), ids)
    assert unused.size >= 3
    assert np.all(dw.k8_dev.cpu().numpy()[unused] == 0)
    assert np.all(dw.kv_scales.cpu().numpy()[unused] == 0)

    o = DequantRun(data, ref)
    tol = ROW_TOL[dtype]
    ref_dense, ref_lse = o.attention()
    for S in (1, 3, 7):
        dw.decode_fp8(sparse=False, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_dense, tol, f"fp8 dense S={S}")
        assert_lse_close(to_f64(dw.lse), ref_lse, tol)
    sel, cnt = wl.random_selection(data, 6, seed=seed)
    dw.set_selection(sel, cnt)
    ref_sparse, _ = o.attention(sel, cnt)
    for S in (1, 2, 5):
        dw.decode_fp8(sparse=True, num_splits=S)
        assert_rows_close(to_f64(dw.out), ref_sparse, tol, f"fp8 sparse S={S}")


def test_fp8_tail_codes_are_ignored(gpu):
    """Code pages written by another producer may hold NaN codes (0x7F) past the
    sequence end; the attention must not read them."""
    data = mk(2, 8, 2, 128, (40, 17), "bf16", seed=5100)
    ref = oracle_fp8(data)
    dw = device(data, gpu)
    dw.quantize_fp8()
    check_codes(dw, data, ref)
    for b, L in enumerate((40, 17)):
        last = int(data.block_table[b, (L - 1) // 16])
        dw.k8_dev[last, :, L % 16:] = 0x7F
        dw.v8_dev[last, :, L % 16:] = 0x7F
    o = DequantRun(data, ref)
    ref_dense, _ = o.attention()
    dw.decode_fp8(sparse=False, num_splits=2)
    assert_rows_close(to_f64(dw.out), ref_dense, ROW_TOL["bf16"], "fp8 with NaN tails")


def test_fp8_error_against_the_unquantised_attention(gpu):
    """Quantisation error itself, as a sanity bound: E4M3 keeps 3 mantissa bits,
    so the output of the 32k GQA shape moves by a few percent at most."""
    data = mk(1, 32, 8, 128, (4096,), "bf16", seed=5200, planted_frac=0.05)
    dw = device(data, gpu)
    dw.quantize_fp8()
    dw.decode_fp8(sparse=False)
    fp8_out = to_f64(dw.out)
    ref, _ = OracleRun(data).attention()
    rel = np.linalg.norm(fp8_out - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert rel.max() < 0.1, rel.max()


@pytest.mark.parametrize("name", ["llama3.1_8b_gqa_b4_32k_bf16", "llama3.1_8b_gqa_b1_128k_bf16",
                                  "llama3.1_8b_gqa_b1_128k_bf16_hostkv",
                                  "opt6.7b_mha_b32_544_f16"])
def test_fp8_named_workload_full_size(gpu, name):
    """Full size, the benchmark's launch configuration (automatic splits); the
    host-KV workload reads its code pages from mapped pinned host memory."""
    spec = wl.WORKLOADS[name]
    print(f"\n[{name}] generating", flush=True)
    data = wl.generate(spec)
    ref = oracle_fp8(data)
    dw = device(data, gpu)
    try:
        dw.quantize_fp8()
        check_codes(dw, data, ref)
        print(f"[{name}] codes ok", flush=True)
        o = DequantRun(data, ref)
        tol = ROW_TOL[spec.dtype]
        if not spec.host_kv:
            S = dw.decode_fp8(sparse=False)
            rel = assert_rows_close(to_f64(dw.out), o.attention()[0], tol, f"{name} fp8 dense")
            print(f"[{name}] fp8 dense ok, S={S}, worst row rel-err {rel:.2e}", flush=True)
        k = spec.topk_blocks or 8
        sel, cnt = wl.random_selection(data, k, seed=7)
        dw.set_selection(sel, cnt)
        S = dw.decode_fp8(sparse=True)
        rel = assert_rows_close(to_f64(dw.out), o.attention(sel, cnt)[0], tol, f"{name} fp8 sparse")
        print(f"[{name}] fp8 sparse ok, S={S}, worst row rel-err {rel:.2e}", flush=True)
    finally:
        torch.cuda.synchronize()
        dw.close()
