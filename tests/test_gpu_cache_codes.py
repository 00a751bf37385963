"""GPU block cache over FP8 / INT4 code pools (KVDrive §5.1 window with §11's
quantised cold blocks) vs the oracle (GPU), through the C ABI.

The host pool holds the oracle-checked code pages of the quantisers; the
cache holds codes and scales.  Over a decode trajectory, every step must:

* keep the plan's invariants (hits keep their slots, misses take free slots,
  then the lowest-mass unselected slots);
* hold, in each listed block's cache page, exactly the pool's code bytes and
  scale pair (the oracle's quantiser output);
* give the oracle's fp64 attention over the dequantised pools (code * scale)
  with the step's selection, within the query dtype's tolerance;
* equal bit for bit the plain code-page attention (kv_paged_decode_attn_fp8 /
  _int4) with the same list and splits: only the page addressing differs;
* give block LSEs and slot masses that match the oracle's over the dequantised
  keys, as attention weights.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import ROW_TOL, OracleRun, assert_rows_close, check_selection_valid, page_lists, to_f64
from test_gpu_cache import check_step_invariants

pytestmark = pytest.mark.gpu


def oracle_codes(data, codes):
    ids, val = page_lists(data)
    quant = oracle.fp8_quantize if codes == "fp8" else oracle.int4_quantize
    kc, ks = quant(data.k64(), ids, val)
    vc, vs = quant(data.v64(), ids, val)
    return kc, ks, vc, vs


class DequantRun(OracleRun):
    """Oracle attention over the dequantised pools."""

    def __init__(self, data, codes, ref):
        super().__init__(data)
        kc, ks, vc, vs = ref
        deq = oracle.fp8_dequantize if codes == "fp8" else oracle.int4_dequantize
        self._k = deq(kc, ks)
        self._v = deq(vc, vs)


def run_code_trajectory(gpu, data, codes, k, C, steps, rho, host_kv=False, check_every=1):
    from kv_cache_decode_amd.step import DeviceWorkload, storage_tensor
    spec = data.spec
    ref = oracle_codes(data, codes)
    kc, ks, vc, vs = ref
    dw = DeviceWorkload(data, device=gpu, host_kv=host_kv)
    try:
        dw.meta_build()
        if codes == "fp8":
            dw.quantize_fp8(host=host_kv)
            gk, gs = dw.k8_dev, dw.kv_scales
        else:
            dw.quantize_int4(host=host_kv)
            gk, gs = dw.k4_dev, dw.kv_scales4
        torch.cuda.synchronize()
        ids, _ = page_lists(data)
        np.testing.assert_array_equal(gk.cpu().numpy()[ids], kc[ids])
        np.testing.assert_array_equal(gs.cpu().numpy()[ids, :, 0], ks[ids])
        dw.cache_init(C, k, codes=codes)
        qs = wl.query_trajectory(data, steps, rho, seed=13)
        tol = ROW_TOL[spec.dtype]
        total_fetch, total_sel = 0, 0
        for t, q_raw in enumerate(qs):
            dw.q = storage_tensor(q_raw, spec.dtype).to(gpu)
            before = [x.cpu().numpy() for x in (dw.slot_block, dw.block_slot, dw.slot_mass)]
            S = dw.cache_step(k)
            torch.cuda.synchronize()
            sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
            sb, bsl, slots = dw.slot_block.cpu().numpy(), dw.block_slot.cpu().numpy(), \
                dw.sel_slots.cpu().numpy()
            fb, fs, fc = dw.fetch_block.cpu().numpy(), dw.fetch_slot.cpu().numpy(), \
                dw.fetch_count.cpu().numpy()
            check_step_invariants(sel, cnt, *before, sb, bsl, slots, fb, fs, fc)
            nb = np.array([spec.blocks(b) for b in range(spec.num_seqs)])
            check_selection_valid(sel, cnt, dw.scores.cpu().numpy(), nb, k)
            total_fetch += int(fc.sum())
            total_sel += int(cnt.sum())
            if t % check_every:
                continue
            out, lse = dw.out.clone(), dw.lse.clone()
            bl = to_f64(dw.block_lse)
            mass = to_f64(dw.slot_mass)
            # the cached pages are the pool's code pages and scale pairs
            ck, cv = dw.cache_k.cpu().numpy(), dw.cache_v.cpu().numpy()
            cs = dw.cache_scales.cpu().numpy()
            for b in range(spec.num_seqs):
                for j in range(spec.num_kv_heads):
                    for pos in range(cnt[b, j]):
                        p = data.block_table[b, sel[b, j, pos]]
                        cp = b * C + slots[b, j, pos]
                        assert ck[cp, j].tobytes() == kc[p, j].tobytes(), (t, b, j, pos)
                        assert cv[cp, j].tobytes() == vc[p, j].tobytes(), (t, b, j, pos)
                        assert cs[cp, j, 0] == ks[p, j] and cs[cp, j, 1] == vs[p, j]
            # the plain code-page attention with the same list and splits
            if codes == "fp8":
                dw.decode_fp8(True, S)
            else:
                dw.decode_int4(True, S)
            torch.cuda.synchronize()
            assert torch.equal(out, dw.out) and torch.equal(lse, dw.lse), f"step {t}"
            step_data = wl.WorkloadData(spec=spec, q_raw=q_raw, k_raw=data.k_raw, v_raw=data.v_raw,
                                        block_table=data.block_table, seq_lens=data.seq_lens,
                                        planted=data.planted)
            o = DequantRun(step_data, codes, ref)
            ref_out, ref_lse = o.attention(sel, cnt)
            assert_rows_close(to_f64(out), ref_out, tol, f"cached {codes} attention step {t}")
            ref_bl = oracle.block_lse(o.q, o.k, data.block_table, data.seq_lens, 16, o.scale, sel,
                                      cnt)
            for b in range(spec.num_seqs):
                for h in range(spec.num_q_heads):
                    c_ = cnt[b, h // spec.group]
                    w_ref = np.exp(ref_bl[b, h, :c_] - ref_lse[b, h])
                    w_got = np.exp(bl[b, h, :c_] - ref_lse[b, h])
                    np.testing.assert_allclose(w_got, w_ref, atol=tol, rtol=0)
            ref_mass = oracle.slot_mass(ref_bl, ref_lse, cnt, slots, C)
            np.testing.assert_allclose(mass, ref_mass, atol=tol, rtol=0)
        return total_fetch, total_sel
    finally:
        torch.cuda.synchronize()
        dw.close()


GRID = [("fp8", "bf16", 4, 128), ("fp8", "f16", 1, 64), ("fp8", "f32", 2, 128),
        ("int4", "bf16", 4, 128), ("int4", "f16", 2, 64), ("int4", "bf16", 1, 128),
        ("int4", "f16", 8, 128)]


@pytest.mark.parametrize("codes,dtype,G,D", GRID,
                         ids=[f"{c}-{d}-G{G}-D{D}" for c, d, G, D in GRID])
def test_code_cache_trajectory(gpu, codes, dtype, G, D):
    """Ragged lengths, a cache smaller than two lists, ten correlated queries."""
    spec = wl.Workload(name="code_cache", num_seqs=2, num_q_heads=2 * G, num_kv_heads=2,
                       head_dim=D, seq_lens=(700, 333), dtype=dtype, seed=6200 + G + D,
                       planted_frac=0.1)
    data = wl.generate(spec)
    fetched, selected = run_code_trajectory(gpu, data, codes, k=8, C=12, steps=10, rho=0.9)
    assert fetched < selected


@pytest.mark.parametrize("codes", ["fp8", "int4"])
def test_code_cache_host_kv(gpu, codes):
    """Zero-copy delta fetch of code pages from pinned host memory."""
    spec = wl.Workload(name="code_cache_host", num_seqs=1, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, seq_lens=(16384,), dtype="bf16", seed=6300,
                       planted_frac=0.05)
    data = wl.generate(spec)
    fetched, selected = run_code_trajectory(gpu, data, codes, k=64, C=128, steps=6, rho=0.95,
                                            host_kv=True)
    assert fetched < selected


def test_code_cache_full_size_128k(gpu):
    """The 128k host-KV shape: INT4 host pages, Top-K 256 through a 1024-slot cache."""
    spec = wl.WORKLOADS["llama3.1_8b_gqa_b1_128k_bf16_hostkv"]
    print("\n[code cache 128k] generating", flush=True)
    data = wl.generate(spec)
    fetched, selected = run_code_trajectory(gpu, data, "int4", k=256, C=1024, steps=4, rho=0.95,
                                            host_kv=True, check_every=3)
    print(f"[code cache 128k] fetched {fetched} of {selected} selected blocks", flush=True)
    assert fetched < selected
