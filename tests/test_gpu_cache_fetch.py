"""The delta fetch fused into the cached attention (GPU), through the C ABI.

Two copies of a workload step through the same decode trajectory, one with
kv_cache_fetch(_codes) then kv_cached_decode_attn(_codes), the other with the
fused kv_cached_decode_attn_fetch(_codes).  After every step the outputs, the
log-sum-exps, the block LSEs, the slot masses, the directory and the whole
cache (pools and scales) must be equal bit for bit; the fused step's output is
also compared with the oracle's attention over the step's selection (over the
dequantised pools for code pages).  The grid covers both attention kernels
(matrix-core and VALU), 16-bit and fp32 pools, FP8 and INT4 pages, and host
memory pools.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import ROW_TOL, OracleRun, assert_rows_close, page_lists, to_f64

pytestmark = pytest.mark.gpu


def dequantised(data, codes):
    ids, val = page_lists(data)
    quant = oracle.fp8_quantize if codes == "fp8" else oracle.int4_quantize
    deq = oracle.fp8_dequantize if codes == "fp8" else oracle.int4_dequantize
    kc, ks = quant(data.k64(), ids, val)
    vc, vs = quant(data.v64(), ids, val)
    return deq(kc, ks), deq(vc, vs)


def run_pair(gpu, data, k, C, steps, rho, codes=None, host_kv=False, oracle_steps=(0, -1)):
    from kv_cache_decode_amd.step import DeviceWorkload, storage_tensor
    spec = data.spec
    pair = [DeviceWorkload(data, device=gpu, host_kv=host_kv) for _ in range(2)]
    try:
        for dw in pair:
            dw.meta_build()
            if codes == "fp8":
                dw.quantize_fp8(host=host_kv)
            elif codes == "int4":
                dw.quantize_int4(host=host_kv)
            dw.cache_init(C, k, codes=codes)
        deq = dequantised(data, codes) if codes else None
        qs = wl.query_trajectory(data, steps, rho, seed=17)
        checks = {t % steps for t in oracle_steps}
        fetched = 0
        for t, q_raw in enumerate(qs):
            for dw in pair:
                dw.q = storage_tensor(q_raw, spec.dtype).to(gpu)
            pair[0].cache_step(k)
            pair[1].cache_step(k, fused=True)
            torch.cuda.synchronize()
            a, b = pair
            fetched += int(a.fetch_count.sum())
            for name in ("out", "lse", "block_lse", "slot_mass", "sel", "sel_slots",
                         "slot_block", "block_slot", "fetch_count", "cache_k", "cache_v"):
                assert torch.equal(getattr(a, name), getattr(b, name)), f"{name} differs at step {t}"
            if codes:
                assert torch.equal(a.cache_scales, b.cache_scales), f"cache scales, step {t}"
            if t in checks:
                sel, cnt = b.sel.cpu().numpy(), b.sel_count.cpu().numpy()
                step_data = wl.WorkloadData(spec=spec, q_raw=q_raw, k_raw=data.k_raw,
                                            v_raw=data.v_raw, block_table=data.block_table,
                                            seq_lens=data.seq_lens, planted=data.planted)
                o = OracleRun(step_data)
                if deq is not None:
                    o._k, o._v = deq
                ref, _ = o.attention(sel, cnt)
                assert_rows_close(to_f64(b.out), ref, ROW_TOL[spec.dtype], f"fused step {t}")
        return fetched
    finally:
        torch.cuda.synchronize()
        for dw in pair:
            dw.close()


GRID = [(None, "bf16", 4, 128), (None, "f16", 1, 64), (None, "f32", 2, 128),
        ("fp8", "bf16", 4, 128), ("fp8", "f32", 1, 64), ("int4", "f16", 2, 128),
        ("int4", "bf16", 1, 64), ("int4", "bf16", 8, 128)]


@pytest.mark.parametrize("codes,dtype,G,D", GRID,
                         ids=[f"{c or 'plain'}-{d}-G{G}-D{D}" for c, d, G, D in GRID])
def test_fused_fetch_equals_fetch_then_attend(gpu, codes, dtype, G, D):
    spec = wl.Workload(name="fused_fetch", num_seqs=2, num_q_heads=2 * G, num_kv_heads=2,
                       head_dim=D, seq_lens=(700, 333), dtype=dtype, seed=6400 + G + D,
                       planted_frac=0.1)
    data = wl.generate(spec)
    assert run_pair(gpu, data, k=8, C=12, steps=10, rho=0.9, codes=codes) > 0


@pytest.mark.parametrize("codes", [None, "int4"])
def test_fused_fetch_host_pools(gpu, codes):
    """Pools in mapped pinned host memory: the fetched tiles cross the host link
    inside the attention launch."""
    spec = wl.Workload(name="fused_fetch_host", num_seqs=1, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, seq_lens=(16384,), dtype="bf16", seed=6500,
                       planted_frac=0.05)
    data = wl.generate(spec)
    assert run_pair(gpu, data, k=64, C=128, steps=6, rho=0.95, codes=codes, host_kv=True) > 0


def test_fused_fetch_full_size_128k(gpu):
    """The 128k host-KV shape with INT4 host pages, Top-K 256, 1024 slots."""
    spec = wl.WORKLOADS["llama3.1_8b_gqa_b1_128k_bf16_hostkv"]
    print("\n[fused fetch 128k] generating", flush=True)
    data = wl.generate(spec)
    n = run_pair(gpu, data, k=256, C=1024, steps=4, rho=0.95, codes="int4", host_kv=True,
                 oracle_steps=(-1,))
    print(f"[fused fetch 128k] {n} blocks fetched over 4 steps", flush=True)
