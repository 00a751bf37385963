"""The quantizers over long, mostly skipped page lists (GPU), through the C ABI.

A list such as kv_tier_plan's demote rows holds a few page ids among many -1
entries.  The quantizer fetches each wave's page ids 64 units at a time, so a
list of more than 64 * (its waves) units takes several rounds; here the list
is long enough for two rounds on a 256-CU part (8 KV heads x 140000 entries),
with pages near its start, at the round boundary and at its end, each with its
own valid count.  Listed pages must carry the oracle's codes and scales bit for
bit; every other page keeps its sentinel bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import kvdecode as kd
from kv_cache_decode_amd import workload as wl

pytestmark = pytest.mark.gpu

N_IDS = 140_000                      # x 8 KV heads = 1,120,000 units > 64 * 16384
POSITIONS = (0, 5, 63, 64, 131_071, 131_072, 131_073, 139_998, 139_999)


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_quantizer_long_mostly_skipped_list(gpu, fmt):
    from kv_cache_decode_amd.step import storage_tensor
    spec = wl.Workload(name=f"qlist_{fmt}", num_seqs=1, num_q_heads=8, num_kv_heads=8,
                       head_dim=128, seq_lens=(300,), dtype="bf16", seed=7700, extra_pages=5)
    data = wl.generate(spec)
    P = spec.num_pages
    rng = np.random.default_rng(7701)
    pages = rng.choice(P, len(POSITIONS), replace=False).astype(np.int32)
    ids = np.full(N_IDS, -1, np.int32)
    ids[list(POSITIONS)] = pages
    val = np.full(N_IDS, 16, np.int32)
    val[list(POSITIONS)] = rng.integers(1, 17, len(POSITIONS))
    val[rng.integers(0, N_IDS, 1000)] = 0        # counts of skipped entries are never read

    shape = kd.make_shape(1, 8, 8, 128, spec.max_blocks, P, "bf16")
    k = storage_tensor(data.k_raw, "bf16").to(gpu)
    v = storage_tensor(data.v_raw, "bf16").to(gpu)
    row = 128 if fmt == "fp8" else 64                # code bytes per token row
    kc = torch.full((P, 8, 16, row), 0xA5, dtype=torch.uint8, device=gpu)
    vc = torch.full_like(kc, 0x5A)
    sc = torch.full((P, 8, 2), -1.0, dtype=torch.float32, device=gpu)
    g_ids = torch.from_numpy(ids).to(gpu)
    g_val = torch.from_numpy(val).to(gpu)
    call = kd.kv_quantize_pages_fp8 if fmt == "fp8" else kd.kv_quantize_pages_int4
    call(shape, k, v, g_ids, g_val, N_IDS, kc, vc, sc)
    torch.cuda.synchronize()

    quant = oracle.fp8_quantize if fmt == "fp8" else oracle.int4_quantize
    vv = val[list(POSITIONS)]
    okc, oks = quant(data.k64(), pages, vv)
    ovc, ovs = quant(data.v64(), pages, vv)
    gk, gv, gs = kc.cpu().numpy(), vc.cpu().numpy(), sc.cpu().numpy()
    np.testing.assert_array_equal(gk[pages], okc[pages])
    np.testing.assert_array_equal(gv[pages], ovc[pages])
    np.testing.assert_array_equal(gs[pages, :, 0], oks[pages])
    np.testing.assert_array_equal(gs[pages, :, 1], ovs[pages])
    others = np.setdiff1d(np.arange(P), pages)
    assert np.all(gk[others] == 0xA5) and np.all(gv[others] == 0x5A)
    assert np.all(gs[others] == -1.0)
