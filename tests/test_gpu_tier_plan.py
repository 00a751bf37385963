"""Hot/cold tier policy (the tiered-offload blog's page replacement with a
hysteresis cooldown; KVDrive §11) on the GPU against the oracle.

* kv_tier_plan equals the oracle's plan bit for bit (heat as fp32 bits, tiers,
  stamps, demote / promote lists and counts) over seeded multi-step
  trajectories: growing sequences, random selections, heat values and
  thresholds with exact ties, sequences of one pass and of several passes of
  the kernel, empty sequences and lists, and the 32k / 128k GQA shapes;
* the demote rows passed whole to the quantizers (negative ids skipped, full
  pages) write exactly the oracle's codes of the demoted pages and touch no
  other page, and the tiered attention over the resulting tiers matches the
  oracle over pools whose cold pages hold their decoded values.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import ROW_TOL, OracleRun, assert_rows_close, page_lists, to_f64

pytestmark = pytest.mark.gpu

BS = 16


def dev(a, gpu, dtype=np.int32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype)).to(gpu)


def random_lists(rng, lens, Hkv, K):
    """Random ascending lists; the entries past each count hold block ids too
    (and -1s), which the plan must ignore: it reads the rows whole."""
    B = len(lens)
    sel = np.full((B, Hkv, K), -1, np.int32)
    cnt = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        N = -(-int(lens[b]) // BS)
        for j in range(Hkv):
            c = int(rng.integers(0, min(K, N) + 1))
            if c:
                sel[b, j, :c] = np.sort(rng.choice(N, c, replace=False))
            if c < K:
                sel[b, j, c:] = rng.integers(-1, max(N, 1), K - c)
            cnt[b, j] = c
    return sel, cnt


def run_trajectory(gpu, B, Hkv, maxN, K, lens, steps, seed, decay, hot_above, cold_below,
                   recent, cooldown, grow=3, dyadic=False):
    from kv_cache_decode_amd import kvdecode as kd
    rng = np.random.default_rng(seed)
    P = B * maxN + 7
    bt = rng.permutation(P)[:B * maxN].astype(np.int32).reshape(B, maxN)
    if dyadic:                                        # heats on a 1/16 grid: exact ties
        heat = (rng.integers(0, 17, P) / 16).astype(np.float32)
    else:
        heat = rng.random(P).astype(np.float32)
    tier = rng.integers(0, 2, P).astype(np.uint8)
    stamp = rng.integers(-3, 3, P).astype(np.int32)
    shape = kd.make_shape(B, Hkv, Hkv, 128, maxN, P, "bf16")
    g_bt = dev(bt, gpu)
    g_heat, g_tier, g_stamp = dev(heat, gpu, np.float32), dev(tier, gpu, np.uint8), dev(stamp, gpu)
    g_dem = torch.full((B, maxN), 12345, dtype=torch.int32, device=gpu)
    g_pro = torch.full_like(g_dem, 12345)
    g_dc = torch.full((B,), -7, dtype=torch.int32, device=gpu)
    g_pc = torch.full_like(g_dc, -7)
    lens = np.array(lens, np.int64)
    moved = 0
    for step in range(1, steps + 1):
        sel, cnt = random_lists(rng, lens, Hkv, K)
        ref = oracle.tier_plan(sel, cnt, bt, lens.astype(np.int32), BS, decay, hot_above,
                               cold_below, recent, cooldown, step, heat, tier, stamp)
        kd.kv_tier_plan(shape, dev(sel, gpu), dev(cnt, gpu), K, g_bt, dev(lens, gpu), decay,
                        hot_above, cold_below, recent, cooldown, step, g_heat, g_tier, g_stamp,
                        g_dem, g_dc, g_pro, g_pc)
        torch.cuda.synchronize()
        heat, tier, stamp, dem, dc, pro, pc = ref
        np.testing.assert_array_equal(g_heat.cpu().numpy().view(np.uint32), heat.view(np.uint32),
                                      err_msg=f"heat bits, step {step}")
        for name, got, want in (("tier", g_tier, tier), ("stamp", g_stamp, stamp),
                                ("demote", g_dem, dem), ("demote_count", g_dc, dc),
                                ("promote", g_pro, pro), ("promote_count", g_pc, pc)):
            np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"{name}, step {step}")
        moved += int(dc.sum() + pc.sum())
        lens = np.minimum(lens + rng.integers(0, grow + 1, B), maxN * BS)
    return moved


CASES = [
    # B, Hkv, maxN, K, lens, decay, hot_above, cold_below, recent, cooldown, dyadic
    (3, 2, 20, 5, (37, 1, 150), 0.8, 0.55, 0.3, 1, 2, False),
    (2, 3, 40, 8, (0, 600), 0.5, 0.75, 0.25, 16, 0, True),      # empty sequence; exact ties
    (4, 8, 130, 24, (17, 2000, 1024, 2063), 0.875, 0.5, 0.125, 17, 3, True),
    (2, 4, 5000, 300, (79_000, 33_333), 0.9, 0.4, 0.2, 64, 5, False),
    (1, 2, 9000, 64, (143_990,), 0.0, 0.5, 0.5, 100, 1, False),  # decay 0; two kernel passes
    (2, 3, 20000, 700, (319_000, 150_001), 0.75, 0.5, 0.25, 40, 2, False),   # three passes
    (2, 1, 300, 300, (4800, 4791), 1.0, 0.5, 0.5, 33, 0, True),  # decay 1: heat frozen
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}-Hkv{c[1]}-N{c[2]}-K{c[3]}" for c in CASES])
def test_tier_plan_matches_oracle(gpu, case):
    B, Hkv, maxN, K, lens, decay, hot, coldb, recent, cooldown, dyadic = case
    moved = run_trajectory(gpu, B, Hkv, maxN, K, lens, 12, 7000 + maxN, decay, hot, coldb,
                           recent, cooldown, dyadic=dyadic)
    if decay < 1.0:
        assert moved > 0, "the trajectory moved no page"


@pytest.mark.parametrize("B,maxN,K", [(4, 2048, 128), (1, 8192, 256)], ids=["32k", "128k"])
def test_tier_plan_full_size(gpu, B, maxN, K):
    """The 32k (batch 4) and 128k (batch 1) GQA shapes: 8 KV heads, Top-K lists."""
    lens = (maxN * BS - 40,) * B
    moved = run_trajectory(gpu, B, 8, maxN, K, lens, 6, 7100 + maxN, 0.875, 0.5, 0.125, 64, 8,
                           grow=1)
    assert moved > 0


@pytest.mark.parametrize("cold", ["fp8", "int4"])
def test_tier_step_quantizes_exactly_the_demoted_pages(gpu, cold):
    from kv_cache_decode_amd.step import DeviceWorkload
    Hkv, G = 2, 4
    spec = wl.Workload(name="tier_step", num_seqs=3, num_q_heads=Hkv * G, num_kv_heads=Hkv,
                       head_dim=128, seq_lens=(700, 33, 1000), dtype="bf16", seed=7300,
                       extra_pages=4)
    data = wl.generate(spec)
    dw = DeviceWorkload(data, device=gpu)
    dw.quantize_fp8(host=False) if cold == "fp8" else dw.quantize_int4(host=False)
    kc, vc, sc = (dw.k8, dw.v8, dw.kv_scales) if cold == "fp8" else (dw.k4, dw.v4, dw.kv_scales4)
    ids, val = page_lists(data)
    quant = oracle.fp8_quantize if cold == "fp8" else oracle.int4_quantize
    deq = oracle.fp8_dequantize if cold == "fp8" else oracle.int4_dequantize
    okc, oks = quant(data.k64(), ids, val)
    ovc, ovs = quant(data.v64(), ids, val)
    P = spec.num_pages
    dw.tier_init(heat=0.25)
    heat = np.full(P, 0.25, np.float32)
    tier = np.zeros(P, np.uint8)
    stamp = np.zeros(P, np.int32)
    bt = data.block_table
    pol = dict(decay=0.75, hot_above=0.4, cold_below=0.2, recent_tokens=48, cooldown_steps=2)
    for step in range(1, 7):
        sel, cnt = wl.random_selection(data, 6, seed=7400 + step)
        dw.set_selection(sel, cnt)
        # sentinel code pools: only the pages demoted in this step may change
        kc.fill_(0xA5)
        vc.fill_(0x5A)
        sc.fill_(-1.0)
        dw.tier_step(step, cold, **pol)
        heat, tier, stamp, dem, dc, pro, pc = oracle.tier_plan(
            sel, cnt, bt, data.seq_lens, BS, pol["decay"], pol["hot_above"], pol["cold_below"],
            pol["recent_tokens"], pol["cooldown_steps"], step, heat, tier, stamp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(dw.page_tier.cpu().numpy(), tier)
        demoted = sorted(int(p) for b in range(spec.num_seqs) for p in dem[b, :dc[b]])
        others = np.setdiff1d(np.arange(P), demoted)
        gk, gv, gs = kc.cpu().numpy(), vc.cpu().numpy(), sc.cpu().numpy()
        np.testing.assert_array_equal(gk[demoted], okc[demoted])
        np.testing.assert_array_equal(gv[demoted], ovc[demoted])
        np.testing.assert_array_equal(gs[demoted, :, 0], oks[demoted])
        np.testing.assert_array_equal(gs[demoted, :, 1], ovs[demoted])
        assert np.all(gk[others] == 0xA5) and np.all(gv[others] == 0x5A)
        assert np.all(gs[others] == -1.0)
        assert dw.demote.cpu().numpy().tolist() == dem.tolist()
    assert int((tier != 0).sum()) > 0, "no page turned cold"
    # attention over the tiers the plan left: refill every cold page's codes
    dw.quantize_fp8(host=False) if cold == "fp8" else dw.quantize_int4(host=False)
    k, v = data.k64().copy(), data.v64().copy()
    cold_pages = np.nonzero(tier)[0]
    k[cold_pages] = deq(okc, oks)[cold_pages]
    v[cold_pages] = deq(ovc, ovs)[cold_pages]
    o = OracleRun(data)
    o._k, o._v = k, v
    ref, _ = o.attention(sel, cnt)
    dw.decode_tiered(True, cold, dw.page_tier, num_splits=3)
    assert_rows_close(to_f64(dw.out), ref, ROW_TOL["bf16"], "tiered attention after the plan")
    dw.close()
