"""Decode-step append: the incremental index equals a full rebuild (GPU).

The final workload is generated, the slots of its last n tokens are replaced by
NaN, the min/max and mean indexes are built over the shorter prefix, and the n
tokens are appended one at a time through kv_append_token.  Afterwards the
pools hold the final bytes in every valid slot, the block meta equals the
oracle's meta of the final lengths and the mean rows equal the oracle's fp64
means rounded to fp32 (both bit-exact), and decode attention matches the
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import workload as wl
from parity import ROW_TOL, OracleRun, assert_rows_close, page_lists, to_f64

pytestmark = pytest.mark.gpu

NAN = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}


@pytest.mark.parametrize("dtype,D,G", [("bf16", 128, 4), ("f16", 64, 1), ("f32", 128, 2)])
def test_append_matches_full_rebuild(gpu, dtype, D, G):
    from kv_cache_decode_amd import kvdecode as kd
    from kv_cache_decode_amd.step import DeviceWorkload, storage_tensor
    n_app = 20
    final = wl.generate(wl.Workload(name="append", num_seqs=3, num_q_heads=2 * G, num_kv_heads=2,
                                    head_dim=D, seq_lens=(50, 21, 33), dtype=dtype, seed=60 + G))
    spec = final.spec
    L_final = np.array(spec.seq_lens)
    L0 = L_final - n_app
    start = wl.WorkloadData(spec=spec, q_raw=final.q_raw, k_raw=final.k_raw.copy(),
                            v_raw=final.v_raw.copy(), block_table=final.block_table,
                            seq_lens=L0.astype(np.int32), planted=final.planted)
    new_k = np.empty((n_app, spec.num_seqs, spec.num_kv_heads, D), dtype=final.k_raw.dtype)
    new_v = np.empty_like(new_k)
    for b in range(spec.num_seqs):
        for i, t in enumerate(range(L0[b], L_final[b])):
            p, s = final.block_table[b, t // 16], t % 16
            new_k[i, b] = final.k_raw[p, :, s]
            new_v[i, b] = final.v_raw[p, :, s]
            start.k_raw[p, :, s] = NAN[dtype]
            start.v_raw[p, :, s] = NAN[dtype]

    dw = DeviceWorkload(start, device=gpu)
    # index of the prefix, built for the prefix lengths
    ids, val = page_lists(start)
    kd.kv_block_meta_build(dw.shape, dw.k_cache, torch.from_numpy(ids).to(gpu),
                           torch.from_numpy(val).to(gpu), len(ids), dw.kmeta)
    kmean = torch.zeros(dw.kmeta.shape[:2] + (D,), dtype=torch.float32, device=gpu)
    kd.kv_block_mean_build(dw.shape, dw.k_cache, torch.from_numpy(ids).to(gpu),
                           torch.from_numpy(val).to(gpu), len(ids), kmean)
    lens = torch.from_numpy(L0.astype(np.int32)).to(gpu)
    for i in range(n_app):
        lens += 1
        kd.kv_append_token(dw.shape, storage_tensor(new_k[i], dtype).to(gpu),
                           storage_tensor(new_v[i], dtype).to(gpu), dw.block_table, lens,
                           dw.k_cache, dw.v_cache, dw.kmeta, kmean)
        if i in (0, 7, n_app - 1):      # the index of the current lengths, every time checked
            cur = wl.WorkloadData(spec=spec, q_raw=final.q_raw, k_raw=final.k_raw,
                                  v_raw=final.v_raw, block_table=final.block_table,
                                  seq_lens=lens.cpu().numpy(), planted=final.planted)
            cids, cval = page_lists(cur)
            ref = oracle.block_meta(final.k64(), cids, cval)
            np.testing.assert_array_equal(to_f64(dw.kmeta)[cids], ref[cids])
            ref_mean = oracle.block_mean(final.k64(), cids, cval)
            np.testing.assert_array_equal(kmean.cpu().numpy()[cids],
                                          ref_mean[cids].astype(np.float32))
    torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), L_final)

    def raw(t):
        t = t.cpu()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        return t.numpy().view(final.k_raw.dtype)

    got_k, got_v = raw(dw.k_cache), raw(dw.v_cache)
    for b in range(spec.num_seqs):
        for t in range(L_final[b]):
            p, s = final.block_table[b, t // 16], t % 16
            assert got_k[p, :, s].tobytes() == final.k_raw[p, :, s].tobytes()
            assert got_v[p, :, s].tobytes() == final.v_raw[p, :, s].tobytes()

    # decode over the appended cache equals the oracle over the final data
    dw.seq_lens.copy_(lens)
    dw.decode(sparse=False, num_splits=2)
    ref_out, _ = OracleRun(final).attention()
    assert_rows_close(to_f64(dw.out), ref_out, ROW_TOL[dtype], "decode after append")
    dw.score_topk(2)
    torch.cuda.synchronize()
    o = OracleRun(final)
    _, _, _, rsel, rcnt = oracle.sparse_step(o.q, o.k, final.block_table, final.seq_lens, 16, 2,
                                             kmeta=o.meta())
    dw.decode(sparse=True, num_splits=1)
    sel, cnt = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    ref_sp, _ = o.attention(sel, cnt)
    assert_rows_close(to_f64(dw.out), ref_sp, ROW_TOL[dtype], "sparse decode after append")


def test_append_without_meta_only_writes_the_slot(gpu):
    from kv_cache_decode_amd import kvdecode as kd
    from kv_cache_decode_amd.step import DeviceWorkload, storage_tensor
    data = wl.generate(wl.Workload(name="app2", num_seqs=2, num_q_heads=4, num_kv_heads=2,
                                   head_dim=128, seq_lens=(40, 16), dtype="bf16", seed=70))
    dw = DeviceWorkload(data, device=gpu)
    before_k = dw.k_cache.clone()
    before_v = dw.v_cache.clone()
    kn = torch.full((2, 2, 128), 3.0, dtype=torch.bfloat16, device=gpu)
    vn = torch.full((2, 2, 128), -2.0, dtype=torch.bfloat16, device=gpu)
    kd.kv_append_token(dw.shape, kn, vn, dw.block_table, dw.seq_lens, dw.k_cache, dw.v_cache, None,
                       None)
    torch.cuda.synchronize()
    changed_k = (dw.k_cache != before_k).any(dim=-1)          # [P, Hkv, 16]
    changed_v = (dw.v_cache != before_v).any(dim=-1)
    expect = torch.zeros_like(changed_k)
    for b, L in enumerate((40, 16)):
        t = L - 1
        expect[int(data.block_table[b, t // 16]), :, t % 16] = True
    assert torch.equal(changed_k, expect) and torch.equal(changed_v, expect)
