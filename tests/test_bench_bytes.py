"""The algorithmic byte counts the benchmark divides by (CPU only).

Each stage's bytes are recounted here from the layouts of the C header for a
small workload, element by element, so a slip in bench.py's formulas (a
missing tensor, a wrong element size, a wrong count of units) shows up.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from kv_cache_decode_amd import workload as wl  # noqa: E402


def spec():
    return wl.Workload(name="bytes", num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
                       seq_lens=(100, 33), dtype="bf16", seed=1, topk_blocks=4)


def test_stage_bytes_recount():
    sp = spec()
    B, Hq, Hkv, D, bs, eb = 2, 8, 2, 64, 16, 2
    N = [7, 3]                                   # ceil(100/16), ceil(33/16)
    maxN = 7
    pages = sum(N)
    k, S_sp, S_de = 4, 3, 5
    keff = min(k, 7) + min(k, 3)
    tile = bs * D * eb
    q = B * Hq * D * eb
    got = bench.stage_bytes(sp, k, S_sp, S_de)
    assert sp.used_pages == pages and sp.max_blocks == maxN
    # K tiles in, (min, max) rows out, the page id and valid count of every listed page
    assert got["meta_build"] == pages * Hkv * (tile + 2 * D * eb) + pages * (4 + 4)
    # new K and V rows in and stored, the page's meta rows read and written, both lengths
    assert got["append"] == B * Hkv * (2 * D * eb + 2 * D * eb + 2 * 2 * D * eb) + 2 * B * 4
    # meta rows + q + table entries + scores written and read back + the selection
    assert got["score_topk"] == (pages * Hkv * 2 * D * eb + q + pages * Hkv * 4
                                 + 2 * B * Hkv * maxN * 4 + B * Hkv * (k + 1) * 4)
    parts = lambda S: B * Hq * S * (D + 2) * 4   # o, m, l per split
    out = B * Hq * (D + 1) * 4                   # out and lse
    assert got["sparse_attn"] == keff * Hkv * 2 * tile + q + keff * Hkv * (4 + 4) + parts(S_sp)
    assert got["dense_attn"] == pages * Hkv * 2 * tile + q + pages * Hkv * 4 + parts(S_de)
    assert got["sparse_combine"] == parts(S_sp) + out
    assert got["dense_combine"] == parts(S_de) + out


def test_code_page_bytes():
    sp = spec()
    f = {"s_sparse": 3, "s_dense": 5, "quantize_us": 1.0, "dense_attn_us": 1.0,
         "sparse_attn_us": 1.0, "decode_sparse_us": 1.0, "decode_dense_us": 1.0,
         "tiered_dense_us": 1.0, "tiered_dense_bytes": 1, "tiered_cold_fraction": 0.5,
         "tiered_splits": 5, "tiered_split_dense_us": 1.0, "tiered_split_splits": [1, 4]}
    pages, Hkv, D, bs = 10, 2, 64, 16
    q = 2 * 8 * D * 2
    parts = lambda S: 2 * 8 * S * (D + 2) * 4
    for fmt, code_bytes in (("fp8", 2 * bs * D), ("int4", bs * D)):
        r = bench.codes_record(sp, f, fmt)
        # codes + 8 B of scales + the 4 B table entry per (page, KV head)
        assert r["dense_attn"]["bytes"] == pages * Hkv * (code_bytes + 8 + 4) + q + parts(5)
        assert r["sparse_attn"]["bytes"] == 7 * Hkv * (code_bytes + 8 + 8) + q + parts(3)
        # 16-bit pages in, codes and scales out, ids and counts
        assert r["quantize"]["bytes"] == pages * Hkv * (2 * bs * D * 2 + code_bytes + 8) + pages * 8


def test_tiered_bytes_recount():
    sp = spec()
    D, Hkv, bs = 64, 2, 16
    # sequence 0 lists pages 0..6, sequence 1 lists 10..12; 13..15 unlisted
    table = np.full((2, 7), -1, np.int32)
    table[0, :7] = np.arange(7)
    table[1, :3] = [10, 11, 12]
    tier = np.zeros(16, np.uint8)
    tier[[0, 1, 2, 10, 13, 14]] = 1              # 4 listed cold pages, 2 unlisted ones ignored
    S = 5
    rest = 10 * Hkv * (4 + 1) + 2 * 8 * D * 2 + 2 * 8 * S * (D + 2) * 4
    for fmt, code_row in (("fp8", D), ("int4", D // 2)):
        got, frac = bench.tiered_bytes(sp, table, tier, fmt, S)
        hot = 6 * Hkv * 2 * bs * D * 2
        cold = 4 * Hkv * (2 * bs * code_row + 8)
        assert got == hot + cold + rest
        assert frac == 0.4


def test_variant_bytes_recount():
    sp = spec()
    D, Hkv, bs, pages, maxN, k = 64, 2, 16, 10, 7, 4
    got = bench.variant_bytes(sp, k)
    rest = 2 * 8 * D * 2 + pages * Hkv * 4 + 2 * 2 * Hkv * maxN * 4 + 2 * Hkv * (k + 1) * 4
    assert got["mean_build"] == pages * Hkv * (bs * D * 2 + D * 4) + pages * 8
    assert got["meta_build"] == pages * Hkv * (bs * D * 2 + 2 * D * 2) + pages * 8
    assert got["mean_select_forced"] == pages * Hkv * D * 4 + rest
    assert got["minmax_select"] == got["minmax_select_forced"] == pages * Hkv * 2 * D * 2 + rest
