"""Pins of the fp64 oracle against things other than itself (no GPU).

Each oracle function is checked against at least one of: a hand-derived golden
fixture (tests/golden), a library routine (numpy reductions, Python's sort,
torch's scaled_dot_product_attention, scipy's softmax / logsumexp), brute force
on tiny inputs (box corners, subset enumeration), closed-form special cases and
invariants of the method.  The pins are chosen so that a plausible slip in the
oracle (a swapped min/max, a dropped scale, a wrong head map, a reversed tie
rule, an off-by-one token mask, K used for V, a dropped l in the merge) fails
at least one of them; tests/test_oracle_mutants.py plants exactly those slips.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from kv_cache_decode_amd import workload as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quest_tiny.json")


def mk(B=2, Hq=4, Hkv=2, D=8, lens=(37, 16), dtype="f32", seed=0, **kw):
    spec = wl.Workload(name="pin", num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       seq_lens=tuple(lens), dtype=dtype, seed=seed, **kw)
    return wl.generate(spec)


def page_lists(data):
    """All (page id, valid tokens) pairs referenced by the block table."""
    spec = data.spec
    ids, val = [], []
    for b in range(spec.num_seqs):
        for n in range(spec.blocks(b)):
            ids.append(int(data.block_table[b, n]))
            val.append(min(spec.block_size, spec.seq_lens[b] - n * spec.block_size))
    return np.array(ids, np.int32), np.array(val, np.int32)


def gather(pool, data, b, j, blocks):
    """Valid token rows of (sequence b, KV head j) over the logical ``blocks``, in order."""
    spec = data.spec
    bs, L = spec.block_size, spec.seq_lens[b]
    rows = []
    for n in blocks:
        p = data.block_table[b, n]
        nv = min(bs, L - n * bs)
        rows.append(pool[p, j, :nv, :])
    return np.concatenate(rows, axis=0)


def sdpa(qv, K, V, scale):
    """torch's fused attention in float64 on the CPU for one query row."""
    q = torch.from_numpy(np.asarray(qv, np.float64)).reshape(1, 1, 1, -1)
    k = torch.from_numpy(np.ascontiguousarray(K, np.float64))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(V, np.float64))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    return out.reshape(-1).numpy()


def full_meta(data):
    ids, val = page_lists(data)
    return oracle.block_meta(data.k64(), ids, val)


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- O1 block meta

def test_meta_golden(golden):
    g = golden["meta_score"]
    k = np.array(g["k_slots"], np.float64).reshape(1, 1, g["block_size"], g["head_dim"])
    km = oracle.block_meta(k, [0], [g["valid_tokens"]])
    assert km[0, 0, 0].tolist() == g["kmin"]
    assert km[0, 0, 1].tolist() == g["kmax"]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_meta_matches_numpy_reduction(dtype):
    data = mk(B=3, Hq=6, Hkv=3, D=16, lens=(45, 16, 3), dtype=dtype, seed=11, extra_pages=2)
    k64 = data.k64()
    ids, val = page_lists(data)
    km = oracle.block_meta(k64, ids, val)
    for p, nv in zip(ids, val):
        np.testing.assert_array_equal(km[p, :, 0], k64[p, :, :nv].min(axis=1))
        np.testing.assert_array_equal(km[p, :, 1], k64[p, :, :nv].max(axis=1))


def test_meta_brackets_and_attains_every_valid_key():
    data = mk(B=2, Hq=2, Hkv=2, D=8, lens=(50, 7), seed=12)
    k64 = data.k64()
    ids, val = page_lists(data)
    km = oracle.block_meta(k64, ids, val)
    for p, nv in zip(ids, val):
        ks = k64[p, :, :nv]                          # [Hkv, nv, D]
        assert np.all(km[p, :, 0][:, None] <= ks) and np.all(ks <= km[p, :, 1][:, None])
        assert np.all(np.any(ks == km[p, :, 0][:, None], axis=1))
        assert np.all(np.any(ks == km[p, :, 1][:, None], axis=1))


# ---------------------------------------------------------------- O2 / O3 scores

def test_score_golden(golden):
    g = golden["meta_score"]
    kmeta = np.array([[[g["kmin"], g["kmax"]]]], np.float64)          # [1, 1, 2, D]
    for qv, want, tok_max in zip(g["queries"], g["scores"], g["token_max_dot"]):
        q = np.array(qv, np.float64).reshape(1, 1, -1)
        s = oracle.head_scores(q, kmeta, np.zeros((1, 1), np.int32), np.array([3], np.int32),
                               g["block_size"])
        assert s[0, 0, 0] == want
        assert s[0, 0, 0] >= tok_max


def test_score_is_support_function_of_the_key_box():
    """Brute force: the Quest score equals max over the 2^D corners of the
    [kmin, kmax] box of q . x -- the largest q . k any key inside the block's
    bounding box can reach.  D = 6 keeps the enumeration at 64 corners."""
    data = mk(B=2, Hq=4, Hkv=2, D=6, lens=(40, 21), seed=13)
    q64 = data.q64()
    km = full_meta(data)
    hs = oracle.head_scores(q64, km, data.block_table, data.seq_lens, 16)
    G = data.spec.group
    corners = np.array(list(itertools.product([0, 1], repeat=6)))         # [64, 6]
    for b in range(2):
        for h in range(4):
            j = h // G
            for n in range(data.spec.blocks(b)):
                p = data.block_table[b, n]
                box = np.where(corners == 0, km[p, j, 0], km[p, j, 1])   # [64, 6]
                want = max(float(np.dot(q64[b, h], x)) for x in box)
                assert hs[b, h, n] == pytest.approx(want, rel=1e-13, abs=1e-13)


def test_score_upper_bounds_every_token_dot():
    data = mk(B=2, Hq=8, Hkv=2, D=16, lens=(70, 33), dtype="bf16", seed=14)
    q64, k64 = data.q64(), data.k64()
    km = full_meta(data)
    hs = oracle.head_scores(q64, km, data.block_table, data.seq_lens, 16)
    gs = oracle.group_scores(hs, 2)
    G = data.spec.group
    for b in range(2):
        for j in range(2):
            for n in range(data.spec.blocks(b)):
                K = gather(k64, data, b, j, [n])
                dots = q64[b, j * G:(j + 1) * G] @ K.T                  # [G, tokens]
                for g in range(G):
                    assert hs[b, j * G + g, n] >= dots[g].max() - 1e-12
                assert gs[b, j, n] >= dots.max() - 1e-12


def test_score_block_size_one_is_the_dot_product():
    data = mk(B=1, Hq=2, Hkv=1, D=16, lens=(9,), block_size=1, seed=15)
    q64, k64 = data.q64(), data.k64()
    ids, val = page_lists(data)
    km = oracle.block_meta(k64, ids, val)
    hs = oracle.head_scores(q64, km, data.block_table, data.seq_lens, 1)
    for h in range(2):
        for n in range(9):
            p = data.block_table[0, n]
            assert hs[0, h, n] == pytest.approx(float(q64[0, h] @ k64[p, 0, 0]), rel=1e-13)


def test_score_shift_adds_q_dot_u():
    """K += u for every key shifts kmin and kmax by u, so every score moves by q . u."""
    data = mk(B=1, Hq=2, Hkv=1, D=8, lens=(64,), seed=16)
    q64, k64 = data.q64(), data.k64()
    ids, val = page_lists(data)
    u = np.linspace(-1.5, 2.0, 8)
    hs0 = oracle.head_scores(q64, oracle.block_meta(k64, ids, val), data.block_table,
                             data.seq_lens, 16)
    hs1 = oracle.head_scores(q64, oracle.block_meta(k64 + u, ids, val), data.block_table,
                             data.seq_lens, 16)
    for h in range(2):
        np.testing.assert_allclose(hs1[0, h], hs0[0, h] + q64[0, h] @ u, rtol=1e-12, atol=1e-12)


def test_score_is_minus_inf_past_the_sequence():
    data = mk(B=2, Hq=2, Hkv=1, D=8, lens=(50, 17), seed=17)
    hs = oracle.head_scores(data.q64(), full_meta(data), data.block_table, data.seq_lens, 16)
    assert np.all(np.isneginf(hs[1, :, 2:]))
    assert np.all(np.isfinite(hs[1, :, :2]))


def test_group_score_is_max_over_the_group_and_reduces_for_g1():
    data = mk(B=2, Hq=8, Hkv=2, D=8, lens=(48, 20), seed=18)
    hs = oracle.head_scores(data.q64(), full_meta(data), data.block_table, data.seq_lens, 16)
    gs = oracle.group_scores(hs, 2)
    np.testing.assert_array_equal(gs, hs.reshape(2, 2, 4, -1).max(axis=2))
    gs1 = oracle.group_scores(hs, 8)
    np.testing.assert_array_equal(gs1, hs)



def test_group_score_is_the_groups_support_function_by_corner_enumeration():
    """Brute force, independent of the per-head formula: the group score is the
    largest q_h . x over the group's heads h and over every corner x of the
    block's [kmin, kmax] box, computed as one library matrix product per block
    (heads x corners).  With the box taken from numpy's min and max over the
    block's valid key rows, no part of the oracle enters the expected value."""
    data = mk(B=2, Hq=8, Hkv=2, D=6, lens=(45, 18), seed=61)
    q64, k64 = data.q64(), data.k64()
    hs = oracle.head_scores(q64, full_meta(data), data.block_table, data.seq_lens, 16)
    gs = oracle.group_scores(hs, 2)                                            # 2 KV heads
    corners = np.array(list(itertools.product([0, 1], repeat=6)), bool)       # [64, 6]
    for b in range(2):
        L = data.spec.seq_lens[b]
        for j in range(2):
            for n in range(data.spec.blocks(b)):
                rows = k64[data.block_table[b, n], j, :min(16, L - 16 * n)]    # valid keys
                box = np.where(corners, rows.max(axis=0), rows.min(axis=0))    # [64, 6]
                want = float((q64[b, 4 * j:4 * j + 4] @ box.T).max())
                assert gs[b, j, n] == pytest.approx(want, rel=1e-13, abs=1e-13)

def test_scores_invariant_under_page_permutation():
    data = mk(B=2, Hq=4, Hkv=2, D=8, lens=(40, 30), seed=19)
    hs0 = oracle.head_scores(data.q64(), full_meta(data), data.block_table, data.seq_lens, 16)
    rng = np.random.default_rng(5)
    P = data.spec.num_pages
    perm = rng.permutation(P)                    # new page of old page p is perm[p]
    k_new = np.empty_like(data.k_raw)
    k_new[perm] = data.k_raw
    data2 = wl.WorkloadData(spec=data.spec, q_raw=data.q_raw, k_raw=k_new, v_raw=data.v_raw,
                            block_table=perm[data.block_table].astype(np.int32),
                            seq_lens=data.seq_lens, planted=data.planted)
    hs1 = oracle.head_scores(data2.q64(), full_meta(data2), data2.block_table, data2.seq_lens, 16)
    np.testing.assert_array_equal(hs0, hs1)


# ---------------------------------------------------------------- O4 Top-K

def test_topk_golden(golden):
    g = golden["topk"]
    s = np.array(g["scores"], np.float64).reshape(1, 1, -1)
    for case in g["cases"]:
        sel, cnt = oracle.topk(s, np.array([6 * 16], np.int32), 16, case["k"])
        want = case["selected"]
        assert cnt[0, 0] == len(want)
        assert sel[0, 0, :len(want)].tolist() == want
        assert np.all(sel[0, 0, len(want):] == -1)


def _sorted_topk(scores, k):
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    return sorted(order[:k])


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_a_library_sort_with_heavy_ties(seed):
    rng = np.random.default_rng(100 + seed)
    B, Hkv = 3, 2
    lens = rng.integers(1, 40 * 16, size=B).astype(np.int32)
    maxN = int(max(-(-lens // 16)))
    gs = rng.integers(-4, 5, size=(B, Hkv, maxN)).astype(np.float64)   # many ties
    for k in (1, 3, 7, 50):
        sel, cnt = oracle.topk(gs, lens, 16, k)
        for b in range(B):
            nb = -(-int(lens[b]) // 16)
            for j in range(Hkv):
                want = _sorted_topk(list(gs[b, j, :nb]), k)
                assert cnt[b, j] == len(want) == min(k, nb)
                assert sel[b, j, :cnt[b, j]].tolist() == want
                assert np.all(sel[b, j, cnt[b, j]:] == -1)


def test_topk_is_the_best_subset_by_enumeration():
    """Brute force: among all K-subsets, the selection has the largest score sum,
    and among the subsets with that sum it is the lexicographically smallest
    (lower indices win ties).  Integer scores keep the sums exact."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(1, 10))
        scores = rng.integers(-3, 4, size=n).astype(np.float64)
        for k in range(1, n + 1):
            best = max(itertools.combinations(range(n), k),
                       key=lambda c: (sum(scores[list(c)]), [-i for i in c]))
            sel, cnt = oracle.topk(scores.reshape(1, 1, n), np.array([n * 16], np.int32), 16, k)
            assert sel[0, 0, :cnt[0, 0]].tolist() == list(best)


def test_topk_duplicate_page_tie_goes_to_lower_block():
    data = mk(B=1, Hq=1, Hkv=1, D=8, lens=(64,), seed=20)
    bt = data.block_table.copy()
    bt[0, 3] = bt[0, 1]                              # blocks 1 and 3 read the same page
    q64 = data.q64()
    km = full_meta(data)
    hs = oracle.head_scores(q64, km, bt, data.seq_lens, 16)
    gs = oracle.group_scores(hs, 1)
    assert gs[0, 0, 1] == gs[0, 0, 3]
    # K such that exactly one of the twins fits: rank of the tied value
    rank = int(np.sum(gs[0, 0, :4] > gs[0, 0, 1]))
    sel, cnt = oracle.topk(gs, data.seq_lens, 16, rank + 1)
    chosen = set(sel[0, 0, :cnt[0, 0]].tolist())
    assert 1 in chosen and 3 not in chosen


def test_topk_k_at_least_n_keeps_all_blocks():
    gs = np.random.default_rng(3).standard_normal((1, 2, 5))
    sel, cnt = oracle.topk(gs, np.array([70], np.int32), 16, 9)
    assert cnt.tolist() == [[5, 5]]
    assert sel[0, 0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1, -1]


# ---------------------------------------------------------------- O5 attention

def test_attention_golden(golden):
    g = golden["attention"]
    q = np.array(g["q"], np.float64).reshape(1, 1, -1)
    k = np.array(g["k"], np.float64).reshape(1, 1, 2, 2)
    v = np.array(g["v"], np.float64).reshape(1, 1, 2, 2)
    out, lse = oracle.attention(q, k, v, np.zeros((1, 1), np.int32), np.array([2], np.int32),
                                g["scale"])
    np.testing.assert_allclose(out[0, 0], g["out"], rtol=1e-14, atol=1e-14)
    assert lse[0, 0] == pytest.approx(g["lse"], rel=1e-14)


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f32", 4, 2), ("f16", 3, 3), ("bf16", 8, 2)])
def test_dense_attention_matches_torch_sdpa(dtype, Hq, Hkv):
    data = mk(B=3, Hq=Hq, Hkv=Hkv, D=16, lens=(70, 16, 5), dtype=dtype, seed=21)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    scale = 1 / math.sqrt(16)
    out, lse = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, scale)
    G = data.spec.group
    for b in range(3):
        blocks = range(data.spec.blocks(b))
        for h in range(Hq):
            K = gather(k64, data, b, h // G, blocks)
            V = gather(v64, data, b, h // G, blocks)
            np.testing.assert_allclose(out[b, h], sdpa(q64[b, h], K, V, scale),
                                       rtol=1e-12, atol=1e-14)
            z = scale * (K @ q64[b, h])
            assert lse[b, h] == pytest.approx(scipy.special.logsumexp(z), rel=1e-13)


def test_sparse_attention_matches_softmax_over_selected_tokens():
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(150, 91), dtype="bf16", seed=22)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    sel, cnt = wl.random_selection(data, 4, seed=3)
    scale = 0.3
    out, _ = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, scale, sel, cnt)
    G = data.spec.group
    for b in range(2):
        for h in range(4):
            j = h // G
            blocks = sel[b, j, :cnt[b, j]]
            K = gather(k64, data, b, j, blocks)
            V = gather(v64, data, b, j, blocks)
            w = scipy.special.softmax(scale * (K @ q64[b, h]))
            np.testing.assert_allclose(out[b, h], w @ V, rtol=1e-12, atol=1e-14)


def test_attention_single_token_returns_its_value():
    data = mk(B=1, Hq=2, Hkv=1, D=8, lens=(1,), seed=23)
    out, lse = oracle.attention(data.q64(), data.k64(), data.v64(), data.block_table,
                                data.seq_lens, 0.5)
    p = data.block_table[0, 0]
    for h in range(2):
        np.testing.assert_array_equal(out[0, h], data.v64()[p, 0, 0])
        assert lse[0, h] == pytest.approx(0.5 * data.q64()[0, h] @ data.k64()[p, 0, 0], rel=1e-14)


def test_attention_equal_keys_give_the_mean_value():
    data = mk(B=1, Hq=1, Hkv=1, D=8, lens=(29,), seed=24)
    k = data.k64()
    k[:] = k[0, 0, 0]                                 # every key identical
    out, lse = oracle.attention(data.q64(), k, data.v64(), data.block_table, data.seq_lens, 0.7)
    V = gather(data.v64(), data, 0, 0, range(2))
    np.testing.assert_allclose(out[0, 0], V.mean(axis=0), rtol=1e-13, atol=1e-15)
    z0 = 0.7 * data.q64()[0, 0] @ k[0, 0, 0]
    assert lse[0, 0] == pytest.approx(z0 + math.log(29), rel=1e-13)


def test_attention_dominant_logit_returns_that_value():
    data = mk(B=1, Hq=1, Hkv=1, D=8, lens=(40,), seed=25)
    q = np.zeros((1, 1, 8)); q[0, 0, 0] = 1.0
    k = np.zeros_like(data.k64())
    p = data.block_table[0, 1]
    k[p, 0, 5, 0] = 60.0                               # token 21 dominates by e^60
    out, _ = oracle.attention(q, k, data.v64(), data.block_table, data.seq_lens, 1.0)
    np.testing.assert_allclose(out[0, 0], data.v64()[p, 0, 5], rtol=1e-20, atol=1e-23)


def test_attention_invariant_under_a_common_key_shift():
    data = mk(B=2, Hq=4, Hkv=2, D=8, lens=(55, 30), seed=26)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    u = np.linspace(2.0, -1.0, 8)
    o0, _ = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, 0.35)
    o1, _ = oracle.attention(q64, k64 + u, v64, data.block_table, data.seq_lens, 0.35)
    np.testing.assert_allclose(o1, o0, rtol=1e-11, atol=1e-13)


def test_attention_invariant_under_page_permutation():
    data = mk(B=2, Hq=2, Hkv=2, D=8, lens=(45, 17), seed=27, extra_pages=3)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    o0, l0 = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, 0.35)
    perm = np.random.default_rng(1).permutation(data.spec.num_pages)
    k2, v2 = np.empty_like(k64), np.empty_like(v64)
    k2[perm], v2[perm] = k64, v64
    o1, l1 = oracle.attention(q64, k2, v2, perm[data.block_table].astype(np.int32),
                              data.seq_lens, 0.35)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_topk_all_blocks_equals_dense():
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(83, 40), dtype="bf16", seed=28)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    _, _, _, sel, cnt = oracle.sparse_step(q64, k64, data.block_table, data.seq_lens, 16,
                                           k=data.spec.max_blocks)
    od, ld = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, 0.25)
    os_, ls = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, 0.25, sel, cnt)
    np.testing.assert_array_equal(od, os_)
    np.testing.assert_array_equal(ld, ls)


def test_mha_is_gqa_with_one_head_per_group():
    """G=1: each query head attends only to its own KV head, so running head h
    alone (as a 1-head problem) gives the same row."""
    data = mk(B=1, Hq=3, Hkv=3, D=8, lens=(35,), seed=29)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    full, _ = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, 0.4)
    for h in range(3):
        one, _ = oracle.attention(q64[:, h:h + 1], k64[:, h:h + 1], v64[:, h:h + 1],
                                  data.block_table, data.seq_lens, 0.4)
        np.testing.assert_array_equal(one[0, 0], full[0, h])


# ---------------------------------------------------------------- O6 splits + merge

def test_combine_golden(golden):
    g = golden["combine"]
    po = np.array(g["part_o"], np.float64).reshape(1, 1, 3, 1)
    pm = np.array([float(x) for x in g["part_m"]]).reshape(1, 1, 3)
    pl = np.array(g["part_l"], np.float64).reshape(1, 1, 3)
    out, lse = oracle.combine(po, pm, pl)
    assert out[0, 0, 0] == pytest.approx(g["out"][0], rel=1e-15)
    assert lse[0, 0] == pytest.approx(g["lse"], rel=1e-15)


def test_each_split_is_attention_over_its_chunk():
    data = mk(B=2, Hq=2, Hkv=1, D=8, lens=(150, 40), seed=30)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    S = 3
    po, pm, pl = oracle.attention_splits(q64, k64, v64, data.block_table, data.seq_lens, 0.5, S)
    for b in range(2):
        nb = data.spec.blocks(b)
        c = -(-nb // S)
        for h in range(2):
            for s in range(S):
                blocks = range(min(s * c, nb), min((s + 1) * c, nb))
                if len(blocks) == 0:
                    assert pm[b, h, s] == -np.inf and pl[b, h, s] == 0
                    assert np.all(po[b, h, s] == 0)
                    continue
                K = gather(k64, data, b, 0, blocks)
                V = gather(v64, data, b, 0, blocks)
                z = 0.5 * (K @ q64[b, h])
                assert pm[b, h, s] == pytest.approx(z.max(), rel=1e-14)
                assert pl[b, h, s] == pytest.approx(np.exp(z - z.max()).sum(), rel=1e-13)
                np.testing.assert_allclose(po[b, h, s], sdpa(q64[b, h], K, V, 0.5),
                                           rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 40])
@pytest.mark.parametrize("sparse", [False, True])
def test_split_then_combine_equals_unsplit(S, sparse):
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(190, 33), dtype="f16", seed=31)
    q64, k64, v64 = data.q64(), data.k64(), data.v64()
    sel, cnt = wl.random_selection(data, 5, seed=4) if sparse else (None, None)
    ref, lref = oracle.attention(q64, k64, v64, data.block_table, data.seq_lens, 0.25, sel, cnt)
    parts = oracle.attention_splits(q64, k64, v64, data.block_table, data.seq_lens, 0.25, S,
                                    sel, cnt)
    out, lse = oracle.combine(*parts)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lref, rtol=1e-13)


# ---------------------------------------------------------------- selection variants
# mean-key index (KVDrive §2.3 spatial blocking, §4) and forced sink / local
# tokens (KVDrive §9.1)

VARIANTS = os.path.join(os.path.dirname(__file__), "golden", "selection_variants.json")


@pytest.fixture(scope="module")
def variants():
    with open(VARIANTS) as f:
        return json.load(f)


def full_mean(data):
    ids, val = page_lists(data)
    return oracle.block_mean(data.k64(), ids, val)


def test_mean_golden(variants):
    g = variants["mean_score"]
    k = np.array(g["k_slots"], np.float64).reshape(1, 1, g["block_size"], g["head_dim"])
    km = oracle.block_mean(k, [0], [g["valid_tokens"]])
    assert km[0, 0].tolist() == g["kmean"]
    for qv, want in zip(g["queries"], g["scores"]):
        s = oracle.head_scores_mean(np.array(qv, np.float64).reshape(1, 1, -1), km,
                                    np.zeros((1, 1), np.int32), np.array([3], np.int32),
                                    g["block_size"])
        assert s[0, 0, 0] == want


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_mean_matches_numpy_reduction(dtype):
    data = mk(B=3, Hq=6, Hkv=3, D=16, lens=(45, 16, 3), dtype=dtype, seed=31, extra_pages=2)
    k64 = data.k64()
    ids, val = page_lists(data)
    km = oracle.block_mean(k64, ids, val)
    for p, nv in zip(ids, val):
        np.testing.assert_allclose(km[p], k64[p, :, :nv].mean(axis=1), rtol=1e-15, atol=1e-15)
    untouched = np.setdiff1d(np.arange(k64.shape[0]), ids)
    assert untouched.size and np.all(km[untouched] == 0)


def test_mean_score_is_the_average_token_dot():
    """Linearity: q . mean(k_t) = mean_t (q . k_t), with the dots taken directly
    from the token rows through the block table (GQA head map h // G)."""
    data = mk(B=2, Hq=6, Hkv=2, D=8, lens=(53, 20), seed=32)
    q64, k64 = data.q64(), data.k64()
    hs = oracle.head_scores_mean(q64, full_mean(data), data.block_table, data.seq_lens, 16)
    G = 3
    for b in range(2):
        nb = data.spec.blocks(b)
        for h in range(6):
            for n in range(nb):
                rows = gather(k64, data, b, h // G, [n])
                want = float(np.mean(rows @ q64[b, h]))
                assert abs(hs[b, h, n] - want) <= 1e-13 * (1 + np.abs(rows @ q64[b, h]).sum())
            assert np.all(np.isneginf(hs[b, h, nb:]))


def test_mean_score_single_token_block_is_the_dot_product():
    data = mk(B=1, Hq=2, Hkv=1, D=8, lens=(48,), seed=33, block_size=1)
    q64, k64 = data.q64(), data.k64()
    ids, val = page_lists(data)
    km = oracle.block_mean(k64, ids, val)
    hs = oracle.head_scores_mean(q64, km, data.block_table, data.seq_lens, 1)
    for h in range(2):
        for n in range(48):
            p = data.block_table[0, n]
            assert hs[0, h, n] == pytest.approx(float(q64[0, h] @ k64[p, 0, 0]), rel=1e-14,
                                                abs=1e-14)


def test_mean_score_is_bounded_by_the_quest_score():
    """The average of q . k_t never exceeds the largest q . k_t, which the
    Quest score bounds from above."""
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(70, 33), seed=34)
    mean_s = oracle.head_scores_mean(data.q64(), full_mean(data), data.block_table,
                                     data.seq_lens, 16)
    quest = oracle.head_scores(data.q64(), full_meta(data), data.block_table, data.seq_lens, 16)
    fin = np.isfinite(quest)
    assert np.all(mean_s[fin] <= quest[fin] + 1e-12)


def test_forced_sets_golden(variants):
    g = variants["forced"]
    bs = g["block_size"]
    for case in g["cases"]:
        L = case["seq_len"]
        nb = -(-L // bs)
        # the scores put every block at -1 except none: K = 1 leaves only forced blocks
        sel, cnt = oracle.select(np.full((1, 1, nb), -1.0), np.array([L], np.int32), bs,
                                 len(case["forced"]), g["sink_tokens"], g["local_tokens"])
        assert sel[0, 0, :cnt[0, 0]].tolist() == case["forced"]


def test_select_golden(variants):
    for case in variants["forced"]["select_cases"]:
        s = np.array(case["scores"], np.float64).reshape(1, 1, -1)
        sel, cnt = oracle.select(s, np.array([case["seq_len"]], np.int32), 16, case["k"],
                                 case["sink_tokens"], case["local_tokens"])
        want = case["selected"]
        assert cnt[0, 0] == len(want)
        assert sel[0, 0, :len(want)].tolist() == want
        assert np.all(sel[0, 0, len(want):] == -1)


def _forced_blocks(L, bs, sink, local):
    """Blocks holding any of the first ``sink`` or the last ``local`` token indices."""
    toks = set(range(min(sink, L))) | set(range(max(L - local, 0), L))
    return {t // bs for t in toks}


@pytest.mark.parametrize("seed", range(4))
def test_select_matches_a_library_sort(seed):
    """Forced blocks by token enumeration, the rest by Python's sort (score
    descending, index ascending); heavy ties from integer scores."""
    rng = np.random.default_rng(200 + seed)
    B, Hkv, bs = 4, 2, 16
    lens = rng.integers(1, 30 * bs, size=B).astype(np.int32)
    maxN = int(max(-(-lens // bs)))
    gs = rng.integers(-3, 4, size=(B, Hkv, maxN)).astype(np.float64)
    for sink, local in ((4, 64), (0, 17), (33, 0), (1, 1)):
        k_min = -(-sink // bs) + -(-local // bs) + 1
        for k in (k_min, k_min + 3, 40):
            sel, cnt = oracle.select(gs, lens, bs, k, sink, local)
            for b in range(B):
                L = int(lens[b])
                nb = -(-L // bs)
                forced = _forced_blocks(L, bs, sink, local)
                rest = [n for n in range(nb) if n not in forced]
                free = min(k, nb) - len(forced)
                assert free >= 0
                for j in range(Hkv):
                    best = sorted(rest, key=lambda n: (-gs[b, j, n], n))[:free]
                    want = sorted(forced | set(best))
                    assert cnt[b, j] == len(want) == min(k, nb)
                    assert sel[b, j, :cnt[b, j]].tolist() == want
                    assert np.all(sel[b, j, cnt[b, j]:] == -1)


def test_select_without_forcing_is_topk():
    rng = np.random.default_rng(9)
    gs = rng.standard_normal((2, 3, 40))
    lens = np.array([640, 333], np.int32)
    for k in (1, 5, 40, 64):
        a = oracle.select(gs, lens, 16, k)
        b = oracle.topk(gs, lens, 16, k)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- FP8 E4M3 cold pages
# OCP 8-bit floating point (E4M3); quantised cold pages per KVDrive §11 and the
# DirectKV review's assumption stress test

def _torch_e4m3(values_f32):
    return torch.from_numpy(np.ascontiguousarray(values_f32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_golden(variants):
    g = variants["fp8_e4m3"]
    for d in g["decode"]:
        v = oracle.fp8_decode(np.array([d["code"]]))[0]
        assert v == d["value"] and np.signbit(v) == np.signbit(d["value"]), d
    codes = oracle.fp8_encode(np.array([e["value"] for e in g["encode"]], np.float32))
    assert codes.tolist() == [e["code"] for e in g["encode"]]
    q = g["quantize"]
    x = np.array(q["x_slots"], np.float64).reshape(1, 1, q["block_size"], q["head_dim"])
    c, s = oracle.fp8_quantize(x, [0], [q["valid_tokens"]])
    assert s[0, 0] == q["scale"]
    assert c[0, 0].tolist() == q["codes"]


def test_fp8_decode_matches_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2      # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("seed", range(3))
def test_fp8_encode_matches_torch_in_range(seed):
    """torch rounds to nearest even; it gives NaN past 464 where the oracle
    saturates, so the comparison stays below 464.  Every grid midpoint is
    included (the ties)."""
    rng = np.random.default_rng(300 + seed)
    y = (rng.standard_normal(100000) * rng.choice([1e-5, 1e-3, 1e-1, 1, 30, 300], 100000))
    grid = oracle.fp8_decode(np.arange(0, 127))                     # the non-negative finite values
    mids = (grid[:-1] + grid[1:]) / 2
    y = np.concatenate([y, grid, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    y = y.astype(np.float32)
    y = y[np.abs(y) < 464]
    np.testing.assert_array_equal(oracle.fp8_encode(y), _torch_e4m3(y))


def test_fp8_encode_saturates_and_round_trips():
    assert oracle.fp8_encode(np.array([464, 480, 1e30, -500], np.float32)).tolist() == [
        0x7E, 0x7E, 0x7E, 0xFE]
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.fp8_decode(codes).astype(np.float32)
    back = oracle.fp8_encode(vals)
    assert np.array_equal(back, codes)          # every finite code, -0 included


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_fp8_quantize_matches_torch_and_error_bound(dtype):
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(45, 16), dtype=dtype, seed=41, extra_pages=1)
    k64 = data.k64()
    ids, val = page_lists(data)
    codes, scales = oracle.fp8_quantize(k64, ids, val)
    x32 = k64.astype(np.float32)
    for p, nv in zip(ids, val):
        for j in range(2):
            tile = x32[p, j, :nv]
            amax = np.abs(tile).max()
            s = scales[p, j]
            # the largest magnitude lands on +-448 (code 0x7E / 0xFE)
            big = np.abs(tile) == amax
            assert np.all((codes[p, j, :nv][big] & 0x7F) == 0x7E)
            # the codes are torch's conversion of x / s taken in fp32
            np.testing.assert_array_equal(codes[p, j, :nv], _torch_e4m3(tile / s))
            # round-to-nearest error: half a grid step
            deq = oracle.fp8_decode(codes[p, j, :nv]) * float(s)
            y = np.abs(tile.astype(np.float64)) / float(s)
            half = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4),
                            2.0 ** -10) * float(s)
            assert np.all(np.abs(deq - tile) <= half * (1 + 1e-6))
            assert np.all(codes[p, j, nv:] == 0)
    untouched = np.setdiff1d(np.arange(k64.shape[0]), ids)
    assert untouched.size and np.all(codes[untouched] == 0) and np.all(scales[untouched] == 0)


def test_fp8_quantize_zero_tile_has_unit_scale():
    x = np.zeros((1, 2, 16, 8))
    x[0, 1, 3, 2] = -1.5
    codes, scales = oracle.fp8_quantize(x, [0], [16])
    assert scales[0, 0] == 1.0 and np.all(codes[0, 0] == 0)
    assert scales[0, 1] == np.float32(1.5) / np.float32(448)
    assert codes[0, 1, 3, 2] == 0xFE


def test_fp8_dequantized_attention_is_attention_over_decoded_values():
    """Attention over fp8 pages is the plain attention over decode(code) * scale:
    checked against torch's fused attention on the decoded tensors."""
    data = mk(B=1, Hq=2, Hkv=1, D=16, lens=(40,), seed=42)
    ids, val = page_lists(data)
    kc, ks = oracle.fp8_quantize(data.k64(), ids, val)
    vc, vs = oracle.fp8_quantize(data.v64(), ids, val)
    kd, vd = oracle.fp8_dequantize(kc, ks), oracle.fp8_dequantize(vc, vs)
    out, _ = oracle.attention(data.q64(), kd, vd, data.block_table, data.seq_lens, 0.25)
    for h in range(2):
        K = gather(kd, data, 0, 0, range(3))
        V = gather(vd, data, 0, 0, range(3))
        np.testing.assert_allclose(out[0, h], sdpa(data.q64()[0, h], K, V, 0.25), rtol=1e-12,
                                   atol=1e-14)


# ---------------------------------------------------------------- INT4 cold pages
# KVDrive §11 and the DirectKV review name INT4 for cold KV; symmetric reading

def test_int4_golden(variants):
    g = variants["int4"]
    for u in g["unpack"]:
        assert oracle.int4_unpack(np.array([u["byte"]], np.uint8)).tolist() == u["codes"], u
    for q in g["quantize"]:
        x = np.array(q["x_slots"], np.float64).reshape(1, 1, q["block_size"], q["head_dim"])
        c, s = oracle.int4_quantize(x, [0], [q["valid_tokens"]])
        assert s[0, 0] == q["scale"], q["derivation"]
        assert c[0, 0].tolist() == q["codes"], q["derivation"]


def test_int4_unpack_c_and_numpy_agree_on_every_byte():
    for b in range(256):
        row = np.array([b], np.uint8)
        assert oracle.int4_unpack(row).tolist() == [oracle.int4_unpack_c(row, 0),
                                                    oracle.int4_unpack_c(row, 1)]


def test_int4_code_rounding_and_clamp():
    cases = {2.5: 2, 3.5: 4, -2.5: -2, -0.5: 0, 0.49999997: 0, 6.5: 6, 7.49: 7, 100.0: 7,
             -7.5: -7, -1e30: -7, 1.5: 2}
    for y, n in cases.items():
        assert oracle.int4_code(y) == n, (y, n)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_int4_quantize_matches_numpy_and_error_bound(dtype):
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(45, 16), dtype=dtype, seed=43, extra_pages=1)
    k64 = data.k64()
    ids, val = page_lists(data)
    codes, scales = oracle.int4_quantize(k64, ids, val)
    n_all = oracle.int4_unpack(codes)
    x32 = k64.astype(np.float32)
    for p, nv in zip(ids, val):
        for j in range(2):
            tile = x32[p, j, :nv]
            amax = np.abs(tile).max()
            s = scales[p, j]
            assert s == np.float32(amax) / np.float32(7)
            n = n_all[p, j, :nv]
            # numpy's fp32 quotient, rounded half to even, clamped
            np.testing.assert_array_equal(n, np.clip(np.rint(tile / s), -7, 7).astype(np.int8))
            big = np.abs(tile) == amax
            assert np.all(np.abs(n[big]) == 7)
            deq = n.astype(np.float64) * float(s)
            assert np.all(np.abs(deq - tile) <= 0.5 * float(s) * (1 + 1e-6))
            assert np.all(codes[p, j, nv:] == 0)
    untouched = np.setdiff1d(np.arange(k64.shape[0]), ids)
    assert untouched.size and np.all(codes[untouched] == 0) and np.all(scales[untouched] == 0)


def test_int4_quantize_zero_tile_has_unit_scale():
    x = np.zeros((1, 2, 16, 8))
    x[0, 1, 3, 2] = -1.5
    codes, scales = oracle.int4_quantize(x, [0], [16])
    assert scales[0, 0] == 1.0 and np.all(codes[0, 0] == 0)
    assert scales[0, 1] == np.float32(1.5) / np.float32(7)
    assert oracle.int4_unpack(codes)[0, 1, 3, 2] == -7


def test_int4_dequantized_attention_is_attention_over_decoded_values():
    data = mk(B=1, Hq=2, Hkv=1, D=16, lens=(40,), seed=44)
    ids, val = page_lists(data)
    kc, ks = oracle.int4_quantize(data.k64(), ids, val)
    vc, vs = oracle.int4_quantize(data.v64(), ids, val)
    kd, vd = oracle.int4_dequantize(kc, ks), oracle.int4_dequantize(vc, vs)
    out, _ = oracle.attention(data.q64(), kd, vd, data.block_table, data.seq_lens, 0.25)
    for h in range(2):
        K = gather(kd, data, 0, 0, range(3))
        V = gather(vd, data, 0, 0, range(3))
        np.testing.assert_allclose(out[0, h], sdpa(data.q64()[0, h], K, V, 0.25), rtol=1e-12,
                                   atol=1e-14)


# ---------------------------------------------------------------- GPU block cache
# KVDrive §5.1: a GPU window of critical blocks with lookahead eviction

def test_cache_plan_golden(variants):
    g = variants["cache_plan"]
    C, N = g["num_slots"], g["num_blocks"]
    sb = np.full((1, 1, C), -1, np.int32)
    bsl = np.full((1, 1, N), -1, np.int32)
    for st in g["steps"]:
        k = len(st["sel"])
        sel = np.array(st["sel"], np.int32).reshape(1, 1, k)
        mass = np.array(st["mass_before"], np.float32).reshape(1, 1, C)
        sb, bsl, slots, fb, fs, fc = oracle.cache_plan(sel, np.array([[k]], np.int32), sb, bsl, mass)
        assert slots[0, 0].tolist() == st["sel_slots"], st["why"]
        assert fc[0, 0] == len(st["fetch"])
        assert [[int(a), int(b)] for a, b in zip(fb[0, 0, :fc[0, 0]], fs[0, 0, :fc[0, 0]])] == st["fetch"]
        assert sb[0, 0].tolist() == st["slot_block"]
        for c, blk in enumerate(st["slot_block"]):
            if blk >= 0:
                assert bsl[0, 0, blk] == c
        assert (bsl[0, 0] >= 0).sum() == sum(1 for x in st["slot_block"] if x >= 0)


def _check_plan_step(sel, cnt, sb0, bsl0, mass, out):
    """Invariants of one cache step, checked independently of the plan's code."""
    sb, bsl, slots, fb, fs, fc = out
    B, Hkv, C = sb.shape
    for b in range(B):
        for j in range(Hkv):
            k = int(cnt[b, j])
            chosen = sel[b, j, :k].tolist()
            before = {int(c): int(x) for c, x in enumerate(sb0[b, j])}
            # every selected block is resident, at the slot reported for it
            for pos, n in enumerate(chosen):
                s = int(slots[b, j, pos])
                assert sb[b, j, s] == n and bsl[b, j, n] == s
            assert np.all(slots[b, j, k:] == -1)
            # the two maps are inverse of each other
            res = {int(x): c for c, x in enumerate(sb[b, j]) if x >= 0}
            assert len(res) == int((sb[b, j] >= 0).sum())
            assert {int(n): int(s) for n, s in enumerate(bsl[b, j]) if s >= 0} == res
            # hits keep their slots; misses are exactly the fetches
            hits = [n for n in chosen if bsl0[b, j, n] >= 0]
            for n in hits:
                assert bsl[b, j, n] == bsl0[b, j, n]
            misses = [n for n in chosen if bsl0[b, j, n] < 0]
            assert int(fc[b, j]) == len(misses)
            assert fb[b, j, :len(misses)].tolist() == misses
            used = fs[b, j, :len(misses)].tolist()
            assert len(set(used)) == len(used)
            assert used == sorted(used), "misses take the reused slots in slot order"
            free = [c for c in range(C) if before[c] < 0]
            # free slots are reused first, in slot order
            if len(used) <= len(free):
                assert used == free[:len(used)]
            else:
                assert set(free) <= set(used)
            victims = [c for c in used if before[c] >= 0]
            survivors = [c for c in range(C) if before[c] >= 0 and before[c] not in chosen
                         and c not in victims]
            for v in victims:
                assert before[v] >= 0 and before[v] not in chosen
                for s in survivors:
                    assert (mass[b, j, v], v) < (mass[b, j, s], s)
            # every other slot keeps its block
            for c in range(C):
                if c not in used:
                    assert sb[b, j, c] == before[c]


@pytest.mark.parametrize("seed", range(4))
def test_cache_plan_invariants_over_many_steps(seed):
    rng = np.random.default_rng(400 + seed)
    B, Hkv, N, C, K = 2, 3, 40, 12, 8
    sb = np.full((B, Hkv, C), -1, np.int32)
    bsl = np.full((B, Hkv, N), -1, np.int32)
    for step in range(25):
        cnt = rng.integers(1, K + 1, size=(B, Hkv)).astype(np.int32)
        sel = np.full((B, Hkv, K), -1, np.int32)
        for b in range(B):
            for j in range(Hkv):
                sel[b, j, :cnt[b, j]] = np.sort(rng.choice(N, cnt[b, j], replace=False))
        # masses with many exact ties (multiples of 1/8, zeros for free slots)
        mass = (rng.integers(0, 4, size=(B, Hkv, C)) / 8).astype(np.float32)
        out = oracle.cache_plan(sel, cnt, sb, bsl, mass)
        _check_plan_step(sel, cnt, sb, bsl, mass, out)
        sb, bsl = out[0], out[1]


def test_block_lse_sums_to_the_row_lse_and_matches_numpy():
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(61, 16), seed=51)
    q64, k64 = data.q64(), data.k64()
    scale = 0.25
    bl = oracle.block_lse(q64, k64, data.block_table, data.seq_lens, 16, scale)
    _, lse = oracle.attention(q64, k64, data.v64(), data.block_table, data.seq_lens, scale)
    for b in range(2):
        nb = data.spec.blocks(b)
        for h in range(4):
            np.testing.assert_allclose(scipy.special.logsumexp(bl[b, h, :nb]), lse[b, h], rtol=1e-13)
            assert np.all(np.isneginf(bl[b, h, nb:]))
            for n in range(nb):
                z = gather(k64, data, b, h // 2, [n]) @ q64[b, h] * scale
                np.testing.assert_allclose(bl[b, h, n], scipy.special.logsumexp(z), rtol=1e-13)


def test_block_lse_over_a_selection():
    data = mk(B=1, Hq=2, Hkv=1, D=8, lens=(100,), seed=52)
    sel = np.array([[[1, 4, 6, -1]]], np.int32)
    cnt = np.array([[3]], np.int32)
    bl = oracle.block_lse(data.q64(), data.k64(), data.block_table, data.seq_lens, 16, 0.5, sel, cnt)
    full = oracle.block_lse(data.q64(), data.k64(), data.block_table, data.seq_lens, 16, 0.5)
    np.testing.assert_array_equal(bl[0, :, :3], full[0, :, [1, 4, 6]].T)
    assert np.all(np.isneginf(bl[0, :, 3]))


def test_slot_mass_is_the_attention_weight_of_each_block():
    data = mk(B=1, Hq=4, Hkv=2, D=16, lens=(90,), seed=53)
    q64, k64 = data.q64(), data.k64()
    sel = np.array([[[0, 2, 5, -1], [1, 3, -1, -1]]], np.int32)
    cnt = np.array([[3, 2]], np.int32)
    slots = np.array([[[4, 0, 2, -1], [1, 5, -1, -1]]], np.int32)
    bl = oracle.block_lse(q64, k64, data.block_table, data.seq_lens, 16, 0.25, sel, cnt)
    _, lse = oracle.attention(q64, k64, data.v64(), data.block_table, data.seq_lens, 0.25, sel, cnt)
    m = oracle.slot_mass(bl, lse, cnt, slots, 6)
    for j in range(2):
        w = np.exp(bl[0, 2 * j:2 * j + 2, :cnt[0, j]] - lse[0, 2 * j:2 * j + 2, None])
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)     # each head's weights
        for pos in range(cnt[0, j]):
            assert m[0, j, slots[0, j, pos]] == pytest.approx(w[:, pos].max(), rel=1e-14)
        untouched = set(range(6)) - set(slots[0, j, :cnt[0, j]].tolist())
        assert all(m[0, j, c] == 0 for c in untouched)



def test_slot_mass_is_the_softmax_mass_of_each_block_over_the_selection():
    """Independent of the oracle's block LSEs: each head's softmax over the
    logits of every token of the selected blocks (scipy), summed per block, max
    over the group's heads, placed at the block's slot; untouched slots 0."""
    data = mk(B=2, Hq=4, Hkv=2, D=16, lens=(90, 41), seed=62)
    q64, k64 = data.q64(), data.k64()
    scale = 0.25
    sel = np.array([[[0, 2, 5, -1], [1, 3, 4, -1]], [[2, -1, -1, -1], [0, 1, 2, -1]]], np.int32)
    cnt = np.array([[3, 3], [1, 3]], np.int32)
    slots = np.array([[[4, 0, 2, -1], [1, 5, 3, -1]], [[3, -1, -1, -1], [2, 0, 1, -1]]], np.int32)
    bl = oracle.block_lse(q64, k64, data.block_table, data.seq_lens, 16, scale, sel, cnt)
    _, lse = oracle.attention(q64, k64, data.v64(), data.block_table, data.seq_lens, scale, sel, cnt)
    m = oracle.slot_mass(bl, lse, cnt, slots, 6)
    for b in range(2):
        L = data.spec.seq_lens[b]
        for j in range(2):
            blocks = sel[b, j, :cnt[b, j]]
            sizes = [min(16, L - 16 * n) for n in blocks]
            K = gather(k64, data, b, j, blocks)                                 # [T, D]
            want = np.zeros(6)
            for h in range(2 * j, 2 * j + 2):
                p = scipy.special.softmax(scale * (K @ q64[b, h]))
                mass = np.add.reduceat(p, np.cumsum([0] + sizes[:-1]))
                for pos, slot in enumerate(slots[b, j, :cnt[b, j]]):
                    want[slot] = max(want[slot], mass[pos])
            np.testing.assert_allclose(m[b, j], want, rtol=1e-12, atol=0)

# ---------------------------------------------------------------- tier plan
# tiered-offload blog page, page replacement (heat, hysteresis cooldown);
# KVDrive §11 (hot blocks at full precision, cold blocks quantised)

TIER = os.path.join(os.path.dirname(__file__), "golden", "tier_plan.json")


def _sel_rows(rows, stride):
    B, Hkv = len(rows), len(rows[0])
    sel = np.full((B, Hkv, stride), -1, np.int32)
    cnt = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        for j in range(Hkv):
            sel[b, j, :len(rows[b][j])] = rows[b][j]
            cnt[b, j] = len(rows[b][j])
    return sel, cnt


def test_tier_plan_golden():
    with open(TIER) as f:
        g = json.load(f)
    bt = np.array(g["block_table"], np.int32)
    heat = np.array(g["initial"]["heat"], np.float32)
    tier = np.array(g["initial"]["tier"], np.uint8)
    stamp = np.array(g["initial"]["stamp"], np.int32)
    for st in g["steps"]:
        sel, cnt = _sel_rows(st["sel"], g["sel_stride"])
        heat, tier, stamp, dem, dc, pro, pc = oracle.tier_plan(
            sel, cnt, bt, np.array(st["seq_lens"], np.int32), g["block_size"], g["decay"],
            g["hot_above"], g["cold_below"], g["recent"], g["cooldown"], st["step"],
            heat, tier, stamp)
        assert heat.tolist() == st["heat"], st["why"]
        assert tier.tolist() == st["tier"], st["why"]
        assert stamp.tolist() == st["stamp"], st["why"]
        for b in range(bt.shape[0]):
            assert dem[b, :dc[b]].tolist() == st["demote"][b], st["why"]
            assert pro[b, :pc[b]].tolist() == st["promote"][b], st["why"]
            assert np.all(dem[b, dc[b]:] == -1) and np.all(pro[b, pc[b]:] == -1)


def _one_page_plan(hit, heat, tier, stamp, step, decay=0.5, hot_above=0.6, cold_below=0.2,
                   recent=0, cooldown=0, L=8, bs=4):
    """One sequence of two blocks on pages 0 and 1; block 0 is hit when ``hit``."""
    sel = np.array([[[0 if hit else -1]]], np.int32)
    cnt = np.array([[1 if hit else 0]], np.int32)
    bt = np.array([[0, 1]], np.int32)
    return oracle.tier_plan(sel, cnt, bt, np.array([L], np.int32), bs, decay, hot_above,
                            cold_below, recent, cooldown, step,
                            np.array([heat, 0.5], np.float32), np.array([tier, 0], np.uint8),
                            np.array([stamp, 0], np.int32))


@pytest.mark.parametrize("decay", [0.75, 0.9, 0.125])
def test_tier_heat_follows_the_geometric_closed_form(decay):
    """n hits from h0 give 1 - decay^n (1 - h0); n misses then give decay^n times that."""
    h0, h = 0.3, np.float32(0.3)
    for n in range(1, 13):
        out = _one_page_plan(True, h, 0, 0, n, decay=decay, hot_above=2.0, cold_below=-1.0)
        h = out[0][0]
        assert out[0][1] == np.float32(np.float32(decay) * np.float32(0.5))  # block 1 missed
        assert abs(float(h) - (1 - decay ** n * (1 - h0))) < 1e-6
    top = float(h)
    for n in range(1, 13):
        h = _one_page_plan(False, h, 0, 0, 12 + n, decay=decay, hot_above=2.0, cold_below=-1.0)[0][0]
        assert abs(float(h) - decay ** n * top) < 1e-6


def test_tier_thresholds_are_strict():
    # a hot page whose heat lands exactly on cold_below stays hot; one ulp above demotes it
    out = _one_page_plan(False, 0.5, 0, 0, 1, cold_below=0.25)
    assert out[0][0] == 0.25 and out[1][0] == 0 and out[4][0] == 0
    # (block 1 holds the recent tokens, so that page 0 alone can move)
    out = _one_page_plan(False, 0.5, 0, 0, 1, recent=4,
                         cold_below=float(np.nextafter(np.float32(0.25), 1)))
    assert out[1][0] == 1 and out[3][0, 0] == 0 and out[4][0] == 1 and out[2][0] == 1
    # a cold page whose heat lands exactly on hot_above stays cold; one ulp below promotes it
    out = _one_page_plan(True, 0.5, 1, 0, 5, hot_above=0.75)
    assert out[0][0] == 0.75 and out[1][0] == 1 and out[6][0] == 0
    out = _one_page_plan(True, 0.5, 1, 0, 5, hot_above=float(np.nextafter(np.float32(0.75), 0)))
    assert out[1][0] == 0 and out[5][0, 0] == 0 and out[6][0] == 1


@pytest.mark.parametrize("cooldown", [0, 1, 4])
def test_tier_cooldown_counts_steps_since_demotion(cooldown):
    # demoted at step 10; hit at every later step; promoted exactly at step 10 + cooldown
    out = _one_page_plan(False, 0.25, 0, 0, 10, cooldown=cooldown)
    h, t, st = out[0][0], out[1][0], out[2][0]
    assert t == 1 and st == 10
    for step in range(11, 20):
        h = np.float32(0.99)
        out = _one_page_plan(True, h, t, st, step, cooldown=cooldown)
        t = out[1][0]
        assert t == (0 if step >= 10 + cooldown else 1), step
        if t == 0:
            break
    assert t == 0


def test_tier_hit_counts_once_over_the_kv_heads():
    bt = np.array([[0, 1, 2]], np.int32)
    L = np.array([12], np.int32)
    base = (np.full(3, 0.5, np.float32), np.zeros(3, np.uint8), np.zeros(3, np.int32))
    outs = []
    for rows in ([[1], []], [[], [1]], [[1], [1]], [[0, 1, 2], [1]]):
        sel, cnt = _sel_rows([rows], 3)
        outs.append(oracle.tier_plan(sel, cnt, bt, L, 4, 0.5, 0.6, 0.2, 0, 0, 1, *base)[0])
    for o in outs:
        assert o[1] == 0.75
    assert outs[3][0] == 0.75 and outs[0][0] == 0.25


def _token_recent(n, bs, L, recent):
    return any(L - recent <= t < L for t in range(n * bs, (n + 1) * bs))


@pytest.mark.parametrize("seed", range(4))
def test_tier_plan_invariants_over_many_steps(seed):
    """Each step's transitions satisfy the policy's conditions, checked token by token."""
    rng = np.random.default_rng(900 + seed)
    B, Hkv, bs, maxN, K = 3, 2, 4, 12, 5
    P = B * maxN + 5
    perm = rng.permutation(P).astype(np.int32)
    bt = perm[:B * maxN].reshape(B, maxN)
    heat = rng.random(P).astype(np.float32)
    tier = rng.integers(0, 2, P).astype(np.uint8)
    stamp = rng.integers(0, 3, P).astype(np.int32)
    lens = rng.integers(1, bs * maxN - 12, B)
    decay, hot_above, cold_below = 0.8, 0.55, 0.3
    recent = [0, 1, bs - 1, bs, bs + 1][seed % 5]
    cooldown = 2
    for step in range(3, 40):
        lens = np.minimum(lens + rng.integers(0, 3, B), bs * maxN)
        sel = np.full((B, Hkv, K), -1, np.int32)
        cnt = np.zeros((B, Hkv), np.int32)
        for b in range(B):
            N = -(-int(lens[b]) // bs)
            for j in range(Hkv):
                c = int(rng.integers(0, min(K, N) + 1))
                sel[b, j, :c] = np.sort(rng.choice(N, c, replace=False))
                cnt[b, j] = c
        h1, t1, s1, dem, dc, pro, pc = oracle.tier_plan(sel, cnt, bt, lens.astype(np.int32), bs,
                                                        decay, hot_above, cold_below, recent,
                                                        cooldown, step, heat, tier, stamp)
        seen = set()
        for b in range(B):
            L = int(lens[b])
            N = -(-L // bs)
            hits = {int(x) for j in range(Hkv) for x in sel[b, j, :cnt[b, j]]}
            moved_down, moved_up = [], []
            for n in range(N):
                p = int(bt[b, n])
                seen.add(p)
                rec = _token_recent(n, bs, L, recent)
                assert (h1[p] > decay * heat[p] - 1e-6) if n in hits else (h1[p] <= heat[p])
                if rec:
                    assert t1[p] == 0
                if tier[p] == 0 and t1[p] == 1:
                    assert not rec and h1[p] < cold_below and s1[p] == step
                    moved_down.append(p)
                elif tier[p] == 1 and t1[p] == 0:
                    assert rec or (h1[p] > hot_above and step - stamp[p] >= cooldown)
                    assert s1[p] == stamp[p]
                    moved_up.append(p)
                elif t1[p] == 0:
                    assert rec or h1[p] >= cold_below
                    assert s1[p] == stamp[p]
                else:
                    assert not rec and (h1[p] <= hot_above or step - stamp[p] < cooldown)
                    assert s1[p] == stamp[p]
            assert dem[b, :dc[b]].tolist() == moved_down
            assert pro[b, :pc[b]].tolist() == moved_up
            assert np.all(dem[b, dc[b]:] == -1) and np.all(pro[b, pc[b]:] == -1)
        rest = [p for p in range(P) if p not in seen]
        assert np.array_equal(h1[rest], heat[rest]) and np.array_equal(t1[rest], tier[rest])
        assert np.array_equal(s1[rest], stamp[rest])
        heat, tier, stamp = h1, t1, s1
