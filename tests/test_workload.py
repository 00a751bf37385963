"""The seeded input generator (no GPU)."""
import numpy as np
import pytest
import torch

from kv_cache_decode_amd import workload as wl


def small(**kw):
    base = dict(name="w", num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=16,
                seq_lens=(100, 16, 33), dtype="bf16", seed=9, planted_frac=0.2)
    base.update(kw)
    return wl.Workload(**base)


def test_same_seed_same_bytes_and_other_seed_differs():
    a, b = wl.generate(small()), wl.generate(small())
    for x, y in ((a.q_raw, b.q_raw), (a.k_raw, b.k_raw), (a.v_raw, b.v_raw),
                 (a.block_table, b.block_table)):
        assert x.tobytes() == y.tobytes()
    c = wl.generate(small(seed=10))
    assert a.k_raw.tobytes() != c.k_raw.tobytes()


def test_chunked_draws_equal_one_draw():
    a = wl.generate(small(planted_frac=0.0), chunk_rows=1)
    b = wl.generate(small(planted_frac=0.0), chunk_rows=10**6)
    assert a.k_raw.tobytes() == b.k_raw.tobytes()
    assert a.v_raw.tobytes() == b.v_raw.tobytes()


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 2**-130]    # exact halfway cases, a subnormal
    ours = wl.round_f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("dtype", wl.DTYPES)
def test_f64_copy_is_exact(dtype):
    d = wl.generate(small(dtype=dtype))
    k64 = d.k64()
    if dtype == "bf16":
        back = wl.round_f32_to_bf16_bits(k64.astype(np.float32))
    elif dtype == "f16":
        back = k64.astype(np.float16)
    else:
        back = k64.astype(np.float32)
    assert back.tobytes() == d.k_raw.tobytes()


def test_page_table_is_a_permutation_of_used_pages():
    spec = small(extra_pages=5)
    d = wl.generate(spec)
    used = np.concatenate([d.block_table[b, :spec.blocks(b)] for b in range(spec.num_seqs)])
    assert sorted(used.tolist()) == list(range(spec.used_pages))
    assert d.k_raw.shape == (spec.used_pages + 5, 2, 16, 16)
    ident = wl.generate(small(page_table="identity"))
    used = np.concatenate([ident.block_table[b, :spec.blocks(b)] for b in range(spec.num_seqs)])
    assert used.tolist() == list(range(spec.used_pages))


def test_planted_blocks_count_and_direction():
    spec = small(planted_frac=0.25, seq_lens=(640, 320, 160), dtype="f32")
    d = wl.generate(spec)
    q = d.q64()
    G = spec.group
    for b in range(spec.num_seqs):
        nb = spec.blocks(b)
        for j in range(spec.num_kv_heads):
            assert d.planted[b, j, :nb].sum() == round(0.25 * nb)
            assert not d.planted[b, j, nb:].any()
            u = q[b, j * G] / np.linalg.norm(q[b, j * G])
            proj = [d.k64()[d.block_table[b, n], j].mean(axis=0) @ u for n in range(nb)]
            proj = np.array(proj)
            # planted keys are shifted by 2u: their mean projection sits about 2 higher
            assert proj[d.planted[b, j, :nb]].mean() - proj[~d.planted[b, j, :nb]].mean() > 1.5


def test_named_workloads_shapes():
    w = wl.WORKLOADS
    c4 = w["llama3.1_8b_gqa_b1_128k_bf16"]
    assert (c4.num_pages, c4.max_blocks, c4.group) == (8192, 8192, 4)
    assert wl.kv_bytes(c4, c4.used_pages * c4.num_kv_heads) == 512 * 2**20
    c3 = w["llama3.1_8b_gqa_b4_32k_bf16"]
    assert (c3.num_pages, c3.max_blocks) == (8192, 2048)
    assert round(c3.planted_frac * 2048) == 102 and round(c4.planted_frac * 8192) == 410
    c2 = w["opt6.7b_mha_b32_544_f16"]
    assert (c2.num_pages, c2.max_blocks) == (1088, 34)
    assert wl.kv_bytes(c2, c2.used_pages * c2.num_kv_heads) == 285212672
    c1 = w["tiny_mha_d64_1k_f32"]
    assert (c1.num_pages, c1.topk_blocks) == (64, 16)


def test_random_selection_is_sorted_unique_and_in_range():
    d = wl.generate(small())
    sel, cnt = wl.random_selection(d, 4, seed=1)
    for b in range(3):
        nb = d.spec.blocks(b)
        for j in range(2):
            s = sel[b, j, :cnt[b, j]]
            assert cnt[b, j] == min(4, nb)
            assert np.all(np.diff(s) > 0) and s.min() >= 0 and s.max() < nb
            assert np.all(sel[b, j, cnt[b, j]:] == -1)
