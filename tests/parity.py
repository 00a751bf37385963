"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances:
* attention outputs, per (sequence, head) row: ||o - ref||_2 / ||ref||_2 <= tol
  with tol = 1e-5 for fp32 inputs and 2e-3 for fp16/bf16 inputs (fp32
  accumulation), and element by element |o_c - ref_c| <= tol * max_c |ref_c|
  over the same row (one wrong channel cannot hide inside the row norm);
* log-sum-exp values (the merged lse, a split's m, m + ln l): |got - ref| <= tol
  in absolute terms, since an lse error e is a relative error e^e - 1 ~ e of
  the softmax normaliser; a split's l (a normaliser itself): rel-err <= tol;
* block meta: bit-exact (compared by value, so -0 == +0);
* scores: |gpu - ref| <= 1e-6 * sum_c |max(q_c kmin_c, q_c kmax_c)| (an fp32 sum
  of D terms is accurate relative to the sum of the terms' magnitudes, not to
  the result, which can cancel; the bound is taken from the oracle's score of
  |q| against |kmin|, |kmax|, which is >= that sum);
* selection: the GPU set equals the oracle set, except for blocks whose oracle
  score lies within 1e-6 * |S_K| of the K-th largest oracle score S_K; the GPU
  list must also be a valid Top-K of the GPU's own scores (ascending, unique,
  lower index first on equal scores);
* mean-key index: bit-exact against the oracle's fp64 mean rounded to fp32
  (the kernel takes the same fp64 sum in slot order and rounds once); mean
  scores within 1e-6 of sum_c |q_c kmean_c|, as above.  A mean score can cancel
  to near zero, so its selection band is also widened to 2e-6 times the row's
  largest magnitude bound: two blocks can only trade places when their oracle
  scores differ by less than the sum of their fp32 errors.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from kv_cache_decode_amd import workload as wl

ROW_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
SCORE_RTOL = 1e-6
TIE_BAND = 1e-6


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


# Worst errors seen by the checks below in this process, printed at the end of a
# pytest session (conftest.py): check name -> {measure: worst value}.
WORST: dict = {}


def _note(what: str, tol: float, **measures: float):
    key = f"{what.split(' S=')[0].split(' step')[0]} [tol {tol:.0e}]"
    cur = WORST.setdefault(key, {})
    for k, v in measures.items():
        cur[k] = max(cur.get(k, 0.0), float(v))


def assert_rows_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str = "out"):
    """Row-norm and element-wise bounds (see the module docstring); returns the
    worst row relative error."""
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    diff = np.abs(got - ref)
    err = np.linalg.norm(got - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    rel = err / np.maximum(nrm, 1e-300)
    worst = int(np.argmax(rel))
    rowmax = np.abs(ref).max(axis=1)
    erel = diff.max(axis=1) / np.maximum(rowmax, 1e-300)
    ew = int(np.argmax(erel))
    _note(what, tol, row_rel=rel.max(), max_abs=diff.max(), elem_rel=erel.max())
    assert rel.max() <= tol, (f"{what}: row rel-err {rel.max():.3e} > {tol:.1e} at row {worst} "
                              f"(max abs err {diff.max():.3e})")
    assert erel.max() <= tol, (f"{what}: element err {diff[ew].max():.3e} > {tol:.1e} * "
                               f"max|ref| ({rowmax[ew]:.3e}) at row {ew}, channel "
                               f"{int(np.argmax(diff[ew]))}")
    return float(rel.max())


def assert_lse_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str = "lse"):
    """|got - ref| <= tol: an lse error is a relative error of the normaliser."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    d = np.abs(got - ref)
    _note(what, tol, max_abs=d.max())
    assert d.max() <= tol, f"{what}: |err| {d.max():.3e} > {tol:.1e} at {np.unravel_index(np.argmax(d), d.shape)}"


def assert_rel_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str):
    """|got - ref| <= tol * |ref| element by element (for positive normalisers)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    r = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)
    _note(what, tol, rel=r.max())
    assert r.max() <= tol, f"{what}: rel-err {r.max():.3e} > {tol:.1e}"


def page_lists(data: wl.WorkloadData):
    """(page ids, valid slot counts) of every page the sequences' current lengths use."""
    bs = data.spec.block_size
    ids, val = [], []
    for b in range(data.spec.num_seqs):
        L = int(data.seq_lens[b])
        for n in range(-(-L // bs)):
            ids.append(int(data.block_table[b, n]))
            val.append(min(bs, L - n * bs))
    return np.array(ids, np.int32), np.array(val, np.int32)


class OracleRun:
    """Lazily computed oracle results for one workload."""

    def __init__(self, data: wl.WorkloadData):
        self.data = data
        self.spec = data.spec
        self.scale = 1.0 / np.sqrt(self.spec.head_dim)
        self._q = self._k = self._v = None
        self._meta = None

    @property
    def q(self):
        if self._q is None:
            self._q = self.data.q64()
        return self._q

    @property
    def k(self):
        if self._k is None:
            self._k = self.data.k64()
        return self._k

    @property
    def v(self):
        if self._v is None:
            self._v = self.data.v64()
        return self._v

    def meta(self):
        if self._meta is None:
            ids, val = page_lists(self.data)
            self._meta = oracle.block_meta(self.k, ids, val)
        return self._meta

    def scores(self):
        hs = oracle.head_scores(self.q, self.meta(), self.data.block_table, self.data.seq_lens,
                                self.spec.block_size)
        return oracle.group_scores(hs, self.spec.num_kv_heads)

    def mean(self):
        if getattr(self, "_mean", None) is None:
            ids, val = page_lists(self.data)
            self._mean = oracle.block_mean(self.k, ids, val)
        return self._mean

    def mean_scores(self):
        hs = oracle.head_scores_mean(self.q, self.mean(), self.data.block_table,
                                     self.data.seq_lens, self.spec.block_size)
        return oracle.group_scores(hs, self.spec.num_kv_heads)

    def mean_score_bound(self):
        hs = oracle.head_scores_mean(np.abs(self.q), np.abs(self.mean()), self.data.block_table,
                                     self.data.seq_lens, self.spec.block_size)
        return oracle.group_scores(hs, self.spec.num_kv_heads)

    def score_bound(self):
        """Per (b, KV head, block): an upper bound of sum_c |term_c| over the group's heads."""
        hs = oracle.head_scores(np.abs(self.q), np.abs(self.meta()), self.data.block_table,
                                self.data.seq_lens, self.spec.block_size)
        return oracle.group_scores(hs, self.spec.num_kv_heads)

    def topk(self, k: int, group_scores=None):
        gs = self.scores() if group_scores is None else group_scores
        return oracle.topk(gs, self.data.seq_lens, self.spec.block_size, k)

    def attention(self, sel=None, cnt=None):
        return oracle.attention(self.q, self.k, self.v, self.data.block_table, self.data.seq_lens,
                                self.scale, sel, cnt)

    def splits(self, S: int, sel=None, cnt=None):
        return oracle.attention_splits(self.q, self.k, self.v, self.data.block_table,
                                       self.data.seq_lens, self.scale, S, sel, cnt)


def check_scores(gpu_scores: np.ndarray, ref: np.ndarray, nblocks: np.ndarray, bound: np.ndarray):
    B, Hkv, maxN = ref.shape
    for b in range(B):
        nb = int(nblocks[b])
        assert np.all(np.isneginf(gpu_scores[b, :, nb:])), "scores past N_b must be -inf"
        r, g, m = ref[b, :, :nb], gpu_scores[b, :, :nb], bound[b, :, :nb]
        bad = np.abs(g - r) > SCORE_RTOL * np.maximum(m, 1e-30)
        assert not bad.any(), (f"score mismatch b={b}: max |err| / bound "
                               f"{(np.abs(g - r) / np.maximum(m, 1e-30)).max():.3e}")


def check_selection_valid(sel: np.ndarray, cnt: np.ndarray, scores: np.ndarray,
                          nblocks: np.ndarray, k: int):
    """The GPU list is a Top-K of the GPU's own scores with the lower-index tie rule."""
    B, Hkv, _ = sel.shape
    for b in range(B):
        nb = int(nblocks[b])
        keff = min(k, nb)
        for j in range(Hkv):
            c = int(cnt[b, j])
            assert c == keff, f"sel_count {c} != K_eff {keff}"
            s = sel[b, j, :c]
            assert np.all(sel[b, j, c:] == -1), "padding must be -1"
            assert np.all(np.diff(s) > 0) and s.min() >= 0 and s.max() < nb, "ascending, in range"
            sc = scores[b, j, :nb].astype(np.float64)
            order = sorted(range(nb), key=lambda i: (-sc[i], i))
            assert sorted(order[:keff]) == s.tolist(), "not the Top-K of the GPU's own scores"


def forced_blocks(L: int, bs: int, sink: int, local: int) -> set:
    """Blocks that hold one of the first ``sink`` or the last ``local`` tokens."""
    nb = -(-L // bs)
    return {n for n in range(nb) if n * bs < sink or (local > 0 and (n + 1) * bs > L - local)}


def check_selection_valid_forced(sel, cnt, scores, seq_lens, k, sink, local, bs=16):
    """Every forced block is in the list and the rest is the Top-(K_eff - #forced)
    of the other blocks by the GPU's own scores, lower index first on ties."""
    B, Hkv, _ = sel.shape
    for b in range(B):
        L = int(seq_lens[b])
        nb = -(-L // bs)
        keff = min(k, nb)
        forced = forced_blocks(L, bs, sink, local)
        for j in range(Hkv):
            c = int(cnt[b, j])
            assert c == keff, f"sel_count {c} != K_eff {keff}"
            s = sel[b, j, :c]
            assert np.all(sel[b, j, c:] == -1), "padding must be -1"
            assert np.all(np.diff(s) > 0) and s.min() >= 0 and s.max() < nb, "ascending, in range"
            sc = scores[b, j, :nb].astype(np.float64)
            rest = sorted((n for n in range(nb) if n not in forced), key=lambda i: (-sc[i], i))
            want = sorted(forced | set(rest[:keff - len(forced)]))
            assert s.tolist() == want, f"b={b} j={j}: not forced + Top-K of the GPU's own scores"


def check_selection_vs_oracle(sel: np.ndarray, cnt: np.ndarray, ref_sel: np.ndarray,
                              ref_cnt: np.ndarray, ref_scores: np.ndarray, nblocks: np.ndarray,
                              bound: np.ndarray = None, forced=None):
    """Same set as the oracle except inside the tie band around the K-th score of
    the competing (not forced) blocks.  ``bound`` (per block magnitude bound of
    the score) widens the band to 2 * SCORE_RTOL * the row's largest bound;
    ``forced(b)`` gives the forced block set of sequence b.
    Returns the number of rows whose sets differ (inside the band)."""
    B, Hkv, _ = sel.shape
    differing = 0
    for b in range(B):
        nb = int(nblocks[b])
        fb = forced(b) if forced else set()
        for j in range(Hkv):
            assert cnt[b, j] == ref_cnt[b, j]
            got = set(sel[b, j, :cnt[b, j]].tolist())
            want = set(ref_sel[b, j, :ref_cnt[b, j]].tolist())
            if got == want:
                continue
            differing += 1
            assert fb <= got, "a forced block is missing"
            sc = ref_scores[b, j, :nb]
            free = int(ref_cnt[b, j]) - len(fb)
            assert free > 0, f"b={b} j={j}: only forced blocks fit, yet the sets differ"
            comp = np.sort([sc[n] for n in range(nb) if n not in fb])[::-1]
            kth = comp[free - 1]
            band = TIE_BAND * abs(kth)
            if bound is not None:
                band = max(band, 2 * SCORE_RTOL * float(bound[b, j, :nb].max()))
            for n in got ^ want:
                assert abs(sc[n] - kth) <= band, (
                    f"block {n} (b={b}, j={j}) differs outside the tie band: "
                    f"score {sc[n]!r}, K-th {kth!r}, band {band:.3e}")
    return differing
