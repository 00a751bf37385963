"""fp64 CPU oracle for paged Top-K decode attention (ctypes binding of oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the library never imports it.  It shares no code with
the HIP path: inputs come from the seeded workload generator as numpy arrays,
are copied exactly to float64 here, and everything after that is oracle.c.

Functions (each computed as oracle.c states it):

* ``block_meta``      channel-wise min/max key per (page, KV head)   (KVDrive §2.2, §2.3)
* ``head_scores``     Quest score per (sequence, query head, block)  (KVDrive §2.2)
* ``group_scores``    max of the head scores over each GQA group
* ``topk``            rank-count Top-K, lower index wins ties, ascending output
* ``block_mean``      mean key per (page, KV head)             (KVDrive §2.3, §4)
* ``head_scores_mean``  q . mean key per (sequence, query head, block)
* ``select``          Top-K with the first / last tokens' blocks forced in  (KVDrive §9.1)
* ``fp8_encode`` / ``fp8_decode``  OCP FP8 E4M3 codes (round to nearest even, saturating)
* ``fp8_quantize``    per-(page, KV head) scaled E4M3 pages      (KVDrive §11; DirectKV review)
* ``fp8_dequantize``  decode(code) * scale
* ``block_lse``       ln sum exp(logits) of each attended block          (KVDrive §5.1)
* ``slot_mass``       eviction mass of each cache slot after a step
* ``cache_plan``      one step of the GPU block cache: hits, misses, victims
* ``tier_plan``       one step of the hot/cold tier policy: page heat, demotions,
                      promotions  (tiered-offload blog, page replacement; KVDrive §11)
* ``attention``       softmax decode attention, dense or over selected blocks
                      (Dual-Blade background; KVDrive §2.3 step 3)
* ``attention_splits``  the same on each contiguous chunk of the block list
* ``combine``         log-sum-exp merge of split partials
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# The pin tests' mutation check points this at a deliberately broken build of
# oracle.c to show that the pins catch the mistake.
_LIB_ENV = "KVD_ORACLE_LIB"
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get(_LIB_ENV) or _LIB_PATH
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    lib.oracle_num_threads.restype = _int
    lib.oracle_block_meta.argtypes = [_D, _int, _int, _int, _I, _I, _int, _D]
    lib.oracle_head_scores.argtypes = [_D, _D, _I, _I, _int, _int, _int, _int, _int, _int, _D]
    lib.oracle_group_scores.argtypes = [_D, _int, _int, _int, _int, _D]
    lib.oracle_block_mean.argtypes = [_D, _int, _int, _int, _I, _I, _int, _D]
    lib.oracle_head_scores_mean.argtypes = [_D, _D, _I, _I, _int, _int, _int, _int, _int, _int, _D]
    lib.oracle_select.argtypes = [_D, _I, _int, _int, _int, _int, _int, _int, _int, _I, _I]
    _U8 = ctypes.POINTER(ctypes.c_uint8)
    _F = ctypes.POINTER(ctypes.c_float)
    lib.oracle_fp8_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_decode.restype = ctypes.c_double
    lib.oracle_fp8_encode.argtypes = [ctypes.c_float]
    lib.oracle_fp8_encode.restype = ctypes.c_uint8
    lib.oracle_fp8_quantize.argtypes = [_D, _int, _int, _int, _I, _I, _int, _U8, _F, _int]
    lib.oracle_fp8_quantize.restype = None
    lib.oracle_int4_code.argtypes = [ctypes.c_float]
    lib.oracle_int4_code.restype = ctypes.c_int
    lib.oracle_int4_quantize.argtypes = [_D, _int, _int, _int, _I, _I, _int, _U8, _F, _int]
    lib.oracle_int4_quantize.restype = None
    lib.oracle_int4_unpack.argtypes = [_U8, _int]
    lib.oracle_int4_unpack.restype = ctypes.c_int
    lib.oracle_block_lse.argtypes = [_D, _D, _I, _I, _I, _I, _int, _int, _int, _int, _int, _int,
                                     _int, ctypes.c_double, _D]
    lib.oracle_block_lse.restype = None
    lib.oracle_slot_mass.argtypes = [_D, _D, _I, _I, _int, _int, _int, _int, _int, _D]
    lib.oracle_slot_mass.restype = None
    lib.oracle_cache_plan.argtypes = [_I, _I, _int, _int, _int, _int, _int, _I, _I, _F, _I, _I,
                                      _I, _I]
    lib.oracle_cache_plan.restype = None
    lib.oracle_tier_plan.argtypes = [_I, _I, _int, _I, _I, _int, _int, _int, _int,
                                     ctypes.c_float, ctypes.c_float, ctypes.c_float, _int, _int,
                                     _int, _F, _U8, _I, _I, _I, _I, _I]
    lib.oracle_tier_plan.restype = None
    lib.oracle_topk.argtypes = [_D, _I, _int, _int, _int, _int, _int, _I, _I]
    lib.oracle_attention.argtypes = [_D, _D, _D, _I, _I, _I, _I, _int, _int, _int, _int, _int,
                                     _int, _int, ctypes.c_double, _D, _D]
    lib.oracle_attention_splits.argtypes = [_D, _D, _D, _I, _I, _I, _I, _int, _int, _int, _int,
                                            _int, _int, _int, ctypes.c_double, _int, _D, _D, _D]
    lib.oracle_combine.argtypes = [_int, _int, _int, _int, _D, _D, _D, _D, _D]
    for f in ("oracle_block_meta", "oracle_head_scores", "oracle_group_scores", "oracle_topk",
              "oracle_block_mean", "oracle_head_scores_mean", "oracle_select",
              "oracle_attention", "oracle_attention_splits", "oracle_combine"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _pd(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_D)


def _pi(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_I)


def block_meta(k_pool, page_ids, valid_tokens, kmeta: Optional[np.ndarray] = None) -> np.ndarray:
    """kmeta [P, Hkv, 2, D] (0 = channel min, 1 = channel max) over each listed page's
    first ``valid_tokens`` slots.  Pages not listed keep the values of ``kmeta``
    (zeros if it is not given)."""
    k = _f64(k_pool)
    P, Hkv, bs, D = k.shape
    ids, val = _i32(page_ids), _i32(valid_tokens)
    out = np.zeros((P, Hkv, 2, D)) if kmeta is None else _f64(kmeta).copy()
    _load().oracle_block_meta(_pd(k), Hkv, bs, D, _pi(ids), _pi(val), len(ids), _pd(out))
    return out


def head_scores(q, kmeta, block_table, seq_lens, block_size: int) -> np.ndarray:
    """Quest score per (b, query head, logical block) [B, Hq, maxN]; -inf past N_b."""
    q, km = _f64(q), _f64(kmeta)
    bt, sl = _i32(block_table), _i32(seq_lens)
    B, Hq, D = q.shape
    Hkv = km.shape[1]
    maxN = bt.shape[1]
    out = np.empty((B, Hq, maxN))
    _load().oracle_head_scores(_pd(q), _pd(km), _pi(bt), _pi(sl), B, Hq, Hkv, D, block_size,
                               maxN, _pd(out))
    return out


def block_mean(k_pool, page_ids, valid_tokens, kmean: Optional[np.ndarray] = None) -> np.ndarray:
    """kmean [P, Hkv, D]: the average key of each listed page's first ``valid_tokens`` slots."""
    k = _f64(k_pool)
    P, Hkv, bs, D = k.shape
    ids, val = _i32(page_ids), _i32(valid_tokens)
    out = np.zeros((P, Hkv, D)) if kmean is None else _f64(kmean).copy()
    _load().oracle_block_mean(_pd(k), Hkv, bs, D, _pi(ids), _pi(val), len(ids), _pd(out))
    return out


def head_scores_mean(q, kmean, block_table, seq_lens, block_size: int) -> np.ndarray:
    """q . kmean per (b, query head, logical block) [B, Hq, maxN]; -inf past N_b."""
    q, km = _f64(q), _f64(kmean)
    bt, sl = _i32(block_table), _i32(seq_lens)
    B, Hq, D = q.shape
    Hkv = km.shape[1]
    maxN = bt.shape[1]
    out = np.empty((B, Hq, maxN))
    _load().oracle_head_scores_mean(_pd(q), _pd(km), _pi(bt), _pi(sl), B, Hq, Hkv, D, block_size,
                                    maxN, _pd(out))
    return out


def select(group_scores_, seq_lens, block_size: int, k: int, sink: int = 0, local: int = 0):
    """Selection with every block that holds one of the first ``sink`` or the last
    ``local`` tokens forced in:
    (sel int32 [B, Hkv, k] ascending, -1 padded;  sel_count int32 [B, Hkv])."""
    gs = _f64(group_scores_)
    sl = _i32(seq_lens)
    B, Hkv, maxN = gs.shape
    sel = np.empty((B, Hkv, k), dtype=np.int32)
    cnt = np.empty((B, Hkv), dtype=np.int32)
    _load().oracle_select(_pd(gs), _pi(sl), B, Hkv, maxN, block_size, k, sink, local, _pi(sel),
                          _pi(cnt))
    return sel, cnt


def fp8_decode(codes) -> np.ndarray:
    """Value of each FP8 E4M3 code (uint8 array), float64."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    table = np.array([lib.oracle_fp8_decode(i) for i in range(256)])
    return table[c]


def fp8_encode(values) -> np.ndarray:
    """E4M3 code of each float32 value (round to nearest even, saturating)."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float32)
    return np.array([lib.oracle_fp8_encode(float(x)) for x in v.ravel()],
                    dtype=np.uint8).reshape(v.shape)


def fp8_quantize(pool, page_ids, valid_tokens):
    """(codes uint8 [P, Hkv, bs, D], scales float32 [P, Hkv]) of the listed pages;
    pages not listed keep code 0 and scale 0."""
    x = _f64(pool)
    P, Hkv, bs, D = x.shape
    ids, val = _i32(page_ids), _i32(valid_tokens)
    codes = np.zeros((P, Hkv, bs, D), dtype=np.uint8)
    scales = np.zeros((P, Hkv), dtype=np.float32)
    _load().oracle_fp8_quantize(_pd(x), Hkv, bs, D, _pi(ids), _pi(val), len(ids),
                                codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                scales.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 1)
    return codes, scales


def fp8_dequantize(codes, scales) -> np.ndarray:
    """decode(code) * scale per (page, KV head), float64 [P, Hkv, bs, D]."""
    return fp8_decode(codes) * np.asarray(scales, np.float64)[:, :, None, None]


def int4_code(y: float) -> int:
    """The INT4 code of an fp32 quotient x / scale: round half to even, clamp to [-7, 7]."""
    return int(_load().oracle_int4_code(float(np.float32(y))))


def int4_quantize(pool, page_ids, valid_tokens):
    """(codes uint8 [P, Hkv, bs, D/2], scales float32 [P, Hkv]) of the listed pages;
    pages not listed keep code 0 and scale 0."""
    x = _f64(pool)
    P, Hkv, bs, D = x.shape
    ids, val = _i32(page_ids), _i32(valid_tokens)
    codes = np.zeros((P, Hkv, bs, D // 2), dtype=np.uint8)
    scales = np.zeros((P, Hkv), dtype=np.float32)
    _load().oracle_int4_quantize(_pd(x), Hkv, bs, D, _pi(ids), _pi(val), len(ids),
                                 codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                 scales.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 1)
    return codes, scales


def int4_unpack(codes) -> np.ndarray:
    """Signed codes int8 [..., D] of packed rows [..., D/2]: byte b holds channel 2b
    in its low nibble and 2b+1 in its high nibble, each 4-bit two's complement."""
    c = np.asarray(codes, dtype=np.uint8)
    nib = np.stack([c & 15, c >> 4], axis=-1).astype(np.int8)      # [..., D/2, 2]
    nib = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return nib.reshape(c.shape[:-1] + (2 * c.shape[-1],))


def int4_unpack_c(packed_row, c: int) -> int:
    """The oracle's C unpack of channel c of one packed row."""
    r = np.ascontiguousarray(packed_row, dtype=np.uint8)
    return int(_load().oracle_int4_unpack(r.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), c))


def int4_dequantize(codes, scales) -> np.ndarray:
    """n * scale per (page, KV head), float64 [P, Hkv, bs, D]."""
    return int4_unpack(codes).astype(np.float64) * np.asarray(scales, np.float64)[:, :, None, None]


def block_lse(q, k_pool, block_table, seq_lens, block_size: int, scale: float, sel=None,
              sel_count=None) -> np.ndarray:
    """ln of the summed exp-logits of every attended block [B, Hq, stride] (-inf past the list)."""
    q, k = _f64(q), _f64(k_pool)
    bt, sl = _i32(block_table), _i32(seq_lens)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    maxN = bt.shape[1]
    stride = maxN if sel is None else np.asarray(sel).shape[-1]
    out = np.empty((B, Hq, stride))
    s_, c_ = (None, None) if sel is None else (_i32(sel), _i32(sel_count))
    _load().oracle_block_lse(_pd(q), _pd(k), _pi(bt), _pi(sl), _pi(s_), _pi(c_), stride, B, Hq,
                             Hkv, D, block_size, maxN, scale, _pd(out))
    return out


def slot_mass(block_lse_, lse, sel_count, sel_slots, num_slots: int) -> np.ndarray:
    """Eviction mass per cache slot [B, Hkv, C]: max over the group's heads of
    exp(block_lse - lse) at the block's slot, 0 elsewhere."""
    bl, ls = _f64(block_lse_), _f64(lse)
    cnt, slots = _i32(sel_count), _i32(sel_slots)
    B, Hq, stride = bl.shape
    Hkv = slots.shape[1]
    out = np.empty((B, Hkv, num_slots))
    _load().oracle_slot_mass(_pd(bl), _pd(ls), _pi(cnt), _pi(slots), stride, B, Hq, Hkv,
                             num_slots, _pd(out))
    return out


def cache_plan(sel, sel_count, slot_block, block_slot, slot_mass_):
    """One cache step; returns (slot_block, block_slot, sel_slots, fetch_block,
    fetch_slot, fetch_count) with the maps updated (inputs are not modified)."""
    sl_ = _i32(sel)
    cnt = _i32(sel_count)
    sb = np.array(slot_block, dtype=np.int32, copy=True)
    bs_ = np.array(block_slot, dtype=np.int32, copy=True)
    mass = np.ascontiguousarray(slot_mass_, dtype=np.float32)
    B, Hkv, stride = sl_.shape
    C, maxN = sb.shape[-1], bs_.shape[-1]
    sel_slots = np.empty((B, Hkv, stride), np.int32)
    fb = np.empty((B, Hkv, stride), np.int32)
    fs = np.empty((B, Hkv, stride), np.int32)
    fc = np.empty((B, Hkv), np.int32)
    _load().oracle_cache_plan(_pi(sl_), _pi(cnt), stride, B, Hkv, maxN, C, _pi(sb), _pi(bs_),
                              mass.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _pi(sel_slots),
                              _pi(fb), _pi(fs), _pi(fc))
    return sb, bs_, sel_slots, fb, fs, fc


def tier_plan(sel, sel_count, block_table, seq_lens, block_size: int, decay: float,
              hot_above: float, cold_below: float, recent: int, cooldown: int, step: int,
              heat, tier, stamp):
    """One step of the tier policy; returns (heat, tier, stamp, demote, demote_count,
    promote, promote_count) with the page state updated (inputs are not modified).

    heat float32 [P], tier uint8 [P] (0 hot, 1 cold), stamp int32 [P];
    demote / promote int32 [B, maxN] in block order, -1 padded."""
    sl_, cnt = _i32(sel), _i32(sel_count)
    bt, sl = _i32(block_table), _i32(seq_lens)
    h = np.array(heat, dtype=np.float32, copy=True)
    t = np.array(tier, dtype=np.uint8, copy=True)
    st = np.array(stamp, dtype=np.int32, copy=True)
    B, Hkv, stride = sl_.shape
    maxN = bt.shape[1]
    # filled with a value the oracle never writes, so that a row it leaves unset shows
    dem = np.full((B, maxN), np.iinfo(np.int32).max, np.int32)
    pro = np.full((B, maxN), np.iinfo(np.int32).max, np.int32)
    dc = np.full(B, -7, np.int32)
    pc = np.full(B, -7, np.int32)
    _load().oracle_tier_plan(_pi(sl_), _pi(cnt), stride, _pi(bt), _pi(sl), B, Hkv, maxN,
                             block_size, float(decay), float(hot_above), float(cold_below),
                             recent, cooldown, step,
                             h.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                             t.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), _pi(st),
                             _pi(dem), _pi(dc), _pi(pro), _pi(pc))
    return h, t, st, dem, dc, pro, pc


def group_scores(head_scores_, num_kv_heads: int) -> np.ndarray:
    """Group score [B, Hkv, maxN]: max over the query heads of each KV head."""
    hs = _f64(head_scores_)
    B, Hq, maxN = hs.shape
    out = np.empty((B, num_kv_heads, maxN))
    _load().oracle_group_scores(_pd(hs), B, Hq, num_kv_heads, maxN, _pd(out))
    return out


def topk(group_scores_, seq_lens, block_size: int, k: int):
    """(sel int32 [B, Hkv, k] ascending, -1 padded;  sel_count int32 [B, Hkv])."""
    gs = _f64(group_scores_)
    sl = _i32(seq_lens)
    B, Hkv, maxN = gs.shape
    sel = np.empty((B, Hkv, k), dtype=np.int32)
    cnt = np.empty((B, Hkv), dtype=np.int32)
    _load().oracle_topk(_pd(gs), _pi(sl), B, Hkv, maxN, block_size, k, _pi(sel), _pi(cnt))
    return sel, cnt


def attention(q, k_pool, v_pool, block_table, seq_lens, scale: float,
              sel=None, sel_count=None):
    """(out [B, Hq, D], lse [B, Hq]) of decode attention; dense when ``sel`` is None."""
    q, k, v = _f64(q), _f64(k_pool), _f64(v_pool)
    bt, sl = _i32(block_table), _i32(seq_lens)
    B, Hq, D = q.shape
    _, Hkv, bs, _ = k.shape
    maxN = bt.shape[1]
    s = None if sel is None else _i32(sel)
    c = None if sel_count is None else _i32(sel_count)
    stride = 0 if s is None else s.shape[-1]
    out = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    _load().oracle_attention(_pd(q), _pd(k), _pd(v), _pi(bt), _pi(sl), _pi(s), _pi(c), stride,
                             B, Hq, Hkv, D, bs, maxN, float(scale), _pd(out), _pd(lse))
    return out, lse


def attention_splits(q, k_pool, v_pool, block_table, seq_lens, scale: float, num_splits: int,
                     sel=None, sel_count=None):
    """(part_o [B, Hq, S, D], part_m [B, Hq, S], part_l [B, Hq, S]) split partials."""
    q, k, v = _f64(q), _f64(k_pool), _f64(v_pool)
    bt, sl = _i32(block_table), _i32(seq_lens)
    B, Hq, D = q.shape
    _, Hkv, bs, _ = k.shape
    maxN = bt.shape[1]
    s = None if sel is None else _i32(sel)
    c = None if sel_count is None else _i32(sel_count)
    stride = 0 if s is None else s.shape[-1]
    S = int(num_splits)
    po = np.empty((B, Hq, S, D))
    pm = np.empty((B, Hq, S))
    pl = np.empty((B, Hq, S))
    _load().oracle_attention_splits(_pd(q), _pd(k), _pd(v), _pi(bt), _pi(sl), _pi(s), _pi(c),
                                    stride, B, Hq, Hkv, D, bs, maxN, float(scale), S,
                                    _pd(po), _pd(pm), _pd(pl))
    return po, pm, pl


def combine(part_o, part_m, part_l):
    """(out [B, Hq, D], lse [B, Hq]) from split partials."""
    po, pm, pl = _f64(part_o), _f64(part_m), _f64(part_l)
    B, Hq, S, D = po.shape
    out = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    _load().oracle_combine(B, Hq, D, S, _pd(po), _pd(pm), _pd(pl), _pd(out), _pd(lse))
    return out, lse


def sparse_step(q, k_pool, block_table, seq_lens, block_size: int, k: int, kmeta=None):
    """Convenience: meta (if not given) -> head scores -> group scores -> Top-K.

    Returns (kmeta, head_scores, group_scores, sel, sel_count)."""
    qa = _f64(q)
    Hkv = np.asarray(k_pool).shape[1]
    if kmeta is None:
        bt, sl = _i32(block_table), _i32(seq_lens)
        ids, val = [], []
        for b in range(bt.shape[0]):
            nb = -(-int(sl[b]) // block_size)
            for n in range(nb):
                ids.append(bt[b, n])
                val.append(min(block_size, int(sl[b]) - n * block_size))
        kmeta = block_meta(k_pool, ids, val)
    hs = head_scores(qa, kmeta, block_table, seq_lens, block_size)
    gs = group_scores(hs, Hkv)
    sel, cnt = topk(gs, seq_lens, block_size, k)
    return kmeta, hs, gs, sel, cnt
