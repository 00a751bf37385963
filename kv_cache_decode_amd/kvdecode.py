"""Thin Python binding of the C ABI in include/kvdecode.h (ctypes).

Argument marshalling only: every function takes the same arguments as its C
counterpart, with device buffers given as torch tensors (their data_ptr is
passed) or as raw integer addresses, and raises :class:`KVError` when the
library returns a status other than KV_OK.  All compute runs in
``libkvdecode.so``; importing this module without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVD_LIBRARY_PATH selects another build of the same library (for example one
# compiled with different launch-shape macros)
LIB_PATH = os.environ.get("KVD_LIBRARY_PATH") or os.path.join(_HERE, "libkvdecode.so")

KV_OK, KV_ERR_INVALID_ARG, KV_ERR_UNSUPPORTED, KV_ERR_ALIGNMENT, KV_ERR_WORKSPACE, KV_ERR_HIP = range(6)
KV_F32, KV_F16, KV_BF16 = 0, 1, 2
KV_INDEX_MINMAX, KV_INDEX_MEAN = 0, 1
KV_FLAG_HOST_KV = 0x1
KV_HOST_COHERENT, KV_HOST_NONCOHERENT = 0x0, 0x1
DTYPE_CODES = {"f32": KV_F32, "f16": KV_F16, "bf16": KV_BF16}

# every symbol the header declares
EXPORTS = (
    "kv_block_meta_build", "kv_block_mean_build", "kv_append_token", "kv_decode_select",
    "kv_decode_score", "kv_select_decode_attn",
    "kv_score_topk_workspace_size", "kv_block_score_topk", "kv_max_forced_blocks",
    "kv_block_select", "kv_block_select_no_alloc", "kv_auto_num_splits",
    "kv_auto_select_splits", "kv_auto_num_splits_fp8",
    "kv_auto_num_splits_tiered", "kv_paged_decode_attn", "kv_decode_combine",
    "kv_quantize_pages_fp8", "kv_paged_decode_attn_fp8", "kv_quantize_pages_int4",
    "kv_paged_decode_attn_int4", "kv_paged_decode_attn_tiered",
    "kv_tiered_split_workspace_size", "kv_paged_decode_attn_tiered_split", "kv_tier_plan",
    "kv_cache_plan",
    "kv_cache_fetch", "kv_cache_fetch_codes", "kv_cached_decode_attn_codes",
    "kv_cached_decode_attn_fetch", "kv_cached_decode_attn_fetch_codes",
    "kv_cached_decode_attn", "kv_cache_slot_mass", "kv_check_tables", "kv_probe_stream_read",
    "kv_probe_gather_read", "kv_probe_fp8_convert", "kv_host_alloc", "kv_host_free",
    "kv_status_string", "kv_last_error_message",
)


class KVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class KVShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


def make_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, num_pages,
               dtype, block_size=16, flags=0) -> KVShape:
    code = DTYPE_CODES.get(dtype, dtype)
    return KVShape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   num_pages, code, flags)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run kv_cache_decode_amd/build.py "
                          "(or __graft_entry__.build()) first")
    # One HIP runtime per process: torch ships its own libamdhip64 under the
    # same soname, so loading torch first makes the library bind to that
    # runtime instead of pulling in a second copy from the ROCm install (two
    # runtimes in one process do not share devices, streams or allocations).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_float
    S = ctypes.POINTER(KVShape)
    sig = {
        "kv_block_meta_build": (I32, [S, P, P, P, I32, P, P]),
        "kv_block_mean_build": (I32, [S, P, P, P, I32, P, P]),
        "kv_append_token": (I32, [S, P, P, P, P, P, P, P, P, P]),
        "kv_max_forced_blocks": (I32, [S, I32, I32]),
        "kv_decode_select": (I32, [S, I32, P, P, P, P, P, P, P, P, P, I32, I32, I32, P, P, P, P,
                                   SZ, P]),
        "kv_block_select": (I32, [S, I32, P, P, P, P, I32, I32, I32, P, P, P, P, SZ, P]),
        "kv_decode_score": (I32, [S, I32, P, P, P, P, P, P, P, P, P, P, P]),
        "kv_select_decode_attn": (I32, [S, P, P, P, I32, I32, I32, P, P, P, F, I32, P, P, P, P, P,
                                        P]),
        "kv_block_select_no_alloc": (I32, [S, I32, P, P, P, P, I32, I32, I32, P, P, P]),
        "kv_score_topk_workspace_size": (SZ, [S, I32]),
        "kv_block_score_topk": (I32, [S, P, P, P, P, I32, P, P, P, P, SZ, P]),
        "kv_auto_num_splits": (I32, [S, I32]),
        "kv_auto_select_splits": (I32, [S, I32]),
        "kv_auto_num_splits_fp8": (I32, [S, I32]),
        "kv_auto_num_splits_tiered": (I32, [S, I32]),
        "kv_paged_decode_attn": (I32, [S, P, P, P, P, P, P, P, I32, F, I32, P, P, P, P]),
        "kv_decode_combine": (I32, [S, I32, P, P, P, P, P, P]),
        "kv_quantize_pages_fp8": (I32, [S, P, P, P, P, I32, P, P, P, P]),
        "kv_paged_decode_attn_fp8": (I32, [S, P, P, P, P, P, P, P, P, I32, F, I32, P, P, P, P]),
        "kv_quantize_pages_int4": (I32, [S, P, P, P, P, I32, P, P, P, P]),
        "kv_paged_decode_attn_int4": (I32, [S, P, P, P, P, P, P, P, P, I32, F, I32, P, P, P, P]),
        "kv_paged_decode_attn_tiered": (I32, [S, P, P, P, P, P, P, I32, P, P, P, P, P, I32, F, I32,
                                              P, P, P, P]),
        "kv_tiered_split_workspace_size": (SZ, [S, I32]),
        "kv_paged_decode_attn_tiered_split": (I32, [S, P, P, P, P, P, P, I32, P, P, P, P, P, I32,
                                                    F, I32, I32, P, P, P, P, SZ, P]),
        "kv_tier_plan": (I32, [S, P, P, I32, P, P, F, F, F, I32, I32, I32, P, P, P, P, P, P, P,
                               P]),
        "kv_cache_plan": (I32, [S, I32, P, P, I32, P, P, P, P, P, P, P, P]),
        "kv_cache_fetch": (I32, [S, I32, P, P, P, P, P, P, I32, P, P, P]),
        "kv_cached_decode_attn": (I32, [S, I32, P, P, P, P, P, P, P, I32, F, I32, P, P, P, P, P]),
        "kv_cache_fetch_codes": (I32, [S, I32, I32, P, P, P, P, P, P, P, I32, P, P, P, P]),
        "kv_cached_decode_attn_codes": (I32, [S, I32, I32, P, P, P, P, P, P, P, P, I32, F, I32,
                                              P, P, P, P, P]),
        "kv_cached_decode_attn_fetch": (I32, [S, I32, P, P, P, P, P, P, P, P, P, P, P, P, I32, F,
                                              I32, P, P, P, P, P]),
        "kv_cached_decode_attn_fetch_codes": (I32, [S, I32, I32, P, P, P, P, P, P, P, P, P, P, P,
                                                    P, P, P, I32, F, I32, P, P, P, P, P]),
        "kv_cache_slot_mass": (I32, [S, I32, P, P, P, P, I32, P, P]),
        "kv_check_tables": (I32, [S, P, P, P, P, I32, P, P]),
        "kv_probe_stream_read": (I32, [P, SZ, P, P]),
        "kv_probe_gather_read": (I32, [S, P, P, P, P, I32, P, P]),
        "kv_probe_fp8_convert": (I32, [P, P, P]),
        "kv_host_alloc": (I32, [SZ, U32, ctypes.POINTER(P), ctypes.POINTER(P)]),
        "kv_host_free": (I32, [P]),
        "kv_status_string": (ctypes.c_char_p, [I32]),
        "kv_last_error_message": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.kv_status_string(status).decode()


def last_error_message() -> str:
    return _lib.kv_last_error_message().decode()


def _check(status: int) -> None:
    if status != KV_OK:
        raise KVError(status, last_error_message())


Buf = Union[None, int, "torch.Tensor"]  # noqa: F821


def _p(x: Buf, need: int = 0, what: str = "buffer", i32: bool = False) -> Optional[int]:
    """The address the C ABI receives for x: None, an int (a device address the
    caller vouches for, such as the one kv_host_alloc returns), or a torch
    tensor, which must be a contiguous tensor in GPU memory of at least `need`
    bytes (int32 where the ABI takes integers).  The library can check only
    null pointers and alignment, and a bad address reaches a kernel."""
    if x is None or isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    if not x.is_cuda:
        raise ValueError(f"{what}: a tensor in GPU memory is required (got one on {x.device}); "
                         "host memory goes in as the device address kv_host_alloc returns")
    if i32 and x.dtype != _torch().int32:
        raise ValueError(f"{what}: int32 required (got {x.dtype})")
    have = x.numel() * x.element_size()
    if have < need:
        raise ValueError(f"{what}: {have} bytes, the shape needs {need}")
    return x.data_ptr()


def _torch():
    import torch
    return torch


class _Lay:
    """Byte counts of the arrays a kv_shape describes."""

    def __init__(self, s: KVShape):
        self.eb = 4 if s.dtype == KV_F32 else 2
        self.B, self.Hq, self.Hkv, self.D = s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim
        self.P, self.maxN, self.bs = s.num_pages, s.max_blocks_per_seq, s.block_size
        self.q = self.B * self.Hq * self.D * self.eb
        self.pool = self.P * self.Hkv * self.bs * self.D * self.eb
        self.kmeta = self.P * self.Hkv * 2 * self.D * self.eb
        self.kmean = self.P * self.Hkv * self.D * 4
        self.table = self.B * self.maxN * 4
        self.lens = self.B * 4
        self.scores = self.B * self.Hkv * self.maxN * 4
        self.rows = self.B * self.Hkv * 4
        self.token = self.B * self.Hkv * self.D * self.eb

    def sel(self, k: int) -> int:
        return self.B * self.Hkv * max(k, 0) * 4

    def index(self, kind: int) -> int:
        return self.kmean if kind == KV_INDEX_MEAN else self.kmeta

    def parts(self, splits: int):
        n = self.B * self.Hq * max(splits, 0)
        return n * self.D * 4, n * 4


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def kv_block_meta_build(shape: KVShape, k_cache: Buf, page_ids: Buf, page_valid_tokens: Buf,
                        num_page_ids: int, kmeta: Buf, stream=None) -> None:
    L, n = _Lay(shape), max(num_page_ids, 0) * 4
    _check(_lib.kv_block_meta_build(ctypes.byref(shape), _p(k_cache, L.pool, "k_cache"),
                                    _p(page_ids, n, "page_ids", True),
                                    _p(page_valid_tokens, n, "page_valid_tokens", True),
                                    num_page_ids, _p(kmeta, L.kmeta, "kmeta"), _stream(stream)))


def kv_block_mean_build(shape: KVShape, k_cache: Buf, page_ids: Buf, page_valid_tokens: Buf,
                        num_page_ids: int, kmean: Buf, stream=None) -> None:
    L, n = _Lay(shape), max(num_page_ids, 0) * 4
    _check(_lib.kv_block_mean_build(ctypes.byref(shape), _p(k_cache, L.pool, "k_cache"),
                                    _p(page_ids, n, "page_ids", True),
                                    _p(page_valid_tokens, n, "page_valid_tokens", True),
                                    num_page_ids, _p(kmean, L.kmean, "kmean"), _stream(stream)))


def kv_append_token(shape: KVShape, k_new: Buf, v_new: Buf, block_table: Buf, seq_lens: Buf,
                    k_cache: Buf, v_cache: Buf, kmeta: Buf = None, kmean: Buf = None,
                    stream=None) -> None:
    L = _Lay(shape)
    _check(_lib.kv_append_token(ctypes.byref(shape), _p(k_new, L.token, "k_new"),
                                _p(v_new, L.token, "v_new"),
                                _p(block_table, L.table, "block_table", True),
                                _p(seq_lens, L.lens, "seq_lens", True),
                                _p(k_cache, L.pool, "k_cache"), _p(v_cache, L.pool, "v_cache"),
                                _p(kmeta, L.kmeta, "kmeta"), _p(kmean, L.kmean, "kmean"),
                                _stream(stream)))


def kv_decode_select(shape: KVShape, index_kind: int, q: Buf, k_new: Buf, v_new: Buf,
                     block_table: Buf, seq_lens: Buf, k_cache: Buf, v_cache: Buf, kmeta: Buf,
                     kmean: Buf, topk_blocks: int, sink_tokens: int, local_tokens: int,
                     scores_out: Buf, sel_blocks: Buf, sel_count: Buf, workspace: Buf = None,
                     workspace_bytes: int = 0, stream=None) -> None:
    L = _Lay(shape)
    _check(_lib.kv_decode_select(ctypes.byref(shape), index_kind, _p(q, L.q, "q"),
                                 _p(k_new, L.token, "k_new"), _p(v_new, L.token, "v_new"),
                                 _p(block_table, L.table, "block_table", True),
                                 _p(seq_lens, L.lens, "seq_lens", True),
                                 _p(k_cache, L.pool, "k_cache"), _p(v_cache, L.pool, "v_cache"),
                                 _p(kmeta, L.kmeta, "kmeta"), _p(kmean, L.kmean, "kmean"),
                                 topk_blocks, sink_tokens, local_tokens,
                                 _p(scores_out, L.scores, "scores_out"),
                                 _p(sel_blocks, L.sel(topk_blocks), "sel_blocks", True),
                                 _p(sel_count, L.rows, "sel_count", True),
                                 _p(workspace, workspace_bytes, "workspace"), workspace_bytes,
                                 _stream(stream)))


def kv_decode_score(shape: KVShape, index_kind: int, q: Buf, k_new: Buf, v_new: Buf,
                    block_table: Buf, seq_lens: Buf, k_cache: Buf, v_cache: Buf, kmeta: Buf,
                    kmean: Buf, scores_out: Buf, stream=None) -> None:
    L = _Lay(shape)
    _check(_lib.kv_decode_score(ctypes.byref(shape), index_kind, _p(q, L.q, "q"),
                                _p(k_new, L.token, "k_new"), _p(v_new, L.token, "v_new"),
                                _p(block_table, L.table, "block_table", True),
                                _p(seq_lens, L.lens, "seq_lens", True),
                                _p(k_cache, L.pool, "k_cache"), _p(v_cache, L.pool, "v_cache"),
                                _p(kmeta, L.kmeta, "kmeta"), _p(kmean, L.kmean, "kmean"),
                                _p(scores_out, L.scores, "scores_out"), _stream(stream)))


def kv_select_decode_attn(shape: KVShape, scores: Buf, block_table: Buf, seq_lens: Buf,
                          topk_blocks: int, sink_tokens: int, local_tokens: int, q: Buf,
                          k_cache: Buf, v_cache: Buf, scale: float, num_splits: int,
                          sel_blocks: Buf, sel_count: Buf, part_o: Buf, part_m: Buf,
                          part_l: Buf, stream=None) -> None:
    L = _Lay(shape)
    po, pm = L.parts(num_splits)
    _check(_lib.kv_select_decode_attn(ctypes.byref(shape), _p(scores, L.scores, "scores"),
                                      _p(block_table, L.table, "block_table", True),
                                      _p(seq_lens, L.lens, "seq_lens", True), topk_blocks,
                                      sink_tokens, local_tokens, _p(q, L.q, "q"),
                                      _p(k_cache, L.pool, "k_cache"),
                                      _p(v_cache, L.pool, "v_cache"), scale, num_splits,
                                      _p(sel_blocks, L.sel(topk_blocks), "sel_blocks", True),
                                      _p(sel_count, L.rows, "sel_count", True),
                                      _p(part_o, po, "part_o"), _p(part_m, pm, "part_m"),
                                      _p(part_l, pm, "part_l"), _stream(stream)))


def kv_score_topk_workspace_size(shape: KVShape, topk_blocks: int) -> int:
    return int(_lib.kv_score_topk_workspace_size(ctypes.byref(shape), topk_blocks))


def kv_block_score_topk(shape: KVShape, q: Buf, kmeta: Buf, block_table: Buf, seq_lens: Buf,
                        topk_blocks: int, scores_out: Buf, sel_blocks: Buf, sel_count: Buf,
                        workspace: Buf = None, workspace_bytes: int = 0, stream=None) -> None:
    L = _Lay(shape)
    _check(_lib.kv_block_score_topk(ctypes.byref(shape), _p(q, L.q, "q"),
                                    _p(kmeta, L.kmeta, "kmeta"),
                                    _p(block_table, L.table, "block_table", True),
                                    _p(seq_lens, L.lens, "seq_lens", True), topk_blocks,
                                    _p(scores_out, L.scores, "scores_out"),
                                    _p(sel_blocks, L.sel(topk_blocks), "sel_blocks", True),
                                    _p(sel_count, L.rows, "sel_count", True),
                                    _p(workspace, workspace_bytes, "workspace"), workspace_bytes,
                                    _stream(stream)))


def kv_auto_num_splits_fp8(shape: KVShape, blocks_per_unit: int) -> int:
    return int(_lib.kv_auto_num_splits_fp8(ctypes.byref(shape), blocks_per_unit))


def kv_auto_num_splits_tiered(shape: KVShape, blocks_per_unit: int) -> int:
    return int(_lib.kv_auto_num_splits_tiered(ctypes.byref(shape), blocks_per_unit))


def kv_max_forced_blocks(shape: KVShape, sink_tokens: int, local_tokens: int) -> int:
    return int(_lib.kv_max_forced_blocks(ctypes.byref(shape), sink_tokens, local_tokens))


def kv_block_select(shape: KVShape, index_kind: int, q: Buf, index: Buf, block_table: Buf,
                    seq_lens: Buf, topk_blocks: int, sink_tokens: int, local_tokens: int,
                    scores_out: Buf, sel_blocks: Buf, sel_count: Buf, workspace: Buf = None,
                    workspace_bytes: int = 0, stream=None) -> None:
    L = _Lay(shape)
    _check(_lib.kv_block_select(ctypes.byref(shape), index_kind, _p(q, L.q, "q"),
                                _p(index, L.index(index_kind), "index"),
                                _p(block_table, L.table, "block_table", True),
                                _p(seq_lens, L.lens, "seq_lens", True), topk_blocks, sink_tokens,
                                local_tokens, _p(scores_out, L.scores, "scores_out"),
                                _p(sel_blocks, L.sel(topk_blocks), "sel_blocks", True),
                                _p(sel_count, L.rows, "sel_count", True),
                                _p(workspace, workspace_bytes, "workspace"), workspace_bytes,
                                _stream(stream)))


def kv_block_select_no_alloc(shape: KVShape, index_kind: int, q: Buf, index: Buf,
                             block_table: Buf, seq_lens: Buf, topk_blocks: int, sink_tokens: int,
                             local_tokens: int, sel_blocks: Buf, sel_count: Buf,
                             stream=None) -> None:
    L = _Lay(shape)
    _check(_lib.kv_block_select_no_alloc(ctypes.byref(shape), index_kind, _p(q, L.q, "q"),
                                         _p(index, L.index(index_kind), "index"),
                                         _p(block_table, L.table, "block_table", True),
                                         _p(seq_lens, L.lens, "seq_lens", True), topk_blocks,
                                         sink_tokens, local_tokens,
                                         _p(sel_blocks, L.sel(topk_blocks), "sel_blocks", True),
                                         _p(sel_count, L.rows, "sel_count", True),
                                         _stream(stream)))


def kv_auto_num_splits(shape: KVShape, blocks_per_unit: int) -> int:
    return int(_lib.kv_auto_num_splits(ctypes.byref(shape), blocks_per_unit))


def kv_auto_select_splits(shape: KVShape, topk_blocks: int) -> int:
    return int(_lib.kv_auto_select_splits(ctypes.byref(shape), topk_blocks))


def kv_paged_decode_attn(shape: KVShape, q: Buf, k_cache: Buf, v_cache: Buf, block_table: Buf,
                         seq_lens: Buf, sel_blocks: Buf, sel_count: Buf, sel_stride: int,
                         scale: float, num_splits: int, part_o: Buf, part_m: Buf, part_l: Buf,
                         stream=None) -> None:
    L = _Lay(shape)
    po, pm = L.parts(num_splits)
    _check(_lib.kv_paged_decode_attn(ctypes.byref(shape), _p(q, L.q, "q"),
                                     _p(k_cache, L.pool, "k_cache"), _p(v_cache, L.pool, "v_cache"),
                                     _p(block_table, L.table, "block_table", True),
                                     _p(seq_lens, L.lens, "seq_lens", True),
                                     _p(sel_blocks, L.sel(sel_stride), "sel_blocks", True),
                                     _p(sel_count, L.rows, "sel_count", True), sel_stride, scale,
                                     num_splits, _p(part_o, po, "part_o"), _p(part_m, pm, "part_m"),
                                     _p(part_l, pm, "part_l"), _stream(stream)))


def kv_decode_combine(shape: KVShape, num_splits: int, part_o: Buf, part_m: Buf, part_l: Buf,
                      out: Buf, lse_out: Buf = None, stream=None) -> None:
    L = _Lay(shape)
    po, pm = L.parts(num_splits)
    _check(_lib.kv_decode_combine(ctypes.byref(shape), num_splits, _p(part_o, po, "part_o"),
                                  _p(part_m, pm, "part_m"), _p(part_l, pm, "part_l"),
                                  _p(out, L.B * L.Hq * L.D * 4, "out"),
                                  _p(lse_out, L.B * L.Hq * 4, "lse_out"), _stream(stream)))


def kv_quantize_pages_fp8(shape: KVShape, k_cache: Buf, v_cache: Buf, page_ids: Buf,
                          page_valid_tokens: Buf, num_page_ids: int, k_fp8: Buf, v_fp8: Buf,
                          kv_scales: Buf, stream=None) -> None:
    _check(_lib.kv_quantize_pages_fp8(ctypes.byref(shape), _p(k_cache), _p(v_cache), _p(page_ids),
                                      _p(page_valid_tokens), num_page_ids, _p(k_fp8), _p(v_fp8),
                                      _p(kv_scales), _stream(stream)))


def kv_paged_decode_attn_fp8(shape: KVShape, q: Buf, k_fp8: Buf, v_fp8: Buf, kv_scales: Buf,
                             block_table: Buf, seq_lens: Buf, sel_blocks: Buf, sel_count: Buf,
                             sel_stride: int, scale: float, num_splits: int, part_o: Buf,
                             part_m: Buf, part_l: Buf, stream=None) -> None:
    _check(_lib.kv_paged_decode_attn_fp8(ctypes.byref(shape), _p(q), _p(k_fp8), _p(v_fp8),
                                         _p(kv_scales), _p(block_table), _p(seq_lens),
                                         _p(sel_blocks), _p(sel_count), sel_stride, scale,
                                         num_splits, _p(part_o), _p(part_m), _p(part_l),
                                         _stream(stream)))


def kv_quantize_pages_int4(shape: KVShape, k_cache: Buf, v_cache: Buf, page_ids: Buf,
                           page_valid_tokens: Buf, num_page_ids: int, k_int4: Buf, v_int4: Buf,
                           kv_scales: Buf, stream=None) -> None:
    _check(_lib.kv_quantize_pages_int4(ctypes.byref(shape), _p(k_cache), _p(v_cache),
                                       _p(page_ids), _p(page_valid_tokens), num_page_ids,
                                       _p(k_int4), _p(v_int4), _p(kv_scales), _stream(stream)))


def kv_paged_decode_attn_int4(shape: KVShape, q: Buf, k_int4: Buf, v_int4: Buf, kv_scales: Buf,
                              block_table: Buf, seq_lens: Buf, sel_blocks: Buf, sel_count: Buf,
                              sel_stride: int, scale: float, num_splits: int, part_o: Buf,
                              part_m: Buf, part_l: Buf, stream=None) -> None:
    _check(_lib.kv_paged_decode_attn_int4(ctypes.byref(shape), _p(q), _p(k_int4), _p(v_int4),
                                          _p(kv_scales), _p(block_table), _p(seq_lens),
                                          _p(sel_blocks), _p(sel_count), sel_stride, scale,
                                          num_splits, _p(part_o), _p(part_m), _p(part_l),
                                          _stream(stream)))


KV_COLD_FP8 = 8
KV_COLD_INT4 = 4


def kv_paged_decode_attn_tiered(shape: KVShape, q: Buf, k_cache: Buf, v_cache: Buf, k_cold: Buf,
                                v_cold: Buf, kv_scales: Buf, cold_format: int, page_tier: Buf,
                                block_table: Buf, seq_lens: Buf, sel_blocks: Buf, sel_count: Buf,
                                sel_stride: int, scale: float, num_splits: int, part_o: Buf,
                                part_m: Buf, part_l: Buf, stream=None) -> None:
    _check(_lib.kv_paged_decode_attn_tiered(ctypes.byref(shape), _p(q), _p(k_cache), _p(v_cache),
                                            _p(k_cold), _p(v_cold), _p(kv_scales), cold_format,
                                            _p(page_tier), _p(block_table), _p(seq_lens),
                                            _p(sel_blocks), _p(sel_count), sel_stride, scale,
                                            num_splits, _p(part_o), _p(part_m), _p(part_l),
                                            _stream(stream)))


def kv_tiered_split_workspace_size(shape: KVShape, sel_stride: int) -> int:
    return int(_lib.kv_tiered_split_workspace_size(ctypes.byref(shape), sel_stride))


def kv_paged_decode_attn_tiered_split(shape: KVShape, q: Buf, k_cache: Buf, v_cache: Buf,
                                      k_cold: Buf, v_cold: Buf, kv_scales: Buf, cold_format: int,
                                      page_tier: Buf, block_table: Buf, seq_lens: Buf,
                                      sel_blocks: Buf, sel_count: Buf, sel_stride: int,
                                      scale: float, num_splits_hot: int, num_splits_cold: int,
                                      part_o: Buf, part_m: Buf, part_l: Buf, workspace: Buf,
                                      workspace_bytes: int, stream=None) -> None:
    _check(_lib.kv_paged_decode_attn_tiered_split(
        ctypes.byref(shape), _p(q), _p(k_cache), _p(v_cache), _p(k_cold), _p(v_cold),
        _p(kv_scales), cold_format, _p(page_tier), _p(block_table), _p(seq_lens),
        _p(sel_blocks), _p(sel_count), sel_stride, scale, num_splits_hot, num_splits_cold,
        _p(part_o), _p(part_m), _p(part_l), _p(workspace), workspace_bytes, _stream(stream)))


def kv_tier_plan(shape: KVShape, sel_blocks: Buf, sel_count: Buf, sel_stride: int,
                 block_table: Buf, seq_lens: Buf, decay: float, hot_above: float,
                 cold_below: float, recent_tokens: int, cooldown_steps: int, step: int,
                 page_heat: Buf, page_tier: Buf, page_stamp: Buf, demote: Buf, demote_count: Buf,
                 promote: Buf, promote_count: Buf, stream=None) -> None:
    L = _Lay(shape)
    lists = L.B * L.maxN * 4
    _check(_lib.kv_tier_plan(ctypes.byref(shape), _p(sel_blocks, L.sel(sel_stride), "sel_blocks", True),
                             _p(sel_count, L.rows, "sel_count", True), sel_stride,
                             _p(block_table, L.table, "block_table", True),
                             _p(seq_lens, L.lens, "seq_lens", True), decay, hot_above, cold_below,
                             recent_tokens, cooldown_steps, step, _p(page_heat, L.P * 4, "page_heat"),
                             _p(page_tier, L.P, "page_tier"),
                             _p(page_stamp, L.P * 4, "page_stamp", True),
                             _p(demote, lists, "demote", True),
                             _p(demote_count, L.B * 4, "demote_count", True),
                             _p(promote, lists, "promote", True),
                             _p(promote_count, L.B * 4, "promote_count", True), _stream(stream)))


def kv_cache_plan(shape: KVShape, num_slots: int, sel_blocks: Buf, sel_count: Buf,
                  sel_stride: int, slot_block: Buf, block_slot: Buf, slot_mass: Buf,
                  sel_slots: Buf, fetch_block: Buf, fetch_slot: Buf, fetch_count: Buf,
                  stream=None) -> None:
    _check(_lib.kv_cache_plan(ctypes.byref(shape), num_slots, _p(sel_blocks), _p(sel_count),
                              sel_stride, _p(slot_block), _p(block_slot), _p(slot_mass),
                              _p(sel_slots), _p(fetch_block), _p(fetch_slot), _p(fetch_count),
                              _stream(stream)))


def kv_cache_fetch(shape: KVShape, num_slots: int, k_cache: Buf, v_cache: Buf,
                   block_table: Buf, fetch_block: Buf, fetch_slot: Buf, fetch_count: Buf,
                   fetch_stride: int, cache_k: Buf, cache_v: Buf, stream=None) -> None:
    _check(_lib.kv_cache_fetch(ctypes.byref(shape), num_slots, _p(k_cache), _p(v_cache),
                               _p(block_table), _p(fetch_block), _p(fetch_slot), _p(fetch_count),
                               fetch_stride, _p(cache_k), _p(cache_v), _stream(stream)))


def kv_cached_decode_attn(shape: KVShape, num_slots: int, q: Buf, cache_k: Buf, cache_v: Buf,
                          seq_lens: Buf, sel_blocks: Buf, sel_count: Buf, sel_slots: Buf,
                          sel_stride: int, scale: float, num_splits: int, part_o: Buf,
                          part_m: Buf, part_l: Buf, block_lse: Buf = None, stream=None) -> None:
    _check(_lib.kv_cached_decode_attn(ctypes.byref(shape), num_slots, _p(q), _p(cache_k),
                                      _p(cache_v), _p(seq_lens), _p(sel_blocks), _p(sel_count),
                                      _p(sel_slots), sel_stride, scale, num_splits, _p(part_o),
                                      _p(part_m), _p(part_l), _p(block_lse), _stream(stream)))


def kv_cache_fetch_codes(shape: KVShape, num_slots: int, code_format: int, k_codes: Buf,
                         v_codes: Buf, kv_scales: Buf, block_table: Buf, fetch_block: Buf,
                         fetch_slot: Buf, fetch_count: Buf, fetch_stride: int, cache_k: Buf,
                         cache_v: Buf, cache_scales: Buf, stream=None) -> None:
    _check(_lib.kv_cache_fetch_codes(ctypes.byref(shape), num_slots, code_format, _p(k_codes),
                                     _p(v_codes), _p(kv_scales), _p(block_table),
                                     _p(fetch_block), _p(fetch_slot), _p(fetch_count),
                                     fetch_stride, _p(cache_k), _p(cache_v), _p(cache_scales),
                                     _stream(stream)))


def kv_cached_decode_attn_codes(shape: KVShape, num_slots: int, code_format: int, q: Buf,
                                cache_k: Buf, cache_v: Buf, cache_scales: Buf, seq_lens: Buf,
                                sel_blocks: Buf, sel_count: Buf, sel_slots: Buf, sel_stride: int,
                                scale: float, num_splits: int, part_o: Buf, part_m: Buf,
                                part_l: Buf, block_lse: Buf = None, stream=None) -> None:
    _check(_lib.kv_cached_decode_attn_codes(ctypes.byref(shape), num_slots, code_format, _p(q),
                                            _p(cache_k), _p(cache_v), _p(cache_scales),
                                            _p(seq_lens), _p(sel_blocks), _p(sel_count),
                                            _p(sel_slots), sel_stride, scale, num_splits,
                                            _p(part_o), _p(part_m), _p(part_l), _p(block_lse),
                                            _stream(stream)))


def kv_cached_decode_attn_fetch(shape: KVShape, num_slots: int, q: Buf, k_pool: Buf, v_pool: Buf,
                                block_table: Buf, fetch_slot: Buf, fetch_count: Buf,
                                cache_k: Buf, cache_v: Buf, seq_lens: Buf, sel_blocks: Buf,
                                sel_count: Buf, sel_slots: Buf, sel_stride: int, scale: float,
                                num_splits: int, part_o: Buf, part_m: Buf, part_l: Buf,
                                block_lse: Buf = None, stream=None) -> None:
    _check(_lib.kv_cached_decode_attn_fetch(
        ctypes.byref(shape), num_slots, _p(q), _p(k_pool), _p(v_pool), _p(block_table),
        _p(fetch_slot), _p(fetch_count), _p(cache_k), _p(cache_v), _p(seq_lens), _p(sel_blocks),
        _p(sel_count), _p(sel_slots), sel_stride, scale, num_splits, _p(part_o), _p(part_m),
        _p(part_l), _p(block_lse), _stream(stream)))


def kv_cached_decode_attn_fetch_codes(shape: KVShape, num_slots: int, code_format: int, q: Buf,
                                      k_codes: Buf, v_codes: Buf, kv_scales: Buf,
                                      block_table: Buf, fetch_slot: Buf, fetch_count: Buf,
                                      cache_k: Buf, cache_v: Buf, cache_scales: Buf,
                                      seq_lens: Buf, sel_blocks: Buf, sel_count: Buf,
                                      sel_slots: Buf, sel_stride: int, scale: float,
                                      num_splits: int, part_o: Buf, part_m: Buf, part_l: Buf,
                                      block_lse: Buf = None, stream=None) -> None:
    _check(_lib.kv_cached_decode_attn_fetch_codes(
        ctypes.byref(shape), num_slots, code_format, _p(q), _p(k_codes), _p(v_codes),
        _p(kv_scales), _p(block_table), _p(fetch_slot), _p(fetch_count), _p(cache_k),
        _p(cache_v), _p(cache_scales), _p(seq_lens), _p(sel_blocks), _p(sel_count),
        _p(sel_slots), sel_stride, scale, num_splits, _p(part_o), _p(part_m), _p(part_l),
        _p(block_lse), _stream(stream)))


def kv_cache_slot_mass(shape: KVShape, num_slots: int, block_lse: Buf, lse: Buf, sel_count: Buf,
                       sel_slots: Buf, sel_stride: int, slot_mass: Buf, stream=None) -> None:
    _check(_lib.kv_cache_slot_mass(ctypes.byref(shape), num_slots, _p(block_lse), _p(lse),
                                   _p(sel_count), _p(sel_slots), sel_stride, _p(slot_mass),
                                   _stream(stream)))


KV_CHECK_BAD_SEQ_LEN = 0x1
KV_CHECK_BAD_PAGE_ID = 0x2
KV_CHECK_BAD_SEL_COUNT = 0x4
KV_CHECK_BAD_SEL_BLOCK = 0x8


def kv_check_tables(shape: KVShape, block_table: Buf, seq_lens: Buf, sel_blocks: Buf,
                    sel_count: Buf, sel_stride: int, result: Buf, stream=None) -> None:
    _check(_lib.kv_check_tables(ctypes.byref(shape), _p(block_table), _p(seq_lens),
                                _p(sel_blocks), _p(sel_count), sel_stride, _p(result),
                                _stream(stream)))


PROBE_SINK_WORDS = 4096


def kv_probe_stream_read(buf: Buf, nbytes: int, sink: Buf, stream=None) -> None:
    _check(_lib.kv_probe_stream_read(_p(buf), nbytes, _p(sink), _stream(stream)))


def kv_probe_gather_read(shape: KVShape, k_cache: Buf, v_cache: Buf, block_table: Buf,
                         seq_lens: Buf, num_splits: int, sink: Buf, stream=None) -> None:
    _check(_lib.kv_probe_gather_read(ctypes.byref(shape), _p(k_cache), _p(v_cache),
                                     _p(block_table), _p(seq_lens), num_splits, _p(sink),
                                     _stream(stream)))


def kv_probe_fp8_convert(counts: Buf, first: Buf, stream=None) -> None:
    _check(_lib.kv_probe_fp8_convert(_p(counts, 32, "counts"), _p(first, 16, "first"),
                                     _stream(stream)))


def kv_host_alloc(nbytes: int, flags: int = KV_HOST_COHERENT):
    """Returns (host_ptr, dev_ptr) as integers."""
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    _check(_lib.kv_host_alloc(nbytes, flags, ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def kv_host_free(host_ptr: int) -> None:
    _check(_lib.kv_host_free(host_ptr))
