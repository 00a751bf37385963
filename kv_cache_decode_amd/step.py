"""A decode step of one layer on the device, driven through the C ABI.

:class:`DeviceWorkload` puts a generated workload in device memory (torch
tensors; the K/V pools optionally in mapped pinned host memory from
``kv_host_alloc``) and owns the output buffers.  Its methods call the C-ABI
entry points in the order of the select -> fetch -> compute step (KVDrive §2.3
and §4): block meta, score + Top-K, split-K attention, merge.  Nothing here
computes; it only allocates and passes pointers.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import numpy as np
import torch

from . import kvdecode as kd
from .workload import WorkloadData

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def storage_tensor(raw: np.ndarray, dtype: str) -> torch.Tensor:
    """CPU torch tensor of the storage dtype sharing the bytes of ``raw``."""
    if dtype == "bf16":
        return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(raw)


class HostBuffer:
    """Pinned, device-mapped host memory holding a copy of a numpy array."""

    def __init__(self, arr: np.ndarray, flags: int = kd.KV_HOST_COHERENT):
        arr = np.ascontiguousarray(arr)
        self.nbytes = arr.nbytes
        self.host, self.dev = kd.kv_host_alloc(self.nbytes, flags)
        ctypes.memmove(self.host, arr.ctypes.data, self.nbytes)

    def free(self):
        if self.host:
            kd.kv_host_free(self.host)
            self.host = self.dev = None

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.free()
        except Exception:
            pass


class DeviceWorkload:
    def __init__(self, data: WorkloadData, device="cuda:0", host_kv: Optional[bool] = None,
                 host_flags: int = kd.KV_HOST_COHERENT):
        spec = data.spec
        self.data, self.spec = data, spec
        self.device = torch.device(device)
        self.host_kv = spec.host_kv if host_kv is None else host_kv
        dt = spec.dtype
        dev = self.device
        self.q = storage_tensor(data.q_raw, dt).to(dev)
        self.block_table = torch.from_numpy(data.block_table).to(dev)
        self.seq_lens = torch.from_numpy(data.seq_lens).to(dev)
        self._host = []
        if self.host_kv:
            hk, hv = HostBuffer(data.k_raw, host_flags), HostBuffer(data.v_raw, host_flags)
            self._host = [hk, hv]
            self.k_cache, self.v_cache = hk.dev, hv.dev
        else:
            self.k_cache = storage_tensor(data.k_raw, dt).to(dev)
            self.v_cache = storage_tensor(data.v_raw, dt).to(dev)
        P, Hkv, bs, D = data.k_raw.shape
        self.kmeta = torch.zeros((P, Hkv, 2, D), dtype=TORCH_DTYPES[dt], device=dev)
        self.kmean = None          # fp32 mean-key index, allocated by mean_build()
        self.k8 = self.v8 = self.kv_scales = None   # E4M3 cold pages, from quantize_fp8()
        self._host8 = []
        self._host4 = []
        self.k4 = self.v4 = self.kv_scales4 = None  # INT4 cold pages, from quantize_int4()
        ids, val = [], []
        for b in range(spec.num_seqs):
            for n in range(spec.blocks(b)):
                ids.append(int(data.block_table[b, n]))
                val.append(min(bs, spec.seq_lens[b] - n * bs))
        # the index build may list pages in any order; physical order turns its
        # K reads and meta writes into sequential streams
        order = np.argsort(np.asarray(ids, dtype=np.int64), kind="stable")
        self.page_ids = torch.tensor(np.asarray(ids, np.int32)[order], device=dev)
        self.page_valid = torch.tensor(np.asarray(val, np.int32)[order], device=dev)
        self.shape = kd.make_shape(spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, D,
                                   spec.max_blocks, P, dt, block_size=bs,
                                   flags=kd.KV_FLAG_HOST_KV if self.host_kv else 0)
        self.scale = 1.0 / math.sqrt(D)
        B, Hq = spec.num_seqs, spec.num_q_heads
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.scores = torch.empty((B, Hkv, spec.max_blocks), dtype=torch.float32, device=dev)
        self._parts = {}
        self.sel = self.sel_count = None
        self.topk = None
        # the K/V rows of each sequence's newest token (position L_b - 1):
        # appending them again leaves the cache and its index unchanged
        last_k = np.empty((spec.num_seqs, Hkv, D), dtype=data.k_raw.dtype)
        last_v = np.empty_like(last_k)
        for b in range(spec.num_seqs):
            t = spec.seq_lens[b] - 1
            p = data.block_table[b, t // bs]
            last_k[b], last_v[b] = data.k_raw[p, :, t % bs], data.v_raw[p, :, t % bs]
        self.last_k = storage_tensor(last_k, dt).to(dev)
        self.last_v = storage_tensor(last_v, dt).to(dev)

    # ------------------------------------------------------------ buffers
    def partials(self, num_splits: int):
        if num_splits not in self._parts:
            B, Hq, D = self.spec.num_seqs, self.spec.num_q_heads, self.spec.head_dim
            dev = self.device
            self._parts[num_splits] = (
                torch.empty((B, Hq, num_splits, D), dtype=torch.float32, device=dev),
                torch.empty((B, Hq, num_splits), dtype=torch.float32, device=dev),
                torch.empty((B, Hq, num_splits), dtype=torch.float32, device=dev),
            )
        return self._parts[num_splits]

    def set_selection(self, sel: np.ndarray, sel_count: np.ndarray):
        self.sel = torch.from_numpy(np.ascontiguousarray(sel, np.int32)).to(self.device)
        self.sel_count = torch.from_numpy(np.ascontiguousarray(sel_count, np.int32)).to(self.device)
        self.topk = int(sel.shape[-1])

    def auto_splits(self, sparse: bool) -> int:
        per_unit = self.topk if sparse else self.spec.max_blocks
        return kd.kv_auto_num_splits(self.shape, per_unit)

    # ------------------------------------------------------------ steps
    def meta_build(self, stream=None):
        kd.kv_block_meta_build(self.shape, self.k_cache, self.page_ids, self.page_valid,
                               int(self.page_ids.numel()), self.kmeta, stream)

    def mean_build(self, stream=None):
        if self.kmean is None:
            P, Hkv, _, D = self.kmeta.shape
            self.kmean = torch.zeros((P, Hkv, D), dtype=torch.float32, device=self.device)
        kd.kv_block_mean_build(self.shape, self.k_cache, self.page_ids, self.page_valid,
                               int(self.page_ids.numel()), self.kmean, stream)

    def append(self, k_new=None, v_new=None, stream=None, meta: bool = True):
        """Store one new token per sequence at position seq_lens - 1 and refresh the
        index rows of its page (min/max when ``meta``; the mean once mean_build ran)."""
        kd.kv_append_token(self.shape, self.last_k if k_new is None else k_new,
                           self.last_v if v_new is None else v_new, self.block_table,
                           self.seq_lens, self.k_cache, self.v_cache,
                           self.kmeta if meta else None, self.kmean, stream)

    def _sel_buffers(self, k: int):
        if self.topk != k or self.sel is None:
            B, Hkv = self.spec.num_seqs, self.spec.num_kv_heads
            self.sel = torch.empty((B, Hkv, k), dtype=torch.int32, device=self.device)
            self.sel_count = torch.empty((B, Hkv), dtype=torch.int32, device=self.device)
            self.topk = k

    def topk_workspace(self, k: int):
        """A workspace of kv_score_topk_workspace_size bytes (with scores_out
        given, its candidate storage lets long rows take the two-level select)."""
        need = kd.kv_score_topk_workspace_size(self.shape, k)
        ws = getattr(self, "_topk_ws", None)
        if ws is None or ws.numel() < need:
            ws = self._topk_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
        return ws, need

    def score_topk(self, k: int, stream=None, workspace: bool = False):
        self._sel_buffers(k)
        ws, need = self.topk_workspace(k) if workspace else (None, 0)
        kd.kv_block_score_topk(self.shape, self.q, self.kmeta, self.block_table, self.seq_lens, k,
                               self.scores, self.sel, self.sel_count, ws, need, stream)

    def select(self, k: int, index: str = "minmax", sink_tokens: int = 0, local_tokens: int = 0,
               stream=None, workspace: bool = False):
        """kv_block_select over the min/max index ("minmax") or the mean index ("mean");
        with ``workspace`` the call also gets kv_score_topk_workspace_size bytes."""
        self._sel_buffers(k)
        kind, idx = ((kd.KV_INDEX_MEAN, self.kmean) if index == "mean"
                     else (kd.KV_INDEX_MINMAX, self.kmeta))
        ws, need = self.topk_workspace(k) if workspace else (None, 0)
        kd.kv_block_select(self.shape, kind, self.q, idx, self.block_table, self.seq_lens, k,
                           sink_tokens, local_tokens, self.scores, self.sel, self.sel_count, ws,
                           need, stream)

    def decode_select(self, k: int, index: str = "minmax", sink_tokens: int = 0,
                      local_tokens: int = 0, k_new=None, v_new=None, meta: bool = True,
                      stream=None, workspace: bool = False):
        """kv_decode_select: append (as append()) and select (as select()) in one call."""
        self._sel_buffers(k)
        kind = kd.KV_INDEX_MEAN if index == "mean" else kd.KV_INDEX_MINMAX
        ws, need = self.topk_workspace(k) if workspace else (None, 0)
        kd.kv_decode_select(self.shape, kind, self.q, self.last_k if k_new is None else k_new,
                            self.last_v if v_new is None else v_new, self.block_table,
                            self.seq_lens, self.k_cache, self.v_cache,
                            self.kmeta if meta else None, self.kmean, k, sink_tokens,
                            local_tokens, self.scores, self.sel, self.sel_count, ws, need, stream)

    def decode_score(self, index: str = "minmax", k_new=None, v_new=None, meta: bool = True,
                     stream=None):
        """kv_decode_score: append (as append()) and the scores of select(), no Top-K."""
        kind = kd.KV_INDEX_MEAN if index == "mean" else kd.KV_INDEX_MINMAX
        kd.kv_decode_score(self.shape, kind, self.q, self.last_k if k_new is None else k_new,
                           self.last_v if v_new is None else v_new, self.block_table,
                           self.seq_lens, self.k_cache, self.v_cache,
                           self.kmeta if meta else None, self.kmean, self.scores, stream)

    def select_attention(self, k: int, num_splits: Optional[int] = None, sink_tokens: int = 0,
                         local_tokens: int = 0, stream=None):
        """kv_select_decode_attn over self.scores: the Top-K (to self.sel /
        self.sel_count) and the sparse attention partials, in one call."""
        self._sel_buffers(k)
        S = num_splits or kd.kv_auto_select_splits(self.shape, k)
        po, pm, pl = self.partials(S)
        kd.kv_select_decode_attn(self.shape, self.scores, self.block_table, self.seq_lens, k,
                                 sink_tokens, local_tokens, self.q, self.k_cache, self.v_cache,
                                 self.scale, S, self.sel, self.sel_count, po, pm, pl, stream)
        return S

    def attention(self, sparse: bool, num_splits: Optional[int] = None, stream=None):
        S = num_splits or self.auto_splits(sparse)
        po, pm, pl = self.partials(S)
        if sparse:
            kd.kv_paged_decode_attn(self.shape, self.q, self.k_cache, self.v_cache,
                                    self.block_table, self.seq_lens, self.sel, self.sel_count,
                                    self.topk, self.scale, S, po, pm, pl, stream)
        else:
            kd.kv_paged_decode_attn(self.shape, self.q, self.k_cache, self.v_cache,
                                    self.block_table, self.seq_lens, None, None, 0, self.scale, S,
                                    po, pm, pl, stream)
        return S

    def quantize_fp8(self, host: Optional[bool] = None, stream=None):
        """E4M3 code pools and (k, v) scales of every used page.  With ``host``
        (default: the workload's host_kv) the code pools then move to mapped
        pinned host memory for zero-copy reads."""
        P, Hkv, bs, D = self.data.k_raw.shape
        dev = self.device
        k8 = torch.zeros((P, Hkv, bs, D), dtype=torch.uint8, device=dev)
        v8 = torch.zeros_like(k8)
        self.kv_scales = torch.zeros((P, Hkv, 2), dtype=torch.float32, device=dev)
        kd.kv_quantize_pages_fp8(self.shape, self.k_cache, self.v_cache, self.page_ids,
                                 self.page_valid, int(self.page_ids.numel()), k8, v8,
                                 self.kv_scales, stream)
        host = self.host_kv if host is None else host
        if host:
            torch.cuda.synchronize(dev)
            hk, hv = HostBuffer(k8.cpu().numpy()), HostBuffer(v8.cpu().numpy())
            self._host8 = [hk, hv]
            self.k8, self.v8 = hk.dev, hv.dev
            self.k8_dev, self.v8_dev = k8, v8
        else:
            self.k8, self.v8 = k8, v8
            self.k8_dev, self.v8_dev = k8, v8

    def attention_fp8(self, sparse: bool, num_splits: Optional[int] = None, stream=None):
        S = num_splits or kd.kv_auto_num_splits_fp8(self.shape,
                                                    self.topk if sparse else self.spec.max_blocks)
        po, pm, pl = self.partials(S)
        sel, cnt, stride = (self.sel, self.sel_count, self.topk) if sparse else (None, None, 0)
        kd.kv_paged_decode_attn_fp8(self.shape, self.q, self.k8, self.v8, self.kv_scales,
                                    self.block_table, self.seq_lens, sel, cnt, stride, self.scale,
                                    S, po, pm, pl, stream)
        return S

    def decode_fp8(self, sparse: bool, num_splits: Optional[int] = None, stream=None):
        S = self.attention_fp8(sparse, num_splits, stream)
        self.combine(S, stream)
        return S

    def quantize_int4(self, host: Optional[bool] = None, stream=None):
        """INT4 code pools ([P, Hkv, bs, D/2], two codes per byte) and (k, v)
        scales of every used page; ``host`` as in quantize_fp8."""
        P, Hkv, bs, D = self.data.k_raw.shape
        dev = self.device
        k4 = torch.zeros((P, Hkv, bs, D // 2), dtype=torch.uint8, device=dev)
        v4 = torch.zeros_like(k4)
        self.kv_scales4 = torch.zeros((P, Hkv, 2), dtype=torch.float32, device=dev)
        kd.kv_quantize_pages_int4(self.shape, self.k_cache, self.v_cache, self.page_ids,
                                  self.page_valid, int(self.page_ids.numel()), k4, v4,
                                  self.kv_scales4, stream)
        host = self.host_kv if host is None else host
        if host:
            torch.cuda.synchronize(dev)
            hk, hv = HostBuffer(k4.cpu().numpy()), HostBuffer(v4.cpu().numpy())
            self._host4 = [hk, hv]
            self.k4, self.v4 = hk.dev, hv.dev
        else:
            self.k4, self.v4 = k4, v4
        self.k4_dev, self.v4_dev = k4, v4

    def attention_int4(self, sparse: bool, num_splits: Optional[int] = None, stream=None):
        S = num_splits or kd.kv_auto_num_splits_fp8(self.shape,
                                                    self.topk if sparse else self.spec.max_blocks)
        po, pm, pl = self.partials(S)
        sel, cnt, stride = (self.sel, self.sel_count, self.topk) if sparse else (None, None, 0)
        kd.kv_paged_decode_attn_int4(self.shape, self.q, self.k4, self.v4, self.kv_scales4,
                                     self.block_table, self.seq_lens, sel, cnt, stride,
                                     self.scale, S, po, pm, pl, stream)
        return S

    def decode_int4(self, sparse: bool, num_splits: Optional[int] = None, stream=None):
        S = self.attention_int4(sparse, num_splits, stream)
        self.combine(S, stream)
        return S

    def attention_tiered(self, sparse: bool, cold: str, page_tier, num_splits: Optional[int] = None,
                         stream=None):
        """kv_paged_decode_attn_tiered: hot pages from the 16-bit pools, pages with
        page_tier != 0 from the FP8 (cold="fp8") or INT4 (cold="int4") code pools."""
        S = num_splits or kd.kv_auto_num_splits_tiered(
            self.shape, self.topk if sparse else self.spec.max_blocks)
        po, pm, pl = self.partials(S)
        sel, cnt, stride = (self.sel, self.sel_count, self.topk) if sparse else (None, None, 0)
        if cold == "fp8":
            kc, vc, sc, fmt = self.k8, self.v8, self.kv_scales, kd.KV_COLD_FP8
        else:
            kc, vc, sc, fmt = self.k4, self.v4, self.kv_scales4, kd.KV_COLD_INT4
        kd.kv_paged_decode_attn_tiered(self.shape, self.q, self.k_cache, self.v_cache, kc, vc, sc,
                                       fmt, page_tier, self.block_table, self.seq_lens, sel, cnt,
                                       stride, self.scale, S, po, pm, pl, stream)
        return S

    def attention_tiered_split(self, sparse: bool, cold: str, page_tier,
                               num_splits_hot: int, num_splits_cold: int, stream=None):
        """kv_paged_decode_attn_tiered_split: the hot and the cold blocks of each
        list as two launches; returns the merged split count."""
        S = num_splits_hot + num_splits_cold
        po, pm, pl = self.partials(S)
        sel, cnt, stride = (self.sel, self.sel_count, self.topk) if sparse else (None, None, 0)
        if cold == "fp8":
            kc, vc, sc, fmt = self.k8, self.v8, self.kv_scales, kd.KV_COLD_FP8
        else:
            kc, vc, sc, fmt = self.k4, self.v4, self.kv_scales4, kd.KV_COLD_INT4
        need = kd.kv_tiered_split_workspace_size(self.shape, stride)
        ws = getattr(self, "_tier_ws", None)
        if ws is None or ws.numel() < need:
            ws = self._tier_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        kd.kv_paged_decode_attn_tiered_split(self.shape, self.q, self.k_cache, self.v_cache, kc,
                                             vc, sc, fmt, page_tier, self.block_table,
                                             self.seq_lens, sel, cnt, stride, self.scale,
                                             num_splits_hot, num_splits_cold, po, pm, pl, ws,
                                             need, stream)
        return S

    def decode_tiered(self, sparse: bool, cold: str, page_tier, num_splits: Optional[int] = None,
                      stream=None):
        S = self.attention_tiered(sparse, cold, page_tier, num_splits, stream)
        self.combine(S, stream)
        return S

    # ------------------------------------------------------------ tier policy
    def tier_init(self, tier=None, heat: float = 0.0):
        """State of the hot/cold tier policy: per page heat (fp32), tier (uint8,
        0 hot; ``tier`` gives the initial one, default all hot) and the step of
        its last demotion, and the [B, maxN] demote / promote lists."""
        P = self.shape.num_pages
        B, maxN = self.spec.num_seqs, self.spec.max_blocks
        dev = self.device
        self.page_heat = torch.full((P,), heat, dtype=torch.float32, device=dev)
        self.page_tier = (torch.zeros(P, dtype=torch.uint8, device=dev) if tier is None else
                          torch.as_tensor(np.asarray(tier, np.uint8)).to(dev))
        self.page_stamp = torch.zeros(P, dtype=torch.int32, device=dev)
        self.demote = torch.empty((B, maxN), dtype=torch.int32, device=dev)
        self.promote = torch.empty_like(self.demote)
        self.demote_count = torch.empty(B, dtype=torch.int32, device=dev)
        self.promote_count = torch.empty_like(self.demote_count)

    def tier_step(self, step: int, cold: Optional[str] = None, decay: float = 0.875,
                  hot_above: float = 0.5, cold_below: float = 0.125, recent_tokens: int = 64,
                  cooldown_steps: int = 8, stream=None):
        """kv_tier_plan over the current selection; with ``cold`` ("fp8" or
        "int4", after quantize_fp8 / quantize_int4) the demoted pages' codes are
        then written into that code pool (the demote rows passed whole, full
        pages), on the same stream and without a host sync."""
        kd.kv_tier_plan(self.shape, self.sel, self.sel_count, self.topk, self.block_table,
                        self.seq_lens, decay, hot_above, cold_below, recent_tokens,
                        cooldown_steps, step, self.page_heat, self.page_tier, self.page_stamp,
                        self.demote, self.demote_count, self.promote, self.promote_count,
                        stream)
        n = int(self.demote.numel())
        if cold == "fp8":
            kd.kv_quantize_pages_fp8(self.shape, self.k_cache, self.v_cache, self.demote, None, n,
                                     self.k8, self.v8, self.kv_scales, stream)
        elif cold == "int4":
            kd.kv_quantize_pages_int4(self.shape, self.k_cache, self.v_cache, self.demote, None,
                                      n, self.k4, self.v4, self.kv_scales4, stream)
        elif cold is not None:
            raise ValueError(f"cold={cold!r}: 'fp8', 'int4' or None")

    # ------------------------------------------------------------ GPU block cache
    def cache_init(self, num_slots: int, k: int, codes: Optional[str] = None):
        """Cache pools [B * C, Hkv, bs, D] and an empty directory for lists of k
        blocks.  With ``codes`` ("fp8" or "int4", after quantize_fp8 /
        quantize_int4) the cache holds code pages and their scales, fetched from
        the code pools."""
        spec, dev = self.spec, self.device
        B, Hq, Hkv, D, bs = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, \
            spec.block_size
        C = num_slots
        self.num_slots = C
        self.cache_codes = codes
        if codes is None:
            self.cache_k = torch.zeros((B * C, Hkv, bs, D), dtype=TORCH_DTYPES[spec.dtype],
                                       device=dev)
            self.cache_scales = None
        else:
            width = D if codes == "fp8" else D // 2
            self.cache_k = torch.zeros((B * C, Hkv, bs, width), dtype=torch.uint8, device=dev)
            self.cache_scales = torch.zeros((B * C, Hkv, 2), dtype=torch.float32, device=dev)
        self.cache_v = torch.zeros_like(self.cache_k)
        self.slot_block = torch.full((B, Hkv, C), -1, dtype=torch.int32, device=dev)
        self.block_slot = torch.full((B, Hkv, spec.max_blocks), -1, dtype=torch.int32, device=dev)
        self.slot_mass = torch.zeros((B, Hkv, C), dtype=torch.float32, device=dev)
        self.sel_slots = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.fetch_block = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.fetch_slot = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.fetch_count = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        self.block_lse = torch.empty((B, Hq, k), dtype=torch.float32, device=dev)

    def cache_plan(self, stream=None):
        kd.kv_cache_plan(self.shape, self.num_slots, self.sel, self.sel_count, self.topk,
                         self.slot_block, self.block_slot, self.slot_mass, self.sel_slots,
                         self.fetch_block, self.fetch_slot, self.fetch_count, stream)

    def _code_pools(self):
        if self.cache_codes == "fp8":
            return kd.KV_COLD_FP8, self.k8, self.v8, self.kv_scales
        return kd.KV_COLD_INT4, self.k4, self.v4, self.kv_scales4

    def cache_fetch(self, stream=None):
        if self.cache_codes is None:
            kd.kv_cache_fetch(self.shape, self.num_slots, self.k_cache, self.v_cache,
                              self.block_table, self.fetch_block, self.fetch_slot,
                              self.fetch_count, self.topk, self.cache_k, self.cache_v, stream)
            return
        fmt, kc, vc, sc = self._code_pools()
        kd.kv_cache_fetch_codes(self.shape, self.num_slots, fmt, kc, vc, sc, self.block_table,
                                self.fetch_block, self.fetch_slot, self.fetch_count, self.topk,
                                self.cache_k, self.cache_v, self.cache_scales, stream)

    def cached_attention(self, num_splits: Optional[int] = None, with_lse: bool = True,
                         stream=None):
        lse = self.block_lse if with_lse else None
        if self.cache_codes is None:
            S = num_splits or self.auto_splits(True)
            po, pm, pl = self.partials(S)
            kd.kv_cached_decode_attn(self.shape, self.num_slots, self.q, self.cache_k,
                                     self.cache_v, self.seq_lens, self.sel, self.sel_count,
                                     self.sel_slots, self.topk, self.scale, S, po, pm, pl, lse,
                                     stream)
            return S
        S = num_splits or kd.kv_auto_num_splits_fp8(self.shape, self.topk)
        po, pm, pl = self.partials(S)
        kd.kv_cached_decode_attn_codes(self.shape, self.num_slots, self._code_pools()[0], self.q,
                                       self.cache_k, self.cache_v, self.cache_scales,
                                       self.seq_lens, self.sel, self.sel_count, self.sel_slots,
                                       self.topk, self.scale, S, po, pm, pl, lse, stream)
        return S

    def cached_attention_fetch(self, num_splits: Optional[int] = None, with_lse: bool = True,
                               stream=None):
        """The step's delta fetch and the attention over the cache in one launch
        (kv_cached_decode_attn_fetch / _codes): what cache_fetch() followed by
        cached_attention() computes."""
        lse = self.block_lse if with_lse else None
        if self.cache_codes is None:
            S = num_splits or self.auto_splits(True)
            po, pm, pl = self.partials(S)
            kd.kv_cached_decode_attn_fetch(self.shape, self.num_slots, self.q, self.k_cache,
                                           self.v_cache, self.block_table, self.fetch_slot,
                                           self.fetch_count, self.cache_k, self.cache_v,
                                           self.seq_lens, self.sel, self.sel_count,
                                           self.sel_slots, self.topk, self.scale, S, po, pm, pl,
                                           lse, stream)
            return S
        fmt, kc, vc, sc = self._code_pools()
        S = num_splits or kd.kv_auto_num_splits_fp8(self.shape, self.topk)
        po, pm, pl = self.partials(S)
        kd.kv_cached_decode_attn_fetch_codes(self.shape, self.num_slots, fmt, self.q, kc, vc, sc,
                                             self.block_table, self.fetch_slot, self.fetch_count,
                                             self.cache_k, self.cache_v, self.cache_scales,
                                             self.seq_lens, self.sel, self.sel_count,
                                             self.sel_slots, self.topk, self.scale, S, po, pm, pl,
                                             lse, stream)
        return S

    def cache_slot_mass(self, stream=None):
        kd.kv_cache_slot_mass(self.shape, self.num_slots, self.block_lse, self.lse,
                              self.sel_count, self.sel_slots, self.topk, self.slot_mass, stream)

    def cache_step(self, k: int, num_splits: Optional[int] = None, stream=None,
                   fused: bool = False):
        """select -> plan -> delta fetch -> attention over the cache -> merge ->
        masses; with ``fused`` the fetch and the attention are one launch."""
        self.score_topk(k, stream)
        self.cache_plan(stream)
        if fused:
            S = self.cached_attention_fetch(num_splits, True, stream)
        else:
            self.cache_fetch(stream)
            S = self.cached_attention(num_splits, True, stream)
        self.combine(S, stream)
        self.cache_slot_mass(stream)
        return S

    def combine(self, num_splits: int, stream=None):
        po, pm, pl = self.partials(num_splits)
        kd.kv_decode_combine(self.shape, num_splits, po, pm, pl, self.out, self.lse, stream)

    def decode(self, sparse: bool, num_splits: Optional[int] = None, stream=None):
        S = self.attention(sparse, num_splits, stream)
        self.combine(S, stream)
        return S

    def close(self):
        for h in self._host + self._host8 + self._host4:
            h.free()
        self._host = []
        self._host8 = []
        self._host4 = []
