"""Seeded synthetic decode workloads: the inputs shared by the HIP path and the oracle.

This module only *makes inputs*.  It holds none of the method's arithmetic:
no block meta, no scores, no selection, no attention.  Both the GPU tests and
the fp64 oracle consume the arrays built here, and nothing else is shared
between them.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64).  Draw order: q, K pool, V pool,
  page permutation, planted blocks.
* q, K and V entries are ``standard_normal`` drawn in float64, cast to float32,
  then rounded to the storage dtype by round-to-nearest-even (fp16 via numpy,
  bf16 by integer RNE on the float32 bit pattern).
* The K/V pools have layout ``[num_pages, num_kv_heads, block_size, head_dim]``;
  a page holds ``block_size`` consecutive tokens of one sequence for every KV
  head (the paged KV cache of the KVDrive paper, §2.2, and the tiered-offload
  blog's page table section).
* ``block_table[b, n]`` is the physical page of logical block ``n`` of sequence
  ``b``; it is the identity map or a uniform random permutation of the
  ``sum_b N_b`` used pages.  Unused table slots hold page 0.
* Planted blocks: in a fraction of the logical blocks of each (sequence,
  KV head), every key gets ``+2u`` with ``u = q[b, j*G] / |q[b, j*G]|`` (the
  first query head of the group), added in float64 to the float32 key before
  the dtype rounding.  This is workload structure (some blocks align with the
  query), not a recall target.
* Slots past a sequence's length in its last page keep their random values;
  every consumer must ignore them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def round_f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round-to-nearest-even.

    Inputs here are finite normals, so the NaN branch of RNE is not needed.
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the storage dtype.

    Returns float32 / float16 arrays, or uint16 bit patterns for bf16.
    """
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return round_f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of a storage array (every fp32/fp16/bf16 value is a double)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(raw).astype(np.float64)
    return raw.astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one synthetic decode step of one layer."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_lens: tuple            # context length of each sequence, current token included
    dtype: str                 # "f32" | "f16" | "bf16"
    seed: int
    block_size: int = 16
    page_table: str = "shuffled"   # "identity" | "shuffled"
    planted_frac: float = 0.0
    topk_blocks: Optional[int] = None   # None: dense only
    host_kv: bool = False      # K/V pools live in mapped pinned host memory
    extra_pages: int = 0       # unreferenced pages appended to the pools

    def __post_init__(self):
        if self.dtype not in DTYPES:
            raise ValueError(f"dtype must be one of {DTYPES}")
        if self.num_q_heads % self.num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        if len(self.seq_lens) != self.num_seqs:
            raise ValueError("one seq_len per sequence")
        if min(self.seq_lens) < 1:
            raise ValueError("every sequence needs at least one token")

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def blocks(self, b: int) -> int:
        return -(-self.seq_lens[b] // self.block_size)

    @property
    def max_blocks(self) -> int:
        return max(self.blocks(b) for b in range(self.num_seqs))

    @property
    def used_pages(self) -> int:
        return sum(self.blocks(b) for b in range(self.num_seqs))

    @property
    def num_pages(self) -> int:
        return self.used_pages + self.extra_pages

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def uniform(name, B, Hq, Hkv, D, L, dtype, seed, **kw) -> Workload:
    return Workload(name=name, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, seq_lens=tuple([L] * B), dtype=dtype, seed=seed, **kw)


# The five seeded workloads of the decode-attention study.  Shapes follow the
# models the pages run (OPT-6.7B with 512 prompt + 32 generated tokens at batch
# 32 on the Dual-Blade page; Llama-3.1-8B at 32k/128k context on the DirectKV
# and KVDrive pages).
WORKLOADS = {
    w.name: w for w in (
        uniform("tiny_mha_d64_1k_f32", 1, 1, 1, 64, 1024, "f32", seed=1,
                page_table="identity", topk_blocks=16),
        uniform("opt6.7b_mha_b32_544_f16", 32, 32, 32, 128, 544, "f16", seed=2,
                page_table="shuffled"),
        uniform("llama3.1_8b_gqa_b4_32k_bf16", 4, 32, 8, 128, 32768, "bf16", seed=3,
                page_table="shuffled", planted_frac=0.05, topk_blocks=128),
        uniform("llama3.1_8b_gqa_b1_128k_bf16", 1, 32, 8, 128, 131072, "bf16", seed=4,
                page_table="shuffled", planted_frac=0.05, topk_blocks=256),
        uniform("llama3.1_8b_gqa_b1_128k_bf16_hostkv", 1, 32, 8, 128, 131072, "bf16", seed=5,
                page_table="shuffled", planted_frac=0.05, topk_blocks=256, host_kv=True),
    )
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclasses.dataclass
class WorkloadData:
    """Arrays of one generated workload.

    ``*_raw`` arrays are in the storage dtype (float32, float16, or uint16 bf16
    bit patterns) and are what the GPU consumes; ``*64()`` give exact float64
    copies for the oracle.
    """

    spec: Workload
    q_raw: np.ndarray          # [B, Hq, D]
    k_raw: np.ndarray          # [P, Hkv, bs, D]
    v_raw: np.ndarray          # [P, Hkv, bs, D]
    block_table: np.ndarray    # int32 [B, maxN]
    seq_lens: np.ndarray       # int32 [B]
    planted: np.ndarray        # bool [B, Hkv, maxN]: logical blocks that got the +2u shift

    def q64(self) -> np.ndarray:
        return storage_to_f64(self.q_raw, self.spec.dtype)

    def k64(self) -> np.ndarray:
        return storage_to_f64(self.k_raw, self.spec.dtype)

    def v64(self) -> np.ndarray:
        return storage_to_f64(self.v_raw, self.spec.dtype)

    def num_blocks(self) -> np.ndarray:
        bs = self.spec.block_size
        return (self.seq_lens.astype(np.int64) + bs - 1) // bs


def _normal_f32(rng: np.random.Generator, shape, chunk_rows: int = 4096) -> np.ndarray:
    """standard_normal in float64, cast to float32, drawn in row chunks to bound memory.

    Chunked draws consume the generator's stream in order, so the values equal
    one draw of the whole shape.
    """
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = rng.standard_normal((r1 - r0, flat.shape[1]))
    return out


def generate(spec: Workload, chunk_rows: int = 4096) -> WorkloadData:
    """Build the seeded arrays of ``spec`` (see the module docstring for the recipe)."""
    rng = np.random.default_rng(spec.seed)
    B, Hq, Hkv, D, bs = (spec.num_seqs, spec.num_q_heads, spec.num_kv_heads,
                         spec.head_dim, spec.block_size)
    G = spec.group
    P = spec.num_pages
    maxN = spec.max_blocks

    q32 = _normal_f32(rng, (B, Hq, D), chunk_rows)
    k32 = _normal_f32(rng, (P, Hkv, bs, D), chunk_rows)
    v32 = _normal_f32(rng, (P, Hkv, bs, D), chunk_rows)

    used = spec.used_pages
    if spec.page_table == "identity":
        perm = np.arange(used, dtype=np.int64)
    elif spec.page_table == "shuffled":
        perm = rng.permutation(used)
    else:
        raise ValueError(f"unknown page_table {spec.page_table!r}")
    block_table = np.zeros((B, maxN), dtype=np.int32)
    off = 0
    for b in range(B):
        nb = spec.blocks(b)
        block_table[b, :nb] = perm[off:off + nb]
        off += nb

    q_raw = to_storage(q32, spec.dtype)
    q64 = storage_to_f64(q_raw, spec.dtype)
    planted = np.zeros((B, Hkv, maxN), dtype=bool)
    if spec.planted_frac > 0:
        for b in range(B):
            nb = spec.blocks(b)
            npl = int(round(spec.planted_frac * nb))
            for j in range(Hkv):
                chosen = rng.choice(nb, size=npl, replace=False)
                planted[b, j, chosen] = True
                qh = q64[b, j * G]
                u = qh / np.linalg.norm(qh)
                pages = block_table[b, chosen]
                k32[pages, j] = (k32[pages, j].astype(np.float64) + 2.0 * u).astype(np.float32)

    return WorkloadData(
        spec=spec,
        q_raw=q_raw,
        k_raw=to_storage(k32, spec.dtype),
        v_raw=to_storage(v32, spec.dtype),
        block_table=block_table,
        seq_lens=np.asarray(spec.seq_lens, dtype=np.int32),
        planted=planted,
    )


def random_selection(data: WorkloadData, k: int, seed: int) -> tuple:
    """A seeded ascending block selection per (sequence, KV head), for attention tests.

    Returns ``(sel int32 [B, Hkv, k] padded with -1, sel_count int32 [B, Hkv])``.
    """
    rng = np.random.default_rng(seed)
    spec = data.spec
    sel = np.full((spec.num_seqs, spec.num_kv_heads, k), -1, dtype=np.int32)
    cnt = np.zeros((spec.num_seqs, spec.num_kv_heads), dtype=np.int32)
    for b in range(spec.num_seqs):
        nb = spec.blocks(b)
        keff = min(k, nb)
        for j in range(spec.num_kv_heads):
            chosen = np.sort(rng.choice(nb, size=keff, replace=False))
            sel[b, j, :keff] = chosen
            cnt[b, j] = keff
    return sel, cnt


def kv_bytes(spec: Workload, blocks: int) -> int:
    """Bytes of K plus V for ``blocks`` (block, KV head) tiles."""
    return 2 * blocks * spec.block_size * spec.head_dim * spec.elem_bytes


def query_trajectory(data: WorkloadData, steps: int, rho: float, seed: int) -> list:
    """Seeded queries of `steps` consecutive decode steps, in the storage dtype.

    Step 0 is the workload's own query.  Each later query follows an AR(1) walk
    per element, q_t = rho * q_{t-1} + sqrt(1 - rho^2) * xi_t with xi_t standard
    normal (float64, then float32, then the storage dtype by round-to-nearest-
    even), so consecutive steps attend to similar blocks (the temporal locality
    of the selections that a GPU block cache relies on) while the marginal
    distribution stays N(0, 1).
    """
    rng = np.random.default_rng(seed)
    spec = data.spec
    q = data.q64()
    out = [data.q_raw]
    for _ in range(1, steps):
        q = rho * q + np.sqrt(1.0 - rho * rho) * rng.standard_normal(q.shape)
        out.append(to_storage(q.astype(np.float32), spec.dtype))
        q = storage_to_f64(out[-1], spec.dtype)
    return out
