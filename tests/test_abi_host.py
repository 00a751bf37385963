"""The C ABI as a library: symbols and host-side validation (no GPU work).

Every call here is built to fail host validation, so it returns before any
launch; the pointer values passed are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

from kv_cache_decode_amd import kvdecode as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvdecode.h")

A16 = 0x10000          # 16-byte aligned stand-in address (never dereferenced)
A4 = 0x10004           # 4-byte aligned, not 16
ODD = 0x10002          # 2-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_exactly_the_binding_exports():
    assert declared_functions() == sorted(kd.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", kd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert getattr(ctypes.CDLL(kd.LIB_PATH), name)


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_compiles_standalone(lang, tmp_path):
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "kvdecode.h"\nint main(void) { kv_shape s; (void)s; return KV_OK; }\n')
    cc = "gcc" if lang == "c" else "g++"
    subprocess.run([cc, "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.dirname(HEADER),
                    str(src)], check=True)


def shape(**kw):
    base = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_blocks_per_seq=4,
                num_pages=8, dtype="bf16")
    base.update(kw)
    return kd.make_shape(**base)


def expect(status, fn, *args, **kw):
    with pytest.raises(kd.KVError) as e:
        fn(*args, **kw, stream=0)
    assert e.value.status == status, str(e.value)
    assert kd.last_error_message()


def attn(s, **kw):
    args = dict(q=A16, k_cache=A16, v_cache=A16, block_table=A16, seq_lens=A16, sel_blocks=None,
                sel_count=None, sel_stride=0, scale=0.1, num_splits=2, part_o=A16, part_m=A16,
                part_l=A16)
    args.update(kw)
    return lambda stream: kd.kv_paged_decode_attn(s, stream=stream, **args)


@pytest.mark.parametrize("bad,status", [
    (dict(num_q_heads=7), kd.KV_ERR_INVALID_ARG),        # not a multiple of Hkv
    (dict(num_q_heads=6), kd.KV_ERR_UNSUPPORTED),        # G = 3
    (dict(num_q_heads=32), kd.KV_ERR_UNSUPPORTED),       # G = 16
    (dict(head_dim=96), kd.KV_ERR_UNSUPPORTED),
    (dict(block_size=8), kd.KV_ERR_UNSUPPORTED),
    (dict(dtype=7), kd.KV_ERR_UNSUPPORTED),
    (dict(num_seqs=0), kd.KV_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), kd.KV_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=0), kd.KV_ERR_INVALID_ARG),
    (dict(num_pages=0), kd.KV_ERR_INVALID_ARG),
    (dict(flags=0x8), kd.KV_ERR_INVALID_ARG),
    (dict(num_pages=2**30, num_kv_heads=4, num_q_heads=4), kd.KV_ERR_INVALID_ARG),
])
def test_shape_validation_in_every_call(bad, status):
    s = shape(**bad)
    expect(status, attn(s))
    expect(status, lambda stream: kd.kv_block_meta_build(s, A16, A16, A16, 4, A16, stream=stream))
    expect(status, lambda stream: kd.kv_block_score_topk(s, A16, A16, A16, A16, 2, A16, A16, A16,
                                                         stream=stream))
    expect(status, lambda stream: kd.kv_decode_combine(s, 2, A16, A16, A16, A16, None,
                                                       stream=stream))
    expect(status, lambda stream: kd.kv_block_mean_build(s, A16, A16, A16, 4, A16, stream=stream))
    expect(status, lambda stream: kd.kv_block_select(s, kd.KV_INDEX_MEAN, A16, A16, A16, A16, 8, 4,
                                                     64, A16, A16, A16, stream=stream))
    expect(status, lambda stream: kd.kv_append_token(s, A16, A16, A16, A16, A16, A16, A16, A16,
                                                     stream=stream))
    assert kd.kv_max_forced_blocks(s, 4, 64) == -1
    assert kd.kv_auto_num_splits(s, 100) == 1
    assert kd.kv_score_topk_workspace_size(s, 2) == 0


def test_null_shape_is_rejected():
    lib = ctypes.CDLL(kd.LIB_PATH)
    lib.kv_paged_decode_attn.restype = ctypes.c_int
    assert lib.kv_decode_combine(None, 1, None, None, None, None, None, None) == kd.KV_ERR_INVALID_ARG
    assert lib.kv_block_meta_build(None, None, None, None, 1, None, None) == kd.KV_ERR_INVALID_ARG


def test_attention_argument_checks():
    s = shape()
    expect(kd.KV_ERR_INVALID_ARG, attn(s, num_splits=0))
    expect(kd.KV_ERR_INVALID_ARG, attn(s, q=None))
    expect(kd.KV_ERR_INVALID_ARG, attn(s, part_l=None))
    expect(kd.KV_ERR_INVALID_ARG, attn(s, sel_blocks=A16))                  # count missing
    expect(kd.KV_ERR_INVALID_ARG, attn(s, sel_blocks=A16, sel_count=A16))   # stride 0
    expect(kd.KV_ERR_INVALID_ARG, attn(s, scale=0.0))
    expect(kd.KV_ERR_INVALID_ARG, attn(s, scale=float("inf")))
    expect(kd.KV_ERR_INVALID_ARG, attn(s, scale=float("nan")))
    expect(kd.KV_ERR_ALIGNMENT, attn(s, k_cache=A4))
    expect(kd.KV_ERR_ALIGNMENT, attn(s, part_o=A4))
    expect(kd.KV_ERR_ALIGNMENT, attn(s, block_table=ODD))
    expect(kd.KV_ERR_ALIGNMENT, attn(s, sel_blocks=ODD, sel_count=A16, sel_stride=4))


def test_score_topk_argument_checks():
    s = shape()
    f = kd.kv_block_score_topk
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, A16, A16, A16, A16, 0, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, None, A16, A16, A16, 2, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: f(s, A4, A16, A16, A16, 2, A16, A16, A16, stream=stream))
    need = kd.kv_score_topk_workspace_size(s, 2)
    assert need >= 2 * 2 * 4 * 4 and need % 256 == 0
    expect(kd.KV_ERR_WORKSPACE, lambda stream: f(s, A16, A16, A16, A16, 2, None, A16, A16, None, 0,
                                                 stream=stream))
    expect(kd.KV_ERR_WORKSPACE, lambda stream: f(s, A16, A16, A16, A16, 2, None, A16, A16, A16,
                                                 need - 4, stream=stream))
    # long rows: the candidate storage of the two-level select (8 bytes per
    # slot, 2K slots per 4096-block chunk) while a row's slots stay within 16384
    def scores_part(sh):
        return (sh.num_seqs * sh.num_kv_heads * sh.max_blocks_per_seq * 4 + 255) // 256 * 256
    for n, k, slots in ((16384, 256, 0), (16385, 256, 5 * 512), (65536, 256, 16 * 512),
                        (65536, 512, 16 * 1024), (65536, 513, 0), (20000, 1, 5 * 2)):
        sh = shape(max_blocks_per_seq=n, num_pages=n)
        rows = sh.num_seqs * sh.num_kv_heads
        assert kd.kv_score_topk_workspace_size(sh, k) == scores_part(sh) + rows * slots * 8, (n, k)
    big = shape(max_blocks_per_seq=65537)
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: f(big, A16, A16, A16, A16, 2, A16, A16, A16,
                                                   stream=stream))


def test_meta_and_combine_argument_checks():
    s = shape()
    m = kd.kv_block_meta_build
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: m(s, A16, A16, A16, -1, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: m(s, None, A16, A16, 3, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: m(s, A4, A16, A16, 3, A16, stream=stream))
    m(s, None, None, None, 0, None, stream=0)            # nothing to do: OK, no launch
    c = kd.kv_decode_combine
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: c(s, 0, A16, A16, A16, A16, None, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: c(s, 2, A16, A16, A16, None, None, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: c(s, 2, A16, A16, A16, A4, None, stream=stream))


def test_host_alloc_argument_checks_and_status_strings():
    with pytest.raises(kd.KVError) as e:
        kd.kv_host_alloc(0)
    assert e.value.status == kd.KV_ERR_INVALID_ARG
    with pytest.raises(kd.KVError) as e:
        kd.kv_host_alloc(64, flags=0x10)
    assert e.value.status == kd.KV_ERR_INVALID_ARG
    kd.kv_host_free(0)                                   # NULL is a no-op
    names = [kd.status_string(i) for i in range(6)]
    assert names == ["KV_OK", "KV_ERR_INVALID_ARG", "KV_ERR_UNSUPPORTED", "KV_ERR_ALIGNMENT",
                     "KV_ERR_WORKSPACE", "KV_ERR_HIP"]
    assert kd.status_string(99) == "unknown kv_status"


def test_auto_splits_bounds():
    s = shape(num_seqs=1, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=8192, num_pages=8192)
    for blocks in (1, 2, 7, 256, 8192):
        S = kd.kv_auto_num_splits(s, blocks)
        assert 1 <= S <= max(1, blocks)
    assert kd.kv_auto_num_splits(s, 0) == 1
    host = shape(num_seqs=1, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=8192,
                 num_pages=8192, flags=kd.KV_FLAG_HOST_KV)
    assert kd.kv_auto_num_splits(host, 256) <= 256 // 8


def test_auto_select_splits():
    """One four-split workgroup per compute unit (256 here, the MI355X count the
    library assumes without a device) where kv_select_decode_attn is one launch;
    the attention rule elsewhere."""
    s32k = shape(num_seqs=4, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=2048,
                 num_pages=8192)
    assert kd.kv_auto_select_splits(s32k, 128) == 32          # 32 rows -> 8 workgroups each
    assert kd.kv_auto_select_splits(s32k, 18) == 20           # at most 4 * ceil(K / 4)
    two = shape(num_seqs=2, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=2048,
                num_pages=4096)
    assert kd.kv_auto_select_splits(two, 128) == 64
    many = shape(num_seqs=64, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=64,
                 num_pages=4096)
    assert kd.kv_auto_select_splits(many, 16) == 4            # at least one workgroup
    for off in (dict(max_blocks_per_seq=8192, num_pages=8192),   # rows too long to fuse
                dict(dtype="f32"), dict(num_q_heads=8)):          # vector path
        o = shape(**{**dict(num_seqs=1, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=2048,
                            num_pages=2048), **off})
        assert kd.kv_auto_select_splits(o, 256) == kd.kv_auto_num_splits(o, 256)
    assert kd.kv_auto_select_splits(s32k, 0) == 1


def test_one_hip_runtime_per_process():
    """The binding loads after torch, so only torch's HIP runtime is mapped."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read()
    libs = set(line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line)
    assert len(libs) == 1, libs


def test_append_argument_checks():
    s = shape()
    f = kd.kv_append_token
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, None, A16, A16, A16, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, A16, A16, A16, A16, A16, None, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: f(s, A4, A16, A16, A16, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: f(s, A16, A16, A16, A16, A16, A16, A4, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: f(s, A16, A16, A16, A16, A16, A16, None, A4,
                                                 stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: f(s, A16, A16, ODD, A16, A16, A16, None, stream=stream))
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: f(shape(head_dim=80), A16, A16, A16, A16, A16, A16,
                                                   None, stream=stream))


def test_mean_build_argument_checks():
    s = shape()
    m = kd.kv_block_mean_build
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: m(s, A16, A16, A16, -1, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: m(s, A16, A16, A16, 3, None, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: m(s, A16, A16, A16, 3, A4, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: m(s, A16, ODD, A16, 3, A16, stream=stream))
    m(s, None, None, None, 0, None, stream=0)            # nothing to do: OK, no launch


@pytest.mark.parametrize("sink,local,want", [
    (0, 0, 0), (4, 0, 1), (16, 0, 1), (17, 0, 2), (0, 1, 1), (0, 16, 2), (0, 17, 2),
    (0, 33, 3), (4, 64, 6), (0, 64, 5),
])
def test_max_forced_blocks(sink, local, want):
    """ceil(sink / 16) for the first tokens; local consecutive tokens touch at most
    ceil((local - 1) / 16) + 1 pages of 16 (checked by sliding the window)."""
    s = shape()
    assert kd.kv_max_forced_blocks(s, sink, local) == want
    worst = 0
    for L in range(1, 300):
        toks = set(range(min(sink, L))) | set(range(max(L - local, 0), L))
        worst = max(worst, len({t // 16 for t in toks}))
    assert worst <= want
    assert kd.kv_max_forced_blocks(s, -1, 0) == -1


def test_select_argument_checks():
    s = shape()
    f = kd.kv_block_select

    def call(kind=kd.KV_INDEX_MEAN, q=A16, index=A16, k=8, sink=4, local=64, scores=A16, **kw):
        return lambda stream: f(s, kind, q, index, A16, A16, k, sink, local, scores, A16, A16,
                                stream=stream, **kw)

    expect(kd.KV_ERR_INVALID_ARG, call(kind=2))
    expect(kd.KV_ERR_INVALID_ARG, call(k=0))
    expect(kd.KV_ERR_INVALID_ARG, call(sink=-1))
    expect(kd.KV_ERR_INVALID_ARG, call(local=-3))
    expect(kd.KV_ERR_INVALID_ARG, call(k=5))                   # 4 + 64 can force 6 blocks
    expect(kd.KV_ERR_INVALID_ARG, call(index=None))
    expect(kd.KV_ERR_ALIGNMENT, call(index=A4))
    expect(kd.KV_ERR_ALIGNMENT, call(q=A4))
    expect(kd.KV_ERR_WORKSPACE, call(scores=None))
    big = shape(max_blocks_per_seq=65537)
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: f(big, 0, A16, A16, A16, A16, 8, 0, 0, A16, A16,
                                                   A16, stream=stream))


def test_select_no_alloc_argument_checks():
    """The no-allocation selection validates like kv_block_select, and refuses
    shapes whose scores exceed the library's scratch before any launch."""
    s = shape()
    f = kd.kv_block_select_no_alloc

    def call(shp=s, kind=kd.KV_INDEX_MINMAX, q=A16, index=A16, k=8, sink=0, local=0, sel=A16):
        return lambda stream: f(shp, kind, q, index, A16, A16, k, sink, local, sel, A16,
                                stream=stream)

    expect(kd.KV_ERR_INVALID_ARG, call(kind=2))
    expect(kd.KV_ERR_INVALID_ARG, call(k=0))
    expect(kd.KV_ERR_INVALID_ARG, call(sink=4, local=64, k=5))
    expect(kd.KV_ERR_INVALID_ARG, call(index=None))
    expect(kd.KV_ERR_INVALID_ARG, call(sel=None))
    expect(kd.KV_ERR_ALIGNMENT, call(q=A4))
    expect(kd.KV_ERR_UNSUPPORTED, call(shp=shape(max_blocks_per_seq=65537)))
    # 64 sequences x 8 KV heads x 4096 blocks = 2 Mi scores > the 1 Mi the scratch holds
    big = shape(num_seqs=64, num_q_heads=32, num_kv_heads=8, max_blocks_per_seq=4096)
    expect(kd.KV_ERR_WORKSPACE, call(shp=big))


def test_fp8_argument_checks():
    s = shape()
    qz = kd.kv_quantize_pages_fp8
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: qz(s, A16, A16, A16, A16, -1, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: qz(s, A16, None, A16, A16, 3, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: qz(s, A16, A16, A16, A16, 3, A16, A16, None, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: qz(s, A16, A16, A16, A16, 3, A4, A16, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: qz(s, A16, A16, A16, A16, 3, A16, A16, A4 + 2, stream=stream))
    qz(s, None, None, None, None, 0, None, None, None, stream=0)     # nothing to do: OK
    # page_valid_tokens may be NULL (full pages): the next missing array still fails
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: qz(s, A16, A16, A16, None, 3, A16, A16, None, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: qz(s, A16, A16, A16, None, 3, A4, A16, A16, stream=stream))
    at = kd.kv_paged_decode_attn_fp8

    def call(scales=A16 + 8, k8=A16, **kw):
        args = dict(q=A16, k_fp8=k8, v_fp8=A16, kv_scales=scales, block_table=A16, seq_lens=A16,
                    sel_blocks=None, sel_count=None, sel_stride=0, scale=0.1, num_splits=2,
                    part_o=A16, part_m=A16, part_l=A16)
        args.update(kw)
        return lambda stream: at(s, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, call(scales=None))
    expect(kd.KV_ERR_ALIGNMENT, call(scales=A4))
    expect(kd.KV_ERR_ALIGNMENT, call(k8=A4))
    expect(kd.KV_ERR_INVALID_ARG, call(num_splits=0))
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: at(shape(head_dim=96), A16, A16, A16, A16, A16, A16,
                                                    None, None, 0, 0.1, 1, A16, A16, A16,
                                                    stream=stream))


def test_cache_argument_checks():
    s = shape()
    pl = kd.kv_cache_plan
    args = lambda C=16, stride=8: (s, C, A16, A16, stride, A16, A16, A16, A16, A16, A16, A16)
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: pl(*args(C=0), stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: pl(*args(C=8193, stride=8), stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: pl(*args(C=16, stride=17), stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: pl(s, 16, None, A16, 8, A16, A16, A16, A16, A16,
                                                    A16, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: pl(s, 16, ODD, A16, 8, A16, A16, A16, A16, A16,
                                                  A16, A16, stream=stream))
    f = kd.kv_cache_fetch
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: f(s, 16, A16, A16, A16, A16, A16, A16, 8, A4, A16,
                                                 stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, 16, A16, None, A16, A16, A16, A16, 8, A16,
                                                   A16, stream=stream))
    at = kd.kv_cached_decode_attn
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: at(s, 16, A16, A16, A16, A16, A16, A16, None, 8,
                                                    0.1, 2, A16, A16, A16, None, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: at(s, 16, A16, A16, A16, A16, A16, A16, A16, 8,
                                                    0.0, 2, A16, A16, A16, None, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: at(s, 16, A16, A4, A16, A16, A16, A16, A16, 8,
                                                  0.1, 2, A16, A16, A16, None, stream=stream))
    m = kd.kv_cache_slot_mass
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: m(s, 16, A16, None, A16, A16, 8, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: m(s, 16, A16, A16, A16, A16, 8, ODD, stream=stream))


def test_probe_argument_checks():
    sr = kd.kv_probe_stream_read
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: sr(A16, 0, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: sr(A16, 24, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: sr(None, 32, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: sr(A4, 32, A16, stream=stream))
    g = kd.kv_probe_gather_read
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: g(shape(), A16, A16, A16, A16, 0, A16,
                                                   stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: g(shape(), A16, None, A16, A16, 2, A16,
                                                   stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: g(shape(), A4, A16, A16, A16, 2, A16,
                                                 stream=stream))
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: g(shape(dtype="f32"), A16, A16, A16, A16, 2,
                                                   A16, stream=stream))
    c = kd.kv_probe_fp8_convert
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: c(None, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: c(A16, None, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: c(A4, A16, stream=stream))


def test_decode_select_argument_checks():
    s = shape()
    f = kd.kv_decode_select

    def call(**kw):
        args = dict(index_kind=kd.KV_INDEX_MINMAX, q=A16, k_new=A16, v_new=A16, block_table=A16,
                    seq_lens=A16, k_cache=A16, v_cache=A16, kmeta=A16, kmean=None, topk_blocks=2,
                    sink_tokens=0, local_tokens=0, scores_out=A16, sel_blocks=A16, sel_count=A16)
        args.update(kw)
        return lambda stream: f(s, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, call(kmeta=None))                       # the chosen index
    expect(kd.KV_ERR_INVALID_ARG, call(index_kind=kd.KV_INDEX_MEAN))       # kmean missing
    expect(kd.KV_ERR_INVALID_ARG, call(index_kind=5))
    expect(kd.KV_ERR_INVALID_ARG, call(topk_blocks=0))
    expect(kd.KV_ERR_INVALID_ARG, call(sink_tokens=64, local_tokens=64))  # forces > topk
    expect(kd.KV_ERR_INVALID_ARG, call(k_new=None))
    expect(kd.KV_ERR_ALIGNMENT, call(v_new=A4))
    expect(kd.KV_ERR_ALIGNMENT, call(index_kind=kd.KV_INDEX_MEAN, kmean=A4))
    expect(kd.KV_ERR_ALIGNMENT, call(sel_count=ODD))
    expect(kd.KV_ERR_WORKSPACE, call(scores_out=None))


def test_decode_score_argument_checks():
    s = shape()
    f = kd.kv_decode_score

    def call(**kw):
        args = dict(index_kind=kd.KV_INDEX_MINMAX, q=A16, k_new=A16, v_new=A16, block_table=A16,
                    seq_lens=A16, k_cache=A16, v_cache=A16, kmeta=A16, kmean=None,
                    scores_out=A16)
        args.update(kw)
        return lambda stream: f(s, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, call(kmeta=None))                       # the chosen index
    expect(kd.KV_ERR_INVALID_ARG, call(index_kind=kd.KV_INDEX_MEAN))       # kmean missing
    expect(kd.KV_ERR_INVALID_ARG, call(index_kind=5))
    expect(kd.KV_ERR_INVALID_ARG, call(k_new=None))
    expect(kd.KV_ERR_INVALID_ARG, call(scores_out=None))                  # always required
    expect(kd.KV_ERR_ALIGNMENT, call(v_new=A4))
    expect(kd.KV_ERR_ALIGNMENT, call(index_kind=kd.KV_INDEX_MEAN, kmean=A4))
    expect(kd.KV_ERR_ALIGNMENT, call(scores_out=ODD))
    expect(kd.KV_ERR_ALIGNMENT, call(block_table=ODD))


def test_select_decode_attn_argument_checks():
    """The Top-K + attention call validates as the two calls it stands for, in
    either of its forms (one launch for rows of up to 2048 blocks, else two)."""
    def call(s, **kw):
        args = dict(scores=A16, block_table=A16, seq_lens=A16, topk_blocks=2, sink_tokens=0,
                    local_tokens=0, q=A16, k_cache=A16, v_cache=A16, scale=0.1, num_splits=2,
                    sel_blocks=A16, sel_count=A16, part_o=A16, part_m=A16, part_l=A16)
        args.update(kw)
        return lambda stream: kd.kv_select_decode_attn(s, stream=stream, **args)

    for s in (shape(), shape(max_blocks_per_seq=4096, num_pages=4096)):
        expect(kd.KV_ERR_INVALID_ARG, call(s, topk_blocks=0))
        expect(kd.KV_ERR_INVALID_ARG, call(s, sink_tokens=64, local_tokens=64))  # forces > K
        expect(kd.KV_ERR_INVALID_ARG, call(s, sink_tokens=-1))
        expect(kd.KV_ERR_INVALID_ARG, call(s, num_splits=0))
        expect(kd.KV_ERR_INVALID_ARG, call(s, scores=None))
        expect(kd.KV_ERR_INVALID_ARG, call(s, sel_blocks=None))
        expect(kd.KV_ERR_INVALID_ARG, call(s, q=None))
        expect(kd.KV_ERR_INVALID_ARG, call(s, part_m=None))
        expect(kd.KV_ERR_INVALID_ARG, call(s, scale=float("nan")))
        expect(kd.KV_ERR_ALIGNMENT, call(s, scores=ODD))
        expect(kd.KV_ERR_ALIGNMENT, call(s, k_cache=A4))
        expect(kd.KV_ERR_ALIGNMENT, call(s, part_o=A4))
        expect(kd.KV_ERR_ALIGNMENT, call(s, sel_count=ODD))
    expect(kd.KV_ERR_UNSUPPORTED, call(shape(max_blocks_per_seq=65537, num_pages=65537)))


def test_int4_argument_checks():
    s = shape()
    qz = kd.kv_quantize_pages_int4
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: qz(shape(dtype="f32"), A16, A16, A16, A16, 2,
                                                    A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: qz(s, A16, A16, A16, A16, -1, A16, A16, A16,
                                                    stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: qz(s, A16, A16, A16, A16, 2, None, A16, A16,
                                                    stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: qz(s, A16, A16, A16, A16, 2, A4, A16, A16,
                                                  stream=stream))
    at = kd.kv_paged_decode_attn_int4
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: at(shape(dtype="f32"), A16, A16, A16, A16, A16,
                                                    A16, None, None, 0, 0.1, 1, A16, A16, A16,
                                                    stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: at(s, A16, A16, A16, None, A16, A16, None, None,
                                                    0, 0.1, 1, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: at(s, A16, A16, A16, A4, A16, A16, None, None, 0,
                                                  0.1, 1, A16, A16, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: at(s, A16, A16, A16, A16, A16, A16, None, None,
                                                    0, 0.1, 0, A16, A16, A16, stream=stream))


def test_check_tables_argument_checks():
    s = shape()
    f = kd.kv_check_tables
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, None, A16, None, None, 0, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, A16, A16, A16, None, 4, A16, stream=stream))
    expect(kd.KV_ERR_INVALID_ARG, lambda stream: f(s, A16, A16, A16, A16, 0, A16, stream=stream))
    expect(kd.KV_ERR_ALIGNMENT, lambda stream: f(s, A16, ODD, None, None, 0, A16, stream=stream))


def test_tiered_argument_checks():
    s = shape()
    f = kd.kv_paged_decode_attn_tiered

    def call(**kw):
        args = dict(q=A16, k_cache=A16, v_cache=A16, k_cold=A16, v_cold=A16, kv_scales=A16,
                    cold_format=kd.KV_COLD_INT4, page_tier=A16, block_table=A16, seq_lens=A16,
                    sel_blocks=None, sel_count=None, sel_stride=0, scale=0.1, num_splits=2,
                    part_o=A16, part_m=A16, part_l=A16)
        args.update(kw)
        return lambda stream: f(s, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, call(cold_format=5))
    expect(kd.KV_ERR_INVALID_ARG, call(page_tier=None))
    expect(kd.KV_ERR_INVALID_ARG, call(k_cold=None))
    expect(kd.KV_ERR_ALIGNMENT, call(v_cold=A4))
    expect(kd.KV_ERR_INVALID_ARG, call(num_splits=0))
    expect(kd.KV_ERR_UNSUPPORTED, lambda stream: f(shape(dtype="f32"), A16, A16, A16, A16, A16,
                                                   A16, kd.KV_COLD_INT4, A16, A16, A16, None,
                                                   None, 0, 0.1, 2, A16, A16, A16, stream=stream))


def test_code_cache_argument_checks():
    s = shape()
    f = kd.kv_cache_fetch_codes

    def fetch(sh=s, **kw):
        args = dict(num_slots=16, code_format=kd.KV_COLD_INT4, k_codes=A16, v_codes=A16,
                    kv_scales=A16, block_table=A16, fetch_block=A16, fetch_slot=A16,
                    fetch_count=A16, fetch_stride=8, cache_k=A16, cache_v=A16, cache_scales=A16)
        args.update(kw)
        return lambda stream: f(sh, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, fetch(code_format=0))
    expect(kd.KV_ERR_INVALID_ARG, fetch(code_format=16))
    expect(kd.KV_ERR_UNSUPPORTED, fetch(sh=shape(dtype="f32")))
    expect(kd.KV_ERR_INVALID_ARG, fetch(kv_scales=None))
    expect(kd.KV_ERR_INVALID_ARG, fetch(cache_scales=None))
    expect(kd.KV_ERR_INVALID_ARG, fetch(v_codes=None))
    expect(kd.KV_ERR_ALIGNMENT, fetch(cache_scales=A4))
    expect(kd.KV_ERR_ALIGNMENT, fetch(k_codes=A4))
    expect(kd.KV_ERR_INVALID_ARG, fetch(fetch_stride=17))
    expect(kd.KV_ERR_INVALID_ARG, fetch(num_slots=0))
    at = kd.kv_cached_decode_attn_codes

    def attend(sh=s, **kw):
        args = dict(num_slots=16, code_format=kd.KV_COLD_FP8, q=A16, cache_k=A16, cache_v=A16,
                    cache_scales=A16, seq_lens=A16, sel_blocks=A16, sel_count=A16,
                    sel_slots=A16, sel_stride=8, scale=0.1, num_splits=2, part_o=A16,
                    part_m=A16, part_l=A16, block_lse=None)
        args.update(kw)
        return lambda stream: at(sh, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, attend(code_format=2))
    expect(kd.KV_ERR_UNSUPPORTED, attend(sh=shape(dtype="f32"), code_format=kd.KV_COLD_INT4))
    expect(kd.KV_ERR_INVALID_ARG, attend(cache_scales=None))
    expect(kd.KV_ERR_ALIGNMENT, attend(cache_scales=A4))
    expect(kd.KV_ERR_INVALID_ARG, attend(sel_slots=None))
    expect(kd.KV_ERR_INVALID_ARG, attend(num_splits=0))
    expect(kd.KV_ERR_INVALID_ARG, attend(scale=-1.0))
    expect(kd.KV_ERR_ALIGNMENT, attend(cache_v=A4))
    expect(kd.KV_ERR_INVALID_ARG, attend(sel_stride=17))


def test_fused_fetch_argument_checks():
    s = shape()
    f = kd.kv_cached_decode_attn_fetch

    def plain(sh=s, **kw):
        args = dict(num_slots=16, q=A16, k_pool=A16, v_pool=A16, block_table=A16,
                    fetch_slot=A16, fetch_count=A16, cache_k=A16, cache_v=A16, seq_lens=A16,
                    sel_blocks=A16, sel_count=A16, sel_slots=A16, sel_stride=8, scale=0.1,
                    num_splits=2, part_o=A16, part_m=A16, part_l=A16, block_lse=None)
        args.update(kw)
        return lambda stream: f(sh, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, plain(k_pool=None))
    expect(kd.KV_ERR_INVALID_ARG, plain(block_table=None))
    expect(kd.KV_ERR_INVALID_ARG, plain(fetch_count=None))
    expect(kd.KV_ERR_ALIGNMENT, plain(v_pool=A4))
    expect(kd.KV_ERR_ALIGNMENT, plain(fetch_slot=ODD))
    expect(kd.KV_ERR_INVALID_ARG, plain(sel_slots=None))
    expect(kd.KV_ERR_INVALID_ARG, plain(num_slots=0))
    expect(kd.KV_ERR_INVALID_ARG, plain(sel_stride=17))
    expect(kd.KV_ERR_INVALID_ARG, plain(num_splits=0))
    g = kd.kv_cached_decode_attn_fetch_codes

    def codes(sh=s, **kw):
        args = dict(num_slots=16, code_format=kd.KV_COLD_INT4, q=A16, k_codes=A16, v_codes=A16,
                    kv_scales=A16, block_table=A16, fetch_slot=A16, fetch_count=A16,
                    cache_k=A16, cache_v=A16, cache_scales=A16, seq_lens=A16, sel_blocks=A16,
                    sel_count=A16, sel_slots=A16, sel_stride=8, scale=0.1, num_splits=2,
                    part_o=A16, part_m=A16, part_l=A16, block_lse=None)
        args.update(kw)
        return lambda stream: g(sh, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, codes(code_format=3))
    expect(kd.KV_ERR_UNSUPPORTED, codes(sh=shape(dtype="f32")))
    expect(kd.KV_ERR_INVALID_ARG, codes(kv_scales=None))
    expect(kd.KV_ERR_INVALID_ARG, codes(cache_scales=None))
    expect(kd.KV_ERR_ALIGNMENT, codes(cache_scales=A4))
    expect(kd.KV_ERR_INVALID_ARG, codes(v_codes=None))


def test_tiered_split_argument_checks():
    s = shape()
    f = kd.kv_paged_decode_attn_tiered_split
    need = kd.kv_tiered_split_workspace_size(s, 0)
    # per (b, j): two lists of maxN ints, two counts, one chunk count, 1024 flag bytes
    assert need == 2 * 2 * ((2 * 4 + 2 + 1) * 4 + 1024)
    assert kd.kv_tiered_split_workspace_size(s, 3) == 2 * 2 * ((2 * 3 + 2 + 1) * 4 + 1024)
    assert kd.kv_tiered_split_workspace_size(s, -1) == 0

    def call(sh=s, **kw):
        args = dict(q=A16, k_cache=A16, v_cache=A16, k_cold=A16, v_cold=A16, kv_scales=A16,
                    cold_format=kd.KV_COLD_FP8, page_tier=A16, block_table=A16, seq_lens=A16,
                    sel_blocks=None, sel_count=None, sel_stride=0, scale=0.1,
                    num_splits_hot=2, num_splits_cold=3, part_o=A16, part_m=A16, part_l=A16,
                    workspace=A16, workspace_bytes=need)
        args.update(kw)
        return lambda stream: f(sh, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, call(cold_format=7))
    expect(kd.KV_ERR_UNSUPPORTED, call(sh=shape(dtype="f32"), cold_format=kd.KV_COLD_INT4))
    expect(kd.KV_ERR_INVALID_ARG, call(num_splits_hot=0))
    expect(kd.KV_ERR_INVALID_ARG, call(num_splits_cold=0))
    expect(kd.KV_ERR_INVALID_ARG, call(page_tier=None))
    expect(kd.KV_ERR_WORKSPACE, call(workspace_bytes=need - 1))
    expect(kd.KV_ERR_WORKSPACE, call(workspace=None))
    expect(kd.KV_ERR_ALIGNMENT, call(workspace=ODD))
    expect(kd.KV_ERR_ALIGNMENT, call(k_cold=A4))
    expect(kd.KV_ERR_INVALID_ARG, call(sel_blocks=A16))
    expect(kd.KV_ERR_INVALID_ARG, call(scale=0.0))


def test_binding_refuses_host_and_strided_tensors():
    """The binding hands the C ABI only contiguous tensors in GPU memory (or an
    int address the caller vouches for); everything else fails in Python."""
    import torch
    s = shape()
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory"):
        kd.kv_block_score_topk(s, q, A16, A16, A16, 4, A16, A16, A16)
    with pytest.raises(ValueError, match="contiguous"):
        kd.kv_block_score_topk(s, q.transpose(0, 1), A16, A16, A16, 4, A16, A16, A16)


def test_tier_plan_argument_checks():
    s = shape()

    def call(shp=s, **kw):
        args = dict(sel_blocks=A16, sel_count=A16, sel_stride=4, block_table=A16, seq_lens=A16,
                    decay=0.5, hot_above=0.6, cold_below=0.2, recent_tokens=16,
                    cooldown_steps=2, step=3, page_heat=A16, page_tier=A16, page_stamp=A16,
                    demote=A16, demote_count=A16, promote=A16, promote_count=A16)
        args.update(kw)
        return lambda stream: kd.kv_tier_plan(shp, stream=stream, **args)

    expect(kd.KV_ERR_INVALID_ARG, call(sel_stride=0))
    # the plan reads the [B, Hkv, sel_stride] rows whole: their positions must fit in int32
    expect(kd.KV_ERR_INVALID_ARG, call(sel_stride=(1 << 30) // s.num_kv_heads + 1))
    expect(kd.KV_ERR_INVALID_ARG, call(decay=1.5))
    expect(kd.KV_ERR_INVALID_ARG, call(decay=-0.1))
    expect(kd.KV_ERR_INVALID_ARG, call(decay=float("nan")))
    expect(kd.KV_ERR_INVALID_ARG, call(hot_above=float("nan")))
    expect(kd.KV_ERR_INVALID_ARG, call(cold_below=float("nan")))
    expect(kd.KV_ERR_INVALID_ARG, call(recent_tokens=0))       # the appended page stays hot
    expect(kd.KV_ERR_INVALID_ARG, call(cooldown_steps=-1))
    for name in ("sel_blocks", "sel_count", "block_table", "seq_lens", "page_heat", "page_tier",
                 "page_stamp", "demote", "demote_count", "promote", "promote_count"):
        expect(kd.KV_ERR_INVALID_ARG, call(**{name: None}))
    for name in ("sel_blocks", "page_heat", "page_stamp", "demote", "promote_count"):
        expect(kd.KV_ERR_ALIGNMENT, call(**{name: ODD}))
    expect(kd.KV_ERR_INVALID_ARG, call(shp=shape(max_blocks_per_seq=262145, num_pages=262145)))
