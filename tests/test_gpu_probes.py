"""The read-ceiling probes read exactly the bytes they claim, and the E4M3
conversion instruction probe finds no mismatch where the quantizers use it (GPU).

Each probe folds what it loads with XOR, so the XOR of its sink words is the
XOR of every 32-bit word it read: for the stream probe, the whole buffer; for
the gather probe, the K and V tiles of every listed page of every sequence, per
KV head (pages shared by two sequences count twice, a cancelling pair).
"""
import numpy as np
import pytest
import torch

from kv_cache_decode_amd import kvdecode as kd
from kv_cache_decode_amd import workload as wl

pytestmark = pytest.mark.gpu


def xor_all(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel()))


# the last size takes the four-loads-per-lane loop on any chip (ranges of >= 1024 chunks)
@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (68 << 20) + 32])
def test_stream_probe_reads_every_word(gpu, nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(gpu)
    sink = torch.zeros(kd.PROBE_SINK_WORDS, dtype=torch.int32, device=gpu)
    kd.kv_probe_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    got = xor_all(sink.cpu().numpy())
    assert got == xor_all(host)


@pytest.mark.parametrize("S,D,dtype", [(1, 128, "bf16"), (3, 128, "bf16"), (8, 64, "f16")])
def test_gather_probe_reads_the_dense_pages(gpu, S, D, dtype):
    from kv_cache_decode_amd.step import DeviceWorkload
    spec = wl.Workload(name="probe", num_seqs=2, num_q_heads=16, num_kv_heads=4, head_dim=D,
                       seq_lens=(1000, 333), dtype=dtype, seed=41, planted_frac=0.0)
    data = wl.generate(spec)
    dw = DeviceWorkload(data, device=gpu)
    sink = torch.zeros(spec.num_seqs * spec.num_kv_heads * S, dtype=torch.int32, device=gpu)
    kd.kv_probe_gather_read(dw.shape, dw.k_cache, dw.v_cache, dw.block_table, dw.seq_lens, S, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().reshape(spec.num_seqs, spec.num_kv_heads, S)
    for j in range(spec.num_kv_heads):
        want = 0
        for b in range(spec.num_seqs):
            for n in range(spec.blocks(b)):
                p = data.block_table[b, n]
                want ^= xor_all(data.k_raw[p, j]) ^ xor_all(data.v_raw[p, j])
        assert xor_all(got[:, j, :]) == want, j
    dw.close()


def test_fp8_conversion_instruction_matches_the_rounding_rule(gpu):
    """The bf16 quantizers take E4M3 codes from the conversion instruction for
    quotients below 464 in magnitude; over all 2^32 fp32 inputs, in both
    operand slots, it must agree there with the codes' rounding rule.  Above
    that it need not (it does not saturate), and the quantizers never ask."""
    counts = torch.full((4,), -1, dtype=torch.int64, device=gpu)
    first = torch.zeros(4, dtype=torch.int32, device=gpu)
    kd.kv_probe_fp8_convert(counts, first)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    f = first.cpu().numpy().view(np.uint32)
    print("fp8 conversion mismatches by class (<464, >=464, inf, NaN):", c.tolist(),
          "first:", [hex(int(x)) for x in f])
    assert c[0] == 0 and f[0] == 0xFFFFFFFF
    assert (c >= 0).all()
