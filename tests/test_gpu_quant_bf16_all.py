"""bf16 pages through the quantizers, every finite bf16 value (GPU), via the C ABI.

For bf16 sources the quantizer takes each quotient x / scale from a per-unit
table of the 128 quotients 1.m / scale, scaled by the value's power of two.
Here every finite bf16 bit pattern (both zeros, subnormals, all binades) is
quantised under a set of unit maxima: ordinary ones, tiny and huge ones whose
quotients fall below the fp32 normal range, and maxima whose scale lies
outside [2^-125, 2^125] (those units divide instead).  A unit holding a NaN
in a valid row divides too; a NaN in a row past the page's valid count is
ignored.  Codes and scales must equal the oracle's bit for bit, except the
code of that NaN's own quotient, which nothing defines: in E4M3 its sign bit
is that of a NaN, so it only has to be a NaN code; in INT4 a NaN has no
nearest integer (the oracle's C conversion of it is undefined), so any code.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_decode_amd import kvdecode as kd
from kv_cache_decode_amd import workload as wl

pytestmark = pytest.mark.gpu

HKV, D, BS = 2, 128, 16
UNIT = BS * D
# unit maxima (rounded to bf16 below): FP8 scale A / 448, INT4 scale A / 7
MAXIMA = (1.0, 0.0123, 7.0, 448.0, 100.3, 3.3e4, 2.5e-20, 1e-30, 1e-36, 3.0e38)


def bf16_bits(x: float) -> np.uint16:
    return np.uint16(wl.to_storage(np.array([x], np.float32), "bf16")[0])


def build_pool(seed):
    rng = np.random.default_rng(seed)
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = b[((b >> 7) & 0xFF) != 0xFF]
    mag = wl.bf16_bits_to_f32(finite & np.uint16(0x7FFF))
    units = []
    for a in MAXIMA:
        A = bf16_bits(a)
        amag = float(wl.bf16_bits_to_f32(np.array([A]))[0])
        vals = finite[mag < amag]
        rng.shuffle(vals)
        per = UNIT - 1
        for i in range(0, len(vals), per):
            u = np.zeros(UNIT, np.uint16)
            chunk = vals[i:i + per]
            u[:len(chunk)] = chunk
            u[-1] = A if rng.random() < 0.5 else A | np.uint16(0x8000)   # the unit's max, either sign
            rng.shuffle(u)
            units.append(u)
    rnd = lambda: wl.to_storage(rng.standard_normal(UNIT).astype(np.float32), "bf16")
    if len(units) % HKV:
        units.append(rnd())
    u = rnd()
    u[5 * D + 3] = 0x7FC0                         # NaN in row 5 (valid)
    units.append(u)
    u = rnd()
    u[(BS - 1) * D + 7] = 0x7FC0                  # NaN in row 15 only: past the valid count
    units.append(u)
    P = len(units) // HKV
    pool = np.stack(units).reshape(P, HKV, BS, D)
    valid = rng.integers(1, BS + 1, P).astype(np.int32)
    valid[-1] = BS - 1                            # the last page holds the two NaN units
    return pool, valid


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_every_finite_bf16_value(gpu, fmt):
    from kv_cache_decode_amd.step import storage_tensor
    pool_k, valid = build_pool(8800)
    P = pool_k.shape[0]
    pool_v = np.ascontiguousarray(pool_k[:, ::-1])      # V: the page's two heads swapped
    shape = kd.make_shape(1, HKV, HKV, D, P, P, "bf16")
    k = storage_tensor(pool_k, "bf16").to(gpu)
    v = storage_tensor(pool_v, "bf16").to(gpu)
    ids = np.arange(P, dtype=np.int32)
    row = D if fmt == "fp8" else D // 2
    kc = torch.full((P, HKV, BS, row), 0xA5, dtype=torch.uint8, device=gpu)
    vc = torch.full_like(kc, 0x5A)
    sc = torch.full((P, HKV, 2), -1.0, dtype=torch.float32, device=gpu)
    call = kd.kv_quantize_pages_fp8 if fmt == "fp8" else kd.kv_quantize_pages_int4
    call(shape, k, v, torch.from_numpy(ids).to(gpu), torch.from_numpy(valid).to(gpu), P, kc, vc, sc)
    torch.cuda.synchronize()

    quant = oracle.fp8_quantize if fmt == "fp8" else oracle.int4_quantize
    k64 = wl.bf16_bits_to_f32(pool_k).astype(np.float64)
    v64 = wl.bf16_bits_to_f32(pool_v).astype(np.float64)
    okc, oks = quant(k64, ids, valid)
    ovc, ovs = quant(v64, ids, valid)
    gk, gv, gs = kc.cpu().numpy(), vc.cpu().numpy(), sc.cpu().numpy()
    # the NaN in a valid row: K head 0 and V head 1 of the last page, row 5, channel 3
    nan_k, nan_v = (P - 1, 0, 5, 3), (P - 1, 1, 5, 3)
    if fmt == "fp8":
        assert gk[nan_k] & 0x7F == 0x7F and gv[nan_v] & 0x7F == 0x7F
        gk[nan_k] = okc[nan_k]
        gv[nan_v] = ovc[nan_v]
    else:                                         # the byte also holds channel 2's code
        assert gk[nan_k[:3] + (1,)] & 0x0F == okc[nan_k[:3] + (1,)] & 0x0F
        assert gv[nan_v[:3] + (1,)] & 0x0F == ovc[nan_v[:3] + (1,)] & 0x0F
        gk[nan_k[:3] + (1,)] = okc[nan_k[:3] + (1,)]
        gv[nan_v[:3] + (1,)] = ovc[nan_v[:3] + (1,)]
    for p in range(P):                            # name the first page that differs
        np.testing.assert_array_equal(gk[p], okc[p], err_msg=f"K codes, page {p}")
        np.testing.assert_array_equal(gv[p], ovc[p], err_msg=f"V codes, page {p}")
    np.testing.assert_array_equal(gs[:, :, 0], oks)
    np.testing.assert_array_equal(gs[:, :, 1], ovs)
