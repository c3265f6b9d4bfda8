"""Pins for the oracle's format decoders and BF16 rounding (CPU only).

E2M1 and E8M0 are checked against their bit-field definitions (the oracle
decodes E2M1 with a value table) and against the OCP MX facts the formats
fix; E4M3FN against torch's float8_e4m3fn (a library routine); BF16
round-to-nearest-even against torch's float32 -> bfloat16 cast, including
ties, subnormals and overflow.
"""
import math

import numpy as np
import torch

from tests import exact_ref as X


def test_e2m1_all_codes(orc):
    vals = [orc.e2m1(c) for c in range(16)]
    for c in range(16):
        assert vals[c] == float(X.e2m1(c))
        assert math.copysign(1.0, vals[c]) == (-1.0 if c & 8 else 1.0)  # code 8 is -0
    # OCP E2M1 facts: largest magnitude 6, smallest nonzero 0.5, 15 distinct values
    assert max(vals) == 6.0 and min(vals) == -6.0
    assert min(abs(v) for v in vals if v != 0) == 0.5
    assert len(set(vals)) == 15


def test_e8m0_all_codes(orc):
    for e in range(255):
        assert orc.e8m0(e) == math.ldexp(1.0, e - 127)
        assert orc.e8m0(e) == float(X.e8m0(e))
    assert math.isnan(orc.e8m0(255))
    assert orc.e8m0(127) == 1.0


def test_e4m3fn_all_codes_vs_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        v = orc.e4m3fn(c)
        r = ref[c].item()
        if math.isnan(r):
            assert math.isnan(v), c
        else:
            assert v == r, (c, v, r)
            assert v == float(X.e4m3fn(c))
    assert orc.e4m3fn(0x7E) == 448.0
    assert orc.e4m3fn(0x08) == 2.0 ** -6
    assert orc.e4m3fn(0x01) == 2.0 ** -9


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_random(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = _torch_bf16_bits(f)
    got = orc.bf16_from_f64(f.astype(np.float64))
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_rne_ties_subnormals_overflow(orc):
    cases = []
    for base in [1.0, 1.0078125, 3.0, 2.0 ** -126, 2.0 ** -130, 2.0 ** 127]:
        b = np.array([base], np.float32).view(np.uint32)[0]
        for low in [0x7FFF, 0x8000, 0x8001, 0x18000, 0x17FFF, 0x0001, 0xFFFF]:
            cases.append(np.array([b + low], np.uint32).view(np.float32)[0])
    cases += [np.float32(3.3895314e38), np.float32(-3.3895314e38), np.float32(1e-45),
              np.float32(-1e-45), np.float32(0.0), np.float32(-0.0)]
    f = np.array(cases, np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(orc.bf16_from_f64(f.astype(np.float64)), _torch_bf16_bits(f))


def test_bf16_single_rounding_from_fp64(orc):
    # 1 + 2^-8 + 2^-40: fp64 -> fp32 first would land on the tie 1 + 2^-8 and
    # round to even (1.0); a single rounding from fp64 goes up.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert orc.bf16_from_f64([v])[0] == X.bf16_bits(X.bf16_round(X.F(v), check_tie=False))
    assert orc.f64_from_bf16(orc.bf16_from_f64([v]))[0] == 1.0 + 2.0 ** -7
    assert orc.bf16_from_f64([1.0 + 2.0 ** -8])[0] == 0x3F80  # exact tie -> even


def test_bf16_roundtrip_all_finite_patterns(orc):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = orc.f64_from_bf16(b)
    fin = np.isfinite(v)
    back = orc.bf16_from_f64(v[fin])
    zero_neg = (b[fin] == 0x8000)
    assert np.array_equal(back[~zero_neg], b[fin][~zero_neg])
    assert back[zero_neg][0] == 0x8000
