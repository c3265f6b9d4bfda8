"""Pins of the oracle's W4A4 variant (CPU only).

"primitive-ai/LFM2.5-24B-A2B-NVFP4A16", "Why this quant": the W4A4 builds make
the expert activations 4-bit as well.  The card gives no activation format;
the reading pinned here is the weights' own MXFP4 format ("LFM2.5-24B-A2B --
Packed MXFP4 Inference", "Model and quantization": E2M1 values, one E8M0
scale per 32 values) with the OCP MX v1.0 shared-scale rule
X = 2^(floor(log2 amax) - 2) (exponent clamped to -127..127, 2^-127 for a
zero block) and nearest-E2M1 elements, ties to the even code, saturating
at 6, sign kept.

The worked blocks below were derived by hand from that rule; the rest is
checked against the exact rational brute force in ``exact_ref`` (all eight
magnitudes tried per element), exhaustively over the BF16 values of one
scale window, and through the whole layer on tiny shapes.
"""
import struct
from fractions import Fraction as F

import numpy as np
import pytest

from packed_bit_expert_amd import synth as S
from tests import exact_ref as X


def _bf(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0] >> 16


def _codes(c, n=32):
    """Unpacked 4-bit codes of one packed row (low nibble = even k)."""
    c = np.asarray(c).ravel()
    return [int((c[k // 2] >> (4 * (k & 1))) & 15) for k in range(n)]


# (values, expected codes of the listed values, expected E8M0 code); the block
# is padded with +0 to 32 values (code 0)
WORKED = [
    # amax 100: floor(log2 100) = 6, X = 2^4.  1/16 -> 0; -0.3125/16 -> -0 (code 8);
    # 100/16 = 6.25 saturates to 6 (code 7); 6.5/16 = 0.406 -> 0.5 (code 1);
    # 3/16 = 0.1875 -> 0; -5/16 = -0.3125 -> -0.5 (code 9)
    ([1.0, -0.3125, 100.0, 6.5, 3.0, -5.0, 0.0], [0, 8, 7, 1, 0, 9, 0], 131),
    # amax 7: X = 1.  Every tie of the E2M1 grid goes to the even code:
    # 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4;
    # 7 lies past the largest value and saturates to 6
    ([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -0.25, -0.75, 5.0, 7.0, 6.0, 0.5, 1.5, 3.0, -6.0],
     [6, 0, 2, 2, 4, 4, 6, 8, 10, 6, 7, 7, 1, 3, 5, 15], 127),
    # amax 1.5 * 2^-126: floor(log2) = -126, -126 - 2 = -128 clamps to -127:
    # 2^-130 / 2^-127 = 0.125 -> 0; 1.5 * 2^-126 / 2^-127 = 3 (code 5);
    # -2^-127 (subnormal BF16) / 2^-127 = -1 (code 10)
    ([2.0 ** -130, 1.5 * 2.0 ** -126, -(2.0 ** -127)], [0, 5, 10], 0),
    # amax 1.5 * 2^127: floor(log2) = 127, X = 2^125: 6 (code 7), 2 (code 4),
    # -0.5 (code 9)
    ([1.5 * 2.0 ** 127, 2.0 ** 126, -(2.0 ** 124)], [7, 4, 9], 252),
    # a zero block takes E8M0 code 0 and all-zero codes; -0 keeps its sign
    ([0.0, -0.0], [0, 8], 0),
]


@pytest.mark.parametrize("case", WORKED, ids=[f"block{i}" for i in range(len(WORKED))])
def test_quant_worked_blocks(orc, case):
    vals, want, want_scale = case
    bits = [_bf(v) for v in vals] + [0] * (32 - len(vals))
    assert all(X.bf16_bits_value(b) == F(v) for b, v in zip(bits, vals)), "inputs are BF16"
    c, s = orc.quant_mxfp4(np.array(bits, np.uint16))
    got = _codes(c)
    assert got[:len(want)] == want
    assert got[len(want):] == [0] * (32 - len(want))
    assert int(s[0, 0]) == want_scale
    # the exact brute force agrees with the hand derivation
    ec, es = X.mxfp4_quant_bits(bits)
    assert ec == got and es == want_scale


def test_quant_exhaustive_one_window(orc):
    """Every BF16 value with |v| in [2^-4, 8) (and its negative) in blocks
    whose amax is 7 (X = 1): six binades x 128 mantissas, each against the
    brute-force nearest code."""
    vals = []
    for e in range(-4, 3):
        for m in range(128):
            v = (1 + m / 128) * 2.0 ** e
            if v < 8:
                vals += [v, -v]
    bits = [_bf(v) for v in vals]
    blocks = []
    for i in range(0, len(bits), 31):
        chunk = bits[i:i + 31]
        blocks.append([_bf(7.0)] + chunk + [0] * (31 - len(chunk)))
    arr = np.array(blocks, np.uint16).reshape(-1)
    c, s = orc.quant_mxfp4(arr.reshape(1, -1))
    assert np.all(s == 127)
    got = _codes(c, arr.size)
    for b in range(len(blocks)):
        ec, es = X.mxfp4_quant_bits(blocks[b])
        assert got[32 * b:32 * b + 32] == ec, f"block {b}"


def test_quant_random_blocks_match_bruteforce(orc):
    rng = np.random.default_rng(3)
    rows = []
    for r in range(64):
        scale = 2.0 ** rng.integers(-20, 20)
        v = rng.standard_normal(64) * scale
        if r % 4 == 1:
            v[rng.integers(0, 64, 8)] = 0.0
        if r % 4 == 2:  # heavy tail: one large value per block
            v[::32] *= 40.0
        rows.append([_bf(float(np.float32(x))) for x in v])
    arr = np.array(rows, np.uint16)
    c, s = orc.quant_mxfp4(arr)
    for r in range(arr.shape[0]):
        got = _codes(c[r], 64)
        for b in range(2):
            ec, es = X.mxfp4_quant_bits(arr[r, 32 * b:32 * b + 32].tolist())
            assert got[32 * b:32 * b + 32] == ec and int(s[r, b]) == es, (r, b)


def test_quant_roundtrip_and_error_bound(orc):
    """Blocks already in MXFP4 (largest magnitude 4 or 6) come back
    unchanged; for any block the error is at most half a step of the E2M1
    grid (0.25, 0.5 or 1 times X), or 2 X in the saturated range (6, 8)."""
    rng = np.random.default_rng(5)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for t in range(50):
        x = int(rng.integers(-100, 100))
        q = rng.choice(grid, 32) * rng.choice([-1.0, 1.0], 32)
        q[int(rng.integers(0, 32))] = rng.choice([4.0, 6.0])
        vals = q * 2.0 ** x
        bits = np.array([_bf(float(v)) for v in vals], np.uint16)
        c, s = orc.quant_mxfp4(bits)
        assert int(s[0, 0]) == x + 127
        deq = [X.e2m1(k) * X.e8m0(int(s[0, 0])) for k in _codes(c)]
        assert deq == [X.bf16_bits_value(b) for b in bits]
    v = (rng.standard_normal((32, 32)) * 3.0).astype(np.float32)
    bits = np.array([[_bf(float(a)) for a in row] for row in v], np.uint16)
    c, s = orc.quant_mxfp4(bits)
    for r in range(32):
        Xs = X.e8m0(int(s[r, 0]))
        for k, code in enumerate(_codes(c[r])):
            a = abs(X.bf16_bits_value(int(bits[r, k]))) / Xs
            err = abs(abs(X.e2m1(code)) - a)
            bound = F(2) if a > 6 else (F(1, 4) if a < 2 else (F(1, 2) if a < 4 else F(1)))
            assert err <= bound, (r, k)


def _tiny(seed, H, I, E, K, T):
    fmt = S.FMT_E8M0_G32
    shape = S.Shape(hidden=H, inter=I, experts=E, top_k=K, layers=1)
    nib = [S.expert_nibbles(shape, fmt, seed, e) for e in range(E)]
    sc = [S.expert_scales(shape, fmt, seed, e) for e in range(E)]
    x = S.activations(seed, 0, 0, T, H)
    ids, rw = S.routing_uniform(seed, 0, 0, T, E, K)
    resid = S.activations(seed + 1, 0, 0, T, H)
    return nib, sc, x, ids, rw, resid


W4A4_CASES = [
    # (seed, H, I, E, K, T, prenorm, residual)
    (21, 64, 32, 8, 4, 2, False, False),
    (22, 96, 64, 8, 4, 1, True, True),
    (23, 64, 96, 6, 3, 2, False, True),
]


@pytest.mark.parametrize("case", W4A4_CASES, ids=[f"seed{c[0]}" for c in W4A4_CASES])
def test_w4a4_layer_matches_exact(orc, case):
    seed, H, I, E, K, T, pre, use_res = case
    nib, sc, x, ids, rw, resid = _tiny(seed, H, I, E, K, T)
    r = resid if use_res else None
    out, d = orc.moe_forward(x, ids, rw, nib, sc, hidden=H, inter=I, num_experts=E,
                             fmt=S.FMT_E8M0_G32, residual=r, prenorm=pre, eps=1e-5, dumps=True,
                             w4a4=True)
    ex = X.layer(x.tolist(), ids.tolist(), rw.tolist(), nib, sc, H, I, S.FMT_E8M0_G32,
                 residual_bits=None if r is None else r.tolist(), use_prenorm=pre, eps=1e-5,
                 w4a4=True)
    for k in ["u", "g", "v", "h", "y"]:
        assert np.array_equal(d[k], np.array(ex[k], np.uint16)), k
    assert np.array_equal(out, np.array(ex["out"], np.uint16))
    # quantising the activations changes the layer
    base = orc.moe_forward(x, ids, rw, nib, sc, hidden=H, inter=I, num_experts=E,
                           fmt=S.FMT_E8M0_G32, residual=r, prenorm=pre, eps=1e-5)
    assert not np.array_equal(base, out)


def test_w4a4_equals_w4a16_on_representable_inputs(orc):
    """When x is already MXFP4 (per block, largest |q| in {4, 6}), its
    quantisation is the identity, so gate and up equal the W4A16 layer's."""
    H, I, E, K, T = 128, 64, 6, 4, 3
    nib, sc, _, ids, rw, _ = _tiny(31, H, I, E, K, T)
    rng = np.random.default_rng(31)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    q = rng.choice(grid, (T, H)) * rng.choice([-1.0, 1.0], (T, H))
    q[:, ::32] = 6.0
    xs = 2.0 ** rng.integers(-3, 3, (T, H // 32)).repeat(32, axis=1)
    x = np.array([[_bf(float(v)) for v in row] for row in q * xs], np.uint16)
    _, d4 = orc.moe_forward(x, ids, rw, nib, sc, hidden=H, inter=I, num_experts=E,
                            fmt=S.FMT_E8M0_G32, dumps=True, w4a4=True)
    _, d16 = orc.moe_forward(x, ids, rw, nib, sc, hidden=H, inter=I, num_experts=E,
                             fmt=S.FMT_E8M0_G32, dumps=True)
    assert np.array_equal(d4["g"], d16["g"]) and np.array_equal(d4["v"], d16["v"])
    assert np.array_equal(d4["h"], d16["h"])


def test_w4a4_rejects_e4m3(orc):
    H, I, E, K, T = 64, 32, 4, 2, 1
    shape = S.Shape(hidden=H, inter=I, experts=E, top_k=K, layers=1)
    fmt = S.FMT_E4M3_G16
    nib = [S.expert_nibbles(shape, fmt, 1, e) for e in range(E)]
    sc = [S.expert_scales(shape, fmt, 1, e) for e in range(E)]
    x = S.activations(1, 0, 0, T, H)
    ids, rw = S.routing_uniform(1, 0, 0, T, E, K)
    with pytest.raises(ValueError):
        orc.moe_forward(x, ids, rw, nib, sc, hidden=H, inter=I, num_experts=E, fmt=fmt,
                        w4a4=True)
