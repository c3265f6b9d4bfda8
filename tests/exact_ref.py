"""Exact rational brute force for tiny MoE layers: the pin for the oracle.

Written independently of ``oracle/moe_oracle.c``: formats are decoded from
their bit fields (not from a value table), every sum is an exact Fraction,
every BF16 rounding is done on the exact rational, and exp/sqrt use 60-digit
decimal arithmetic.  Where the exact value lies within 2^-40 (relative) of a
BF16 rounding boundary the result is flagged as a near tie, because the
oracle's fp64 arithmetic may then legitimately round the other way.

Definitions follow "LFM2.5-24B-A2B -- Packed MXFP4 Inference" ("Model and
quantization": E2M1 values, two per byte, one E8M0 scale per 32 values, BF16
activations, FP32-or-better accumulation with BF16 outputs; "Grouped top-4
expert execution": gate, up, activation*multiply, down, routing-weighted
combine with sequential BF16 multiply/add rounding) and
"primitive-ai/LFM2.5-24B-A2B-NVFP4A16" ("What's quantized to what": one
global scale shared by gate and up).
"""
from __future__ import annotations

import decimal
import struct
from fractions import Fraction as F

_CTX = decimal.Context(prec=60)


class NearTie(Exception):
    pass


# -- formats from their bit fields ----------------------------------------------

def e2m1(code: int) -> F:
    code = int(code)
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = F(m, 2) if e == 0 else F(2) ** (e - 1) * (1 + F(m, 2))
    return -mag if s else mag


def e8m0(code: int) -> F:
    code = int(code)
    assert code != 255
    return F(2) ** (code - 127)


def e4m3fn(code: int) -> F:
    code = int(code)
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    assert not (e == 15 and m == 7)
    mag = F(m, 8) * F(2) ** -6 if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 7)
    return -mag if s else mag


def f32_exact(v: float) -> F:
    return F(struct.unpack("<f", struct.pack("<f", v))[0])


def bf16_bits_value(bits: int) -> F:
    return F(struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0])


# -- exact BF16 rounding ----------------------------------------------------------

def _floor_log2(a: F) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    elif F(2) ** (e + 1) <= a:
        e += 1
    return e


def bf16_round(v: F, check_tie: bool = True) -> F:
    """Round an exact rational to BF16, nearest-even (finite results only)."""
    if v == 0:
        return F(0)
    a = abs(v)
    E = max(_floor_log2(a), -126)
    quantum = F(2) ** (E - 7)
    q = a / quantum
    f = q.numerator // q.denominator
    d = q - f
    if check_tie and abs(abs(d - F(1, 2))) * quantum < a * F(2) ** -40 and d != F(1, 2):
        raise NearTie(str(v))
    if d > F(1, 2) or (d == F(1, 2) and f % 2 == 1):
        f += 1
    r = f * quantum
    assert r < F(2) ** 128, "overflow is never generated here"
    return r if v > 0 else -r


def bf16_bits(v: F) -> int:
    """Bit pattern of an exact BF16 value (+0 for zero)."""
    if v == 0:
        return 0
    f = float(v)
    assert F(f) == v
    return struct.unpack("<I", struct.pack("<f", f))[0] >> 16


def _dec(v: F) -> decimal.Decimal:
    return _CTX.divide(decimal.Decimal(v.numerator), decimal.Decimal(v.denominator))


def silu_mul_bf16(g: F, u: F) -> F:
    gd = _dec(g)
    s = _CTX.divide(gd, _CTX.add(decimal.Decimal(1), _CTX.exp(_CTX.minus(gd))))
    return bf16_round(F(_CTX.multiply(s, _dec(u))))


# -- MXFP4 activations (W4A4) ------------------------------------------------------
# Reading of "primitive-ai/LFM2.5-24B-A2B-NVFP4A16" ("Why this quant": the W4A4
# builds make the expert activations 4-bit): the weights' MXFP4 format of
# "LFM2.5-24B-A2B -- Packed MXFP4 Inference" ("Model and quantization"), with
# the OCP MX v1.0 shared scale 2^(floor(log2 amax) - 2) (exponent clamped to
# -127..127, 2^-127 for a zero block) and nearest-E2M1 elements, ties to the
# even code.  Here the nearest element is found by trying all eight
# magnitudes on exact rationals, a different procedure from the oracle's.

def mxfp4_quant_bits(bits: list) -> tuple:
    """One block of 32 BF16 bit patterns -> (codes list, E8M0 scale code)."""
    vals = [bf16_bits_value(b) for b in bits]
    amax = max(abs(v) for v in vals)
    x = -127 if amax == 0 else min(127, max(-127, _floor_log2(amax) - 2))
    X = F(2) ** x
    codes = []
    for b, v in zip(bits, vals):
        r = abs(v) / X
        best = None
        for c in range(8):
            d = abs(e2m1(c) - r)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        codes.append(best[1] | (8 if (int(b) >> 15) & 1 else 0))
    return codes, x + 127


def mxfp4_values(bits: list) -> list:
    """Quantised values (exact) of a BF16 row whose length is a multiple of 32."""
    out = []
    for i in range(0, len(bits), 32):
        codes, sc = mxfp4_quant_bits(bits[i:i + 32])
        out += [e2m1(c) * e8m0(sc) for c in codes]
    return out


def signed_zero_product_bits(h: F, g: F, v: F) -> int:
    """BF16 bits of h = silu(g) * v.  Exact rationals carry no sign of zero;
    IEEE arithmetic gives a zero product the XOR of its factors' signs, with
    silu(g) negative exactly when g is and every exact-zero sum being +0."""
    if h != 0:
        return bf16_bits(h)
    neg = (g < 0) != (v < 0)
    return 0x8000 if neg else 0


# -- the layer ----------------------------------------------------------------------

def _weight(nib: bytes, sc: bytes, cols: int, fmt: int, n: int, k: int, tscale: F) -> F:
    G = 16 if fmt == 1 else 32
    byte = nib[n * (cols // 2) + k // 2]
    code = (byte >> 4) if (k % 2) else (byte & 15)
    scode = sc[n * (cols // G) + k // G]
    s = e4m3fn(scode) if fmt == 1 else e8m0(scode)
    return e2m1(code) * s * tscale


def prenorm(x: list, eps: float) -> list:
    H = len(x)
    ms = sum(v * v for v in x) / H + F(eps)
    root = F(_CTX.sqrt(_dec(ms)))
    return [bf16_round(v / root) for v in x]


def layer(x_bits, ids, w_bits, nibbles, scales, H, I, fmt, tscales=None,
          residual_bits=None, use_prenorm=False, eps=1e-5, w4a4=False):
    """Exact layer for tiny shapes.  Returns dict of BF16 bit-pattern lists:
    out [T][H], u [T][H], g/v/h [T][K][I], y [T][K][H].  With ``w4a4`` the
    GEMVs read the MXFP4 quantisation of u and of each h."""
    T, K = len(ids), len(ids[0])
    res = {"out": [], "u": [], "g": [], "v": [], "h": [], "y": []}
    for t in range(T):
        x = [bf16_bits_value(b) for b in x_bits[t]]
        u = prenorm(x, eps) if use_prenorm else x
        res["u"].append([bf16_bits(v) for v in u])
        if w4a4:
            u = mxfp4_values(res["u"][-1])
        gs, vs, hs, ys = [], [], [], []
        for j in range(K):
            e = int(ids[t][j])
            nib = bytes(nibbles[e])
            sc = bytes(scales[e])
            G = 16 if fmt == 1 else 32
            tg = f32_exact(float(tscales[e][0])) if tscales is not None else F(1)
            td = f32_exact(float(tscales[e][1])) if tscales is not None else F(1)
            gate_n, up_n, down_n = 0, I * H // 2, I * H
            gate_s, up_s, down_s = 0, I * H // G, 2 * I * H // G
            g = [bf16_round(sum(u[k] * _weight(nib[gate_n:], sc[gate_s:], H, fmt, n, k, tg)
                                for k in range(H))) for n in range(I)]
            v = [bf16_round(sum(u[k] * _weight(nib[up_n:], sc[up_s:], H, fmt, n, k, tg)
                                for k in range(H))) for n in range(I)]
            h = [silu_mul_bf16(g[n], v[n]) for n in range(I)]
            hbits = [signed_zero_product_bits(h[n], g[n], v[n]) for n in range(I)]
            hq = mxfp4_values(hbits) if w4a4 else h
            y = [bf16_round(sum(hq[n] * _weight(nib[down_n:], sc[down_s:], I, fmt, m, n, td)
                                for n in range(I))) for m in range(H)]
            gs.append([bf16_bits(a) for a in g])
            vs.append([bf16_bits(a) for a in v])
            hs.append(hbits)
            ys.append(y)
        out = []
        for m in range(H):
            acc = F(0)
            for j in range(K):
                p = bf16_round(bf16_bits_value(w_bits[t][j]) * ys[j][m])
                acc = bf16_round(acc + p)
            if residual_bits is not None:
                acc = bf16_round(bf16_bits_value(residual_bits[t][m]) + acc)
            out.append(bf16_bits(acc))
        res["out"].append(out)
        res["g"].append(gs)
        res["v"].append(vs)
        res["h"].append(hs)
        res["y"].append([[bf16_bits(a) for a in y] for y in ys])
    return res
