"""The oracle against exact rational brute force on tiny shapes (CPU only).

Every intermediate the oracle dumps (pre-normed u, gate g, up v, h, y) and
the final output must match the exact computation bit for bit.  Shapes are
non-square and not powers of two where possible, so a transposed operand,
a swapped nibble order, a wrong scale index, a dropped term, a wrong sign,
a fused multiply-add in the combine or a different slot order all change
some bit.
"""
import numpy as np
import pytest

from packed_bit_expert_amd import synth as S
from tests import exact_ref as X


def _tiny_layer(seed, H, I, E, K, T, fmt, ids=None, dup=False):
    shape = S.Shape(hidden=H, inter=I, experts=E, top_k=K, layers=1)
    rng = np.random.default_rng(seed)
    nib = [S.expert_nibbles(shape, fmt, seed, e) for e in range(E)]
    sc = [S.expert_scales(shape, fmt, seed, e) for e in range(E)]
    ts = S.tensor_scales(shape, fmt, seed)
    x = S.activations(seed, 0, 0, T, H)
    if ids is None:
        ids, rw = S.routing_uniform(seed, 0, 0, T, E, K)
    else:
        _, rw = S.routing_uniform(seed, 0, 0, T, E, K)
    if dup:
        ids[0, :] = ids[0, 0]
    resid = S.activations(seed + 1, 0, 0, T, H)
    return shape, nib, sc, ts, x, ids, rw, resid


CASES = [
    # (seed, H, I, E, K, T, fmt, prenorm, residual)
    (1, 64, 32, 8, 4, 2, S.FMT_E8M0_G32, False, False),
    (2, 96, 64, 8, 4, 1, S.FMT_E8M0_G32, True, True),
    (3, 64, 96, 6, 3, 2, S.FMT_E8M0_G32, False, True),
    (4, 64, 32, 8, 4, 2, S.FMT_E4M3_G16, False, False),
    (5, 48, 80, 5, 2, 1, S.FMT_E4M3_G16, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_oracle_matches_exact(orc, case):
    seed, H, I, E, K, T, fmt, pre, use_res = case
    shape, nib, sc, ts, x, ids, rw, resid = _tiny_layer(seed, H, I, E, K, T, fmt, dup=(seed == 3))
    r = resid if use_res else None
    out, d = orc.moe_forward(x, ids, rw, nib, sc, hidden=H, inter=I, num_experts=E, fmt=fmt,
                             tensor_scales=ts, residual=r, prenorm=pre, eps=1e-5, dumps=True)
    ex = X.layer(x.tolist(), ids.tolist(), rw.tolist(), nib, sc, H, I, fmt,
                 tscales=ts, residual_bits=None if r is None else r.tolist(),
                 use_prenorm=pre, eps=1e-5)
    assert np.array_equal(d["u"], np.array(ex["u"], np.uint16))
    assert np.array_equal(d["g"], np.array(ex["g"], np.uint16))
    assert np.array_equal(d["v"], np.array(ex["v"], np.uint16))
    assert np.array_equal(d["h"], np.array(ex["h"], np.uint16))
    assert np.array_equal(d["y"], np.array(ex["y"], np.uint16))
    assert np.array_equal(out, np.array(ex["out"], np.uint16))
    # the values are not degenerate: outputs span many distinct BF16 values
    assert len(np.unique(out)) > H // 2


def test_oracle_exact_detects_planted_mistakes(orc):
    """The brute force is sharp enough to see small mistakes: perturb one
    nibble, one scale code, one routing weight -> some output bit changes."""
    seed, H, I, E, K, T, fmt = 11, 64, 32, 4, 2, 1, S.FMT_E8M0_G32
    shape, nib, sc, ts, x, ids, rw, _ = _tiny_layer(seed, H, I, E, K, T, fmt)
    base = orc.moe_forward(x, ids, rw, nib, sc, hidden=H, inter=I, num_experts=E, fmt=fmt)
    e = int(ids[0, 0])
    nib2 = [a.copy() for a in nib]
    nib2[e][5] ^= 0x10  # high nibble of byte 5 of gate row 0
    sc2 = [a.copy() for a in sc]
    sc2[e][-1] = 120 if sc2[e][-1] != 120 else 121  # last down-scale block
    rw2 = rw.copy()
    rw2[0, 1] ^= 1
    for n_, s_, w_ in [(nib2, sc, rw), (nib, sc2, rw), (nib, sc, rw2)]:
        o = orc.moe_forward(x, ids, w_, n_, s_, hidden=H, inter=I, num_experts=E, fmt=fmt)
        assert not np.array_equal(o, base)
        ex = X.layer(x.tolist(), ids.tolist(), w_.tolist(), n_, s_, H, I, fmt)
        assert np.array_equal(o, np.array(ex["out"], np.uint16))
