"""Pins of the oracle's router ("GPU routing inside resident-layer graphs":
router projection, sigmoid scores, expert bias where configured, dynamic
top-k, routing coefficients).  None of them re-types the oracle's formula:
they check exact sums against rational arithmetic, the top-k set against a
brute-force search over all k-subsets, closed-form special cases, and
invariants (permutation equivariance, bias dominance, monotone and
normalised coefficients, composition with the pinned pre-norm)."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from packed_bit_expert_amd import synth as S


def small_int_bf16(rng, shape, lo=-4, hi=4):
    """BF16 bits of small integers (exact in BF16; products and sums exact)."""
    v = rng.integers(lo, hi + 1, shape).astype(np.float32)
    return S.to_bf16_bits(v)


def test_logits_are_exact_sums_on_integer_inputs():
    rng = np.random.default_rng(1)
    x = small_int_bf16(rng, (3, 32))
    w = small_int_bf16(rng, (8, 32))
    _, _, lg = O.route(x, w, top_k=2, logits=True)
    for t in range(3):
        for e in range(8):
            exact = sum(Fraction(O.f64_from_bf16(x[t, k]).item()) * Fraction(O.f64_from_bf16(w[e, k]).item())
                        for k in range(32))
            assert lg[t, e] == float(exact)


def test_topk_set_is_the_best_k_subset():
    """With no ties, the selected set maximises the sum of the selection keys
    over all C(E, k) subsets, and the slots are in descending key order."""
    rng = np.random.default_rng(2)
    E, K, H = 8, 3, 64
    for trial in range(20):
        x = S.to_bf16_bits(rng.standard_normal((1, H)).astype(np.float32))
        w = S.to_bf16_bits(rng.standard_normal((E, H)).astype(np.float32) / 8)
        bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
        ids, _, lg = O.route(x, w, bias, top_k=K, logits=True)
        key = [1.0 / (1.0 + math.exp(-lg[0, e])) + float(bias[e]) for e in range(E)]
        best = max(itertools.combinations(range(E), K), key=lambda c: sum(key[e] for e in c))
        assert set(ids[0].tolist()) == set(best)
        ks = [key[e] for e in ids[0]]
        assert ks == sorted(ks, reverse=True)


def test_zero_logits_tie_to_smallest_ids_and_equal_coefficients():
    """x orthogonal to every router row: all scores are sigmoid(0) = 1/2, every
    key ties, the slots are experts 0..k-1 and each coefficient is bf16(1/k)."""
    H, E = 64, 16
    x = np.zeros((2, H), np.uint16)
    x[:, 0] = S.to_bf16_bits(np.array([3.0], np.float32))[0]
    w = S.to_bf16_bits(np.random.default_rng(3).standard_normal((E, H)).astype(np.float32))
    w[:, 0] = 0
    for K in (1, 3, 4):
        ids, rw = O.route(x, w, top_k=K)
        assert ids.tolist() == [list(range(K))] * 2
        assert np.all(rw == O.bf16_from_f64(1.0 / K))


def test_permuting_experts_permutes_the_choice():
    rng = np.random.default_rng(4)
    E, H, K = 16, 128, 4
    x = S.to_bf16_bits(rng.standard_normal((5, H)).astype(np.float32))
    w = S.to_bf16_bits(rng.standard_normal((E, H)).astype(np.float32) / 11)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    ids, rw = O.route(x, w, bias, top_k=K)
    perm = rng.permutation(E)          # new expert i is old expert perm[i]
    inv = np.argsort(perm)
    ids2, rw2 = O.route(x, w[perm], bias[perm], top_k=K)
    assert np.array_equal(inv[ids], ids2)
    assert np.array_equal(rw, rw2)


def test_bias_selects_but_does_not_weight():
    """A large bias forces an expert into slot 0 and a large negative one
    keeps it out; the coefficients still come from the scores alone: forcing
    the unbiased choice's own set in another order leaves every expert's
    coefficient unchanged."""
    rng = np.random.default_rng(5)
    E, H, K = 16, 128, 4
    x = S.to_bf16_bits(rng.standard_normal((1, H)).astype(np.float32))
    w = S.to_bf16_bits(rng.standard_normal((E, H)).astype(np.float32) / 11)
    ids, rw = O.route(x, w, top_k=K)
    target = int(np.setdiff1d(np.arange(E), ids[0])[0])
    b = np.zeros(E, np.float32)
    b[target] = 10.0
    ids_b, _ = O.route(x, w, b, top_k=K)
    assert ids_b[0, 0] == target
    b2 = np.zeros(E, np.float32)
    b2[ids[0, 0]] = -10.0
    ids_c, _ = O.route(x, w, b2, top_k=K)
    assert ids[0, 0] not in ids_c[0]
    # same set, reversed by the bias: coefficients follow the experts
    b3 = np.zeros(E, np.float32)
    for j, e in enumerate(ids[0]):
        b3[e] = 2.0 + j
    ids_d, rw_d = O.route(x, w, b3, top_k=K)
    assert ids_d[0].tolist() == ids[0][::-1].tolist()
    assert rw_d[0].tolist() == rw[0][::-1].tolist()


def test_coefficients_monotone_and_normalised():
    rng = np.random.default_rng(6)
    sh = S.LFM24B
    w = S.router_weights(sh, 7, 0)
    x = S.activations(7, 0, 0, 16, sh.hidden)
    ids, rw, lg = O.route(x, w, S.expert_bias(sh, 7, 0), top_k=4, logits=True)
    for t in range(16):
        assert len(set(ids[t].tolist())) == 4
        c = O.f64_from_bf16(rw[t])
        assert abs(c.sum() - 1.0) <= 4 * 2.0 ** -9
        s = 1.0 / (1.0 + np.exp(-lg[t, ids[t]]))
        order = np.argsort(-s, kind="stable")
        assert np.all(np.diff(c[order]) <= 0)


def test_prenorm_composes_with_the_pinned_prenorm():
    sh = S.LFM24B
    w = S.router_weights(sh, 7, 1)
    x = S.to_bf16_bits(np.random.default_rng(8).standard_normal((4, sh.hidden)).astype(np.float32) * 23)
    eps = float(np.float32(1e-5))
    a = O.route(x, w, top_k=4, prenorm=True, eps=eps)
    b = O.route(O.prenorm(x, eps), w, top_k=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_router_rejects_bad_k():
    x = np.zeros((1, 32), np.uint16)
    w = np.zeros((4, 32), np.uint16)
    with pytest.raises(ValueError):
        O.route(x, w, top_k=5)


def test_coefficients_hand_worked_normalised_scores():
    """A hand-worked value that separates the coefficient rule (selected
    sigmoid scores normalised to sum 1) from a softmax over the selected
    logits.  x = e_0 and router rows whose first entries are 0, bf16(ln 3) =
    1.1015625 and -2 give logits (0, 1.1015625, -2).  Scores: sigmoid(0) =
    1/2 and sigmoid(1.1015625) = 1 / (1 + e^-1.1015625) = 0.750553 (ln 3
    would give exactly 3/4), so the top-2 slots are experts (1, 0) with
    coefficients 0.750553 / 1.250553 = 0.600177 and 0.399823 (exactly 0.6 and
    0.4 at ln 3).  Rounded to BF16 (spacing 2^-8 on [1/2, 1), 2^-9 on
    [1/4, 1/2)): 154 * 2^-8 = 0.6015625 (0x3F1A) and 205 * 2^-9 =
    0.400390625 (0x3ECD).  A softmax of the two logits would give 0.7505 and
    0.2495 instead."""
    H, E = 512, 3
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80  # 1.0
    w = np.zeros((E, H), np.uint16)
    w[1, 0] = 0x3F8D  # 1.1015625, the BF16 nearest to ln 3
    w[2, 0] = 0xC000  # -2.0
    assert O.f64_from_bf16(np.array([0x3F8D], np.uint16))[0] == 1.1015625
    ids, rw, lg = O.route(x, w, top_k=2, logits=True)
    assert lg[0].tolist() == [0.0, 1.1015625, -2.0]
    assert ids[0].tolist() == [1, 0]
    assert rw[0].tolist() == [0x3F1A, 0x3ECD]
