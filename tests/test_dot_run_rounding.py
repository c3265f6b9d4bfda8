"""Host model of the decode dot products' rounding (no GPU).

The decode GEMVs sum the exact FP32 products of BF16 activations and
dequantised E2M1 x E8M0 weights in FP32 runs of 16 products, add the runs in
FP64 and round the row sum once to BF16 ("LFM2.5-24B-A2B -- Packed MXFP4
Inference", "Model and quantization": FP32 accumulation, BF16 outputs).  The
BF16 result equals the correctly rounded exact sum unless an inexact run
moves the sum across a rounding boundary.  This model rounds after every
product (more often than the hardware's dot instruction, which adds two
products per rounding) on rows drawn like the synthetic workloads, and checks
that runs of 16 leave every BF16 row sum equal to the exact one, as runs of 8
do.  The exact reference is math.fsum of the products (exact in FP64).
"""
import math

import numpy as np

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def _bf16_rne(f32):
    b = np.asarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32)


def _bf16_of_f64(d):
    """Single rounding FP64 -> BF16: round-to-odd to FP32, then RNE."""
    f = d.astype(np.float32)
    u = f.view(np.uint32).copy()
    inexact = (f.astype(np.float64) != d) & (f != 0)
    fix = inexact & ((u & 1) == 0)
    up = (f.astype(np.float64) < d) == (f > 0)
    u[fix & up] += 1
    u[fix & ~up] -= 1
    return _bf16_rne(u.view(np.float32))


def _rows(rng, n, k):
    codes = rng.integers(0, 16, (n, k))
    scales = np.exp2(rng.integers(117, 124, (n, k // 32)) - 127.0)
    w = E2M1[codes] * np.repeat(scales, 32, axis=1)
    x = _bf16_rne(rng.standard_normal(k).astype(np.float32)).view(np.float32).astype(np.float64)
    return w * x  # exact in FP64 and in FP32


def _runs_to_bf16(prod, run):
    n, k = prod.shape
    p32 = prod.astype(np.float32).reshape(n, k // run, run)
    acc = np.zeros((n, k // run), np.float32)
    for i in range(run):
        acc = (acc + p32[:, :, i]).astype(np.float32)
    return _bf16_of_f64(acc.astype(np.float64).sum(axis=1))


def test_runs_of_16_keep_the_correctly_rounded_bf16_sum():
    rng = np.random.default_rng(7)
    prod = _rows(rng, 3000, 2048)
    exact = _bf16_of_f64(np.array([math.fsum(r) for r in prod]))
    for run in (8, 16):
        got = _runs_to_bf16(prod, run)
        assert int(np.sum(got != exact)) == 0, f"runs of {run}"


def test_the_model_detects_a_coarser_accumulation():
    """The same rows summed entirely in FP32 (one run of 2,048) do change
    some BF16 results, so the check above can fail."""
    rng = np.random.default_rng(7)
    prod = _rows(rng, 3000, 2048)
    exact = _bf16_of_f64(np.array([math.fsum(r) for r in prod]))
    assert int(np.sum(_runs_to_bf16(prod, 2048) != exact)) > 0
