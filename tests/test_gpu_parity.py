"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Bit-exact: dequantisation, the combine, the pair sort, and the GEMV outputs
of inputs whose sums are exact in any FP32 order.  Everything else: the
tolerance of tests/gpu_helpers.py.  All inputs come from the seeded
generator; no oracle input or expected value comes from the GPU.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from packed_bit_expert_amd import moe as M
from packed_bit_expert_amd import synth as S
from tests import gpu_helpers as GH

pytestmark = pytest.mark.gpu

LFM = S.LFM24B
SMALL = S.Shape(hidden=512, inter=256, experts=16, top_k=4, layers=1)
MID = S.Shape(hidden=1024, inter=768, experts=24, top_k=4, layers=1)


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def layer_mx():
    banner("upload LFM 2048/1536 E8M0 layer 0")
    return GH.Layer(LFM, S.FMT_E8M0_G32, 0)


@pytest.fixture(scope="module")
def layer_nv():
    banner("upload LFM 2048/1536 E4M3 layer 0")
    return GH.Layer(LFM, S.FMT_E4M3_G16, 0)


# -- bit-exact building blocks ------------------------------------------------------

def test_dequant_e8m0_bitexact():
    """Every supported E8M0 code, 1..254, with every E2M1 code: code 1 with
    the 0.5 nibble gives the BF16 subnormal 2^-127, and codes 253..254 with
    large nibbles overflow to +-inf; both must come out exactly as the
    oracle's correctly rounded values."""
    banner("dequant E8M0 codes 1..254, all nibbles")
    codes = np.arange(1, 255, dtype=np.uint8)
    rows, cols = codes.size, 256
    rng = np.random.default_rng(1)
    nib = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    # every (low, high) nibble pair in the first block: all 16 codes at even
    # and at odd positions under the row's own scale code
    nib[:, :16] = (np.arange(16, dtype=np.uint8) | (np.arange(16, dtype=np.uint8)[::-1] << 4))[None, :]
    sc = np.repeat(codes[:, None], cols // 32, axis=1)
    sc[:, 1:] = rng.integers(1, 255, size=(rows, cols // 32 - 1), dtype=np.uint8)
    assert {int(c) for c in codes} <= set(np.unique(sc[:, 0]).tolist())
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=GH.dev())
    M.moe_w4a16_dequant(GH.u8_dev(nib), GH.u8_dev(sc), rows, cols, M.SCALE_E8M0_G32, out)
    torch.cuda.synchronize()
    got = GH.bits_host(out)
    ref = O.bf16_from_f64(O.dequant(nib, sc, rows, cols, O.FMT_E8M0_G32))  # -0 codes stay -0
    assert np.array_equal(got, ref)


def test_dequant_e4m3_bitexact():
    banner("dequant E4M3FN all finite codes, all nibbles")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rows, cols = codes.size, 128
    rng = np.random.default_rng(2)
    nib = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    sc = np.repeat(codes[:, None], cols // 16, axis=1)
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=GH.dev())
    M.moe_w4a16_dequant(GH.u8_dev(nib), GH.u8_dev(sc), rows, cols, M.SCALE_E4M3_G16, out)
    torch.cuda.synchronize()
    ref = O.bf16_from_f64(O.dequant(nib, sc, rows, cols, O.FMT_E4M3_G16))
    assert np.array_equal(GH.bits_host(out), ref)


@pytest.mark.parametrize("T,K,H,res", [(1, 4, 2048, False), (37, 4, 2048, True), (5, 8, 512, True),
                                       (3, 1, 1024, False), (64, 4, 2048, True)])
def test_combine_bitexact(T, K, H, res):
    banner(f"combine T={T} K={K} H={H} residual={res}")
    rng = np.random.default_rng(T * 100 + K)
    scale = rng.choice([1e-3, 1.0, 30.0, 1e4], size=(T, K, 1))
    y = S.to_bf16_bits((rng.standard_normal((T, K, H)) * scale).astype(np.float32))
    y[:, :, :16] = S.to_bf16_bits(rng.integers(-4, 5, size=(T, K, 16)).astype(np.float32) * 0.25)
    w = S.to_bf16_bits(rng.dirichlet(np.ones(K), size=T).astype(np.float32))
    r = S.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * 8) if res else None
    out = torch.empty((T, H), dtype=torch.bfloat16, device=GH.dev())
    M.moe_w4a16_combine(GH.bf16_dev(y), GH.bf16_dev(w), None if r is None else GH.bf16_dev(r), out,
                        T, K, H)
    torch.cuda.synchronize()
    assert np.array_equal(GH.bits_host(out), O.combine(y, w, r))


@pytest.mark.parametrize("T,kind", [(1, "uniform"), (32, "zipf"), (64, "uniform"), (0, "uniform"),
                                    (300, "zipf"), (40, "one"), (2048, "uniform")])
def test_sort_pairs_exact(T, kind):
    banner(f"sort T={T} {kind}")
    E, K = 64, 4
    if T == 0:
        ids = np.zeros((0, K), np.int32)
    elif kind == "zipf":
        ids, _ = S.routing_zipf(9, 0, T, T, E, K)
    elif kind == "one":
        ids = np.full((T, K), 17, np.int32)
    else:
        ids, _ = S.routing_uniform(9, 0, T, T, E, K)
    ids = ids.reshape(T, K).astype(np.int32)
    counts = torch.full((E,), -1, dtype=torch.int32, device=GH.dev())
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device=GH.dev())
    perm = torch.full((max(T * K, 1),), -1, dtype=torch.int32, device=GH.dev())
    M.moe_w4a16_sort_pairs(GH.i32_dev(ids) if T else GH.i32_dev(np.zeros(1)), T, K, E, counts,
                           offsets, perm)
    torch.cuda.synchronize()
    c, o, p = O.sort_pairs(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy()[: T * K], p)


# -- exactness-forcing full-kernel cases -------------------------------------------------

def _integer_case(shape, seed):
    """x integers in [-8, 8], scales 1.0, weights in {0, +-1, +-2}: every gate
    and up sum is an integer below 2^24, exact in any FP32 order."""
    rng = np.random.default_rng(seed)
    E = shape.experts
    codes = np.array([0, 2, 4, 10, 12], np.uint8)  # 0, 1, 2, -1, -2
    nib, sc = [], []
    for _ in range(E):
        c = rng.choice(codes, size=shape.nibble_bytes() * 2)
        nib.append((c[0::2] | (c[1::2] << 4)).astype(np.uint8))
        sc.append(np.full(shape.scale_bytes(0), 127, np.uint8))
    return nib, sc


@pytest.mark.parametrize("shape,flags", [(LFM, 0), (LFM, M.FLAG_FORCE_BATCHED), (SMALL, 0),
                                         (MID, 0), (SMALL, M.FLAG_FORCE_BATCHED)])
def test_integer_inputs_bitexact_gate_up(shape, flags):
    banner(f"integer-exact gate/up H={shape.hidden} I={shape.inter} flags={flags}")
    from packed_bit_expert_amd.residency import ResidentExperts
    nib, sc = _integer_case(shape, 3)
    store = ResidentExperts(shape, 0, 1)
    for e in range(shape.experts):
        store.buf[0, e, : store.nib_bytes].copy_(torch.from_numpy(nib[e]))
        store.buf[0, e, store.nib_bytes:].copy_(torch.from_numpy(sc[e]))
    L = GH.Layer(shape, 0, 0, store=store)
    L._host = {e: (nib[e], sc[e]) for e in range(shape.experts)}
    rng = np.random.default_rng(4)
    T = 3
    x = S.to_bf16_bits(rng.integers(-8, 9, size=(T, shape.hidden)).astype(np.float32))
    ids = np.stack([rng.choice(shape.experts, 4, replace=False) for _ in range(T)]).astype(np.int32)
    ids[1] = ids[1, 0]  # duplicates in one token
    rw = S.to_bf16_bits(np.full((T, 4), 0.25, np.float32))
    flags |= M.FLAG_FORCE_DECODE if not (flags & M.FLAG_FORCE_BATCHED) else 0
    out, d, st = L.gpu(x, ids, rw, flags=flags, dumps=True)
    ref, rd = L.oracle(x, ids, rw, dumps=True)
    assert st == 0
    assert np.array_equal(d["u"], rd["u"])
    assert np.array_equal(d["g"], rd["g"])
    assert np.array_equal(d["v"], rd["v"])
    GH.compare(d["h"], rd["h"], "h")
    GH.compare(out, ref, "out")
    for j in range(1, 4):  # same expert in every slot: identical y
        assert np.array_equal(d["y"][1, j], d["y"][1, 0])


@pytest.mark.parametrize("flags", [M.FLAG_FORCE_DECODE, M.FLAG_FORCE_BATCHED])
def test_one_hot_reads_weight_columns(layer_mx, flags):
    banner(f"one-hot x flags={flags}")
    T, H = 4, LFM.hidden
    x = np.zeros((T, H), np.uint16)
    ks = [0, 33, 1027, 2047]
    for t, k in enumerate(ks):
        x[t, k] = 0x3F80
    ids, rw = S.routing_uniform(0, 0, 7, T, LFM.experts, 4)
    out, d, st = layer_mx.gpu(x, ids, rw, flags=flags, dumps=True)
    _, rd = layer_mx.oracle(x, ids, rw, dumps=True)
    assert np.array_equal(d["g"], rd["g"]) and np.array_equal(d["v"], rd["v"])
    e = int(ids[2, 1])
    nib, sc = layer_mx.host(e)
    W = O.dequant(nib[: LFM.inter * H // 2], sc[: LFM.inter * H // 32], LFM.inter, H, 0)
    assert np.array_equal(d["g"][2, 1], O.bf16_from_f64(W[:, ks[2]] + 0.0))


# -- tolerance parity on the workloads ------------------------------------------------------

def test_c0_decode(layer_mx):
    banner("c0: one layer, T=1, E8M0, decode kernel")
    w = S.WORKLOADS["c0"]
    x, ids, rw = S.inputs(w, 0, 0)
    out, d, st = layer_mx.gpu(x, ids, rw, dumps=True)
    ref, rd = layer_mx.oracle(x, ids, rw, dumps=True)
    assert st == 0
    for k in ["g", "v", "h", "y"]:
        GH.compare(d[k], rd[k], k)
    s = GH.compare(out, ref, "out")
    assert s["bit_identical"] > 0.5
    # the fused combine equals the standalone combine kernel on the same y
    o2 = torch.empty((1, LFM.hidden), dtype=torch.bfloat16, device=GH.dev())
    M.moe_w4a16_combine(GH.bf16_dev(d["y"]), GH.bf16_dev(rw), None, o2, 1, 4, LFM.hidden)
    torch.cuda.synchronize()
    assert np.array_equal(GH.bits_host(o2), out)


def test_c0_forced_batched(layer_mx):
    banner("c0 through the batched MFMA path (T=1)")
    x, ids, rw = S.inputs(S.WORKLOADS["c0"], 0, 0)
    out, st = layer_mx.gpu(x, ids, rw, flags=M.FLAG_FORCE_BATCHED)
    GH.compare(out, layer_mx.oracle(x, ids, rw), "out")


@pytest.mark.parametrize("step", [0, 1])
def test_c2_concurrency32(layer_mx, step):
    banner(f"c2: T=32 Zipf, step {step}")
    x, ids, rw = S.inputs(S.WORKLOADS["c2"], 0, step)
    out, d, st = layer_mx.gpu(x, ids, rw, dumps=True)
    ref, rd = layer_mx.oracle(x, ids, rw, dumps=True)
    GH.compare(d["h"], rd["h"], "h")
    GH.compare(d["y"], rd["y"], "y")
    s = GH.compare(out, ref, "out")
    assert s["bit_identical"] > 0.5


@pytest.mark.parametrize("chunk", [0, 77])
def test_c3_prefill_chunk(layer_mx, chunk):
    banner(f"c3: T=64 uniform, chunk {chunk}")
    x, ids, rw = S.inputs(S.WORKLOADS["c3"], 0, chunk)
    out, st = layer_mx.gpu(x, ids, rw)
    GH.compare(out, layer_mx.oracle(x, ids, rw), "out")


def test_c4_nvfp4_batch1(layer_nv):
    banner("c4: E4M3/16 + tensor scales, T=1")
    x, ids, rw = S.inputs(S.WORKLOADS["c4"], 0, 0)
    out, d, st = layer_nv.gpu(x, ids, rw, dumps=True)
    ref, rd = layer_nv.oracle(x, ids, rw, dumps=True)
    GH.compare(d["g"], rd["g"], "g")
    GH.compare(d["y"], rd["y"], "y")
    GH.compare(out, ref, "out")


def test_c4_nvfp4_batch32(layer_nv):
    banner("c4: E4M3/16 + tensor scales, T=32 Zipf")
    x, ids, rw = S.inputs(S.WORKLOADS["c4b32"], 0, 0)
    out, st = layer_nv.gpu(x, ids, rw)
    GH.compare(out, layer_nv.oracle(x, ids, rw), "out")


@pytest.mark.parametrize("shape,T,flags", [(SMALL, 1, 0), (SMALL, 19, 0), (MID, 1, 0), (MID, 33, 0),
                                           (SMALL, 5, M.FLAG_FORCE_DECODE), (LFM, 17, 0),
                                           (MID, 2, M.FLAG_PRENORM)])
def test_ragged_and_small_shapes(shape, T, flags):
    banner(f"ragged H={shape.hidden} I={shape.inter} E={shape.experts} T={T} flags={flags}")
    L = GH.Layer(shape, S.FMT_E8M0_G32, 5)
    x = S.activations(7, 0, T, T, shape.hidden)
    ids, rw = S.routing_zipf(7, 0, T, T, shape.experts, shape.top_k)
    r = S.activations(8, 0, T, T, shape.hidden)
    out, st = L.gpu(x, ids, rw, residual=r, flags=flags)
    ref = L.oracle(x, ids, rw, residual=r, prenorm=bool(flags & M.FLAG_PRENORM))
    GH.compare(out, ref, "out")


@pytest.mark.parametrize("K,T,flags", [(1, 1, 0), (2, 1, 0), (3, 1, M.FLAG_PRENORM), (5, 1, 0),
                                       (6, 3, M.FLAG_FORCE_DECODE), (7, 1, M.FLAG_PRENORM),
                                       (8, 2, M.FLAG_FORCE_DECODE | M.FLAG_PRENORM)])
def test_decode_top_k_other_than_four(K, T, flags):
    """The decode kernels at top-k below and above four: below, waves without
    a slot of their own work on the last one and discard it; above, the down
    kernel's waves take a second slot each (its top-8 build)."""
    banner(f"decode top_k={K} H={MID.hidden} T={T} flags={flags}")
    L = GH.Layer(MID, S.FMT_E8M0_G32, 6)
    x = S.activations(9, 0, T, T, MID.hidden)
    ids, rw = S.routing_uniform(9, 0, T, T, MID.experts, K)
    r = S.activations(10, 0, T, T, MID.hidden)
    out, d, st = L.gpu(x, ids, rw, residual=r, flags=flags, dumps=True)
    assert st == 0
    ref, rd = L.oracle(x, ids, rw, residual=r, prenorm=bool(flags & M.FLAG_PRENORM), dumps=True)
    for k in ("h", "y"):
        GH.compare(d[k], rd[k], f"k={K} {k}")
    GH.compare(out, ref, f"k={K} out")


@pytest.mark.parametrize("K,flags", [(2, 0), (6, M.FLAG_PRENORM), (8, 0)])
def test_decode_top_k_other_than_four_full_shape(layer_mx, K, flags):
    """The same at the LFM2.5-24B-A2B shape, where two down waves share each
    slot's rows (one load set each) and the top-8 build gives each of them a
    second slot."""
    banner(f"decode top_k={K} H={LFM.hidden} T=1 flags={flags}")
    x = S.activations(11, 0, 1, 1, LFM.hidden)
    ids, rw = S.routing_uniform(11, 0, 1, 1, LFM.experts, K)
    r = S.activations(12, 0, 1, 1, LFM.hidden)
    out, d, st = layer_mx.gpu(x, ids, rw, residual=r, flags=flags, dumps=True)
    assert st == 0
    ref, rd = layer_mx.oracle(x, ids, rw, residual=r, prenorm=bool(flags & M.FLAG_PRENORM),
                              dumps=True)
    for k in ("h", "y"):
        GH.compare(d[k], rd[k], f"k={K} {k}")
    GH.compare(out, ref, f"k={K} out")


def test_prenorm_residual_decode(layer_mx):
    banner("pre-norm + residual, T=1 decode and T=3 batched")
    for T in (1, 3):
        x = S.to_bf16_bits(np.random.default_rng(T).standard_normal((T, LFM.hidden)).astype(np.float32) * 37)
        ids, rw = S.routing_uniform(11, 0, T, T, LFM.experts, 4)
        out, d, st = layer_mx.gpu(x, ids, rw, residual=x, flags=M.FLAG_PRENORM, dumps=True)
        ref, rd = layer_mx.oracle(x, ids, rw, residual=x, prenorm=True, dumps=True)
        GH.compare(d["u"], rd["u"], "u")
        GH.compare(out, ref, "out")


@pytest.mark.parametrize("path", [M.FLAG_FORCE_DECODE, M.FLAG_FORCE_BATCHED])
def test_prenorm_special_values(layer_mx, path):
    """The pre-norm's FP32 rescale hands values next to a BF16 rounding
    midpoint, and subnormal products, to FP64: rows with exact zeros and BF16
    subnormals, a row spanning 2^-60 .. 2^60, and a constant row must give
    the oracle's u bit for bit on both paths."""
    banner(f"pre-norm special values, flags={path}")
    rng = np.random.default_rng(21)
    H = LFM.hidden
    rows = rng.standard_normal((3, H)).astype(np.float32)
    rows[1] *= np.exp2(rng.integers(-60, 61, size=H)).astype(np.float32)
    x = S.to_bf16_bits(rows)
    idx = rng.permutation(H)
    x[0, idx[:64]] = 0                                                    # exact zeros
    sub = rng.integers(1, 128, size=64).astype(np.uint16)                 # BF16 subnormals
    x[0, idx[64:128]] = sub | (rng.integers(0, 2, size=64).astype(np.uint16) << 15)
    x[2] = S.to_bf16_bits(np.full(H, 3.0, np.float32))                    # constant row
    ids, rw = S.routing_uniform(13, 0, 3, 3, LFM.experts, 4)
    out, d, st = layer_mx.gpu(x, ids, rw, residual=x, flags=M.FLAG_PRENORM | path, dumps=True)
    ref, rd = layer_mx.oracle(x, ids, rw, residual=x, prenorm=True, dumps=True)
    assert st == 0
    assert np.array_equal(d["u"], rd["u"]), f"{int(np.sum(d['u'] != rd['u']))} u values differ"
    for k in ("h", "y"):
        GH.compare(d[k], rd[k], f"special {k}")
    GH.compare(out, ref, "special out")


def test_determinism_and_zero_tokens(layer_mx):
    banner("determinism (3 runs) and T=0")
    x, ids, rw = S.inputs(S.WORKLOADS["c2"], 0, 3)
    a, _ = layer_mx.gpu(x, ids, rw)
    b, _ = layer_mx.gpu(x, ids, rw)
    assert np.array_equal(a, b)
    x1, ids1, rw1 = S.inputs(S.WORKLOADS["c0"], 0, 3)
    a1, _ = layer_mx.gpu(x1, ids1, rw1)
    b1, _ = layer_mx.gpu(x1, ids1, rw1)
    assert np.array_equal(a1, b1)
    cfg = M.make_cfg(0)
    M.moe_w4a16_forward(0, 0, 0, 0, 0, 0, cfg)


def test_check_ids_flags_bad_slots(layer_mx):
    banner("device checks: out-of-range id")
    x, ids, rw = S.inputs(S.WORKLOADS["c0"], 0, 5)
    bad = ids.copy()
    bad[0, 2] = 64
    out, st = layer_mx.gpu(x, bad, rw, flags=M.FLAG_CHECK_IDS)
    assert st == 1
    assert np.all(np.isfinite(O.f64_from_bf16(out)))
    x2, ids2, rw2 = S.inputs(S.WORKLOADS["c2"], 0, 5)
    bad2 = ids2.copy()
    bad2[3, 1] = -5
    out2, st2 = layer_mx.gpu(x2, bad2, rw2, flags=M.FLAG_CHECK_IDS)
    assert st2 == 1
    assert np.all(np.isfinite(O.f64_from_bf16(out2)))
    # a valid call afterwards reports 0
    _, st3 = layer_mx.gpu(x, ids, rw, flags=M.FLAG_CHECK_IDS)
    assert st3 == 0


@pytest.mark.parametrize("fmt_layer,prenorm", [("layer_mx", False), ("layer_mx", True), ("layer_nv", False)])
def test_serial_expert_execution_equals_grouped(fmt_layer, prenorm, request):
    """The serial ablation (one gate/up and one down launch per selected
    expert, then the combine) runs the same device functions as the grouped
    path, so every dump and the output are bitwise equal to it; both are
    checked against the oracle."""
    L = request.getfixturevalue(fmt_layer)
    banner(f"serial expert execution vs grouped ({fmt_layer}, prenorm={prenorm})")
    w = S.WORKLOADS["c4" if L.fmt else "c0"]
    for step in (0, 9):
        x, ids, rw = S.inputs(w, 0, step)
        res = x if prenorm else None
        fl = M.FLAG_PRENORM if prenorm else 0
        g_out, g_d, g_st = L.gpu(x, ids, rw, residual=res, flags=fl, dumps=True)
        s_out, s_d, s_st = L.gpu(x, ids, rw, residual=res, flags=fl | M.FLAG_SERIAL, dumps=True)
        assert g_st == s_st == 0
        for k in ("u", "g", "v", "h", "y"):
            assert np.array_equal(g_d[k], s_d[k]), k
        assert np.array_equal(g_out, s_out)
        GH.compare(s_out, L.oracle(x, ids, rw, residual=res, prenorm=prenorm), "out")


def test_serial_check_ids(layer_mx):
    banner("serial expert execution with a rejected slot")
    x, ids, rw = S.inputs(S.WORKLOADS["c0"], 0, 5)
    bad = ids.copy()
    bad[0, 1] = 99
    g_out, g_st = layer_mx.gpu(x, bad, rw, flags=M.FLAG_CHECK_IDS)
    s_out, s_st = layer_mx.gpu(x, bad, rw, flags=M.FLAG_CHECK_IDS | M.FLAG_SERIAL)
    assert g_st == s_st == 1
    assert np.array_equal(g_out, s_out)


def test_e4m3_every_scale_code_through_both_paths():
    """Every finite E4M3FN scale code, subnormals, zeros and negative codes
    included, at random positions of every selected expert's scales, through
    the decode kernels (T = 1) and the batched kernels (T = 32, Zipf routing:
    passes on both sides of the two-groups-per-MFMA limit).  The device
    decodes E4M3 with the gfx950 OCP FP8 conversion in several lane
    positions (the dequant test covers one); the oracle decodes the format
    from its definition."""
    banner("E4M3: every finite scale code in every expert used, T=1 and T=32")
    L = GH.Layer(LFM, S.FMT_E4M3_G16, 6)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rng = np.random.default_rng(7)
    x1, ids1, rw1 = S.inputs(S.WORKLOADS["c4"], 0, 3)
    x32, ids32, rw32 = S.inputs(S.WORKLOADS["c4b32"], 0, 3)
    used = sorted({int(e) for e in np.concatenate([ids1.ravel(), ids32.ravel()])})
    nb = L.store.nib_bytes
    for e in used:
        nib, sc = L.host(e)
        sc = rng.choice(codes, size=sc.size).astype(np.uint8)
        L._host[e] = (nib, sc)
        L.store.buf[0, e, nb:].copy_(torch.from_numpy(sc))
    torch.cuda.synchronize()
    for x, ids, rw, what in ((x1, ids1, rw1, "T=1"), (x32, ids32, rw32, "T=32")):
        out, st = L.gpu(x, ids, rw)
        assert st == 0
        GH.compare(out, L.oracle(x, ids, rw), f"E4M3 every code {what}")
