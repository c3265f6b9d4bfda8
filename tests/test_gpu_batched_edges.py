"""GPU: edge cases of the batched (sorted, MFMA) path.

"LFM2.5-24B-A2B -- Packed MXFP4 Inference", "Grouped top-4 expert
execution": the (token, slot) pairs of a call are grouped by expert and each
selected expert's packed weights are read once.  Situations the workload
tests do not reach:

* more than 256 pairs (the workgroups hold the first 256 routing ids in
  registers and read the rest from memory) with hot experts of more than 16
  pairs, which take several passes of 16 token rows over the same weights;
* the layer stack at H = 4096, where one workgroup per token cannot finish a
  row's pre-norm inside the combine, so a separate pre-norm launch follows it;
* the largest expert count and top-k the ABI admits (1024 experts, top-8), on
  both paths;
* every token routed to the same four experts (three passes each).

Each case is compared with the oracle under the stated tolerance; the stack
must also equal the chained single-layer calls bit for bit.
"""
import numpy as np
import pytest
import torch

from packed_bit_expert_amd import moe as M
from packed_bit_expert_amd import synth as S
from packed_bit_expert_amd.residency import ResidentExperts
from tests import gpu_helpers as GH

pytestmark = pytest.mark.gpu
LFM = S.LFM24B
WIDE = S.Shape(hidden=4096, inter=512, experts=8, top_k=2, layers=3)


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def layer_mx():
    banner("upload LFM 2048/1536 E8M0 layer 3")
    return GH.Layer(LFM, S.FMT_E8M0_G32, 3)


@pytest.mark.parametrize("w4a4", [False, True])
def test_many_pairs_and_multi_pass_experts(layer_mx, w4a4):
    T = 150
    banner(f"T={T} ({4 * T} pairs), Zipf routing, w4a4={w4a4}")
    x = S.activations(9, 3, 0, T, LFM.hidden)
    ids, rw = S.routing_zipf(9, 3, 0, T, LFM.experts, LFM.top_k)
    counts = np.bincount(ids.ravel(), minlength=LFM.experts)
    assert ids.size > 256 and counts.max() > 32, "the case must reach the paths it names"
    flags = M.FLAG_W4A4 if w4a4 else 0
    out, st = layer_mx.gpu(x, ids, rw, flags=flags)
    assert st == 0
    GH.compare(out, layer_mx.oracle(x, ids, rw, w4a4=w4a4), f"out T={T} w4a4={w4a4}")


def test_wide_hidden_stack():
    sh = WIDE
    assert M.moe_w4a16_shape_supported(sh.hidden, sh.inter)
    banner(f"stack of {sh.layers} layers at H={sh.hidden} I={sh.inter}, T=6")
    store = ResidentExperts(sh, S.FMT_E8M0_G32, sh.layers).fill_synthetic()
    T, L = 6, sh.layers
    x = S.activations(4, 0, 0, T, sh.hidden)
    routes = [S.routing_uniform(4, l, 0, T, sh.experts, sh.top_k) for l in range(L)]
    ids = np.stack([r[0] for r in routes])
    rw = np.stack([r[1] for r in routes])
    # the one-call stack
    out = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device=GH.dev())
    cfg = M.make_cfg(T, sh.hidden, sh.inter, sh.experts, sh.top_k, prenorm_eps=GH.EPS)
    ws = torch.zeros(M.moe_w4a16_workspace_bytes(cfg), dtype=torch.uint8, device=GH.dev())
    cfg.workspace, cfg.workspace_bytes = ws.data_ptr(), ws.numel()
    M.moe_w4a16_stack_forward(L, GH.bf16_dev(x), GH.i32_dev(ids), GH.bf16_dev(rw), store.wtab,
                              store.stab, None, out, cfg)
    torch.cuda.synchronize()
    got = GH.bits_host(out)
    # the same layers as single calls, each on the previous call's output
    h = GH.bf16_dev(x)
    for l in range(L):
        wt, stb, _ = store.layer_tables(l)
        o = torch.empty_like(h)
        c = M.make_cfg(T, sh.hidden, sh.inter, sh.experts, sh.top_k, flags=M.FLAG_PRENORM,
                       residual=h, prenorm_eps=GH.EPS)
        w2 = torch.zeros(M.moe_w4a16_workspace_bytes(c), dtype=torch.uint8, device=GH.dev())
        c.workspace, c.workspace_bytes = w2.data_ptr(), w2.numel()
        M.moe_w4a16_forward(h, GH.i32_dev(ids[l]), GH.bf16_dev(rw[l]), wt, stb, o, c)
        h = o
    torch.cuda.synchronize()
    assert np.array_equal(got, GH.bits_host(h)), "stack call == chained single-layer calls"
    # every layer against the oracle, on the oracle chain's input
    hh = x
    for l in range(L):
        lay = GH.Layer(sh, S.FMT_E8M0_G32, l, store=store, l=l)
        nxt = lay.oracle(hh, ids[l], rw[l], residual=hh, prenorm=True)
        g, st = lay.gpu(hh, ids[l], rw[l], residual=hh, flags=M.FLAG_PRENORM)
        assert st == 0
        GH.compare(g, nxt, f"wide layer {l}")
        hh = nxt
    GH.compare(got, hh, "wide stack free-running", check=False)


MAXSH = S.Shape(hidden=512, inter=256, experts=1024, top_k=8, layers=1)


@pytest.mark.parametrize("T", [1, 9])
def test_most_experts_and_largest_top_k(T):
    """E = 1024 experts (the largest the ABI admits) and top-8 routing, on the
    decode path (T = 1) and the batched path (T = 9)."""
    banner(f"E={MAXSH.experts} top_k={MAXSH.top_k} T={T}")
    L = GH.Layer(MAXSH, S.FMT_E8M0_G32, 2)
    x = S.activations(6, 2, T, T, MAXSH.hidden)
    ids, rw = S.routing_zipf(6, 2, T, T, MAXSH.experts, MAXSH.top_k)
    r = S.activations(7, 2, T, T, MAXSH.hidden)
    out, st = L.gpu(x, ids, rw, residual=r)
    assert st == 0
    GH.compare(out, L.oracle(x, ids, rw, residual=r), f"E=1024 k=8 T={T}")


def test_every_token_the_same_experts(layer_mx):
    """All 40 tokens pick the same four experts (in rotating slot order):
    four experts with 40 pairs each, three passes of 16 token rows apiece."""
    T = 40
    banner(f"T={T}, every token routed to the same four experts")
    x = S.activations(8, 3, 1, T, LFM.hidden)
    base = np.array([5, 9, 2, 60], np.int32)
    ids = np.stack([np.roll(base, t % 4) for t in range(T)]).astype(np.int32)
    _, rw = S.routing_uniform(8, 3, 1, T, LFM.experts, LFM.top_k)
    out, st = layer_mx.gpu(x, ids, rw)
    assert st == 0
    GH.compare(out, layer_mx.oracle(x, ids, rw), "same experts")
    again, _ = layer_mx.gpu(x, ids, rw)
    assert np.array_equal(out, again)


def _routing_with_counts(counts, T, K, E, filler_from):
    """ids [T, K] in which expert e is routed exactly counts[e] times, every
    token to K distinct experts; slots left over go to single-use experts
    numbered from filler_from."""
    ids = -np.ones((T, K), np.int32)
    for e, c in sorted(counts.items(), key=lambda kv: -kv[1]):
        free = sorted(range(T), key=lambda t: -int(np.sum(ids[t] < 0)))
        n = 0
        for t in free:
            if n == c:
                break
            if e in ids[t] or not np.any(ids[t] < 0):
                continue
            ids[t, int(np.argmax(ids[t] < 0))] = e
            n += 1
        assert n == c, "the construction must place every pair"
    nxt = filler_from
    for t in range(T):
        for j in range(K):
            if ids[t, j] < 0:
                ids[t, j] = nxt
                nxt += 1
    assert nxt <= E
    return ids


@pytest.fixture(scope="module")
def layer_nv():
    banner("upload LFM 2048/1536 E4M3 layer 2")
    return GH.Layer(LFM, S.FMT_E4M3_G16, 2)


def test_e4m3_pass_size_boundaries(layer_nv):
    """E4M3 passes of at most 8 tokens put two scale groups in one MFMA and
    larger passes one, and the tiles are split over the CUs by that cost:
    experts routed 8, 9, 16, 17, 24 and 25 times give passes of 8 | 9 | 16 |
    16 + 1 | 16 + 8 | 16 + 9 tokens next to single-token experts."""
    T, K = 25, LFM.top_k
    counts = {3: 25, 11: 24, 20: 17, 31: 16, 40: 9, 47: 8}
    ids = _routing_with_counts(counts, T, K, LFM.experts, 48)
    got = np.bincount(ids.ravel(), minlength=LFM.experts)
    assert all(got[e] == c for e, c in counts.items())
    assert all(len(set(row)) == K for row in ids.tolist())
    banner(f"E4M3 T={T}, expert counts {sorted(counts.values())} + singletons")
    x = S.activations(10, 2, 0, T, LFM.hidden)
    _, rw = S.routing_uniform(10, 2, 0, T, LFM.experts, K)
    r = S.activations(11, 2, 0, T, LFM.hidden)
    out, st = layer_nv.gpu(x, ids, rw, residual=r)
    assert st == 0
    GH.compare(out, layer_nv.oracle(x, ids, rw, residual=r), "E4M3 pass-size boundaries")
    again, _ = layer_nv.gpu(x, ids, rw, residual=r)
    assert np.array_equal(out, again)
