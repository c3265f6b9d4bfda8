"""GPU: the measurement helpers that stand next to the decode path.

The decode floor replaces each layer's two decode kernels by kernels that
load the same bytes and compute nothing ("LFM2.5-24B-A2B on Your Own
Hardware", "What speed should I expect? A bandwidth ceiling, not a
promise": decode speed is bounded by the bytes each token must read).  Its
figures only mean something if those kernels read what the decode kernels
read, so the first test recomputes, on the host, the XOR folds they store
from the expert bytes, x, the coefficients and the residual, for a one-layer
stack: every stored word depends on the exact addresses of its loads.  The
other tests check that the empty launch, the burst read and the bounded
grid barrier run and report as documented.
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
H, I, K = LFM.hidden, LFM.inter, LFM.top_k


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def _fold16(b):
    """XOR of the four little-endian dwords of each 16-byte row of b."""
    return np.bitwise_xor.reduce(np.ascontiguousarray(b).view("<u4").reshape(-1, 4), axis=1)


def _floor_reference(x, ids, rw, experts):
    """What the floor kernels of one layer store, from the same inputs:
    h [K * I] (the gate/up floor) and the layer's output words [H]."""
    xb = np.ascontiguousarray(x.reshape(-1)).view(np.uint8)       # H BF16
    xpiece = _fold16(xb)                                         # 16 bytes per thread
    h = np.zeros(K * I, np.uint32)
    for sj in range(K):
        nib, sc = experts[int(ids[sj])]
        gate_w = nib[: I * H // 2].reshape(I, H // 2)
        gate_s = sc[: I * H // 32].reshape(I, H // 32)
        for nb in range(I // 2):
            gw = sj * (I // 2) + nb
            wave = gw % 4
            for q in (0, 2):                                   # the two storing lanes
                n = 2 * nb + q // 2
                acc = int(xpiece[64 * wave + 16 * q])
                for i in range(4):
                    acc ^= int(gate_s[n, 16 * i])
                    acc ^= int(_fold16(gate_w[n, 16 * (16 * i): 16 * (16 * i) + 16])[0])
                h[sj * I + n] = acc & 0xFFFF
    h16 = h.astype(np.uint16)
    hb = h16.view(np.uint8)
    nib0, sc0 = experts[int(ids[0])]                             # wave 0: slot 0, rows m0..m0+3
    down_w = nib0[I * H:].reshape(H, I // 2)
    down_s = sc0[2 * I * H // 32:].reshape(H, I // 32)
    rwv = [int(v) for v in rw.reshape(-1)]
    xv = x.reshape(-1)
    out = np.zeros(H, np.uint16)
    for m0 in range(0, H, 8):
        for tid in range(8):                                   # the storing lanes: li = tid, q = 0
            acc = 0
            for j in range(K):
                acc ^= rwv[j]
            acc ^= int(xv[m0 + tid])
            for u in range(3):                                 # slot 0's h, piece tid + 64 u
                e0 = 8 * (tid + 64 * u)
                acc ^= int(_fold16(hb[2 * e0: 2 * e0 + 16])[0])
            for i in range(3):
                acc ^= int(down_s[m0, tid + 16 * i])
                c = 16 * (tid + 16 * i)
                acc ^= int(_fold16(down_w[m0, c: c + 16])[0])
            out[m0 + tid] = acc & 0xFFFF
    return h16, out


def test_decode_floor_reads_the_decode_kernels_bytes():
    banner("decode floor, one layer, T=1: host recomputation of the stored folds")
    store = ResidentExperts(LFM, S.FMT_E8M0_G32, 1).fill_synthetic([5])
    x = S.activations(12, 5, 0, 1, H)
    ids, rw = S.routing_uniform(12, 5, 0, 1, LFM.experts, K)
    dev = GH.dev()
    cfg = M.make_cfg(1, H, I, LFM.experts, K, prenorm_eps=GH.EPS)
    ws = torch.zeros(M.moe_w4a16_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    cfg.workspace, cfg.workspace_bytes = ws.data_ptr(), ws.numel()
    sink = torch.zeros(8192, dtype=torch.int16, device=dev)
    M.moe_w4a16_decode_floor(1, GH.bf16_dev(x), GH.i32_dev(ids[None]), GH.bf16_dev(rw[None]),
                             store.wtab, store.stab, sink, cfg)
    torch.cuda.synchronize()
    got = sink[:H].cpu().numpy().view(np.uint16)
    experts = {int(e): store.host_expert(0, int(e)) for e in ids.reshape(-1)}
    _, want = _floor_reference(x, ids.reshape(-1), rw, experts)
    assert np.array_equal(got, want), f"{int(np.sum(got != want))} of {H} floor words differ"
    # a second call on the same inputs stores the same words
    sink2 = torch.zeros_like(sink)
    M.moe_w4a16_decode_floor(1, GH.bf16_dev(x), GH.i32_dev(ids[None]), GH.bf16_dev(rw[None]),
                             store.wtab, store.stab, sink2, cfg)
    torch.cuda.synchronize()
    assert torch.equal(sink, sink2)


def test_empty_launch_and_burst_read():
    banner("empty launch; burst read of 1, 2, 4, 8 loads per lane")
    dev = GH.dev()
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    for wg, th in ((1, 1), (768, 256), (256, 1024)):
        M.moe_w4a16_empty_launch(wg, th, sink, stream)
    src = torch.arange(1 << 20, dtype=torch.int32, device=dev)    # 4 MiB
    for lpl in (1, 2, 4, 8):
        M.moe_w4a16_read_burst(src.data_ptr(), src.numel() * 4, lpl, sink, stream)
    with pytest.raises(M.MoeError):
        M.moe_w4a16_read_burst(src.data_ptr(), src.numel() * 4, 3, sink, stream)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0, "the sinks are never written for these inputs"


@pytest.mark.parametrize("wg", [64, "cus"])
def test_grid_barrier_completes(wg):
    dev = GH.dev()
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    n = ncu if wg == "cus" else wg
    banner(f"grid barrier, {n} workgroups, 50 barriers")
    stream = torch.cuda.current_stream().cuda_stream
    ctr = torch.zeros(2, dtype=torch.int32, device=dev)
    M.moe_w4a16_grid_barrier(n, 50, ctr, stream)
    torch.cuda.synchronize()
    assert int(ctr[1].item()) == 0, "a bounded poll gave up"
    assert int(ctr[0].item()) == n * 50
    with pytest.raises(M.MoeError):
        M.moe_w4a16_grid_barrier(ncu + 1, 1, ctr, stream)
