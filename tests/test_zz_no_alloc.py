"""GPU: moe_w4a16_forward_noalloc, the entry point for callers that cannot
allocate (its workspace is the library's own device array), against
moe_w4a16_forward with a caller workspace on the same inputs: two calls in a
row, the second with fewer tokens, both bit-identical to the workspace
entry point (same kernels) and within the oracle's tolerance."""
import numpy as np
import pytest
import torch

from packed_bit_expert_amd import moe as M
from packed_bit_expert_amd import synth as S
from tests import gpu_helpers as GH

pytestmark = pytest.mark.gpu
LFM = S.LFM24B


def _forward(lay, x, ids, rw, residual, flags, noalloc):
    T = ids.shape[0]
    out = torch.empty((T, LFM.hidden), dtype=torch.bfloat16, device=GH.dev())
    rd = None if residual is None else GH.bf16_dev(residual)
    cfg = M.make_cfg(T, flags=flags, residual=rd, prenorm_eps=GH.EPS)
    args = (GH.bf16_dev(x), GH.i32_dev(ids), GH.bf16_dev(rw), lay.wtab, lay.stab, out)
    if noalloc:
        # a workspace the call must not use: left unset
        M.moe_w4a16_forward_noalloc(*args, cfg)
    else:
        ws = torch.zeros(M.moe_w4a16_workspace_bytes(cfg), dtype=torch.uint8, device=GH.dev())
        cfg.workspace, cfg.workspace_bytes = ws.data_ptr(), ws.numel()
        M.moe_w4a16_forward(*args, cfg)
    torch.cuda.synchronize()
    return GH.bits_host(out)


@pytest.mark.parametrize("flags", [M.FLAG_PRENORM, 0, M.FLAG_W4A4])
def test_noalloc_matches_workspace_entry_point(flags):
    print(f"\n[case] forward_noalloc flags={flags}: T=48 then T=1 (then T=5)", flush=True)
    lay = GH.Layer(LFM, S.FMT_E8M0_G32, 6)
    w = S.WORKLOADS["c2"]
    for T, step in ((48, 1), (1, 2), (5, 3)):
        x = S.activations(w.family, 6, step, T, LFM.hidden)
        ids, rw = S.routing_zipf(w.family, 6, step, T, LFM.experts, LFM.top_k)
        res = x if flags & M.FLAG_PRENORM else None
        got = _forward(lay, x, ids, rw, res, flags, True)
        ref = _forward(lay, x, ids, rw, res, flags, False)
        assert np.array_equal(got, ref), f"T={T}: no-alloc differs from the workspace call"
        orc = lay.oracle(x, ids, rw, residual=res, prenorm=bool(flags & M.FLAG_PRENORM),
                         w4a4=bool(flags & M.FLAG_W4A4))
        GH.compare(got, orc, f"no-alloc T={T}")


def test_noalloc_rejects_beyond_its_scratch():
    cfg = M.make_cfg(78)
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_forward_noalloc(1 << 40, 1 << 40, 1 << 40, 1 << 40, 1 << 40,
                                    (1 << 40) + (1 << 30), cfg)
    assert e.value.code == M.ERR_WORKSPACE_TOO_SMALL
    cfg = M.make_cfg(4, flags=M.FLAG_CHECK_IDS)
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_forward_noalloc(1 << 40, 1 << 40, 1 << 40, 1 << 40, 1 << 40,
                                    (1 << 40) + (1 << 30), cfg)
    assert e.value.code == M.ERR_INVALID_ARG
