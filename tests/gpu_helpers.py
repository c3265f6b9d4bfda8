"""Helpers for the GPU parity tests: upload seeded inputs, call the C-ABI,
and compare with the oracle under the stated tolerance.

Tolerance (per output tensor of one call): every element satisfies
|gpu - ref| <= 1e-2 * max(|ref|, rms(ref)) and the relative L2 error
||gpu - ref|| / ||ref|| <= 5e-3, where ref is the oracle's BF16 result.
The fraction of bit-identical elements is reported as a bug detector.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O
from packed_bit_expert_amd import moe as M
from packed_bit_expert_amd import synth as S

ELEM_TOL = 1e-2
L2_TOL = 5e-3
EPS = float(np.float32(1e-5))  # the pre-norm epsilon, as the FP32 value the library receives


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(
        torch.bfloat16).to(dev())


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev())


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(dev())


def compare(gpu_bits, ref_bits, what="out", check=True):
    g = O.f64_from_bf16(gpu_bits).ravel()
    r = O.f64_from_bf16(ref_bits).ravel()
    assert np.all(np.isfinite(r)), f"{what}: oracle produced non-finite values"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    bound = ELEM_TOL * np.maximum(np.abs(r), rms)
    nrm = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r)) / nrm if nrm > 0 else float(np.linalg.norm(g))
    ident = float(np.mean(np.asarray(gpu_bits).ravel() == np.asarray(ref_bits).ravel())) if r.size else 1.0
    stats = {"what": what, "n": int(r.size), "rel_l2": rel, "max_ratio": float(np.max(err / np.maximum(bound, 1e-300))) if r.size else 0.0,
             "bit_identical": ident, "finite": bool(np.all(np.isfinite(g)))}
    print(f"[parity] {what}: n={stats['n']} rel_l2={rel:.3e} max|d|/bound={stats['max_ratio']:.3f} "
          f"bit-identical={ident:.5f}", flush=True)
    if check:
        assert stats["finite"], f"{what}: GPU produced non-finite values"
        assert np.all(err <= bound), f"{what}: element bound violated ({stats})"
        assert rel <= L2_TOL, f"{what}: relative L2 {rel} > {L2_TOL}"
    return stats


class Layer:
    """One resident layer of seeded experts plus host copies for the oracle."""

    def __init__(self, shape: S.Shape, fmt: int, gen_layer: int, store=None, l: int = 0):
        from packed_bit_expert_amd.residency import ResidentExperts
        self.shape, self.fmt, self.gen_layer = shape, fmt, gen_layer
        if store is None:
            store = ResidentExperts(shape, fmt, 1).fill_synthetic([gen_layer])
            l = 0
        self.store, self.l = store, l
        self.wtab, self.stab, self.tsc = store.layer_tables(l)
        self._host = {}

    def host(self, e):
        if e not in self._host:
            self._host[e] = (S.expert_nibbles(self.shape, self.fmt, self.gen_layer, e),
                             S.expert_scales(self.shape, self.fmt, self.gen_layer, e))
        return self._host[e]

    def host_tables(self, ids):
        nib = [None] * self.shape.experts
        sc = [None] * self.shape.experts
        for e in np.unique(ids):
            nib[int(e)], sc[int(e)] = self.host(int(e))
        return nib, sc

    def host_tscales(self):
        return S.tensor_scales(self.shape, self.fmt, self.gen_layer)

    def oracle(self, x, ids, rw, residual=None, prenorm=False, eps=EPS, dumps=False, w4a4=False):
        nib, sc = self.host_tables(ids)
        return O.moe_forward(x, ids, rw, nib, sc, hidden=self.shape.hidden, inter=self.shape.inter,
                             num_experts=self.shape.experts, fmt=self.fmt,
                             tensor_scales=self.host_tscales(), residual=residual,
                             prenorm=prenorm, eps=eps, dumps=dumps, w4a4=w4a4)

    def gpu(self, x, ids, rw, residual=None, flags=0, eps=EPS, dumps=False, wtab=None):
        sh = self.shape
        T, K = ids.shape
        xd = bf16_dev(x)
        idd = i32_dev(ids)
        rwd = bf16_dev(rw)
        rd = None if residual is None else bf16_dev(residual)
        out = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device=dev())
        cfg = M.make_cfg(T, sh.hidden, sh.inter, sh.experts, K, self.fmt, flags=flags,
                         tensor_scales=self.tsc, residual=rd, prenorm_eps=eps)
        ws = torch.zeros(M.moe_w4a16_workspace_bytes(cfg), dtype=torch.uint8, device=dev())
        cfg.workspace, cfg.workspace_bytes = ws.data_ptr(), ws.numel()
        d = {}
        if dumps:
            d = {"u": torch.empty((T, sh.hidden), dtype=torch.bfloat16, device=dev()),
                 "g": torch.empty((T, K, sh.inter), dtype=torch.bfloat16, device=dev()),
                 "v": torch.empty((T, K, sh.inter), dtype=torch.bfloat16, device=dev()),
                 "h": torch.empty((T, K, sh.inter), dtype=torch.bfloat16, device=dev()),
                 "y": torch.empty((T, K, sh.hidden), dtype=torch.bfloat16, device=dev())}
        M.moe_w4a16_forward_debug(xd, idd, rwd, self.wtab if wtab is None else wtab, self.stab,
                                  out, cfg, **d)
        torch.cuda.synchronize()
        status = M.moe_w4a16_device_status(ws)
        res = bits_host(out)
        if dumps:
            return res, {k: bits_host(v) for k, v in d.items()}, status
        return res, status
