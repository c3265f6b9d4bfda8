"""Resident packed experts and their persistent device pointer tables.

"LFM2.5-24B-A2B -- Packed MXFP4 Inference", "Direct reads from GPU-resident
weights" and "Full GPU mode": every packed expert stays in device memory,
each expert is one contiguous triplet buffer (gate, up, down nibbles then
their scales; "Bounded pinned RAM expert cache"), and the kernels reach the
selected experts through per-layer device tables of base pointers that are
built once and kept, so no expert is ever staged or copied per call.

On MI355X all 38 layers x 64 experts (12.19 GB for the MXFP4 format) fit in
one GPU's HBM, so one allocation holds the whole stack; the tables for layer
l are rows l of two [L][E] int64 device tensors.
"""
from __future__ import annotations

import concurrent.futures as cf

import torch

from . import synth


class ResidentExperts:
    """Packed experts of ``layers`` MoE layers resident on ``device``.

    ``buf``      uint8 [L][E][triplet] -- per expert: nibbles, then scales
    ``wtab``     int64 [L][E] device pointers to each expert's nibbles
    ``stab``     int64 [L][E] device pointers to each expert's scales
    ``tscales``  float32 [L][E][2] tensor scales (E4M3 format) or None
    """

    def __init__(self, shape: synth.Shape, fmt: int, layers: int, device="cuda"):
        self.shape, self.fmt, self.layers = shape, fmt, layers
        self.nib_bytes = shape.nibble_bytes()
        self.sc_bytes = shape.scale_bytes(fmt)
        self.triplet = self.nib_bytes + self.sc_bytes
        assert self.triplet % 256 == 0 and self.nib_bytes % 256 == 0, "bases stay 256-byte aligned"
        E = shape.experts
        self.buf = torch.empty((layers, E, self.triplet), dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        idx = torch.arange(layers * E, dtype=torch.int64).reshape(layers, E)
        self.wtab = (base + idx * self.triplet).to(device)
        self.stab = (base + idx * self.triplet + self.nib_bytes).to(device)
        self.tscales = None
        if fmt == synth.FMT_E4M3_G16:
            self.tscales = torch.empty((layers, E, 2), dtype=torch.float32, device=device)

    def layer_tables(self, l: int):
        """(wtab, stab, tscales) device tensors of layer l."""
        ts = None if self.tscales is None else self.tscales[l]
        return self.wtab[l], self.stab[l], ts

    def fill_synthetic(self, layer_ids=None, threads: int = 8):
        """Fill every expert from the seeded generator (layer l of the store
        holds generator layer layer_ids[l])."""
        E = self.shape.experts
        layer_ids = list(range(self.layers)) if layer_ids is None else list(layer_ids)
        pinned = torch.empty((E, self.triplet), dtype=torch.uint8).pin_memory()
        host = pinned.numpy()

        def one(args):
            gl, e = args
            host[e, : self.nib_bytes] = synth.expert_nibbles(self.shape, self.fmt, gl, e)
            host[e, self.nib_bytes:] = synth.expert_scales(self.shape, self.fmt, gl, e)

        with cf.ThreadPoolExecutor(threads) as ex:
            for l, gl in enumerate(layer_ids):
                list(ex.map(one, [(gl, e) for e in range(E)]))
                self.buf[l].copy_(pinned, non_blocking=False)
                if self.tscales is not None:
                    self.tscales[l].copy_(torch.from_numpy(synth.tensor_scales(self.shape, self.fmt, gl)))
        return self

    def host_expert(self, l: int, e: int):
        """(nibbles, scales) of one resident expert, copied back to numpy."""
        t = self.buf[l, e].cpu().numpy()
        return t[: self.nib_bytes], t[self.nib_bytes:]
