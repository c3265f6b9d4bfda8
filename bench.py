"""Benchmark of the grouped top-4 W4A16 MoE FFN on one MI355X.

Default workload (the metric's configuration): the 38-layer LFM2.5-24B-A2B
MoE stack, batch-1 decode -- one step is one token through all 38 MoE layers
(weightless pre-norm + BF16 residual between layers, fresh top-4 routing per
layer and step), 64 steps timed warm after warm-up steps, as in the MXFP4
card's benchmark protocol ("Benchmark decode separately from prefill":
repeated 64-forward decode runs, first run excluded).  Inputs are seeded
synthetic data already resident in HBM when timing starts; the weights of all
38 x 64 experts (12.19 GB) stay resident and are read through the pointer
tables.

Prints one JSON line.  `value` is MoE-layer tokens/s (tokens through one MoE
layer per second, i.e. 38 x the stack's tokens/s for the default workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
EPS = 1e-5


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default="c1",
                   choices=["c1", "c0", "c2", "c2stack", "c3", "c4", "c4b32", "c1serial",
                            "c1routed", "c2w4a4", "c3w4a4", "c2stackw4a4", "c1hybrid"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-batch32", action="store_true",
                   help="skip the concurrency-32 sub-record of the default (c1) run")
    p.add_argument("--batch32-steps", type=int, default=64,
                   help="timed layer calls of the concurrency-32 sub-record")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--calib", action="store_true",
                   help="also run a 1 GiB stream read and a 256 MiB copy (counter calibration)")
    p.add_argument("--eager", action="store_true",
                   help="launch every step from the host instead of replaying a captured HIP graph")
    p.add_argument("--timing-steps", type=int, default=16,
                   help="steps of the per-kernel event timing pass (0 = skip)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                        "`bench.py --calib` into profiles/ and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(expert-parallel sharding is a design note, not code). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from packed_bit_expert_amd import synth as S
    from packed_bit_expert_amd.residency import ResidentExperts

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "c1hybrid":
        run_hybrid(args, dev)
        return
    shape = S.LFM24B
    w = S.WORKLOADS[base_workload(args.workload)]
    # layers resident: the whole 38-layer stack for every workload, so single-
    # layer workloads rotate over 38 layers and the reuse distance (762 MB+ per
    # token) exceeds the 256 MB Infinity Cache.
    L = shape.layers
    t0 = time.time()
    store = ResidentExperts(shape, w.fmt, L, device=dev).fill_synthetic()
    print(f"[bench] {L} layers x {shape.experts} experts resident ({store.buf.numel() / 1e9:.2f} GB) "
          f"in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()  # capture needs a non-default stream; every launch and event uses it
    torch.cuda.set_stream(stream)
    res = measure(args, args.workload, store, stream, dev, args.steps, args.warmup,
                  args.cpu_seconds)
    # The metric is quoted at batch 1 and at batch 32: the default run adds the
    # concurrency-32 workload (T = 32, Zipf(1.1) routing, one layer per call
    # rotating over the 38 resident layers, graph replay) as a sub-record with
    # its own roofline, MFMA use and oracle baseline.
    if args.workload == "c1" and not args.no_batch32:
        sub = measure(args, "c2", store, stream, dev, args.batch32_steps, max(16, args.warmup),
                      args.cpu_seconds * 2 / 3, calib=False)
        res["batch32"] = {k: sub[k] for k in ("metric", "value", "unit", "ms_per_step", "steps",
                                                 "warmup", "dtype", "config", "roofline",
                                                 "kernels", "cpu_baseline")}
        res["batch32"]["ms_per_call"] = sub["ms_per_step"]
    print(json.dumps(res), flush=True)


def decode_floor(args, store, stream, dev, xs, ids, rws, cfg, warmup, steps, buf, sink):
    """What the batch-1 decode kernels cost without their arithmetic, each
    figure event-timed like the kernels themselves (the library's
    per-dispatch events, launches queued behind a delay kernel):
      loads_only_us   the stack's launches with each layer's two decode
                      kernels replaced by kernels of the same grid that read
                      the same bytes in the same order after the same
                      dependent slot load, with no arithmetic (per kind: 1 =
                      gate/up, 2 = down);
      empty_us        an empty kernel with each decode kernel's grid;
      burst_read_us   a read of each kernel's algorithmic byte count in which
                      every lane issues all of its 16-byte loads before using
                      any (1, 2, 4 or 8 per lane), each launch at a new
                      offset of a 1 GiB buffer."""
    import numpy as np

    from packed_bit_expert_amd import moe as M
    L = store.layers
    nt = min(args.timing_steps, steps)
    durs = {}
    for c0 in range(0, nt, 4):
        M.moe_w4a16_delay(30000, stream)
        M.moe_w4a16_timing_begin(1024)
        for s in range(warmup + c0, warmup + min(nt, c0 + 4)):
            M.moe_w4a16_decode_floor(L, xs[s], ids[s], rws[s], store.wtab, store.stab, sink, cfg)
        msl, kinds = M.moe_w4a16_timing_end(1024)
        for d, k in zip(msl, kinds):
            durs.setdefault(k, []).append(d)
    loads_only = {"1": float(np.mean(durs[15]) * 1e3), "2": float(np.mean(durs[16]) * 1e3)}

    def timed(launch, n=128):
        ts = []
        for c0 in range(0, n, 64):
            M.moe_w4a16_delay(30000, stream)
            M.moe_w4a16_timing_begin(64)
            for i in range(c0, c0 + 64):
                launch(i)
            msl, _ = M.moe_w4a16_timing_end(64)
            ts += msl
        return float(np.mean(ts) * 1e3)

    empty = {"1": timed(lambda i: M.moe_w4a16_empty_launch(768, 256, sink, stream)),
             "2": timed(lambda i: M.moe_w4a16_empty_launch(256, 512, sink, stream))}

    # the same two floors inside a captured graph, as the step itself runs:
    # the decode launches of a step with no arithmetic, and as many empty
    # kernels of the same grids as a step launches
    import torch

    def graph_ms(fn, nrep):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(nrep):
                fn(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / nrep

    floor_step_ms = graph_ms(lambda r: M.moe_w4a16_decode_floor(
        L, xs[warmup + r], ids[warmup + r], rws[warmup + r], store.wtab, store.stab, sink, cfg),
        steps)

    def empty_step(r):
        M.moe_w4a16_empty_launch(1, 256, sink, stream)  # the slot resolve's place
        for _ in range(L):
            M.moe_w4a16_empty_launch(768, 256, sink, stream)
            M.moe_w4a16_empty_launch(256, 512, sink, stream)

    empty_step_ms = graph_ms(empty_step, steps)

    # a grid-wide barrier inside one kernel (what a persistent kernel would
    # pay per in-kernel dependency): one workgroup per CU, 0 and 200 barriers
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    ctr = torch.zeros(2, dtype=torch.int32, device=dev)
    barrier_us = {}
    for wg in (64, ncu):
        t = {}
        for nb in (0, 200):
            ts = []
            for _ in range(8):
                ctr.zero_()
                M.moe_w4a16_timing_begin(1)
                M.moe_w4a16_grid_barrier(wg, nb, ctr, stream)
                msl, _ = M.moe_w4a16_timing_end(1)
                ts += msl
            t[nb] = float(np.median(ts) * 1e3)
        torch.cuda.synchronize()
        if int(ctr[1].item()) != 0:
            raise RuntimeError("grid barrier probe: a bounded poll gave up")
        barrier_us[str(wg)] = (t[200] - t[0]) / 200
    burst = {}
    for kind, nb in (("1", 13373440), ("2", 6692864)):
        nreg = buf.numel() // nb
        burst[kind] = {str(lpl): timed(lambda i, lpl=lpl: M.moe_w4a16_read_burst(
            buf.data_ptr() + (i % nreg) * nb, nb, lpl, sink, stream)) for lpl in (1, 2, 4, 8)}
    return {"loads_only_us": loads_only, "empty_us": empty, "burst_read_us": burst,
            "graph_loads_only_step_ms": floor_step_ms, "graph_empty_step_ms": empty_step_ms,
            "grid_barrier_us_by_workgroups": barrier_us,
            "launches_per_step": 2 * L + 1,
            "burst_read_best_us": {k: min(v.values()) for k, v in burst.items()},
            "note": "kinds: 1 = decode gate/up (13,373,440 B per launch), 2 = decode down + "
                    "combine (6,692,864 B per launch)"}


def base_workload(k):
    """The synthetic input family (synth.WORKLOADS key) of a bench workload."""
    return {"c2stack": "c2", "c1serial": "c1", "c1routed": "c1", "c2w4a4": "c2", "c3w4a4": "c3",
            "c2stackw4a4": "c2", "c1floor": "c1"}.get(k, k)


def measure(args, wkey, store, stream, dev, steps, warmup, cpu_seconds, calib=None):
    """Time `steps` steps of workload `wkey` (after `warmup` untimed ones) on
    the resident experts, then the per-kernel durations, the read ceilings and
    the oracle baseline; returns the result record."""
    import numpy as np
    import torch

    from packed_bit_expert_amd import moe as M
    from packed_bit_expert_amd import synth as S

    shape = S.LFM24B
    routed = wkey == "c1routed"
    w4a4 = wkey.endswith("w4a4")
    w = S.WORKLOADS[base_workload(wkey)]
    stack = wkey in ("c1", "c2stack", "c1serial", "c1routed", "c2stackw4a4")
    T, E, K, H = w.tokens, shape.experts, shape.top_k, shape.hidden
    L = shape.layers
    nsteps = warmup + steps
    # per-step inputs (resident before timing)
    if stack:
        xs = torch.stack([torch.from_numpy(S.activations(w.family, 0, s, T, H).view(np.int16))
                          for s in range(nsteps)]).view(torch.bfloat16).to(dev)
        routes = [[S.routing(w, l, s) for l in range(L)] for s in range(nsteps)]
        ids = torch.from_numpy(np.stack([[r[0] for r in rs] for rs in routes])).to(dev)  # [S][L][T][K]
        rws = torch.from_numpy(np.stack([[r[1].view(np.int16) for r in rs] for rs in routes])).view(
            torch.bfloat16).to(dev)
    else:
        xs = torch.stack([torch.from_numpy(S.activations(w.family, s % L, s, T, H).view(np.int16))
                          for s in range(nsteps)]).view(torch.bfloat16).to(dev)
        routes = [S.routing(w, s % L, s) for s in range(nsteps)]
        ids = torch.from_numpy(np.stack([r[0] for r in routes])).to(dev)
        rws = torch.from_numpy(np.stack([r[1].view(np.int16) for r in routes])).view(torch.bfloat16).to(dev)
    out = torch.empty((nsteps, T, H), dtype=torch.bfloat16, device=dev)
    if routed:
        # the routing is an output of every step (router on the device)
        ids = torch.zeros((nsteps, L, T, K), dtype=torch.int32, device=dev)
        rws = torch.zeros((nsteps, L, T, K), dtype=torch.bfloat16, device=dev)
        wr = torch.from_numpy(np.stack([S.router_weights(shape, w.family, l).view(np.int16)
                                        for l in range(L)])).view(torch.bfloat16).to(dev)
        rbias = torch.from_numpy(np.stack([S.expert_bias(shape, w.family, l)
                                           for l in range(L)])).to(dev)
    flags = M.FLAG_SERIAL if wkey == "c1serial" else 0
    if w4a4:
        flags |= M.FLAG_W4A4
    cfg = M.make_cfg(T, H, shape.inter, E, K, w.fmt, prenorm_eps=EPS, stream=stream, flags=flags)
    if w.fmt == S.FMT_E4M3_G16:
        cfg.tensor_scales = store.tscales[0].data_ptr()
    ws = torch.zeros(M.moe_w4a16_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    cfg.workspace, cfg.workspace_bytes = ws.data_ptr(), ws.numel()

    def step(s):
        if routed:
            M.moe_w4a16_stack_forward_routed(L, xs[s], wr, rbias, store.wtab, store.stab, None,
                                             out[s], ids[s], rws[s], cfg)
        elif stack:
            ts = None if store.tscales is None else store.tscales
            M.moe_w4a16_stack_forward(L, xs[s], ids[s], rws[s], store.wtab, store.stab, ts,
                                      out[s], cfg)
        else:
            l = s % L
            if store.tscales is not None:
                cfg.tensor_scales = store.tscales[l].data_ptr()
            M.moe_w4a16_forward(xs[s], ids[s], rws[s], store.wtab[l], store.stab[l], out[s], cfg)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for s in range(warmup, nsteps):
                step(s)
        torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for s in range(warmup, nsteps):
            step(s)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / steps
    print(f"[bench] {wkey}: {steps} steps in {ms:.3f} ms ({ms_step:.4f} ms per step)",
          file=sys.stderr, flush=True)

    # algorithmic bytes: each call reads its distinct selected experts' packed
    # bytes once, plus activations in and out
    ids_h = ids[warmup:].cpu().numpy()
    if stack:
        distinct = [len(np.unique(ids_h[s, l])) for s in range(steps) for l in range(L)]
    else:
        distinct = [len(np.unique(ids_h[s])) for s in range(steps)]
    layer_calls = len(distinct)
    act = T * H * 2
    if wkey == "c1serial":
        per_kind = kernel_bytes_serial(shape, w, T)
    else:
        per_kind = kernel_bytes(shape, w, T, float(np.mean(distinct)), chained=w.chained)
    alg_bytes = sum(distinct) * shape.expert_bytes(w.fmt) + layer_calls * act * (3 if w.chained else 2)
    secs = ms / 1e3
    achieved_step = alg_bytes / secs / 1e9
    tok_layer_per_s = T * layer_calls / secs

    # per-kernel durations: HIP events on the launch stream around every
    # launch, the same steps replayed eagerly behind a delay kernel so that
    # the queue is full and each event pair brackets only its kernel
    kernels = []
    dominant = None
    if args.timing_steps > 0:
        nt = min(args.timing_steps, steps)
        chunk = 4 if stack else 64
        cap = 4096
        durs = {}
        for c0 in range(0, nt, chunk):
            M.moe_w4a16_delay(30000, stream)
            M.moe_w4a16_timing_begin(cap)
            for s in range(warmup + c0, warmup + min(nt, c0 + chunk)):
                step(s)
            msl, kinds = M.moe_w4a16_timing_end(cap)
            for d, k in zip(msl, kinds):
                durs.setdefault(k, []).append(d)
        torch.cuda.synchronize()
        for k, v in sorted(durs.items()):
            v = np.array(v)
            rec = {"kernel": M.KERNEL_KINDS.get(k, str(k)), "launches_per_step": len(v) / nt,
                   "mean_us": float(v.mean() * 1e3), "median_us": float(np.median(v) * 1e3),
                   "min_us": float(v.min() * 1e3), "share_of_kernel_time": None}
            if k in per_kind:
                rec["alg_bytes_per_launch"] = per_kind[k]
                rec["achieved_GBps"] = per_kind[k] / (v.mean() / 1e3) / 1e9
            rec["_kind"] = k
            rec["_total"] = float(v.sum())
            kernels.append(rec)
        tot = sum(r["_total"] for r in kernels)
        for r in kernels:
            r["share_of_kernel_time"] = r["_total"] / tot
        dominant = max(kernels, key=lambda r: r["_total"])

    # achievable HBM read bandwidth on this GPU (16-byte loads over 1 GiB)
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    for _ in range(2):
        M.moe_w4a16_stream_read(buf, buf.numel(), sink, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        M.moe_w4a16_stream_read(buf, buf.numel(), sink, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    stream_gbps = 5 * buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    # the dominant kernel's bytes read by one launch of the plain stream read
    # (16-byte loads, no arithmetic, no dependent loads), each launch at a new
    # offset of the 1 GiB buffer so that it reads HBM, not the memory-side
    # cache: what launch and memory latency alone cost a kernel of this size
    plain_us = None
    if dominant is not None and dominant.get("alg_bytes_per_launch"):
        nb = int(dominant["alg_bytes_per_launch"]) // 4096 * 4096
        nreg = buf.numel() // nb
        ts = []
        for c0 in range(0, 256, 64):
            M.moe_w4a16_delay(30000, stream)
            M.moe_w4a16_timing_begin(64)
            for i in range(c0, c0 + 64):
                M.moe_w4a16_stream_read(buf.data_ptr() + (i % nreg) * nb, nb, sink, stream)
            msl, _ = M.moe_w4a16_timing_end(64)
            ts += msl
        torch.cuda.synchronize()
        plain_us = float(np.mean(ts) * 1e3)
    # the decode path's floor: the same launches with no arithmetic, empty
    # launches of the same grids, and reads of the same byte counts in which
    # every lane issues all of its loads up front
    floor = None
    if wkey == "c1" and args.timing_steps > 0:
        floor = decode_floor(args, store, stream, dev, xs, ids, rws, cfg, warmup, steps, buf, sink)
    if args.calib if calib is None else calib:
        # counter calibration: one more 1 GiB read and a 256 MiB device copy
        M.moe_w4a16_stream_read(buf, buf.numel(), sink, stream)
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    del buf

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, shape, cpu_seconds, w4a4=w4a4)
        # the same oracle on one thread, over a shorter sample
        cpu1 = cpu_baseline(w, shape, cpu_seconds / 2, w4a4=w4a4, nthreads=1)

    if dominant is not None and "achieved_GBps" in dominant:
        roof = {"bound": "hbm", "achieved": dominant["achieved_GBps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": dominant["achieved_GBps"] / HBM_PEAK_GBPS,
                # counters of this exact workload only: the serial, routed, stacked
                # and W4A4 variants launch other kernels or other byte counts
                "traffic": traffic_for(dominant["_kind"], wkey),
                "kernel": dominant["kernel"],
                "alg_bytes_per_launch": dominant["alg_bytes_per_launch"],
                "mean_launch_us": dominant["mean_us"],
                "plain_read_same_bytes_us": plain_us,
                "frac_of_plain_read": plain_us / dominant["mean_us"] if plain_us else None}
        if floor is not None and dominant["_kind"] in (1, 2):
            # the step's floor: the same launches moving the same bytes with
            # no arithmetic, replayed from a graph like the step itself (the
            # event-timed single kernels carry a ~4 us timing floor that hides
            # the difference; see floor["empty_us"])
            roof["floor"] = floor
            roof["floor_step_ms"] = floor["graph_loads_only_step_ms"]
            roof["frac_of_floor"] = floor["graph_loads_only_step_ms"] / ms_step
            roof["launch_floor_step_ms"] = floor["graph_empty_step_ms"]
        if dominant["_kind"] in (4, 5):
            fl = kernel_flops(shape, T, dominant["_kind"])
            roof["mfma_useful_TFLOPs"] = fl / (dominant["mean_us"] / 1e6) / 1e12
            if w4a4:  # E2M1 x E2M1 on the block-scaled FP4 MFMA: dense peak 10.1 PFLOP/s
                roof["mfma_useful_frac_of_fp4_peak"] = roof["mfma_useful_TFLOPs"] / 10100.0
            else:
                roof["mfma_useful_frac_of_bf16_peak"] = roof["mfma_useful_TFLOPs"] / 2500.0
    else:
        roof = {"bound": "hbm", "achieved": achieved_step, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved_step / HBM_PEAK_GBPS, "traffic": None, "kernel": "whole step"}
    for r in kernels:
        r.pop("_kind")
        r.pop("_total")

    return {
        "metric": "MoE-layer tokens/s & achieved HBM GB/s (% of peak), 24B-A2B shape, batch 1/32",
        "value": tok_layer_per_s,
        "unit": "tokens/s per MoE layer",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4" if w4a4 else "bf16",
        "data": "synthetic (seeded E2M1 nibbles, E8M0 117..123 or E4M3 normal scales, x ~ N(0,1) BF16)",
        "config": {
            "workload": workload_name(wkey),
            "hidden": H, "inter": shape.inter, "experts": E, "top_k": K,
            "layers_per_step": L if stack else 1, "tokens_per_step": T,
            "weights": "E2M1 + E4M3/16 + FP32 tensor scale" if w.fmt else "E2M1 + E8M0/32",
            "stack_tokens_per_s": T * steps / secs if stack else None,
            "graph_replay": not args.eager,
            "step_achieved_GBps": achieved_step,
            "step_frac_of_peak": achieved_step / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_step": alg_bytes / steps,
            "mean_distinct_experts_per_layer_call": float(np.mean(distinct)),
        },
        "roofline": roof,
        "kernels": kernels,
        "hbm_stream_read_GBps": stream_gbps,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
    }


def run_hybrid(args, dev):
    """c1 with the MXFP4 card's hybrid split ("Hybrid mode"): the first 1,854
    experts resident (28 full layers and 62 experts of layer 28), the other
    578 CPU-backed in a pageable checkpoint copy behind a 2 GiB pinned LRU
    cache (the card's automatic limit, min(2 GiB, RAM / 4)).  Resident layers
    run as one stack call; each partially resident layer runs through
    moe_w4a16_hybrid_forward (ids to the host, cache, one H2D copy per routed
    CPU expert, grouped layer).  Eager launches: the host steps cannot be
    captured."""
    import numpy as np
    import torch

    from packed_bit_expert_amd import moe as M
    from packed_bit_expert_amd import synth as S
    from packed_bit_expert_amd.residency import ResidentExperts

    shape, w = S.LFM24B, S.WORKLOADS["c1"]
    L, E, K, H, T = shape.layers, shape.experts, shape.top_k, shape.hidden, 1
    n_res = 1854
    full, part = n_res // E, n_res % E  # 28 full layers, 62 experts of layer 28
    t0 = time.time()
    store = ResidentExperts(shape, w.fmt, full + 1, device=dev).fill_synthetic()
    nib = shape.nibble_bytes()
    trip = nib + shape.scale_bytes(w.fmt)
    ckpt = {}
    for l in range(full, L):
        for e in range(E):
            if l == full and e < part:
                continue
            ckpt[(l, e)] = np.concatenate([S.expert_nibbles(shape, w.fmt, l, e),
                                           S.expert_scales(shape, w.fmt, l, e)])
    print(f"[bench] {n_res} experts resident, {len(ckpt)} CPU-backed ({len(ckpt) * trip / 1e9:.2f} GB "
          f"checkpoint in pageable RAM) in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    wt = store.wtab.cpu().numpy()
    st = store.stab.cpu().numpy()
    tables = {}
    for l in range(full, L):
        rw_ = [int(wt[l, e]) if (l == full and e < part) else 0 for e in range(E)]
        rs_ = [int(st[l, e]) if (l == full and e < part) else 0 for e in range(E)]
        src = [0 if (l == full and e < part) else ckpt[(l, e)].ctypes.data for e in range(E)]
        tables[l] = (rw_, rs_, src)
    cache_bytes = 2 << 30
    staging = torch.empty((T * K, trip), dtype=torch.uint8, device=dev)
    hy = M.moe_w4a16_hybrid_create(trip, nib, cache_bytes, T * K, staging, E, T * K)

    nsteps = args.warmup + args.steps
    xs = torch.stack([torch.from_numpy(S.activations(w.family, 0, s, T, H).view(np.int16))
                      for s in range(nsteps)]).view(torch.bfloat16).to(dev)
    routes = [[S.routing(w, l, s) for l in range(L)] for s in range(nsteps)]
    ids = torch.from_numpy(np.stack([[r[0] for r in rs] for rs in routes])).to(dev)
    rws = torch.from_numpy(np.stack([[r[1].view(np.int16) for r in rs] for rs in routes])).view(
        torch.bfloat16).to(dev)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    cfg = M.make_cfg(T, prenorm_eps=EPS, stream=stream)
    ws = torch.zeros(M.moe_w4a16_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    cfg.workspace, cfg.workspace_bytes = ws.data_ptr(), ws.numel()
    hbuf = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    out = torch.empty((nsteps, T, H), dtype=torch.bfloat16, device=dev)

    def step(s):
        M.moe_w4a16_stack_forward(full, xs[s], ids[s, :full], rws[s, :full], store.wtab[:full],
                                  store.stab[:full], None, hbuf[0], cfg)
        h = hbuf[0]
        for l in range(full, L):
            dst = out[s] if l == L - 1 else hbuf[(l - full + 1) % 2]
            c = M.make_cfg(T, flags=M.FLAG_PRENORM, residual=h, prenorm_eps=EPS, stream=stream)
            c.workspace, c.workspace_bytes = ws.data_ptr(), ws.numel()
            rw_, rs_, src = tables[l]
            M.moe_w4a16_hybrid_forward(hy, h, ids[s, l], rws[s, l], rw_, rs_, src, dst, c)
            h = dst

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    st0 = M.moe_w4a16_hybrid_stats(hy)
    t_start = time.perf_counter()
    for s in range(args.warmup, nsteps):
        step(s)
    torch.cuda.synchronize()
    secs = time.perf_counter() - t_start
    st1 = M.moe_w4a16_hybrid_stats(hy)
    moved = st1["h2d_bytes"] - st0["h2d_bytes"]
    hits = st1["hits"] - st0["hits"]
    reqs = hits + st1["misses"] - st0["misses"]

    # the host link's ceiling: one 256 MiB pinned-to-device copy
    src_p = torch.empty(256 << 20, dtype=torch.uint8).pin_memory()
    dst_d = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst_d.copy_(src_p, non_blocking=True)
    torch.cuda.synchronize()
    tc = time.perf_counter()
    for _ in range(4):
        dst_d.copy_(src_p, non_blocking=True)
    torch.cuda.synchronize()
    link = 4 * (256 << 20) / (time.perf_counter() - tc) / 1e9
    achieved = moved / secs / 1e9
    M.moe_w4a16_hybrid_destroy(hy)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, shape, args.cpu_seconds)
    res = {
        "metric": "MoE-layer tokens/s & achieved HBM GB/s (% of peak), 24B-A2B shape, batch 1/32",
        "value": L * T * args.steps / secs,
        "unit": "tokens/s per MoE layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": secs / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded E2M1 nibbles, E8M0 117..123 scales, x ~ N(0,1) BF16)",
        "config": {"workload": workload_name("c1hybrid"), "hidden": H, "inter": shape.inter,
                   "experts": E, "top_k": K, "layers_per_step": L, "tokens_per_step": T,
                   "resident_experts": n_res, "cpu_backed_experts": len(ckpt),
                   "pinned_cache_bytes": cache_bytes, "graph_replay": False,
                   "stack_tokens_per_s": T * args.steps / secs},
        "roofline": {"bound": "host link", "achieved": achieved, "peak": link, "unit": "GB/s",
                     "frac": achieved / link, "traffic": None,
                     "note": "H2D bytes of routed CPU experts per second of whole steps, against a "
                             "256 MiB pinned H2D copy measured in the same run"},
        "host_transfers": {"h2d_bytes_per_step": moved / args.steps,
                           "routed_cpu_experts_per_step": reqs / args.steps,
                           "pinned_cache_hit_rate": hits / reqs if reqs else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def kernel_bytes(shape, w, T, distinct, chained):
    """Algorithmic bytes per launch of each kernel kind: the packed weights and
    scales of the distinct selected experts that kernel reads, plus the
    activations it reads or writes in HBM by definition (x in; out and the
    residual).  Intermediates (h, y) are not counted."""
    H, I = shape.hidden, shape.inter
    G = shape.group(w.fmt)
    gu = 2 * I * (H // 2 + H // G)
    dn = H * (I // 2 + I // G)
    act = T * H * 2
    return {1: distinct * gu + act, 2: distinct * dn + act * (2 if chained else 1),
            4: distinct * gu + act, 5: distinct * dn, 6: act * (2 if chained else 1),
            12: shape.experts * H * 2 + act}


def kernel_bytes_serial(shape, w, T):
    """As kernel_bytes for serial expert execution: each gate/up and down
    launch reads one expert; the combine reads the residual and writes out."""
    H, I = shape.hidden, shape.inter
    G = shape.group(w.fmt)
    act = T * H * 2
    return {1: 2 * I * (H // 2 + H // G) + act, 2: H * (I // 2 + I // G), 6: 2 * act}


def kernel_flops(shape, T, kind):
    H, I, K = shape.hidden, shape.inter, shape.top_k
    return 2 * T * K * (2 * I * H if kind == 4 else H * I)


def source_hash(kind):
    import hashlib
    files = {1: "decode.hip", 2: "decode.hip", 4: "batched.hip", 5: "batched.hip", 6: "batched.hip"}
    h = hashlib.sha256()
    for f in (files.get(kind, "api.hip"), "common.h"):
        with open(os.path.join(ROOT, "packed_bit_expert_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KIND_FILE = {1: "dec_gateup", 2: "dec_down", 4: "bat_gateup", 5: "bat_down", 6: "combine"}
TRAFFIC_FILE = "hbm_traffic_{kind}_{workload}.txt"


def traffic_for(kind, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload, or None if there is none or the kernel source
    changed since the counters were taken."""
    if kind not in KIND_FILE:
        return None
    p = os.path.join(ROOT, "profiles", TRAFFIC_FILE.format(kind=KIND_FILE[kind], workload=workload))
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash(kind):
        return None
    return float(kv["hbm_bytes_per_launch"])


def pmc_summary(args):
    """Read rocprofv3 counter CSVs of `bench.py --calib` runs (one with
    FETCH_SIZE, one with WRITE_SIZE), scale each counter by what it reads for
    the calibration kernels of known size (1 GiB stream read, 256 MiB copy),
    and write per-kernel HBM bytes per launch to profiles/."""
    import csv
    import glob

    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        if not rows:
            sys.exit(f"no {counter} rows under {d}")
        return rows

    fetch = load(args.pmc_summary[0], "FETCH_SIZE")
    write = load(args.pmc_summary[1], "WRITE_SIZE")

    def per_kernel(rows, pat):
        v = [x for n, x in rows if pat in n]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    gib_kib = float(1 << 20)
    sr, _ = per_kernel(fetch, "k_stream_read")
    cp_w, _ = per_kernel(write, "copyBuffer")
    if cp_w is None:
        cp_w, _ = per_kernel(write, "elementwise")
    f_fetch = gib_kib / max(v for n, v in fetch if "k_stream_read" in n)
    f_write = (256 * 1024.0) / max(v for n, v in write if ("copyBuffer" in n or "elementwise" in n))
    wl = os.environ.get("PMC_WORKLOAD", "c1")
    fmt = 1 if wl.startswith("c4") else 0  # the E4M3 workloads' kernels carry FMT = 1
    names = {1: "k_dec_gateup", 2: "k_dec_down", 4: f"k_bat_gemm<{fmt}, 0", 5: f"k_bat_gemm<{fmt}, 1"}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for kind, pat in names.items():
        fk, nf = per_kernel(fetch, pat)
        wk, nw = per_kernel(write, pat)
        if fk is None or wk is None:
            continue
        hbm = (fk * f_fetch + wk * f_write) * 1024.0
        p = os.path.join(ROOT, "profiles", TRAFFIC_FILE.format(kind=KIND_FILE[kind], workload=wl))
        with open(p, "w") as fh:
            fh.write(f"# HBM traffic per launch of {pat}* ({wl}), from rocprofv3 --pmc FETCH_SIZE and\n"
                     f"# WRITE_SIZE runs of: {os.environ.get('PMC_COMMAND', 'bench.py --calib')}\n"
                     f"# counters scaled by their reading for kernels of known size: FETCH_SIZE of\n"
                     f"# the 1 GiB stream read, WRITE_SIZE of the 256 MiB device copy\n")
            fh.write(f"kernel: {pat}\nworkload: {wl}\n")
            fh.write(f"dispatches_fetch: {nf}\ndispatches_write: {nw}\n")
            fh.write(f"fetch_kib_per_launch_raw: {fk:.1f}\nwrite_kib_per_launch_raw: {wk:.1f}\n")
            fh.write(f"fetch_factor: {f_fetch:.4f}\nwrite_factor: {f_write:.4f}\n")
            fh.write(f"calib_stream_read_fetch_kib: {1 / f_fetch * gib_kib:.1f}\n")
            fh.write(f"hbm_bytes_per_launch: {hbm:.0f}\n")
            fh.write(f"source_sha256: {source_hash(kind)}\n")
        print(open(p).read())


def workload_name(k):
    return {
        "c1": "38-layer MoE stack, batch-1 decode (LFM2.5-24B-A2B, 2048/1536, 64 experts, top-4, E2M1+E8M0/32)",
        "c1serial": "38-layer MoE stack, batch-1 decode, serial expert execution (ablation: one "
                    "gate/up and one down launch per selected expert, then the combine)",
        "c1routed": "38-layer MoE stack, batch-1 decode, routing on the device per layer (router "
                    "projection, sigmoid, expert bias, top-4, coefficients) from the layer input",
        "c0": "one MoE layer, 1 token (rotating over 38 resident layers)",
        "c2": "concurrency-32 decode, Zipf(1.1) routing, one layer per call (rotating over 38 layers)",
        "c2stack": "concurrency-32 decode through the 38-layer stack",
        "c3": "prefill: S=64 chunks through one layer (rotating over 38 layers)",
        "c4": "NVFP4-style E2M1+E4M3/16+FP32 tensor scale, batch 1",
        "c4b32": "NVFP4-style E2M1+E4M3/16+FP32 tensor scale, batch 32",
        "c2w4a4": "concurrency-32 decode, one layer per call, W4A4 (MXFP4 activations on the "
                  "block-scaled FP4 MFMA)",
        "c3w4a4": "prefill S=64 chunks through one layer, W4A4 (MXFP4 activations on the "
                  "block-scaled FP4 MFMA)",
        "c2stackw4a4": "concurrency-32 decode through the 38-layer stack, W4A4",
        "c1hybrid": "38-layer batch-1 decode, hybrid: 1,854 experts resident, 578 CPU-backed behind "
                    "a 2 GiB pinned LRU cache (one H2D copy per routed CPU expert)",
    }[k]


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def cpu_baseline(w, shape, target_s, w4a4=False, nthreads=0):
    """The oracle as it stands on this host's cores (all of them, or
    `nthreads`), on a bounded sample of the workload: layer calls of the
    workload's batch in the workload's order (consecutive layers of one step,
    chained through the pre-norm and residual for the stack), until about
    `target_s` seconds of oracle time."""
    import numpy as np

    from oracle import oracle as O
    from packed_bit_expert_amd import synth as S
    threads = nthreads or O.threads_available()
    T = w.tokens
    busy = 0.0
    calls = 0
    h = None
    while busy < target_s:
        layer, step = calls % shape.layers, 10_000 + calls // shape.layers
        if w.chained:
            if layer == 0:
                h = S.activations(w.family, 0, step, T, shape.hidden)
        else:
            h = S.activations(w.family, layer, step, T, shape.hidden)
        ids, rw = S.routing(w, layer, step)
        nib = [None] * shape.experts
        sc = [None] * shape.experts
        for e in np.unique(ids):
            nib[int(e)] = S.expert_nibbles(shape, w.fmt, layer, int(e))
            sc[int(e)] = S.expert_scales(shape, w.fmt, layer, int(e))
        ts = S.tensor_scales(shape, w.fmt, layer)
        t0 = time.perf_counter()
        out = O.moe_forward(h, ids, rw, nib, sc, hidden=shape.hidden, inter=shape.inter,
                            num_experts=shape.experts, fmt=w.fmt, tensor_scales=ts,
                            residual=h if w.chained else None, prenorm=w.chained, eps=EPS,
                            w4a4=w4a4, nthreads=threads)
        busy += time.perf_counter() - t0
        if w.chained:
            h = out
        calls += 1
    return {"value": T * calls / busy, "unit": "tokens/s per MoE layer", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus_online": os.cpu_count(),
            "sample": f"{calls} {'W4A4 ' if w4a4 else ''}layer calls of {T} token(s) on {w.name} inputs (layers 0..{min(calls, shape.layers) - 1}"
                      f"{', chained' if w.chained else ''}), fp64 scalar C oracle with {threads} OpenMP "
                      f"threads, {busy:.1f} s of oracle time (input generation excluded)"}


if __name__ == "__main__":
    main()
