"""The benchmark's host logic (CPU only): the one-GPU rule, the algorithmic
byte and flop counts behind the roofline, and the rule that a counter summary
of an older kernel source is not reported as traffic.

The byte counts are pinned to the pages' parameter count ("LFM2.5-24B-A2B on
Your Own Hardware: The RAM, KV Cache and Bandwidth Budget", "Where do the 2.45B
active parameters actually go?": three hidden x expert-intermediate matrices
per expert) and the bits per weight of the two packed formats: 4 + 8/32 for
E2M1 with one E8M0 per 32 ("LFM2.5-24B-A2B -- Packed MXFP4 Inference", "Model
and quantization") and 4 + 8/16 for E2M1 with one E4M3 per 16
("primitive-ai/LFM2.5-24B-A2B-NVFP4A16", "What's quantized to what").
"""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench
from packed_bit_expert_amd import synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "closed_forms.json")))
PARAMS = GOLD["per_expert_params"]["value"]  # 3 * 2048 * 1536


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("wname,bits", [("c1", 4 + 8 / 32), ("c4", 4 + 8 / 16)])
def test_decode_bytes_per_launch(wname, bits):
    """T = 1, four distinct experts: gate/up reads two of the three matrices
    of each expert and x; down reads the third, the residual, and writes out
    (chained stack) or only writes out."""
    w = S.WORKLOADS[wname]
    sh = S.LFM24B
    per_matrix = PARAMS // 3 * bits / 8
    assert sh.expert_bytes(w.fmt) == pytest.approx(3 * per_matrix, abs=0)
    act = sh.hidden * 2
    kb = bench.kernel_bytes(sh, w, 1, 4.0, chained=w.chained)
    assert kb[1] == pytest.approx(4 * 2 * per_matrix + act, abs=0)
    assert kb[2] == pytest.approx(4 * per_matrix + act * (2 if w.chained else 1), abs=0)
    if wname == "c1":  # the figures the roofline reports for the headline workload
        assert (kb[1], kb[2]) == (13373440, 6692864)


def test_batched_bytes_and_flops():
    w = S.WORKLOADS["c2"]
    sh = S.LFM24B
    per_matrix = PARAMS // 3 * (4 + 8 / 32) / 8
    kb = bench.kernel_bytes(sh, w, 32, 39.0, chained=False)
    assert kb[4] == pytest.approx(39 * 2 * per_matrix + 32 * sh.hidden * 2, abs=0)
    assert kb[5] == pytest.approx(39 * per_matrix, abs=0)
    # useful flops: two per multiply-add of every (token, slot) pair's GEMV
    assert bench.kernel_flops(sh, 32, 4) == 2 * 32 * 4 * (2 * PARAMS // 3)
    assert bench.kernel_flops(sh, 32, 5) == 2 * 32 * 4 * (PARAMS // 3)


def test_serial_bytes_one_expert_per_launch():
    w = S.WORKLOADS["c1"]
    sh = S.LFM24B
    serial = bench.kernel_bytes_serial(sh, w, 1)
    grouped = bench.kernel_bytes(sh, w, 1, 1.0, chained=False)
    assert serial[1] == grouped[1] and serial[2] == grouped[5]


def test_every_workload_has_a_name():
    names = set(bench.workload_name(k) for k in
                ["c1", "c0", "c2", "c2stack", "c3", "c4", "c4b32", "c1serial", "c1routed",
                 "c2w4a4", "c3w4a4", "c2stackw4a4", "c1hybrid"])
    assert len(names) == 13


def test_traffic_needs_the_current_source(tmp_path, monkeypatch):
    """A counter summary is reported only while the kernel's source hash
    matches the one recorded with the counters."""
    csrc = tmp_path / "packed_bit_expert_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("decode.hip", "common.h"):
        shutil.copy(os.path.join(ROOT, "packed_bit_expert_amd", "csrc", f), csrc / f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    p = tmp_path / "profiles" / bench.TRAFFIC_FILE.format(kind="dec_gateup", workload="c1")
    assert bench.traffic_for(1, "c1") is None  # no summary
    p.write_text(f"hbm_bytes_per_launch: 123456\nsource_sha256: {bench.source_hash(1)}\n")
    assert bench.traffic_for(1, "c1") == 123456.0
    with open(csrc / "decode.hip", "a") as fh:
        fh.write("\n// changed\n")
    assert bench.traffic_for(1, "c1") is None  # the kernel changed since
    assert bench.traffic_for(3, "c1") is None  # no summary kind for the slot resolve


def test_cpu_baseline_thread_count_is_per_call():
    """The bench times the oracle on every host core and then on one; the
    one-thread run must not leave the process at one thread, or a later
    all-cores baseline (the batch-32 sub-record's) runs on one core."""
    import numpy as np

    from oracle import oracle as O
    sh = S.Shape(hidden=256, inter=128, experts=8, top_k=2, layers=1)
    x = S.activations(1, 0, 0, 3, sh.hidden)
    ids, rw = S.routing_uniform(1, 0, 0, 3, sh.experts, sh.top_k)
    nib = [S.expert_nibbles(sh, S.FMT_E8M0_G32, 0, e) for e in range(sh.experts)]
    sc = [S.expert_scales(sh, S.FMT_E8M0_G32, 0, e) for e in range(sh.experts)]
    before = O.threads_available()
    kw = dict(hidden=sh.hidden, inter=sh.inter, num_experts=sh.experts, fmt=S.FMT_E8M0_G32)
    one = O.moe_forward(x, ids, rw, nib, sc, nthreads=1, **kw)
    assert O.threads_available() == before
    assert np.array_equal(one, O.moe_forward(x, ids, rw, nib, sc, **kw))
