"""Closed forms the pages print, pinning the shapes and byte counts (CPU only).

The numbers come from tests/golden/closed_forms.json, each with its page and
section.  They pin the expert shape used by the layout, the oracle and the
roofline's algorithmic bytes: per-expert parameters 3*h*inter, the
active/total split, and the bits per weight of both packed formats (4.25 for
E2M1 + E8M0/32, 4.5 for E2M1 + E4M3/16), the latter through the published
checkpoint sizes.
"""
import json
import os

import pytest

from packed_bit_expert_amd import synth as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def g(name):
    return GOLD[name]["value"]


def close(x, name):
    d = GOLD[name].get("decimals", 0)
    return round(x, d) == pytest.approx(g(name), abs=10 ** -d / 2 + 1e-12)


def test_shape_constants():
    s = S.LFM24B
    assert (s.hidden, s.inter, s.experts, s.top_k, s.layers) == (
        g("hidden"), g("moe_intermediate"), g("experts"), g("top_k"), g("moe_layers"))


def test_parameter_counts():
    s = S.LFM24B
    per_expert = s.nibble_bytes() * 2          # two E2M1 values per byte
    assert per_expert == g("per_expert_params") == 3 * s.hidden * s.inter
    all_e = per_expert * s.experts * s.layers
    act = per_expert * s.top_k * s.layers
    assert close(all_e / 1e9, "all_expert_params_billions")
    assert close(act / 1e9, "active_expert_params_billions")
    always = g("total_params") - all_e
    assert close(always / 1e9, "always_on_params_billions")
    assert close((always + act) / 1e9, "active_total_params_billions")
    assert close(100.0 * all_e / g("total_params"), "expert_share_percent")


def test_bits_per_weight_from_checkpoint_sizes():
    s = S.LFM24B
    per_expert = 3 * s.hidden * s.inter
    n_exp = s.experts * s.layers
    all_e = per_expert * n_exp
    always = g("total_params") - all_e
    # NVFP4A16 build: experts at E2M1 + one E4M3 byte per 16 values (4.5 bits),
    # everything else BF16 -> the published 14.95 GB.
    nv_bytes = S.LFM24B.expert_bytes(S.FMT_E4M3_G16) * n_exp + 2 * always
    assert S.LFM24B.expert_bytes(S.FMT_E4M3_G16) * 8 == per_expert * 4.5
    assert close(nv_bytes / 1e9, "nvfp4a16_file_gigabytes")
    # BF16 everything -> 47.94 GB
    assert close(2 * g("total_params") / 1e9, "bf16_file_gigabytes")
    # MXFP4 checkpoint: the hub counts each U8 byte (nibbles + E8M0 scales) as a
    # parameter next to the BF16/F32 ones -> ~13B "params".
    mx = S.LFM24B.expert_bytes(S.FMT_E8M0_G32)
    assert mx * 8 == per_expert * 4.25 and mx == 5_013_504
    assert close((mx * n_exp + always) / 1e9, "mxfp4_checkpoint_params_billions")


def test_launch_counts():
    s = S.LFM24B
    assert s.layers * s.top_k == g("moe_launches_serial")
    assert s.layers == g("moe_launches_grouped")
    assert g("moe_launches_serial") + g("rms_conv_launches") == g("graph_launches_before")
    assert g("moe_launches_grouped") + g("rms_conv_launches") == g("graph_launches_after")


def test_algorithmic_bytes_per_token_layer():
    """Bytes the roofline counts: the 4 selected experts' packed bytes."""
    s = S.LFM24B
    assert 4 * s.expert_bytes(S.FMT_E8M0_G32) == 20_054_016
    assert 4 * s.expert_bytes(S.FMT_E4M3_G16) == 21_233_664
    assert 38 * 4 * s.expert_bytes(S.FMT_E8M0_G32) == 762_052_608
