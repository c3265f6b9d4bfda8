"""The C-ABI library on a host without a GPU: it loads, exports every symbol
the header declares, and rejects bad arguments with the documented codes
before anything is enqueued (argument checks read host values only)."""
import os
import re

import pytest

from packed_bit_expert_amd import moe as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe_w4a16.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_w4a16_\w+)\s*\(", src)))


def test_header_exports_match_library():
    names = header_functions()
    assert names == sorted(M.EXPORTS)
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n


def test_constants_match_header():
    src = open(os.path.join(ROOT, "include", "moe_w4a16.h")).read()
    defs = dict(re.findall(r"#define (MOE_\w+) \(?(-?\w+(?: << \d+)?)\)?", src))
    assert int(defs["MOE_W4A16_ABI_VERSION"]) == M.ABI_VERSION == M.moe_w4a16_abi_version()
    assert int(defs["MOE_ERR_WORKSPACE_TOO_SMALL"]) == M.ERR_WORKSPACE_TOO_SMALL
    assert int(defs["MOE_ERR_DEVICE_CHECK"]) == M.ERR_DEVICE_CHECK
    assert int(defs["MOE_SCALE_E4M3_G16"]) == M.SCALE_E4M3_G16
    for n in ["PRENORM", "FORCE_DECODE", "FORCE_BATCHED", "CHECK_IDS", "SERIAL", "W4A4"]:
        assert eval(defs["MOE_FLAG_" + n].replace("u", "")) == getattr(M, "FLAG_" + n), n


def test_shape_support():
    assert M.moe_w4a16_shape_supported(2048, 1536)
    assert M.moe_w4a16_shape_supported(512, 256)
    assert not M.moe_w4a16_shape_supported(2048, 1000)
    assert not M.moe_w4a16_shape_supported(0, 1536)
    assert not M.moe_w4a16_shape_supported(8192, 1536)


FAKE = 1 << 40  # aligned host-side pointer values; never dereferenced


def call(cfg, **over):
    args = dict(x=FAKE, ids=FAKE, rw=FAKE, w=FAKE, s=FAKE, out=FAKE + (1 << 30))
    args.update(over)
    M.moe_w4a16_forward(args["x"], args["ids"], args["rw"], args["w"], args["s"], args["out"], cfg)


def cfg(**kw):
    c = M.make_cfg(kw.pop("T", 1))
    c.workspace = kw.pop("workspace", FAKE + (2 << 30))
    c.workspace_bytes = kw.pop("workspace_bytes", 1 << 30)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("over,code", [
    (dict(abi_version=2), M.ERR_ABI_MISMATCH),
    (dict(num_tokens=-1), M.ERR_INVALID_ARG),
    (dict(hidden=2000), M.ERR_UNSUPPORTED_SHAPE),
    (dict(inter=100), M.ERR_UNSUPPORTED_SHAPE),
    (dict(top_k=0), M.ERR_UNSUPPORTED_SHAPE),
    (dict(top_k=9), M.ERR_UNSUPPORTED_SHAPE),
    (dict(num_experts=0), M.ERR_UNSUPPORTED_SHAPE),
    (dict(scale_fmt=7), M.ERR_INVALID_ARG),
    (dict(scale_fmt=M.SCALE_E4M3_G16), M.ERR_INVALID_ARG),           # no tensor scales
    (dict(tensor_scales=FAKE), M.ERR_INVALID_ARG),                     # E8M0 with tensor scales
    (dict(flags=1 << 9), M.ERR_INVALID_ARG),
    (dict(flags=M.FLAG_FORCE_DECODE | M.FLAG_FORCE_BATCHED), M.ERR_INVALID_ARG),
    (dict(hidden=4096, inter=1024, flags=M.FLAG_FORCE_DECODE), M.ERR_UNSUPPORTED_SHAPE),
    (dict(workspace=0), M.ERR_INVALID_ARG),
    (dict(workspace=FAKE + 8), M.ERR_MISALIGNED),
    (dict(workspace_bytes=100), M.ERR_WORKSPACE_TOO_SMALL),
    (dict(flags=M.FLAG_PRENORM, prenorm_eps=-1.0), M.ERR_INVALID_ARG),
    (dict(flags=M.FLAG_W4A4, scale_fmt=M.SCALE_E4M3_G16, tensor_scales=FAKE), M.ERR_INVALID_ARG),
    (dict(flags=M.FLAG_W4A4 | M.FLAG_FORCE_DECODE), M.ERR_INVALID_ARG),
    (dict(flags=M.FLAG_W4A4 | M.FLAG_SERIAL), M.ERR_INVALID_ARG),
])
def test_cfg_errors(over, code):
    with pytest.raises(M.MoeError) as ei:
        call(cfg(**over))
    assert ei.value.code == code, str(ei.value)


@pytest.mark.parametrize("over,code", [
    (dict(x=0), M.ERR_INVALID_ARG),
    (dict(ids=0), M.ERR_INVALID_ARG),
    (dict(out=0), M.ERR_INVALID_ARG),
    (dict(w=0), M.ERR_INVALID_ARG),
    (dict(x=FAKE + 2), M.ERR_MISALIGNED),
    (dict(out=FAKE + (1 << 30) + 4), M.ERR_MISALIGNED),
    (dict(ids=FAKE + 2), M.ERR_MISALIGNED),
    (dict(w=FAKE + 4), M.ERR_MISALIGNED),
    (dict(out=FAKE + 1024), M.ERR_INVALID_ARG),   # overlaps x (T=1, H=2048 -> 4 KiB)
])
def test_pointer_errors(over, code):
    with pytest.raises(M.MoeError) as ei:
        call(cfg(), **over)
    assert ei.value.code == code, str(ei.value)


def test_zero_tokens_is_noop_without_pointers():
    M.moe_w4a16_forward(0, 0, 0, 0, 0, 0, cfg(T=0))


def test_workspace_bytes_grows_with_tokens():
    b1 = M.moe_w4a16_workspace_bytes(cfg(T=1))
    b64 = M.moe_w4a16_workspace_bytes(cfg(T=64))
    assert 0 < b1 < b64
    assert b1 % 256 == 0 and b64 % 256 == 0
    assert M.moe_w4a16_workspace_bytes(cfg(hidden=100)) == 0


def test_stack_and_hook_errors():
    with pytest.raises(M.MoeError) as ei:
        M.moe_w4a16_stack_forward(0, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + (1 << 30), cfg())
    assert ei.value.code == M.ERR_INVALID_ARG
    with pytest.raises(M.MoeError) as ei:
        M.moe_w4a16_dequant(FAKE, FAKE, 4, 48, 0, FAKE)
    assert ei.value.code == M.ERR_UNSUPPORTED_SHAPE
    with pytest.raises(M.MoeError) as ei:
        M.moe_w4a16_combine(FAKE, FAKE, None, FAKE, 1, 4, 2052)
    assert ei.value.code == M.ERR_UNSUPPORTED_SHAPE
    with pytest.raises(M.MoeError) as ei:
        M.moe_w4a16_sort_pairs(FAKE + 1, 4, 4, 64, FAKE, FAKE, FAKE)
    assert ei.value.code == M.ERR_MISALIGNED
    with pytest.raises(M.MoeError) as ei:
        M.moe_w4a16_stream_read(FAKE, 100, FAKE)
    assert ei.value.code == M.ERR_MISALIGNED
    assert "16-byte" in M.moe_w4a16_last_error()


def test_measurement_helpers_reject_bad_arguments():
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_delay(1_000_001)
    assert e.value.code == M.ERR_INVALID_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_timing_begin(0)
    assert e.value.code == M.ERR_INVALID_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_timing_end(16)  # never begun on this thread
    assert e.value.code == M.ERR_INVALID_ARG


def test_kernel_kind_constants_match_header():
    src = open(os.path.join(ROOT, "include", "moe_w4a16.h")).read()
    kinds = {int(v): n for n, v in re.findall(r"#define MOE_KERNEL_(\w+) (\d+)", src)}
    assert sorted(kinds) == sorted(M.KERNEL_KINDS)


def test_serial_flag_limits():
    for over in ({"T": 2}, {"flags": M.FLAG_SERIAL | M.FLAG_FORCE_BATCHED}):
        c = cfg(**{"flags": M.FLAG_SERIAL, **over})
        with pytest.raises(M.MoeError) as e:
            call(c)
        assert e.value.code == M.ERR_INVALID_ARG


def test_router_zero_tokens_and_bad_shape():
    cfg = M.make_cfg(0)
    M.moe_w4a16_route(0, 0, None, 0, 0, cfg)
    c2 = M.make_cfg(1, num_experts=300, top_k=4)
    c2.workspace, c2.workspace_bytes = FAKE, 1 << 30
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_route(FAKE, FAKE, None, FAKE, FAKE, c2)
    assert e.value.code == M.ERR_UNSUPPORTED_SHAPE
    c3 = M.make_cfg(1, top_k=4)
    c3.workspace, c3.workspace_bytes = FAKE, 16
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_route(FAKE, FAKE, None, FAKE, FAKE, c3)
    assert e.value.code == M.ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("args,code", [
    ((1000, 512, 1 << 20, 1, FAKE, 64, 4), M.ERR_INVALID_ARG),        # triplet not a multiple of 256
    ((4096, 4096, 1 << 20, 1, FAKE, 64, 4), M.ERR_INVALID_ARG),       # nibbles fill the triplet
    ((4096, 2048, 1 << 20, 0, FAKE, 64, 4), M.ERR_INVALID_ARG),       # no staging slot
    ((4096, 2048, 1 << 20, 4, 0, 64, 4), M.ERR_INVALID_ARG),          # no staging buffer
    ((4096, 2048, 1 << 20, 4, FAKE + 16, 64, 4), M.ERR_MISALIGNED),
    ((4096, 2048, 3 * 4096, 4, FAKE, 64, 4), M.ERR_INVALID_ARG),     # cache smaller than the staging
    ((4096, 2048, 1 << 20, 4, FAKE, 2000, 4), M.ERR_INVALID_ARG),     # too many experts
])
def test_hybrid_create_argument_errors(args, code):
    """Checked on the host before anything is allocated."""
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_hybrid_create(*args)
    assert e.value.code == code


def test_hybrid_null_handle_errors():
    with pytest.raises(M.MoeError):
        M.moe_w4a16_hybrid_stats(None)
    with pytest.raises(M.MoeError):
        M.moe_w4a16_hybrid_last_requests(None)
    M.moe_w4a16_hybrid_destroy(None)


def test_floor_helpers_reject_bad_arguments():
    """The decode floor mirrors only T = 1 at the 2048/1536/top-4 E8M0 shape;
    the empty launch and the burst read check their own arguments."""
    for over in ({"T": 2}, {"hidden": 1024, "inter": 768}, {"top_k": 2},
                 {"scale_fmt": M.SCALE_E4M3_G16, "tensor_scales": FAKE}):
        with pytest.raises(M.MoeError) as e:
            M.moe_w4a16_decode_floor(38, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + (1 << 30), cfg(**over))
        assert e.value.code in (M.ERR_UNSUPPORTED_SHAPE, M.ERR_INVALID_ARG), over
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_decode_floor(0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + (1 << 30), cfg())
    assert e.value.code == M.ERR_INVALID_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_empty_launch(1, 2048, FAKE)
    assert e.value.code == M.ERR_INVALID_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_read_burst(FAKE, 4096, 3, FAKE)
    assert e.value.code == M.ERR_INVALID_ARG
    with pytest.raises(M.MoeError) as e:
        M.moe_w4a16_read_burst(FAKE + 8, 4096, 4, FAKE)
    assert e.value.code == M.ERR_MISALIGNED
    for args in ((0, 10, FAKE), (8, -1, FAKE), (8, 200000, FAKE), (8, 10, 0), (8, 10, FAKE + 2)):
        with pytest.raises(M.MoeError) as e:
            M.moe_w4a16_grid_barrier(*args)
        assert e.value.code == M.ERR_INVALID_ARG, args


def test_workspace_control_words_do_not_move_with_cfg():
    """The router's counters live in the control region at the start of every
    workspace, so workspace sizes grow by the same fixed control region for
    every cfg and a T = 1 workspace is never smaller than that region."""
    b1 = M.moe_w4a16_workspace_bytes(cfg(T=1))
    assert b1 >= 256 + 4 * 2048
