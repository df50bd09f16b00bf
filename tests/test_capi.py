"""Host-only checks of the C ABI (no GPU needed): every symbol moe.h declares
is exported by libmoe.so, and invalid arguments are rejected on the host with
the documented status before anything is enqueued."""
import ctypes
import os
import re

import pytest

import routing_expert_ffn_sigmoid_amd as moe
from routing_expert_ffn_sigmoid_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

needs_lib = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH),
                               reason="libmoe.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_load_stats",
              "moe_layer_forward", "moe_workspace_size", "moe_status_string"]:
        assert n in names
    assert set(names) == set(moe.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(moe.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), f"libmoe.so does not export {n}"


@needs_lib
def test_status_strings():
    for code in range(6):
        assert moe.status_string(code).startswith("MOE_")


def _ws_size(cfg):
    n = ctypes.c_size_t(0)
    return moe.lib().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), n.value


@needs_lib
@pytest.mark.parametrize("name", list(workloads.SHORT))
def test_workspace_size_for_presets(name):
    cfg = moe.make_cfg(workloads.get(name))
    rc, n = _ws_size(cfg)
    assert rc == moe.MOE_OK and n > 0


@needs_lib
@pytest.mark.parametrize("override,code", [
    ({"N": 0}, moe.MOE_ERR_INVALID_ARG),
    ({"T": -1}, moe.MOE_ERR_INVALID_ARG),
    ({"n_groups": 3}, moe.MOE_ERR_INVALID_ARG),          # 3 does not divide 16
    ({"topk_groups": 5}, moe.MOE_ERR_INVALID_ARG),
    ({"k": 9}, moe.MOE_ERR_INVALID_ARG),                  # > 2 kept groups x 4 experts
    ({"group_topn": 3}, moe.MOE_ERR_INVALID_ARG),
    ({"score_fn": 7}, moe.MOE_ERR_INVALID_ARG),
    ({"capacity": -1}, moe.MOE_ERR_INVALID_ARG),
    ({"act_dtype": 5}, moe.MOE_ERR_INVALID_ARG),
    ({"N": 260, "n_groups": 4}, moe.MOE_ERR_UNSUPPORTED),
    ({"N": 18, "n_groups": 1, "topk_groups": 1}, moe.MOE_ERR_UNSUPPORTED),
    ({"H": 100}, moe.MOE_ERR_UNSUPPORTED),
    ({"I": 96}, moe.MOE_ERR_UNSUPPORTED),
    ({"N": 16, "n_groups": 8, "topk_groups": 2}, moe.MOE_ERR_UNSUPPORTED),  # groups of 2
    ({"w_dtype": 1}, moe.MOE_ERR_UNSUPPORTED),
    ({"group_capacity": -2}, moe.MOE_ERR_INVALID_ARG),
    ({"w_layout": 5}, moe.MOE_ERR_INVALID_ARG),
    ({"w_layout": 1}, moe.MOE_ERR_UNSUPPORTED),           # fp32 weights are read row-major
    ({"group_capacity": -1, "capacity": 4}, moe.MOE_ERR_INVALID_ARG),  # one policy at a time
    ({"T": 1 << 24, "capacity": 4}, moe.MOE_ERR_UNSUPPORTED),  # 24-bit token field of the keys
    ({"T": 1 << 24, "group_capacity": -1}, moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_configs_rejected_on_host(override, code):
    cfg = moe.make_cfg(workloads.TINY, **override)
    rc, _ = _ws_size(cfg)
    assert rc == code
    # the layer entry point rejects the same configuration before any launch
    w = moe.MoeWeights()
    rc2 = moe.lib().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), None, None, None,
                                      None, None, 0, None)
    assert rc2 == code


@needs_lib
def test_missing_workspace_and_pointers_rejected():
    cfg = moe.make_cfg(workloads.TINY)
    w = moe.MoeWeights()
    L = moe.lib()
    # NULL x / out with T > 0
    assert L.moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), None, None, None, None,
                               None, 0, None) == moe.MOE_ERR_INVALID_ARG
    # all pointers present (never dereferenced), workspace too small
    fake = ctypes.c_void_p(0x1000)
    w = moe.MoeWeights(fake, fake, fake, fake, fake)
    assert L.moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), fake, None, fake, None,
                               fake, 16, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_load_stats(ctypes.byref(cfg), fake, fake, fake, fake, fake, fake, None, 0,
                            None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_permute(ctypes.byref(cfg), fake, fake, None, fake, fake, fake, fake, None,
                         None, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_grouped_ffn(ctypes.byref(cfg), 0, None, 4, 64, fake, None, fake, fake, fake,
                             fake, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    # the router GEMM needs workspace: K-split partials, and with bf16
    # activations the bf16 pieces of the router weight even when K is not
    # split (6 k-steps of 32 below); checked before any launch
    for c in (cfg, moe.make_cfg(workloads.V1, T=300, H=192)):
        assert L.moe_route(ctypes.byref(c), fake, fake, fake, None, fake, fake, fake, None,
                           fake, 16, None) == moe.MOE_ERR_WORKSPACE
        rc, need = _ws_size(c)
        assert rc == moe.MOE_OK and need > 16
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(cfg), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_size(None, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(moe, "_LIB", None)
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()


@needs_lib
def test_bf16_weights_must_be_tiled():
    cfg = moe.make_cfg(workloads.V1)
    assert cfg.w_layout == moe.MOE_LAYOUT_TILED
    assert _ws_size(cfg)[0] == moe.MOE_OK
    cfg.w_layout = moe.MOE_LAYOUT_ROWS
    assert _ws_size(cfg)[0] == moe.MOE_ERR_UNSUPPORTED


@needs_lib
def test_pack_weights_argument_checks():
    L = moe.lib()
    fake = ctypes.c_void_p(0x10000)
    other = ctypes.c_void_p(0x10000 + 3 * 32 * 64 * 2)
    assert L.moe_pack_weights(3, 32, 64, moe.MOE_F32, fake, other, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_weights(3, 24, 64, moe.MOE_BF16, fake, other, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_weights(3, 32, 48, moe.MOE_BF16, fake, other, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_weights(-1, 32, 64, moe.MOE_BF16, fake, other, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(3, 32, 64, moe.MOE_BF16, None, other, None) == moe.MOE_ERR_INVALID_ARG
    # overlapping source and destination
    near = ctypes.c_void_p(0x10000 + 1024)
    assert L.moe_pack_weights(3, 32, 64, moe.MOE_BF16, fake, near, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(3, 32, 64, moe.MOE_BF16, fake, fake, None) == moe.MOE_ERR_INVALID_ARG
    # nothing to do
    assert L.moe_pack_weights(0, 32, 64, moe.MOE_BF16, None, None, None) == moe.MOE_OK


@needs_lib
def test_noalloc_forward_rejects_on_the_host():
    """moe_layer_forward_noalloc checks its arguments and the fixed scratch
    limit before it touches a device: invalid configurations and missing
    pointers as moe_layer_forward, MOE_ERR_TOO_LARGE beyond the scratch."""
    L = moe.lib()
    w = moe.MoeWeights()
    for override, code in (({"N": 0}, moe.MOE_ERR_INVALID_ARG), ({"H": 100}, moe.MOE_ERR_UNSUPPORTED)):
        cfg = moe.make_cfg(workloads.TINY, **override)
        assert L.moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), None, None, None,
                                           None, None) == code
    cfg = moe.make_cfg(workloads.TINY)
    assert L.moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), None, None, None,
                                       None, None) == moe.MOE_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)
    wf = moe.MoeWeights(fake, fake, fake, fake, fake)
    for wl in (workloads.V3_PREFILL, workloads.V3_DECODE.with_(T=512), workloads.V1):
        c = moe.make_cfg(wl)
        assert _ws_size(c)[1] > moe.NOALLOC_SCRATCH_BYTES
        assert L.moe_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(wf), fake, None, fake,
                                           None, None) == moe.MOE_ERR_TOO_LARGE
    # the decode-sized V3 layer fits
    assert _ws_size(moe.make_cfg(workloads.V3_DECODE))[1] <= moe.NOALLOC_SCRATCH_BYTES
