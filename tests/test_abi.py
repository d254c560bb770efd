"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/moe_decode.h declares, and its configuration checks
and workspace sizing behave as documented."""
import ctypes
import os
import re

import pytest

from sparse_moe_decode_router_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_decode_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(binding.EXPORTED) == declared_functions()


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_refuses_to_run_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(binding.MoEError):
        binding.lib()


def cfg(**kw):
    base = dict(hidden=7168, latent=2048, n_experts=896, expert_inter=2048, shared_inter=4096,
                max_batch=64, max_top_k=16, router_dtype=0)
    base.update(kw)
    return binding.Config(**base)


def validate(c):
    return binding.lib().moe_decode_validate_config(ctypes.byref(c))


@pytest.mark.parametrize("kw,want", [
    ({}, binding.MOE_OK),
    (dict(hidden=512, latent=256, n_experts=64, expert_inter=256, shared_inter=512,
          max_batch=1, max_top_k=4, router_dtype=1), binding.MOE_OK),
    (dict(expert_inter=256, shared_inter=512), binding.MOE_OK),
    (dict(max_batch=0), binding.MOE_ERR_INVALID_ARG),
    (dict(max_batch=65), binding.MOE_ERR_UNSUPPORTED),
    (dict(max_top_k=0), binding.MOE_ERR_INVALID_ARG),
    (dict(max_top_k=65, n_experts=128), binding.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=8, max_top_k=16), binding.MOE_ERR_INVALID_ARG),
    (dict(hidden=7200), binding.MOE_ERR_UNSUPPORTED),
    (dict(latent=2080), binding.MOE_ERR_UNSUPPORTED),
    (dict(expert_inter=2000), binding.MOE_ERR_UNSUPPORTED),
    (dict(shared_inter=100), binding.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=900), binding.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=1056), binding.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=1024), binding.MOE_OK),
    (dict(router_dtype=2), binding.MOE_ERR_INVALID_ARG),
    (dict(hidden=-128), binding.MOE_ERR_INVALID_ARG),
])
def test_validate_config(kw, want):
    assert validate(cfg(**kw)) == want


def test_validate_null_config():
    assert binding.lib().moe_decode_validate_config(None) == binding.MOE_ERR_INVALID_ARG


def test_workspace_size():
    lib = binding.lib()
    k3 = cfg()
    n = lib.moe_decode_workspace_size(ctypes.byref(k3))
    assert n > 0 and n % 256 == 0
    # a smaller batch capacity needs no more memory
    assert lib.moe_decode_workspace_size(ctypes.byref(cfg(max_batch=1))) <= n
    assert lib.moe_decode_workspace_size(ctypes.byref(cfg(hidden=7200))) == 0
    # the workspace is far below the layer's weights (6.2 GB)
    assert n < 512 << 20


def test_init_rejects_bad_arguments_before_touching_the_device():
    lib = binding.lib()
    c = cfg()
    h = ctypes.c_void_p()
    w = binding.Weights()
    assert lib.moe_decode_init(ctypes.byref(c), ctypes.byref(w), None, 0, ctypes.byref(h)) == \
        binding.MOE_ERR_INVALID_ARG       # null weight pointers
    assert lib.moe_decode_init(ctypes.byref(c), None, None, 0, ctypes.byref(h)) == \
        binding.MOE_ERR_INVALID_ARG
    assert lib.moe_decode_init(ctypes.byref(c), ctypes.byref(w), None, 0, None) == \
        binding.MOE_ERR_INVALID_ARG
    fake = binding.Weights(*([0x1000] * 10))
    assert lib.moe_decode_init(ctypes.byref(c), ctypes.byref(fake), None, 0,
                               ctypes.byref(h)) == binding.MOE_ERR_WORKSPACE
    odd = binding.Weights(*([0x1008] * 10))   # not 16-byte aligned
    assert lib.moe_decode_init(ctypes.byref(c), ctypes.byref(odd), 0x100000, 1 << 40,
                               ctypes.byref(h)) == binding.MOE_ERR_INVALID_ARG
    bad = cfg(hidden=7200)
    assert lib.moe_decode_init(ctypes.byref(bad), ctypes.byref(fake), 0x100000, 1 << 40,
                               ctypes.byref(h)) == binding.MOE_ERR_UNSUPPORTED


def test_step_and_graph_reject_null_context():
    lib = binding.lib()
    assert lib.moe_decode_step(None, 0x1000, 1, 1, 0x1000, None, None, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert lib.moe_decode_destroy(None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_decode_graph_launch(None, None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_decode_graph_destroy(None) == binding.MOE_ERR_INVALID_ARG
    info = binding.DispatchInfo()
    assert lib.moe_decode_last_dispatch(None, ctypes.byref(info)) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_decode_status_string(-4).decode().startswith("workspace")


def test_workload_configs_are_supported():
    for name in ("tiny", "k3", "k3_zipf", "k3_flat", "k3_tp8"):
        d = synth.RECIPES[name].dims
        assert binding.validate(d, 64 if name != "tiny" else 1, d.top_k) == binding.MOE_OK
