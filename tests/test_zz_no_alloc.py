"""The step that allocates nothing (moe_decode_step_static, for callers that
cannot allocate device memory), through the C ABI: two calls in a row, the
second with a smaller batch, each against the step of an ordinary context on
its own workspace (same kernels: identical expert ids and weights, outputs
equal up to the order of the latent combine's atomic adds) and against the
oracle; a configuration whose workspace exceeds the static array is refused."""
import ctypes
import sys

import numpy as np
import pytest

from gpu_util import check_step, run, to_dev_tokens
from sparse_moe_decode_router_amd import binding, synth

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield


def same_step(a, b):
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])
    fa = (a[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fb = (b[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rms = np.sqrt(np.mean(fa * fa, axis=1, keepdims=True))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(fa), np.abs(fb)) + 1e-300)) - 7)
    assert np.all(np.abs(fa - fb) <= np.maximum(ulp, rms * 2.0 ** -16))


@pytest.mark.parametrize("recipe,max_batch,calls", [
    ("small", 16, [(16, 6), (5, 6)]),
    ("k3_tp8", 64, [(64, 16), (3, 16)]),
])
def test_static_step_matches_context_step(recipe, max_batch, calls):
    import torch
    if recipe == "small":
        dims = synth.LayerDims(hidden=1024, latent=512, n_experts=96, expert_inter=384,
                               shared_inter=384, top_k=6, router_f32=False)
        rec = synth.LayerRecipe(dims=dims, router_std=0.05, dense_std=0.05, scale_exp_lo=-7,
                                scale_exp_hi=-3, bias="normal:0.1")
        layer = synth.make_layer(rec, 3)
    else:
        layer = synth.make_layer(synth.K3_TP8, synth.TP8_STACK_SEED0 + 5)
    dev = binding.DeviceLayer(layer)
    max_k = max(k for _, k in calls)
    ctx = binding.MoEDecode(dev, max_batch, max_k)
    for i, (B, k) in enumerate(calls):
        log(f"static step {recipe}: call {i}, B={B} k={k}")
        x = synth.make_tokens(layer.dims, 50 + i, B)
        out, idx, w = binding.step_static(dev, max_batch, max_k, to_dev_tokens(x), k)
        torch.cuda.synchronize()
        got = (out.cpu().numpy().view(np.uint16), idx.cpu().numpy(), w.cpu().numpy())
        want = run(ctx, x, k)
        same_step(got, want)
        r = check_step(layer, x, k, *got)
        log("  ", r)


def test_static_step_refuses_a_workspace_beyond_the_array():
    dims = synth.LayerDims(hidden=8192, latent=4096, n_experts=1024, expert_inter=8192,
                           shared_inter=4096, top_k=64, router_f32=False)
    assert binding.workspace_size(dims, 64, 64) > binding.STATIC_WORKSPACE_BYTES
    cfg = binding.make_config(dims, 64, 64)
    wts = binding.Weights(*([16] * 10))  # never dereferenced: refused before any launch
    rc = binding.lib().moe_decode_step_static(ctypes.byref(cfg), ctypes.byref(wts), 16, 1, 1,
                                              16, None, None, None)
    assert rc == binding.MOE_ERR_WORKSPACE
