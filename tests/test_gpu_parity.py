"""GPU parity of the HIP decode step against the CPU oracle (through the C ABI).

Sizes: small layers that the oracle finishes in seconds but that still span
several MFMA tiles, K splits, column groups and ragged tails; then the K3-scale
layer (896 experts, top-16, hidden 7168) at batch 1, 8 and 64 and one
tensor-parallel rank's share, in the launch configuration the benchmark times,
with the oracle evaluating sampled tokens end to end and every token's expert
selection.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
from sparse_moe_decode_router_amd import binding, synth

from gpu_util import (TAU, bf16_f64, check_step, oracle_keys, rel_l2, run, to_dev_tokens,
                      with_k)

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


def small_recipe(H=256, L=256, E=64, I=256, Is=256, k=4, bias="normal:0.1", router_f32=False,
                 std=0.05):
    dims = synth.LayerDims(hidden=H, latent=L, n_experts=E, expert_inter=I, shared_inter=Is,
                           top_k=k, router_f32=router_f32)
    return synth.LayerRecipe(dims=dims, router_std=std, dense_std=std, scale_exp_lo=-7,
                             scale_exp_hi=-3, bias=bias)


def make_ctx(layer, max_batch, max_top_k=None):
    dl = binding.DeviceLayer(layer)
    return binding.MoEDecode(dl, max_batch, max_top_k or layer.dims.top_k)


# ---------------------------------------------------------------------------
# Number format and routing primitives
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lo,hi", [(100, 150), (8, 247)])
def test_dequant_matches_oracle_decode(lo, hi):
    import torch
    rng = np.random.default_rng(lo)
    n = 32 * 4096
    q = rng.integers(0, 256, n // 2, dtype=np.uint8)
    s = rng.integers(lo, hi + 1, n // 32, dtype=np.uint8)
    got = binding.dequant(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    want = np.array([oracle.mxfp4_element(q, s, j) for j in range(0, n, 97)])
    np.testing.assert_array_equal(got[::97], want)
    # every byte value (every pair of codes) with unit scale: the E2M1 table
    q1 = np.arange(256, dtype=np.uint8)
    s1 = np.full(512 // 32, 127, np.uint8)
    got1 = binding.dequant(torch.from_numpy(q1).cuda(), torch.from_numpy(s1).cuda()).cpu()
    want1 = [oracle.mxfp4_element(q1, s1, j) for j in range(512)]
    np.testing.assert_array_equal(got1.numpy().astype(np.float64), want1)


# ---------------------------------------------------------------------------
# Small layers: many tiles, splits, column groups and ragged tails
# ---------------------------------------------------------------------------

def test_tiny_layer_batch1():
    layer = synth.make_layer(synth.TINY, 0)
    ctx = make_ctx(layer, 1)
    x = synth.make_tokens(layer.dims, 0, 1)
    out, idx, w = run(ctx, x, 4)
    r = check_step(layer, x, 4, out, idx, w)
    log("tiny B=1", r)
    assert ctx.last_dispatch()["router_f32"] == 1


SMALL = small_recipe(H=1024, L=512, E=96, I=384, Is=384, k=6)


@pytest.fixture(scope="module")
def small_layer():
    return synth.make_layer(SMALL, 3)


@pytest.fixture(scope="module")
def small_ctx(small_layer):
    return make_ctx(small_layer, 64, 8)


@pytest.mark.parametrize("B", [1, 2, 3, 8, 9, 16, 17, 33, 64])
@pytest.mark.parametrize("k", [1, 6, 8])
def test_small_layer_batches(small_layer, small_ctx, B, k):
    log(f"small layer B={B} k={k}")
    x = synth.make_tokens(small_layer.dims, 100 + B, B)
    out, idx, w = run(small_ctx, x, k)
    assert small_ctx.last_dispatch()["out_staged"] == (1 if B <= 2 else 2 if B <= 8 else 0)
    if B * k <= 8:  # few gate/up units: waves share each tile
        assert small_ctx.last_dispatch()["split_w13"] >= 2
    r = check_step(small_layer, x, k, out, idx, w)
    if k == 1:
        assert np.all(w == 1.0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=k * 2.0 ** -23)
    log("  ", r)


@pytest.mark.parametrize("B", [1, 3, 8])
def test_small_layer_dense_routing(small_layer, B):
    """Up to 8 tokens with the routing at the end of the dense-in launch."""
    ctx = make_ctx(small_layer, 8, 8)
    ctx.set_mode(binding.MODE_DENSE_ROUTING)
    x = synth.make_tokens(small_layer.dims, 120 + B, B)
    out, idx, w = run(ctx, x, 8)
    assert ctx.last_dispatch()["routing"] == 0
    check_step(small_layer, x, 8, out, idx, w)


def test_small_layer_without_bias():
    layer = synth.make_layer(small_recipe(bias="none", k=4), 4)
    ctx = make_ctx(layer, 16)
    x = synth.make_tokens(layer.dims, 4, 16)
    out, idx, w = run(ctx, x, 4)
    check_step(layer, x, 4, out, idx, w)


def test_intermediates_match_oracle(small_layer, small_ctx):
    """Each stage against the oracle's binary64 intermediates (same selection)."""
    import torch
    B, k = 5, 6
    x = synth.make_tokens(small_layer.dims, 7, B)
    out, idx, w = run(small_ctx, x, k)
    dbg = {n: t.cpu().numpy() for n, t in small_ctx.debug_export(B, k).items()}
    torch.cuda.synchronize()
    ref = oracle.moe_step(with_k(small_layer, k), x, rounding="none", forced_idx=idx, want="all")
    np.testing.assert_allclose(dbg["score"], ref["score"], rtol=0, atol=2e-6)
    bias = small_layer.bias.astype(np.float64)
    np.testing.assert_allclose(dbg["key"], ref["score"] + bias, rtol=0, atol=3e-6)
    for name, tol in (("z", 2e-5), ("act", 5e-5), ("ylat", 5e-5), ("ash", 5e-5)):
        e = rel_l2(dbg[name], ref[name])
        log(f"  {name}: rel L2 {e:.2e}")
        assert e < tol, (name, e)
    assert dbg["n_active"][0] == len(np.unique(idx))


@pytest.mark.parametrize("B", [12, 33])
def test_f32_router_layer_several_tokens(B):
    """f32 router (its own launch first): routing units that load the keys
    from memory, beside the dense-in kernel of up to 16 tokens and beside the
    K-sliced one above 16."""
    log(f"f32 router B={B}")
    layer = synth.make_layer(small_recipe(router_f32=True, bias="none", k=4), 5)
    ctx = make_ctx(layer, B)
    x = synth.make_tokens(layer.dims, 5, B)
    out, idx, w = run(ctx, x, 4)
    check_step(layer, x, 4, out, idx, w)
    assert ctx.last_dispatch()["n_kernels"] == 5


# Routing forms of up to 8 tokens: the default (this small layer's dense-in
# launch is one round, so the gate/up launch routes, by threshold selection)
# and the routing at the end of the dense-in launch (selection by rounds).
ROUTING_FORMS = ["four_launches", "dense_routing"]


@pytest.mark.parametrize("form", ROUTING_FORMS)
def test_zero_router_picks_lowest_ids_with_equal_weights(form):
    layer = synth.make_layer(small_recipe(bias="none", k=5), 6)
    layer.router_w[:] = 0
    ctx = make_ctx(layer, 4)
    ctx.set_mode(mode_const(form))
    x = synth.make_tokens(layer.dims, 6, 4)
    out, idx, w = run(ctx, x, 5)
    np.testing.assert_array_equal(idx, np.tile(np.arange(5), (4, 1)))
    assert np.all(w == np.float32(0.2))
    check_step(layer, x, 5, out, idx, w)


@pytest.mark.parametrize("form", ROUTING_FORMS)
@pytest.mark.parametrize("B", [4, 12, 20])
@pytest.mark.parametrize("k,want", [(5, [3, 7, 69, 130, 200]),
                                    (8, [3, 7, 69, 130, 131, 192, 200, 250])])
def test_ties_at_the_threshold_go_to_the_lowest_ids(B, k, want, form):
    """Keys equal at the k-th largest value, spread over several lane slots
    (expert e sits in slot e // 64): the selection takes the lowest ids among
    them, also when the cut falls between two ids of one slot (130 taken,
    131 not).  Zero router: every score is 0.5, so the keys are exactly
    1.5, 0.75 or 0.5 and the weights 1/k.  B = 12 routes through the routing
    units, B = 20 through the ones that add the K-sliced router's partials
    (with more than 64 keys at the threshold: the rounds)."""
    layer = synth.make_layer(small_recipe(E=256, bias="none", k=k), 11)
    layer.router_w[:] = 0
    layer.bias = np.zeros(256, np.float32)
    layer.bias[[200, 3]] = 1.0
    layer.bias[[250, 7, 69, 130, 131, 192]] = 0.25
    ctx = make_ctx(layer, B, 8)
    ctx.set_mode(mode_const(form))
    x = synth.make_tokens(layer.dims, 11, B)
    out, idx, w = run(ctx, x, k)
    np.testing.assert_array_equal(idx, np.tile(np.array(want), (B, 1)))
    assert np.all(w == np.float32(1.0 / k))
    check_step(layer, x, k, out, idx, w)


def test_hot_experts_serve_every_token():
    """A bias that sends all 64 tokens to the same experts: more than 8
    tokens per expert, several column units per expert."""
    layer = synth.make_layer(small_recipe(bias="none", k=4), 8)
    layer.bias = np.zeros(layer.dims.n_experts, np.float32)
    layer.bias[[3, 17, 40]] = 5.0
    ctx = make_ctx(layer, 64)
    x = synth.make_tokens(layer.dims, 8, 64)
    out, idx, w = run(ctx, x, 4)
    assert np.all(np.isin([3, 17, 40], idx[0]))
    check_step(layer, x, 4, out, idx, w)


@pytest.mark.parametrize("form", ROUTING_FORMS)
@pytest.mark.parametrize("B", [3, 20])
def test_all_experts_selected(form, B):
    layer = synth.make_layer(small_recipe(E=32, k=32), 9)
    ctx = make_ctx(layer, B)
    ctx.set_mode(mode_const(form))
    x = synth.make_tokens(layer.dims, 9, B)
    out, idx, w = run(ctx, x, 32)
    np.testing.assert_array_equal(idx, np.tile(np.arange(32), (B, 1)))
    check_step(layer, x, 32, out, idx, w)


# Hidden 4096: four 128-element steps per wave, so the dense-in launch stages
# x in LDS (up to 8 tokens).
STAGED_MID = small_recipe(H=4096, L=512, E=96, I=384, Is=384, k=6)


@pytest.mark.parametrize("form", ["four_launches", "dense_routing"])
def test_staged_dense_in_up_to_8_tokens(form):
    """The dense-in launch with x staged in LDS: 2 rows up to 2 tokens, all 8
    rows (one workgroup per compute unit, this layer's 86 tiles fitting one
    round) from 3 to 8; every token's output against the oracle, with the
    routing after it (dense routing) or at the start of the gate/up launch."""
    layer = synth.make_layer(STAGED_MID, 21)
    ctx = make_ctx(layer, 8)
    ctx.set_mode(mode_const(form))
    for B in (1, 2, 3, 5, 8):
        log(f"staged dense-in, {form}, B={B}")
        x = synth.make_tokens(layer.dims, 30 + B, B)
        out, idx, w = run(ctx, x, 6)
        assert ctx.last_dispatch()["in_staged"] == (1 if B <= 2 else 3)
        check_step(layer, x, 6, out, idx, w)
    ctx.close()


def assert_same_step(a, b):
    """Two runs of one step: identical expert ids and weights; outputs equal
    up to the order of the f32 atomic adds of the expert combine.  A different
    order moves each latent value by a few f32 rounding steps (about
    k * 2^-24 relative); after the latent-up contraction that is far below
    2^-16 of the row's rms, plus the one bf16 step a value near a rounding
    boundary can take.  Outputs that cancel to almost zero can differ by more
    bf16 steps of their own, never by more than this absolute bound."""
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])
    fa, fb = bf16_f64(a[0]), bf16_f64(b[0])
    rms = np.sqrt(np.mean(fa * fa, axis=1, keepdims=True))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(fa), np.abs(fb)) + 1e-300)) - 7)
    assert np.all(np.abs(fa - fb) <= np.maximum(ulp, rms * 2.0 ** -16))
    assert np.mean(a[0] != b[0]) < 1e-2


def assert_modes_agree(a, b):
    """Two execution modes of one step.  The modes reduce in different
    orders: above 16 tokens the router's K slices (so scores can differ in
    their last f32 bits and a near tie may select another expert), and the
    output either as one sum over latent-up and shared-down or as two.  Two
    f32 reduction trees over K = 6144 terms of size up to the row's rms differ
    by far less than K 2^-24 rms (typically sqrt(K) 2^-24 rms); the bound is
    one bf16 step of the value or 2^-12 rms.  Tokens with the same experts
    must have weights within 2e-6 and outputs within that bound; at most 5 %
    of the tokens may differ in their experts."""
    same = np.all(a[1] == b[1], axis=1)
    assert np.mean(same) >= 0.95
    np.testing.assert_allclose(a[2][same], b[2][same], rtol=0, atol=2e-6)
    fa, fb = bf16_f64(a[0][same]), bf16_f64(b[0][same])
    rms = np.sqrt(np.mean(fa * fa, axis=1, keepdims=True))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(fa), np.abs(fb)) + 1e-300)) - 7)
    assert np.all(np.abs(fa - fb) <= np.maximum(ulp, rms * 2.0 ** -12))


def test_repeated_steps_agree(small_layer, small_ctx):
    x = synth.make_tokens(small_layer.dims, 11, 24)
    a = run(small_ctx, x, 6)
    for _ in range(3):
        assert_same_step(a, run(small_ctx, x, 6))


def test_graph_replays_match_eager_and_track_new_inputs(small_layer):
    """A captured two-layer graph gives the eager result; replays with a
    changed input (the same device buffer) give the new input's result, not
    a stale one; eager work runs between replays."""
    import torch
    ctxs = [make_ctx(small_layer, 8, 6) for _ in range(2)]
    B, k = 8, 6
    x1 = synth.make_tokens(small_layer.dims, 12, B)
    x2 = synth.make_tokens(small_layer.dims, 13, B)
    xd = [to_dev_tokens(x1), to_dev_tokens(x1)]
    outs = [torch.empty((B, small_layer.dims.hidden), dtype=torch.int16, device="cuda")
            for _ in range(2)]
    idxs = [torch.empty((B, k), dtype=torch.int32, device="cuda") for _ in range(2)]
    ws = [torch.empty((B, k), dtype=torch.float32, device="cuda") for _ in range(2)]
    g = binding.Graph(ctxs, xd, B, k, outs, idxs, ws)
    eager1 = run(ctxs[0], x1, k)
    eager2 = run(ctxs[0], x2, k)
    stream = torch.cuda.Stream()
    for rep in range(4):
        src = x1 if rep % 2 == 0 else x2
        want = eager1 if rep % 2 == 0 else eager2
        for t in xd:
            t.copy_(to_dev_tokens(src))
        torch.cuda.synchronize()
        g.launch(stream)
        stream.synchronize()
        for layer_i in range(2):
            got = (outs[layer_i].cpu().numpy().view(np.uint16), idxs[layer_i].cpu().numpy(),
                   ws[layer_i].cpu().numpy())
            assert_same_step(got, want)
        run(ctxs[1], x2, k)        # eager work between replays
    g.close()


def test_timing_events_time_each_kernel(small_layer, small_ctx):
    """Events attached to the dispatches: one positive duration per kernel,
    together no longer than the step; a wrong event count is refused."""
    import torch
    x = synth.make_tokens(small_layer.dims, 15, 4)
    run(small_ctx, x, 6)
    n = small_ctx.last_dispatch()["n_kernels"]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    small_ctx.set_timing_events(evs)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    run(small_ctx, x, 6)
    t1.record()
    torch.cuda.synchronize()
    small_ctx.set_timing_events(None)
    d = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n)]
    log("  kernel ms", d, "step ms", t0.elapsed_time(t1))
    assert all(v > 0 for v in d)
    assert sum(d) <= t0.elapsed_time(t1)
    with pytest.raises(binding.MoEError):
        small_ctx.set_timing_events(evs[:-1])


def test_dispatch_follows_the_batch(small_layer, small_ctx):
    for B, cg in ((1, 1), (16, 1), (17, 2), (64, 4)):
        x = synth.make_tokens(small_layer.dims, 14, B)
        run(small_ctx, x, 6)
        d = small_ctx.last_dispatch()
        assert d["batch"] == B and d["col_tiles"] == cg
        assert d["fused"] == 0 and d["n_kernels"] == 4
        assert d["grid_in"] >= 1 and d["grid_w13"] >= 1 and d["grid_step"] == 0
        # Up to two tokens the output launch stages its whole operand in LDS,
        # up to eight its latent part.
        assert d["out_staged"] == (1 if B <= 2 else 2 if B <= 8 else 0)
        # Above 16 tokens the dense-in launch splits K into slices; this
        # small layer's launch also fits one round at 16.
        assert d["in_staged"] == (2 if B >= 9 else 0 if B > 2 else d["in_staged"])
    try:
        for mode, fused, n in ((binding.MODE_FUSED, 1, 1), (binding.MODE_TWO_LAUNCHES, 2, 2),
                               (binding.MODE_SIDE_STREAM, 3, 6)):
            small_ctx.set_mode(mode)
            run(small_ctx, synth.make_tokens(small_layer.dims, 14, 5), 6)
            d = small_ctx.last_dispatch()
            assert d["fused"] == fused and d["n_kernels"] == n
            assert (d["grid_step"] >= 1) == (fused in (1, 2))  # persistent launches only
    finally:
        small_ctx.set_mode(binding.MODE_FOUR_LAUNCHES)


PERSISTENT_MODES = [("fused", 1), ("two_launches", 2), ("side_stream", 3)]


def mode_const(name):
    return {"fused": binding.MODE_FUSED, "two_launches": binding.MODE_TWO_LAUNCHES,
            "four_launches": binding.MODE_FOUR_LAUNCHES,
            "side_stream": binding.MODE_SIDE_STREAM,
            "late_routing": binding.MODE_LATE_ROUTING,
            "dense_routing": binding.MODE_DENSE_ROUTING,
            "ordered": binding.MODE_ORDERED}[name]


@pytest.mark.parametrize("B,k", [(1, 1), (1, 6), (2, 8), (3, 6), (8, 8), (8, 1), (9, 6), (16, 8)])
def test_late_routing_matches_four_launches(small_layer, B, k):
    """The routing at the start of the gate/up launch (up to 8 tokens and 128
    pairs; larger batches route in the dense-in launch as before) selects the
    same experts with the same weights; outputs agree up to the order of the
    latent combine; both against the oracle."""
    late = make_ctx(small_layer, 64, 8)
    late.set_mode(binding.MODE_LATE_ROUTING)
    four = make_ctx(small_layer, 64, 8)
    four.set_mode(binding.MODE_DENSE_ROUTING)
    auto = make_ctx(small_layer, 64, 8)  # default: this layer's dense-in launch is one round
    x = synth.make_tokens(small_layer.dims, 500 + B, B)
    a = run(late, x, k)
    b = run(four, x, k)
    c = run(auto, x, k)
    assert late.last_dispatch()["routing"] == (2 if B <= 8 else 1)
    assert four.last_dispatch()["routing"] == (0 if B <= 8 else 1)
    assert auto.last_dispatch()["routing"] == (2 if B <= 8 else 1)
    assert_same_step(a, c)
    assert_same_step(a, b)
    check_step(small_layer, x, k, *a)


def assert_bits_equal(a, b):
    for u, v in zip(a, b):
        np.testing.assert_array_equal(np.asarray(u), np.asarray(v))


@pytest.mark.parametrize("B,k", [(1, 1), (1, 8), (3, 6), (8, 8), (24, 6), (64, 8)])
def test_ordered_combine_is_bit_reproducible(small_layer, B, k):
    """MOE_MODE_ORDERED: repeated steps, on one context and on a fresh one,
    give the same bits; the four-launch step's experts and weights, outputs
    up to the order of the latent combine; every token against the oracle."""
    ordered = make_ctx(small_layer, 64, 8)
    ordered.set_mode(binding.MODE_ORDERED)
    x = synth.make_tokens(small_layer.dims, 900 + B, B)
    a = run(ordered, x, k)
    for _ in range(3):
        assert_bits_equal(a, run(ordered, x, k))
    assert ordered.last_dispatch()["ordered"] == 1
    fresh = make_ctx(small_layer, 64, 8)
    fresh.set_mode(binding.MODE_ORDERED)
    assert_bits_equal(a, run(fresh, x, k))
    four = make_ctx(small_layer, 64, 8)
    b = run(four, x, k)
    assert four.last_dispatch()["ordered"] == 0
    assert_same_step(a, b)
    check_step(small_layer, x, k, *a)


def test_ordered_combine_graph_replays_equal_eager_bits(small_layer):
    """A captured two-layer graph of the ordered form replays the eager
    step's bits, with eager steps of other batches between the replays."""
    import torch
    B, k = 8, 6
    ctxs = [make_ctx(small_layer, 16, 6) for _ in range(2)]
    for c in ctxs:
        c.set_mode(binding.MODE_ORDERED)
    x = synth.make_tokens(small_layer.dims, 14, B)
    xd = [to_dev_tokens(x), to_dev_tokens(x)]
    outs = [torch.empty((B, small_layer.dims.hidden), dtype=torch.int16, device="cuda")
            for _ in range(2)]
    idxs = [torch.empty((B, k), dtype=torch.int32, device="cuda") for _ in range(2)]
    ws = [torch.empty((B, k), dtype=torch.float32, device="cuda") for _ in range(2)]
    want = run(ctxs[0], x, k)
    g = binding.Graph(ctxs, xd, B, k, outs, idxs, ws)
    stream = torch.cuda.Stream()
    for rep in range(3):
        g.launch(stream)
        stream.synchronize()
        for li in range(2):
            assert_bits_equal((outs[li].cpu().numpy().view(np.uint16), idxs[li].cpu().numpy(),
                               ws[li].cpu().numpy()), want)
        run(ctxs[1], synth.make_tokens(small_layer.dims, 15 + rep, 3), k)
    g.close()


def test_late_routing_repeated_steps_and_graph(small_layer):
    """Steps of several batches in a row on one context, eager and replayed
    from a graph: the gate/up launch's own routing leaves nothing stale."""
    import torch
    ctx = make_ctx(small_layer, 8, 8)
    ctx.set_mode(binding.MODE_LATE_ROUTING)
    for i, B in enumerate((8, 1, 5, 8, 2)):
        x = synth.make_tokens(small_layer.dims, 600 + i, B)
        check_step(small_layer, x, 6, *run(ctx, x, 6))
    B, k = 4, 6
    x = synth.make_tokens(small_layer.dims, 610, B)
    xd = [to_dev_tokens(x)]
    outs = [torch.empty((B, small_layer.dims.hidden), dtype=torch.int16, device="cuda")]
    idxs = [torch.empty((B, k), dtype=torch.int32, device="cuda")]
    ws = [torch.empty((B, k), dtype=torch.float32, device="cuda")]
    g = binding.Graph([ctx], xd, B, k, outs, idxs, ws)
    want = run(ctx, x, k)
    stream = torch.cuda.Stream()
    for _ in range(3):
        g.launch(stream)
        stream.synchronize()
        got = (outs[0].cpu().numpy().view(np.uint16), idxs[0].cpu().numpy(), ws[0].cpu().numpy())
        assert_same_step(got, want)
        run(ctx, synth.make_tokens(small_layer.dims, 611, 7), 6)   # eager work between replays
    g.close()


@pytest.mark.parametrize("mode,kind", PERSISTENT_MODES)
@pytest.mark.parametrize("B", [1, 9, 33, 64])
def test_four_launch_step_matches_persistent(small_layer, B, mode, kind):
    """The four-launch step and the persistent-kernel steps compute the same
    values (up to the order of the latent combine's atomic adds); both against
    the oracle."""
    k = 6
    fused = make_ctx(small_layer, 64, 8)
    fused.set_mode(mode_const(mode))
    four = make_ctx(small_layer, 64, 8)
    x = synth.make_tokens(small_layer.dims, 200 + B, B)
    a = run(fused, x, k)
    b = run(four, x, k)
    assert fused.last_dispatch()["fused"] == kind and four.last_dispatch()["fused"] == 0
    assert_modes_agree(a, b)
    check_step(small_layer, x, k, *a)


@pytest.mark.parametrize("mode,kind", PERSISTENT_MODES)
def test_persistent_step_other_shapes(mode, kind):
    """Persistent kernels of other chunk shapes: K3 latent with a short down
    row (16, 2) is covered by the TP8 tests; here the (2, 2) shape of a small
    layer, several steps in a row on one context."""
    layer = synth.make_layer(small_recipe(k=4), 21)
    ctx = make_ctx(layer, 16)
    ctx.set_mode(mode_const(mode))
    for B in (1, 7, 16):
        x = synth.make_tokens(layer.dims, 21 + B, B)
        out, idx, w = run(ctx, x, 4)
        assert ctx.last_dispatch()["fused"] == kind
        check_step(layer, x, 4, out, idx, w)


def test_contexts_of_different_shapes_share_a_workspace(small_layer):
    """Two contexts of different configurations (experts, top-k, maximum
    batch) on one workspace, stepped alternately in the four-launch, two-launch
    and one-launch forms: every step matches the oracle.  The counters that a
    step returns to zero sit at the same offsets for both configurations."""
    import torch
    other = synth.make_layer(small_recipe(H=512, L=256, E=64, I=256, Is=256, k=4), 17)
    da, db = binding.DeviceLayer(small_layer), binding.DeviceLayer(other)
    size = max(binding.workspace_size(small_layer.dims, 64, 8),
               binding.workspace_size(other.dims, 8, 4))
    ws = torch.empty(size, dtype=torch.uint8, device="cuda")
    a = binding.MoEDecode(da, 64, 8, workspace=ws)
    b = binding.MoEDecode(db, 8, 4, workspace=ws)
    steps = [(a, small_layer, 33, 8, "fused"), (b, other, 8, 4, "four_launches"),
             (a, small_layer, 64, 6, "two_launches"), (b, other, 3, 4, "fused"),
             (a, small_layer, 9, 8, "four_launches"), (b, other, 1, 2, "two_launches"),
             (a, small_layer, 17, 6, "fused"), (b, other, 8, 4, "fused"),
             (a, small_layer, 64, 8, "four_launches")]
    for i, (ctx, layer, B, k, mode) in enumerate(steps):
        log(f"  shared workspace step {i}: B={B} k={k} {mode}")
        ctx.set_mode(mode_const(mode))
        x = synth.make_tokens(layer.dims, 300 + i, B)
        out, idx, w = run(ctx, x, k)
        check_step(layer, x, k, out, idx, w)


# ---------------------------------------------------------------------------
# K3-scale layer (configuration of the benchmark)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def k3_layer():
    log("generating the K3-scale layer")
    return synth.make_layer(synth.K3, 0)


@pytest.fixture(scope="module")
def k3_dev(k3_layer):
    return binding.DeviceLayer(k3_layer)


def k3_ctx(k3_dev, bias_kind, max_batch):
    dl = k3_dev
    if bias_kind != "normal":
        recipe = {"zipf": synth.K3_ZIPF, "flat": synth.K3_FLAT}[bias_kind]
        dl = k3_dev.with_bias(synth.make_bias(recipe, 0))
    return binding.MoEDecode(dl, max_batch, 16), dl


def layer_with_bias(layer, bias_kind):
    if bias_kind == "normal":
        return layer
    recipe = {"zipf": synth.K3_ZIPF, "flat": synth.K3_FLAT}[bias_kind]
    return dataclasses.replace(layer, bias=synth.make_bias(recipe, 0))


@pytest.mark.parametrize("bias_kind,B", [("normal", 1), ("zipf", 8), ("flat", 64), ("normal", 64)])
def test_k3_layer(k3_layer, k3_dev, bias_kind, B):
    log(f"K3 layer, {bias_kind} bias, B={B}")
    ctx, _ = k3_ctx(k3_dev, bias_kind, 64)
    layer = layer_with_bias(k3_layer, bias_kind)
    x = synth.make_tokens(layer.dims, 0, B)
    out, idx, w = run(ctx, x, 16)
    # Batch 1 leaves the down kernel short of units: two waves per tile; the
    # output launch stages its operands in LDS.
    assert ctx.last_dispatch()["split_w2"] == (2 if B == 1 else 1)
    assert ctx.last_dispatch()["out_staged"] == (1 if B == 1 else 2 if B == 8 else 0)
    # x staged in LDS at batch 1; at batch 8 the 1.4-round launch reads it
    # through the caches; K slices at 64.
    assert ctx.last_dispatch()["in_staged"] == {1: 1, 8: 0, 64: 2}[B]
    r = check_step(layer, x, 16, out, idx, w)
    log("  ", r, "distinct experts", len(np.unique(idx)))


@pytest.mark.parametrize("mode,kind", PERSISTENT_MODES)
@pytest.mark.parametrize("bias_kind,B", [("normal", 1), ("zipf", 8), ("normal", 64)])
def test_k3_persistent_step_matches_four_launches(k3_layer, k3_dev, bias_kind, B, mode, kind):
    """The persistent-kernel steps on the K3 layer (chunk shape 16x16) give
    the four-launch step's values."""
    four, _ = k3_ctx(k3_dev, bias_kind, 64)
    fused, _ = k3_ctx(k3_dev, bias_kind, 64)
    fused.set_mode(mode_const(mode))
    x = synth.make_tokens(k3_dev.dims, 5, B)
    a = run(four, x, 16)
    b = run(fused, x, 16)
    assert fused.last_dispatch()["fused"] == kind and four.last_dispatch()["fused"] == 0
    assert_modes_agree(a, b)
    r = check_step(layer_with_bias(k3_layer, bias_kind), x, 16, *b)
    log(f"  K3 {mode} {bias_kind} B={B}:", r)


@pytest.mark.parametrize("bias_kind,B", [("normal", 1), ("flat", 64)])
def test_k3_ordered_combine(k3_layer, k3_dev, bias_kind, B):
    """The ordered latent combine on the K3 layer (batch 1: two waves per
    down tile, their sums added in LDS first): two runs give the same bits,
    the four-launch step's experts and weights, every token against the
    oracle."""
    four, _ = k3_ctx(k3_dev, bias_kind, 64)
    ordered, _ = k3_ctx(k3_dev, bias_kind, 64)
    ordered.set_mode(binding.MODE_ORDERED)
    x = synth.make_tokens(k3_dev.dims, 17, B)
    a = run(ordered, x, 16)
    assert_bits_equal(a, run(ordered, x, 16))
    assert ordered.last_dispatch()["split_w2"] == (2 if B == 1 else 1)
    assert_modes_agree(a, run(four, x, 16))
    r = check_step(layer_with_bias(k3_layer, bias_kind), x, 16, *a)
    log(f"  K3 ordered {bias_kind} B={B}:", r)


@pytest.mark.parametrize("bias_kind,B", [("normal", 1), ("zipf", 8)])
def test_k3_late_routing(k3_layer, k3_dev, bias_kind, B):
    """The routing in the gate/up launch on the K3 layer: the four-launch
    step's experts and weights, every token against the oracle."""
    four, _ = k3_ctx(k3_dev, bias_kind, 8)
    late, _ = k3_ctx(k3_dev, bias_kind, 8)
    late.set_mode(binding.MODE_LATE_ROUTING)
    x = synth.make_tokens(k3_dev.dims, 9, B)
    a = run(four, x, 16)
    b = run(late, x, 16)
    # The K3 dense-in launch takes more than one round: by default the
    # routing stays at its end.
    assert four.last_dispatch()["routing"] == 0
    assert late.last_dispatch()["routing"] == 2
    assert_same_step(a, b)
    r = check_step(layer_with_bias(k3_layer, bias_kind), x, 16, *b)
    log(f"  K3 late routing {bias_kind} B={B}:", r)


@pytest.mark.parametrize("users,drafts", [(1, 7), (8, 3)])
def test_k3_spec_verify_batch(k3_layer, k3_dev, users, drafts):
    """Speculative-decoding verify batches (tokens of one user correlated):
    parity with the oracle, and the correlation shows as shared experts."""
    ctx, _ = k3_ctx(k3_dev, "normal", 64)
    x = synth.make_spec_tokens(k3_layer.dims, 3, users, drafts)
    out, idx, w = run(ctx, x, 16)
    r = check_step(k3_layer, x, 16, out, idx, w)
    B = users * (drafts + 1)
    log(f"  spec u{users} d{drafts}:", r, "distinct experts", len(np.unique(idx)), "of", B * 16)
    assert len(np.unique(idx)) < 0.75 * min(B * 16, 896)


def test_k3_tp8_share_layer():
    layer = synth.make_layer(synth.K3_TP8, synth.TP8_STACK_SEED0)
    ctx = make_ctx(layer, 64, 16)
    for B in (1, 8, 9, 16, 64):
        log(f"K3 TP8 share B={B}")
        x = synth.make_tokens(layer.dims, 1, B)
        out, idx, w = run(ctx, x, 16)
        d = ctx.last_dispatch()
        # Batch 1 leaves the gate/up kernel short of units (16 experts x 4
        # tile groups): eight waves share each tile.
        assert d["split_w13"] == (8 if B == 1 else 1)
        # x staged once per workgroup up to 8 tokens (all 8 rows from 3);
        # from 9 tokens this one-round dense-in launch splits K into slices.
        assert d["in_staged"] == (1 if B == 1 else 3 if B == 8 else 2)
        r = check_step(layer, x, 16, out, idx, w)
        log("  ", r)


# ---------------------------------------------------------------------------
# Invariances on the GPU
# ---------------------------------------------------------------------------

def test_k3_batch64_rows_match_batch1_steps(k3_layer, k3_dev):
    """Tokens are independent: each row of a 64-token step (large-batch
    kernels, K split across workgroups) against the same token stepped alone
    (batch-1 kernels).  The two reduce in different orders, so ids may differ
    only at a near tie (each a valid choice), and weights and outputs agree to
    the cross-mode bound."""
    ctx64, _ = k3_ctx(k3_dev, "normal", 64)
    ctx1, _ = k3_ctx(k3_dev, "normal", 1)
    x = synth.make_tokens(k3_layer.dims, 77, 64)
    a = run(ctx64, x, 16)
    rows = [run(ctx1, x[b:b + 1], 16) for b in range(64)]
    b = tuple(np.concatenate([r[i] for r in rows]) for i in range(3))
    assert ctx64.last_dispatch()["col_tiles"] == 4 and ctx1.last_dispatch()["col_tiles"] == 1
    assert_modes_agree(a, b)
    diff = np.nonzero(np.any(a[1] != b[1], axis=1))[0]
    key64 = oracle_keys(k3_layer, x[diff])
    for i, t in enumerate(diff):
        is_near, alts = oracle.near_tie_alternatives(key64[i], 16, TAU)
        assert is_near and all(any(np.array_equal(s[1][t], c) for c in alts) for s in (a, b))
    log(f"  batch 64 vs batch 1: {len(diff)} tokens with other experts (near ties)")


def permuted_layer(layer, perm):
    """The layer with expert j of the new layer = expert perm[j] of the old."""
    return dataclasses.replace(
        layer, router_w=np.ascontiguousarray(layer.router_w[perm]),
        bias=None if layer.bias is None else np.ascontiguousarray(layer.bias[perm]),
        w13_q=np.ascontiguousarray(layer.w13_q[perm]), w13_s=np.ascontiguousarray(layer.w13_s[perm]),
        w2_q=np.ascontiguousarray(layer.w2_q[perm]), w2_s=np.ascontiguousarray(layer.w2_s[perm]))


@pytest.mark.parametrize("which,B", [("small", 9), ("tp8", 16)])
def test_expert_permutation_permutes_ids_only(small_layer, which, B):
    """Renumbering the experts (router rows, bias, expert weights) renumbers
    the selection and leaves weights and outputs unchanged: each expert's
    score is formed in the same order wherever its router row sits, so the
    mapped ids and weights are bit-identical; the outputs may differ only by
    the order of the latent combine."""
    layer = small_layer if which == "small" else \
        synth.make_layer(synth.K3_TP8, synth.TP8_STACK_SEED0 + 3)
    k = 6 if which == "small" else 16
    perm = np.random.default_rng(5).permutation(layer.dims.n_experts)
    lp = permuted_layer(layer, perm)
    x = synth.make_tokens(layer.dims, 31, B)
    a = run(make_ctx(layer, B, k), x, k)
    b = run(make_ctx(lp, B, k), x, k)
    mapped = np.sort(perm[b[1]], axis=1)
    np.testing.assert_array_equal(mapped, a[1])
    order = np.argsort(perm[b[1]], axis=1)
    np.testing.assert_array_equal(np.take_along_axis(b[2], order, axis=1), a[2])
    assert_same_step(a, (b[0], a[1], a[2]))
    check_step(lp, x, k, *b)


@pytest.fixture(scope="module")
def c4_layers():
    log("generating the eight TP8-share layers")
    layers = [synth.make_layer(synth.K3_TP8, synth.TP8_STACK_SEED0 + l) for l in range(8)]
    return layers, [binding.DeviceLayer(la) for la in layers]


def c4_graph_run(c4_layers, B, mode, replays=2):
    """Eight TP8-share layers (own seeds and inputs) captured in one HIP graph,
    the configuration the stacked benchmark replays; returns the inputs and
    each replay's per-layer results (out, idx, w as numpy)."""
    import torch
    layers, devs = c4_layers
    n_layers, k = len(layers), 16
    ctxs = [binding.MoEDecode(dv, B, k) for dv in devs]
    for c in ctxs:
        c.set_mode(mode_const("four_launches" if mode == "prefetch" else mode))
    xs = [synth.make_tokens(la.dims, synth.TP8_STACK_SEED0 + l, B) for l, la in enumerate(layers)]
    xd = [to_dev_tokens(x) for x in xs]
    H = layers[0].dims.hidden
    outs = [torch.empty((B, H), dtype=torch.int16, device="cuda") for _ in range(n_layers)]
    idxs = [torch.empty((B, k), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    ws = [torch.empty((B, k), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    # "prefetch": each layer prefetches the next layer's router and
    # latent-down rows while it routes; results are unchanged.
    g = binding.Graph(ctxs, xd, B, k, outs, idxs, ws, prefetch_next=mode == "prefetch")
    stream = torch.cuda.Stream()
    reps = []
    for rep in range(replays):
        g.launch(stream)
        stream.synchronize()
        reps.append([(outs[l].cpu().numpy().view(np.uint16), idxs[l].cpu().numpy(),
                      ws[l].cpu().numpy()) for l in range(n_layers)])
        for c in ctxs:
            assert c.read_flags() == 0
    g.close()
    return ctxs, xs, reps


@pytest.mark.parametrize("mode", ["four_launches", "prefetch", "side_stream", "two_launches",
                                  "fused", "late_routing", "dense_routing", "ordered"])
def test_c4_eight_layer_graph(c4_layers, mode):
    """Every execution mode: each layer's replayed result equals its eager
    step, and the replayed outputs of the first and last layers match the
    oracle on every token."""
    B, k = 4, 16
    ctxs, xs, reps = c4_graph_run(c4_layers, B, mode)
    for rep in reps:
        for l in range(len(xs)):
            assert_same_step(rep[l], run(ctxs[l], xs[l], k))
    for l in (0, len(xs) - 1):
        r = check_step(c4_layers[0][l], xs[l], k, *reps[-1][l])
        log(f"  C4 {mode} layer {l}:", r)


@pytest.mark.parametrize("mode", ["prefetch", "dense_routing", "late_routing"])
@pytest.mark.parametrize("B", [1, 2])
def test_c4_graph_small_batch_forms(c4_layers, mode, B):
    """Up to two tokens the dense-in launch stages x in LDS (with the routing
    at its end, with prefetch units after it, or with the routing in the
    gate/up launch): replays equal eager steps, and the first and last
    layers match the oracle on every token."""
    k = 16
    ctxs, xs, reps = c4_graph_run(c4_layers, B, mode)
    for rep in reps:
        for l in range(len(xs)):
            assert_same_step(rep[l], run(ctxs[l], xs[l], k))
    for l in (0, len(xs) - 1):
        r = check_step(c4_layers[0][l], xs[l], k, *reps[-1][l])
        log(f"  C4 {mode} B={B} layer {l}:", r)


@pytest.mark.parametrize("B", [1, 64])
def test_c4_graph_replay_matches_oracle(c4_layers, B):
    """The default form at batch 1 and 64: the outputs of both replays of
    the eight-layer graph, every layer and every token, against the oracle."""
    ctxs, xs, reps = c4_graph_run(c4_layers, B, "four_launches")
    for rep in reps:
        for l in range(len(xs)):
            r = check_step(c4_layers[0][l], xs[l], 16, *rep[l])
            log(f"  C4 B={B} layer {l}:", r)
