"""The GPU parity gate itself, on the CPU: results that equal the oracle's pass,
and a planted error of the kind a kernel could make fails -- one output
element off by 20 % on one token, one token's output off by a little more
than the tolerance while the batch as a whole stays within it, a routing
weight off by 2e-5, a swapped expert at a token with no near tie, too many
near-tie tokens in a batch."""
import numpy as np
import pytest

import oracle
from gpu_util import TAU, check_step, near_tie_max, oracle_keys, oracle_step
from sparse_moe_decode_router_amd import synth


def bf16_bits(v: np.ndarray) -> np.ndarray:
    return np.vectorize(oracle.bf16_bits_rne, otypes=[np.uint16])(v)


@pytest.fixture(scope="module")
def case():
    layer = synth.make_layer(synth.TINY, 0)
    x = synth.make_tokens(layer.dims, 41, 6)
    ref = oracle_step(layer, x, threads=3)
    out = bf16_bits(ref["out"])
    return layer, x, out, ref["idx"].astype(np.int32), ref["weight"].astype(np.float32)


def test_threaded_oracle_equals_one_call(case):
    layer, x, *_ = case
    a = oracle_step(layer, x, threads=4)
    b = oracle.moe_step(layer, x, rounding="output")
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_oracle_results_pass(case):
    layer, x, out, idx, w = case
    r = check_step(layer, x, 4, out, idx, w)
    assert r["tokens"] == 6 and r["near_ties"] == 0 and r["max_elem_over_bound"] <= 1


def test_one_element_off_fails(case):
    """An element of about a fifth of the token's rms, 20 % off: too small a
    change for the token's relative L2 error to exceed 2e-3 at hidden 512."""
    layer, x, out, idx, w = case
    f = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rms = np.sqrt(np.mean(f[2] ** 2))
    h = int(np.argmin(np.abs(np.abs(f[2]) - 0.2 * rms)))
    bad = out.copy()
    bad[2, h] = bf16_bits(np.array([f[2, h] * 1.2]))[0]
    with pytest.raises(AssertionError, match=f"element {h}:"):
        check_step(layer, x, 4, bad, idx, w)


def test_one_token_beyond_tolerance_fails(case):
    """Noise of 2.5e-3 relative on one of six tokens: the batch norm stays
    below 2e-3, the token's own does not."""
    layer, x, out, idx, w = case
    ref = oracle_step(layer, x, threads=2)["out"]
    noisy = ref.copy()
    rng = np.random.default_rng(0)
    d = rng.standard_normal(ref.shape[1])
    noisy[4] += 2.5e-3 * np.linalg.norm(ref[4]) * d / np.linalg.norm(d)
    bad = out.copy()
    bad[4] = bf16_bits(noisy[4])
    with pytest.raises(AssertionError):
        check_step(layer, x, 4, bad, idx, w)


def test_weight_off_fails(case):
    layer, x, out, idx, w = case
    bad = w.copy()
    bad[1, 2] += 2e-5
    with pytest.raises(AssertionError, match="weights differ"):
        check_step(layer, x, 4, out, idx, bad)


def test_swapped_expert_without_near_tie_fails(case):
    layer, x, out, idx, w = case
    key = oracle_keys(layer, x)[3]
    order = np.lexsort((np.arange(key.size), -key))
    assert key[order[3]] - key[order[4]] > TAU
    bad = idx.copy()
    bad[3] = np.sort(np.concatenate([order[:3], order[4:5]]))
    with pytest.raises(AssertionError, match="without a near tie"):
        check_step(layer, x, 4, out, bad, w)


def test_too_many_near_ties_fail():
    """Six experts whose keys tie exactly at every token (zero router, equal
    bias), the GPU taking another valid four of them each time: every token
    is a near tie, more than a batch of three may hold."""
    layer = synth.make_layer(synth.TINY, 0)
    layer.router_w[:] = 0
    layer.bias = np.zeros(layer.dims.n_experts, np.float32)
    layer.bias[10:16] = 1.0
    x = synth.make_tokens(layer.dims, 41, 3)
    ref = oracle_step(layer, x, threads=1)
    np.testing.assert_array_equal(ref["idx"], np.tile(np.arange(10, 14), (3, 1)))
    idx = np.tile(np.arange(12, 16, dtype=np.int32), (3, 1))
    assert near_tie_max(3) < 3
    with pytest.raises(AssertionError, match="near-tie tokens"):
        check_step(layer, x, 4, bf16_bits(ref["out"]), idx, np.full((3, 4), 0.25, np.float32))
