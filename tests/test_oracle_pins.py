"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with an independent authority: a table
from the OCP MX v1.0 specification, bit-level format formulas, brute-force
enumeration (all bf16 values, all k-subsets), a separately written dense
NumPy evaluation of the layer (every expert computed, then masked), library
routines (matmul, ldexp), and special cases whose answer is known in closed
form.  A plausible slip in the oracle (a dropped term, a wrong sign, index or
nibble order, a transposed operand, a missing rounding point) fails one of them.
"""
import dataclasses
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_moe_decode_router_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# ---------------------------------------------------------------------------
# Independent helpers (written from the format definitions, not from the oracle)
# ---------------------------------------------------------------------------

_PATTERNS = np.arange(65536, dtype=np.uint32)
with np.errstate(invalid="ignore"):
    _BF16_VALUES = (_PATTERNS << 16).view(np.float32).astype(np.float64)
_POS_FINITE = _BF16_VALUES[:0x7F80]            # 0x0000 .. 0x7F7F, ascending


def bf16_round_bruteforce(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 value by search over every positive finite bf16 value;
    exact ties go to the pattern with an even last bit."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    assert np.all(a < _POS_FINITE[-1]), "test values stay below bf16 max"
    i = np.searchsorted(_POS_FINITE, a, side="left")   # _POS_FINITE[i-1] < a <= [i]
    i = np.clip(i, 1, _POS_FINITE.size - 1)
    lo, hi = _POS_FINITE[i - 1], _POS_FINITE[i]
    pick_hi = (hi - a) < (a - lo)
    tie = (hi - a) == (a - lo)
    pick_hi = np.where(tie, (i % 2) == 0, pick_hi)
    r = np.where(pick_hi, hi, lo)
    r = np.where(a == 0, 0.0, r)
    return np.copysign(r, v)


def e2m1_formula(code: int) -> float:
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return math.copysign(mag, sign)


_E2M1_TAB = np.array([e2m1_formula(c) for c in range(16)])


def decode_mx(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Dense decode of MXFP4 rows [..., K/2] codes + [..., K/32] scales."""
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    scale = np.exp2(s.astype(np.float64) - 127.0)
    return _E2M1_TAB[codes] * np.repeat(scale, 32, axis=-1)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def dense_reference(layer, x, rounding="output", forced_idx=None):
    """The layer evaluated densely with NumPy: every expert is computed for
    every token, then masked by the selection and weighted.  `rounding` as in
    oracle.moe_step."""
    d = layer.dims
    E, I, k = d.n_experts, d.expert_inter, d.top_k
    ident = lambda a: a  # noqa: E731
    rnd = bf16_round_bruteforce if rounding == "bf16_all" else ident
    rnd_out = ident if rounding == "none" else bf16_round_bruteforce
    xv = bf16_f64(x)
    rw = layer.router_w.astype(np.float64) if d.router_f32 else bf16_f64(layer.router_w)
    logit = xv @ rw.T
    score = 1.0 / (1.0 + np.exp(-logit))
    bias = np.zeros(E) if layer.bias is None else layer.bias.astype(np.float64)
    key = score + bias
    B = xv.shape[0]
    idx = np.empty((B, k), np.int64)
    for b in range(B):
        if forced_idx is not None:
            idx[b] = np.sort(forced_idx[b])
        else:
            order = np.lexsort((np.arange(E), -key[b]))
            idx[b] = np.sort(order[:k])
    sel = np.take_along_axis(score, idx, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    z = rnd(xv @ bf16_f64(layer.lat_down).T)
    W13 = decode_mx(layer.w13_q, layer.w13_s)      # [E][2I][L]
    W2 = decode_mx(layer.w2_q, layer.w2_s)         # [E][L][I]
    ylat = np.zeros((B, d.latent))
    for b in range(B):
        mask_w = np.zeros(E)
        mask_w[idx[b]] = w[b]
        for e in range(E):                         # ascending id, every expert
            gu = W13[e] @ z[b]
            g, u = gu[:I], gu[I:]
            a = rnd(g / (1.0 + np.exp(-g)) * u)
            ylat[b] += mask_w[e] * (W2[e] @ a)
    ylat = rnd(ylat)
    S13 = bf16_f64(layer.sh_w13)
    Is = d.shared_inter
    gs, us = xv @ S13[:Is].T, xv @ S13[Is:].T
    ash = rnd(gs / (1.0 + np.exp(-gs)) * us)
    sh = ash @ bf16_f64(layer.sh_w2).T
    up = ylat @ bf16_f64(layer.lat_up).T
    out = rnd_out(up + sh)
    return dict(idx=idx, weight=w, score=score, key=key, z=z, ylat=ylat, ash=ash, sh=sh, up=up,
                out=out)


def small_recipe(H=64, L=64, E=8, I=32, Is=64, k=2, router_f32=False, bias="normal:0.1",
                 router_std=0.1, dense_std=0.1):
    dims = synth.LayerDims(hidden=H, latent=L, n_experts=E, expert_inter=I, shared_inter=Is,
                           top_k=k, router_f32=router_f32)
    return synth.LayerRecipe(dims=dims, router_std=router_std, dense_std=dense_std,
                             scale_exp_lo=-6, scale_exp_hi=-2, bias=bias)


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def test_e2m1_matches_ocp_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 16
    for code_s, val_s in rows:
        code, val = int(code_s, 16), float(val_s)
        got = oracle.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


def test_e2m1_matches_bit_formula():
    for c in range(16):
        got, want = oracle.e2m1_value(c), e2m1_formula(c)
        assert got == want and math.copysign(1, got) == math.copysign(1, want)


def test_e8m0_matches_ldexp():
    for byte in range(255):
        assert oracle.e8m0_value(byte) == math.ldexp(1.0, byte - 127)
    assert math.isnan(oracle.e8m0_value(255))


def test_bf16_widening_exact_for_every_pattern():
    vals = [oracle.bf16_value(p) for p in range(0, 65536, 7)]
    want = _BF16_VALUES[::7]
    finite = np.isfinite(want)
    np.testing.assert_array_equal(np.array(vals)[finite], want[finite])


def test_bf16_rounding_matches_bruteforce():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
        rng.standard_normal(2000),
        # exact midpoints between neighbouring bf16 values: ties to even
        0.5 * (_POS_FINITE[100:2100:1] + _POS_FINITE[101:2101:1]),
        -0.5 * (_POS_FINITE[30000:32000] + _POS_FINITE[30001:32001]),
        # bf16 subnormal range
        rng.uniform(-2.0 ** -126, 2.0 ** -126, 500),
        np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -133, 3 * 2.0 ** -134]),
    ])
    got = np.array([oracle.bf16_round(float(t)) for t in v])
    want = bf16_round_bruteforce(v)
    np.testing.assert_array_equal(got, want)
    assert math.copysign(1, oracle.bf16_round(-0.0)) == -1.0
    # a value exactly halfway rounds to the even neighbour, not up
    assert oracle.bf16_bits_rne(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_bits_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82


def test_mxfp4_nibble_order_and_block_scale():
    q = np.zeros(32, np.uint8)
    s = np.array([127, 130], np.uint8)       # blocks of 32 elements: scale 1, then 8
    q[0] = 0x21                              # element 0 <- low nibble 1 (0.5), 1 <- 2 (1.0)
    q[16] = 0xF7                             # element 32 <- 7 (6.0), 33 <- 0xF (-6.0)
    assert oracle.mxfp4_element(q, s, 0) == 0.5
    assert oracle.mxfp4_element(q, s, 1) == 1.0
    assert oracle.mxfp4_element(q, s, 32) == 48.0
    assert oracle.mxfp4_element(q, s, 33) == -48.0
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, 64, dtype=np.uint8)
    s = rng.integers(100, 150, 4, dtype=np.uint8)
    dense = decode_mx(q, s)
    for j in range(128):
        assert oracle.mxfp4_element(q, s, j) == dense[j]


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------

def bruteforce_topk(key: np.ndarray, k: int):
    """argmax over all k-subsets of the exact key sum; among equal sums the
    lexicographically smallest ascending index tuple."""
    exact = [Fraction(float(t)) for t in key]
    best, best_sum = None, None
    for combo in itertools.combinations(range(len(key)), k):
        tot = sum(exact[i] for i in combo)
        if best_sum is None or tot > best_sum:
            best, best_sum = combo, tot
    return np.array(best)


@pytest.mark.parametrize("E,k", [(5, 1), (6, 2), (8, 3), (10, 4), (12, 4), (12, 2)])
def test_topk_matches_bruteforce_over_all_subsets(E, k):
    rng = np.random.default_rng(E * 31 + k)
    for trial in range(40):
        if trial % 2:
            key = rng.standard_normal(E).astype(np.float32)
        else:                                    # heavy ties
            key = rng.integers(-2, 3, E).astype(np.float32) * np.float32(0.25)
        np.testing.assert_array_equal(oracle.topk(key, k), bruteforce_topk(key, k))


def test_topk_tiny_layer_all_635376_subsets():
    layer = synth.make_layer(synth.TINY, 0, experts=False)
    d = layer.dims
    x = synth.make_tokens(d, 0, 1)
    _, score = oracle.router_scores(d, x, layer.router_w)
    key, idx, _ = oracle.select(d, score, layer.bias)
    combos = np.array(list(itertools.combinations(range(d.n_experts), d.top_k)))
    # Sums of 4 binary64 keys in [1/8, 2) need at most 53 + 4 + 2 significant
    # bits: exact in the 64-bit significand of the x87 extended format.
    assert np.finfo(np.longdouble).nmant >= 63
    assert key.min() >= 0.125 and key.max() < 2.0
    sums = key[0].astype(np.longdouble)[combos].sum(axis=1)
    best = combos[np.flatnonzero(sums == sums.max())[0]]    # first = lexicographically least
    np.testing.assert_array_equal(idx[0], best)


def test_topk_threshold_invariant_large():
    rng = np.random.default_rng(3)
    for _ in range(20):
        key = rng.standard_normal(896)
        key[rng.integers(0, 896, 50)] = key[0]                 # plant ties
        sel = oracle.topk(key, 16)
        assert np.all(np.diff(sel) > 0)
        rest = np.setdiff1d(np.arange(896), sel)
        assert key[sel].min() >= key[rest].max()
        # ties at the boundary resolved toward lower ids
        t = key[sel].min()
        assert not np.any((key[rest] == t) & (rest < sel[key[sel] == t].max()))


def test_select_decides_on_binary64_keys():
    """The top-k is taken on the binary64 keys s + bias: two experts whose keys
    differ by 2^-40 (below binary32 resolution at 0.5) are ordered by that
    difference, not by the id tie-break that binary32 keys would force."""
    dims = small_recipe(E=8, k=1).dims
    score = np.full((1, 8), 0.25)
    score[0, 3] = 0.5
    score[0, 5] = 0.5 + 2.0 ** -40
    assert np.float32(score[0, 3]) == np.float32(score[0, 5])
    key, idx, w = oracle.select(dims, score, None)
    assert idx.tolist() == [[5]] and w.tolist() == [[1.0]]
    assert key[0, 5] - key[0, 3] == 2.0 ** -40
    # the same through a bias: equal scores, biases apart by 2^-30 in binary32
    bias = np.zeros(8, np.float32)
    bias[2] = np.float32(2.0 ** -30)
    _, idx2, _ = oracle.select(dims, np.full((1, 8), 0.75), bias)
    assert idx2.tolist() == [[2]]


# ---------------------------------------------------------------------------
# Near ties: the selections the parity tests accept from the GPU
# ---------------------------------------------------------------------------

def explainable_bruteforce(key: np.ndarray, k: int, tau: float):
    """Every k-subset S for which some key vector within tau / 2 of `key`, per
    element, has S among its top-k sets: raise S by tau / 2, lower the rest by
    tau / 2 and ask whether S's smallest key is still at least the largest
    other key (equal keys may then be ordered either way)."""
    E = key.size
    res = []
    for combo in itertools.combinations(range(E), k):
        up = np.array([key[e] + tau / 2 if e in combo else key[e] - tau / 2 for e in range(E)])
        rest = [e for e in range(E) if e not in combo]
        if not rest or min(up[list(combo)]) >= max(up[rest]):
            res.append(combo)
    return res


def planted_keys(rng, E, k, tau, case):
    """Keys with a planted configuration at the k-th / (k+1)-th boundary (no
    two keys exactly tau apart, where rounding would decide the comparison)."""
    key = 0.5 + rng.permutation(E).astype(np.float64) * 4 * tau   # distinct, 4 tau apart
    order = np.argsort(-key, kind="stable")
    if k >= E:                                  # no boundary: every expert is chosen
        return key
    kth, k1 = order[k - 1], order[k]
    if case == "exact tie":
        key[k1] = key[kth]
    elif case == "gap just below tau":
        key[k1] = key[kth] - 0.999 * tau
    elif case == "gap just above tau":
        key[k1] = key[kth] - 1.001 * tau
    elif case == "key within tau above the k-th":
        if k >= 2:
            key[order[k - 2]] = key[kth] + 0.4 * tau
        key[k1] = key[kth] - 0.45 * tau
    elif case == "many within tau":
        band = order[max(0, k - 3):k + 3]
        key[band] = key[kth] + rng.uniform(-tau / 2, tau / 2, band.size)
    elif case == "all equal":
        key[:] = 0.5
    return key


@pytest.mark.parametrize("case", ["exact tie", "gap just below tau", "gap just above tau",
                                  "key within tau above the k-th", "many within tau",
                                  "all equal", "random"])
@pytest.mark.parametrize("E,k", [(6, 1), (8, 3), (10, 4), (12, 2), (9, 9)])
def test_near_tie_alternatives_match_bruteforce(case, E, k):
    tau = 1e-5
    rng = np.random.default_rng(E * 100 + k * 7 + len(case))
    for trial in range(6):
        key = planted_keys(rng, E, k, tau, case) if case != "random" else \
            0.5 + rng.uniform(-3 * tau, 3 * tau, E)
        want = explainable_bruteforce(key, k, tau)
        is_near, alts = oracle.near_tie_alternatives(key, k, tau)
        got = sorted(tuple(int(e) for e in a) for a in alts)
        assert got == sorted(want), (case, key)
        assert is_near == (len(want) > 1)
        # the oracle's own selection is always among them
        assert tuple(oracle.topk(key, k).tolist()) in got
        if k < E:
            srt = np.sort(key)[::-1]
            assert is_near == (srt[k - 1] - srt[k] <= tau)
            # an expert more than tau above the (k+1)-th key is in every set
            for e in np.nonzero(key > srt[k] + tau)[0]:
                assert all(e in a for a in got)


def test_near_tie_gap_above_tau_accepts_only_the_oracle_selection():
    rng = np.random.default_rng(11)
    key = rng.uniform(0, 1, 896)
    srt = np.sort(key)[::-1]
    key[key == srt[16]] = srt[15] - 1.5e-5
    is_near, alts = oracle.near_tie_alternatives(key, 16, 1e-5)
    assert not is_near and len(alts) == 1
    np.testing.assert_array_equal(alts[0], oracle.topk(key, 16))


def test_weights_invariants():
    rng = np.random.default_rng(4)
    dims = small_recipe(E=32, k=6).dims
    score = rng.uniform(0.01, 0.99, (50, 32))
    key, idx, w = oracle.select(dims, score, rng.standard_normal(32).astype(np.float32) * 0.1)
    assert np.all(w > 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    np.testing.assert_allclose(w, np.take_along_axis(score, idx, 1)
                               / np.take_along_axis(score, idx, 1).sum(1, keepdims=True),
                               rtol=1e-15)
    d1 = small_recipe(E=32, k=1).dims
    _, _, w1 = oracle.select(d1, score, None)
    assert np.all(w1 == 1.0)
    _, idx_eq, w_eq = oracle.select(dims, np.full((3, 32), 0.3), None)
    np.testing.assert_array_equal(idx_eq, np.tile(np.arange(6), (3, 1)))
    np.testing.assert_allclose(w_eq, 1.0 / 6, rtol=1e-15)


@pytest.mark.parametrize("router_f32", [False, True])
def test_router_scores_match_matmul_and_logistic(router_f32):
    layer = synth.make_layer(small_recipe(H=256, E=40, router_f32=router_f32), 5, experts=False)
    d = layer.dims
    x = synth.make_tokens(d, 5, 6)
    logit, score = oracle.router_scores(d, x, layer.router_w)
    rw = layer.router_w.astype(np.float64) if router_f32 else bf16_f64(layer.router_w)
    np.testing.assert_allclose(logit, bf16_f64(x) @ rw.T, rtol=1e-12, atol=1e-14)
    from scipy.special import expit
    np.testing.assert_allclose(score, expit(logit), rtol=1e-14)


# ---------------------------------------------------------------------------
# The whole step against the dense NumPy evaluation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rounding", ["output", "bf16_all", "none"])
@pytest.mark.parametrize("recipe_name,B", [("small", 3), ("small_f32router", 2),
                                           ("tiny", 2)])
def test_step_matches_dense_reference(recipe_name, B, rounding):
    recipe = {"small": small_recipe(), "small_f32router": small_recipe(router_f32=True, E=12,
                                                                       k=3, bias="none"),
              "tiny": synth.TINY}[recipe_name]
    layer = synth.make_layer(recipe, 7)
    x = synth.make_tokens(layer.dims, 7, B)
    got = oracle.moe_step(layer, x, rounding=rounding, want="all")
    ref = dense_reference(layer, x, rounding=rounding)
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    np.testing.assert_allclose(got["weight"], ref["weight"], rtol=1e-14)
    for name in ("z", "ylat", "ash", "sh", "up", "out"):
        rounded = {"bf16_all": ("z", "ylat", "ash", "out"), "output": ("out",),
                   "none": ()}[rounding]
        if name in rounded:
            # both sides round the same binary64 value; only a sum-order
            # difference of ~1e-16 could move a value across a rounding edge
            diff = got[name] != ref[name]
            assert diff.mean() < 1e-3, name
        else:
            assert rel_l2(got[name], ref[name]) < 1e-12, name


def test_output_policy_rounds_only_the_output():
    layer = synth.make_layer(small_recipe(), 17)
    x = synth.make_tokens(layer.dims, 17, 3)
    got = oracle.moe_step(layer, x, rounding="output", want="all")
    exact = oracle.moe_step(layer, x, rounding="none", want="all")
    for name in ("z", "act", "ylat", "ash", "sh", "up"):
        np.testing.assert_array_equal(got[name], exact[name])
    np.testing.assert_array_equal(got["out"], bf16_round_bruteforce(exact["out"]))
    np.testing.assert_array_equal(got["out"], bf16_round_bruteforce(got["up"] + got["sh"]))


def test_zero_gate_weights_leave_only_the_shared_expert():
    layer = synth.make_layer(small_recipe(), 8)
    layer.w13_q[:] = 0                                          # every E2M1 code +0
    x = synth.make_tokens(layer.dims, 8, 2)
    got = oracle.moe_step(layer, x, want="all")
    assert np.all(got["ylat"] == 0)
    np.testing.assert_array_equal(got["out"], bf16_round_bruteforce(got["sh"]))


def test_zero_shared_expert_leaves_only_the_routed_path():
    layer = synth.make_layer(small_recipe(), 9)
    layer.sh_w13[:] = 0
    x = synth.make_tokens(layer.dims, 9, 2)
    got = oracle.moe_step(layer, x, want="all")
    assert np.all(got["sh"] == 0)
    up = got["ylat"] @ bf16_f64(layer.lat_up).T
    np.testing.assert_array_equal(got["out"], bf16_round_bruteforce(up))


def test_unit_codes_reduce_experts_to_matmul():
    """Codes in {0, +1, -1} with one scale per layer: each expert is a
    +-1/0 matrix times 2^(s-127), i.e. a plain matmul."""
    rng = np.random.default_rng(10)
    layer = synth.make_layer(small_recipe(), 10)
    d = layer.dims
    codes = np.array([0x0, 0x2, 0xA], np.uint8)                 # 0, +1, -1
    for name in ("w13_q", "w2_q"):
        arr = getattr(layer, name)
        arr[:] = codes[rng.integers(0, 3, arr.shape)] | (codes[rng.integers(0, 3, arr.shape)] << 4)
    layer.w13_s[:] = 125
    layer.w2_s[:] = 126
    x = synth.make_tokens(d, 10, 1)
    got = oracle.moe_step(layer, x, rounding="none", want="all")

    def signs(q):
        lo, hi = q & 0xF, q >> 4
        to = {0x0: 0.0, 0x2: 1.0, 0xA: -1.0}
        v = np.stack([np.vectorize(to.get)(lo), np.vectorize(to.get)(hi)], -1)
        return v.reshape(*q.shape[:-1], q.shape[-1] * 2)

    z = got["z"][0]
    I = d.expert_inter
    ylat = np.zeros(d.latent)
    for j, e in enumerate(got["idx"][0]):
        gu = (signs(layer.w13_q[e]) * 2.0 ** -2) @ z
        a = gu[:I] / (1 + np.exp(-gu[:I])) * gu[I:]
        np.testing.assert_allclose(got["act"][0, j], a, rtol=1e-12, atol=1e-300)
        ylat += got["weight"][0, j] * ((signs(layer.w2_q[e]) * 2.0 ** -1) @ a)
    np.testing.assert_allclose(got["ylat"][0], ylat, rtol=1e-12)


def test_k_equal_E_is_a_dense_weighted_moe():
    layer = synth.make_layer(small_recipe(E=4, k=4), 11)
    x = synth.make_tokens(layer.dims, 11, 2)
    got = oracle.moe_step(layer, x, rounding="none", want="all")
    np.testing.assert_array_equal(got["idx"], np.tile(np.arange(4), (2, 1)))
    np.testing.assert_allclose(got["weight"], got["score"] / got["score"].sum(1, keepdims=True),
                               rtol=1e-14)


def test_identity_latent_projections_give_a_plain_moe():
    """H = L with identity down/up projections: z = x and out = ylat + sh."""
    layer = synth.make_layer(small_recipe(H=64, L=64), 12)
    eye = synth.to_bf16_bits(np.eye(64, dtype=np.float32))
    layer.lat_down[:] = eye
    layer.lat_up[:] = eye
    x = synth.make_tokens(layer.dims, 12, 2)
    got = oracle.moe_step(layer, x, rounding="none", want="all")
    np.testing.assert_array_equal(got["z"], bf16_f64(x))
    np.testing.assert_allclose(got["out"], got["ylat"] + got["sh"], rtol=1e-15)


def test_zero_router_selects_lowest_ids_with_equal_weights():
    layer = synth.make_layer(small_recipe(E=16, k=5, bias="none"), 13)
    layer.router_w[:] = 0
    x = synth.make_tokens(layer.dims, 13, 3)
    got = oracle.moe_step(layer, x, want="all")
    np.testing.assert_array_equal(got["idx"], np.tile(np.arange(5), (3, 1)))
    assert np.all(got["weight"] == 0.2)


def test_expert_permutation_permutes_indices_only():
    layer = synth.make_layer(small_recipe(E=10, k=3), 14)
    x = synth.make_tokens(layer.dims, 14, 3)
    base = oracle.moe_step(layer, x, want="all")
    perm = np.random.default_rng(14).permutation(10)            # new id of old expert e
    inv = np.argsort(perm)
    p = dataclasses.replace(layer)
    p.router_w = layer.router_w[inv]
    p.bias = layer.bias[inv]
    p.w13_q, p.w13_s = layer.w13_q[inv], layer.w13_s[inv]
    p.w2_q, p.w2_s = layer.w2_q[inv], layer.w2_s[inv]
    got = oracle.moe_step(p, x, want="all")
    np.testing.assert_array_equal(np.sort(perm[base["idx"]], axis=1), got["idx"])
    np.testing.assert_array_equal(got["out"], base["out"])


def test_tokens_are_independent():
    layer = synth.make_layer(synth.TINY, 15)
    x = synth.make_tokens(layer.dims, 15, 5)
    batch = oracle.moe_step(layer, x, want="all")
    for b in range(5):
        one = oracle.moe_step(layer, x[b:b + 1], want="all")
        for name in ("idx", "weight", "z", "ylat", "out"):
            np.testing.assert_array_equal(one[name][0], batch[name][b])


def test_forced_selection_is_used_as_given():
    layer = synth.make_layer(small_recipe(E=8, k=2), 16)
    x = synth.make_tokens(layer.dims, 16, 2)
    forced = np.array([[7, 1], [3, 4]], np.int32)
    got = oracle.moe_step(layer, x, forced_idx=forced, want="all")
    np.testing.assert_array_equal(got["idx"], np.sort(forced, axis=1))
    ref = dense_reference(layer, x, forced_idx=forced)
    assert (got["out"] != ref["out"]).mean() < 1e-3


def test_zipf_bias_fixture_is_well_formed():
    b = synth.load_zipf_bias()
    assert b.shape == (896,) and np.all(np.isfinite(b))
    assert b.max() - b.min() > 0.3          # the calibration spread popularity
