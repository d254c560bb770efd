"""Seeded synthetic inputs for the sparse latent-MoE decode layer.

Both the GPU library's tests/benchmark and the CPU oracle take their inputs
from here, and from nothing else.  This module holds no arithmetic of the
method (no scoring, selection, dequantisation or contraction): it only draws
numbers with NumPy's PCG64 and lays them out in the library's formats.

Shapes follow the Kimi-K3 layer the pages describe (896 experts, 16 active per
token, MXFP4 expert weights: page "快是可以生成的，可信只能证明（vLLM 重写 Kimi K3
解码路径…）", section "为什么一条请求会慢").  The remaining dimensions and all
value distributions are assumptions of this implementation, listed with the
workloads below.

Layouts (all row-major, each row contiguous along its reduction dimension):
  x          bf16 [B][H]
  router_w   bf16 [E][H]   (float32 for the tiny layer)
  bias       f32  [E]      (None = no bias)
  lat_down   bf16 [L][H]
  lat_up     bf16 [H][L]
  w13_q      u8   [E][2I][L/2]   two E2M1 codes per byte, rows 0..I-1 gate, I..2I-1 up
  w13_s      u8   [E][2I][L/32]  E8M0 scale bytes, one per 32 elements
  w2_q       u8   [E][L][I/2]
  w2_s       u8   [E][L][I/32]
  sh_w13     bf16 [2Is][H]  gate rows then up rows
  sh_w2      bf16 [H][Is]
bf16 tensors are numpy uint16 arrays holding the bit patterns.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# Stream ids: every tensor draws from its own PCG64 stream, derived from
# (seed, tensor id, index), so any expert or token batch can be regenerated
# on its own.
_T_X, _T_ROUTER, _T_BIAS, _T_LDOWN, _T_LUP = 1, 2, 3, 4, 5
_T_W13Q, _T_W13S, _T_W2Q, _T_W2S, _T_SH13, _T_SH2 = 6, 7, 8, 9, 10, 11
_T_CALIB, _T_ZIPF_RANK, _T_FLAT_BIAS, _T_SPEC = 12, 13, 14, 15

REPO_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ZIPF_BIAS_FILE = os.path.join(REPO_ROOT, "tests", "golden", "k3_zipf_bias.txt")


@dataclasses.dataclass(frozen=True)
class LayerDims:
    hidden: int
    latent: int
    n_experts: int
    expert_inter: int
    shared_inter: int
    top_k: int
    router_f32: bool = False

    @property
    def expert_bytes(self) -> int:
        """MXFP4 bytes of one expert (gate/up + down, codes + scales)."""
        L, I = self.latent, self.expert_inter
        return 2 * I * (L // 2 + L // 32) + L * (I // 2 + I // 32)


@dataclasses.dataclass(frozen=True)
class LayerRecipe:
    """How to draw one layer's weights."""
    dims: LayerDims
    router_std: float
    dense_std: float          # latent projections and shared expert
    scale_exp_lo: int         # E8M0 exponent range, inclusive
    scale_exp_hi: int
    bias: str                 # "none" | "normal:<std>" | "uniform:<half-width>" | "zipf"


# The workloads.  Names say what they are; sizes are in the dims.
TINY = LayerRecipe(
    dims=LayerDims(hidden=512, latent=256, n_experts=64, expert_inter=256, shared_inter=512,
                   top_k=4, router_f32=True),
    router_std=0.02, dense_std=0.02, scale_exp_lo=-8, scale_exp_hi=-4, bias="none")

K3_DIMS = LayerDims(hidden=7168, latent=2048, n_experts=896, expert_inter=2048,
                    shared_inter=4096, top_k=16)
K3 = LayerRecipe(dims=K3_DIMS, router_std=0.01, dense_std=0.02, scale_exp_lo=-9,
                 scale_exp_hi=-5, bias="normal:0.1")
# Same layer, bias calibrated so expert popularity follows Zipf(1.1).
K3_ZIPF = dataclasses.replace(K3, bias="zipf")
# Same layer, near-uniform routing (bias uniform in (-0.01, 0.01)).
K3_FLAT = dataclasses.replace(K3, bias="uniform:0.01")
# One tensor-parallel rank's share (1/8) of the K3 layer: expert and shared
# intermediates divided by 8.  Layers of a stack use seeds 1000 + layer.
K3_TP8_DIMS = dataclasses.replace(K3_DIMS, expert_inter=256, shared_inter=512)
K3_TP8 = dataclasses.replace(K3, dims=K3_TP8_DIMS)

RECIPES = {"tiny": TINY, "k3": K3, "k3_zipf": K3_ZIPF, "k3_flat": K3_FLAT, "k3_tp8": K3_TP8}
TP8_STACK_SEED0 = 1000


def _rng(*ids: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(i) for i in ids]))


def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round binary32 samples to bf16 (nearest, ties to even) and return the
    bit patterns.  Used only to put generated inputs into bf16 storage."""
    f = np.ascontiguousarray(f32, dtype=np.float32)
    if not np.isfinite(f).all():
        raise ValueError("generated inputs must be finite")
    u = f.view(np.uint32)
    r = (u >> 16) & 1          # finite patterns: the sums below cannot wrap
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 patterns to float32 (for plotting / stats)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(seed: int, tid: int, shape, std: float) -> np.ndarray:
    g = _rng(seed, tid)
    return to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


@dataclasses.dataclass
class Layer:
    dims: LayerDims
    seed: int
    router_w: np.ndarray
    bias: Optional[np.ndarray]
    lat_down: np.ndarray
    lat_up: np.ndarray
    w13_q: np.ndarray
    w13_s: np.ndarray
    w2_q: np.ndarray
    w2_s: np.ndarray
    sh_w13: np.ndarray
    sh_w2: np.ndarray

    def nbytes(self) -> int:
        return sum(a.nbytes for a in (self.router_w, self.lat_down, self.lat_up, self.w13_q,
                                      self.w13_s, self.w2_q, self.w2_s, self.sh_w13, self.sh_w2))


def expert_codes(seed: int, tid: int, e: int, shape) -> np.ndarray:
    """Uniform bytes = two uniform E2M1 codes 0..15 each."""
    return _rng(seed, tid, e).integers(0, 256, size=shape, dtype=np.uint8)


def expert_scales(seed: int, tid: int, e: int, shape, lo: int, hi: int) -> np.ndarray:
    """E8M0 bytes 127+lo .. 127+hi, uniform."""
    return _rng(seed, tid, e).integers(127 + lo, 127 + hi + 1, size=shape, dtype=np.uint8)


def load_zipf_bias() -> np.ndarray:
    """Router bias calibrated for Zipf(1.1) expert popularity on the K3 layer
    (seed 0); written by tests/golden/make_zipf_bias.py."""
    vals = np.loadtxt(ZIPF_BIAS_FILE, dtype=np.float64, comments="#")
    return vals.astype(np.float32)


def make_bias(recipe: LayerRecipe, seed: int) -> Optional[np.ndarray]:
    E = recipe.dims.n_experts
    kind = recipe.bias
    if kind == "none":
        return None
    if kind.startswith("normal:"):
        std = float(kind.split(":")[1])
        return (_rng(seed, _T_BIAS).standard_normal(E) * std).astype(np.float32)
    if kind.startswith("uniform:"):
        hw = float(kind.split(":")[1])
        return _rng(seed, _T_FLAT_BIAS).uniform(-hw, hw, E).astype(np.float32)
    if kind == "zipf":
        if seed != 0 or recipe.dims != K3_DIMS:
            raise ValueError("the stored Zipf bias belongs to the K3 layer with seed 0")
        return load_zipf_bias()
    raise ValueError(f"unknown bias kind {kind!r}")


def make_layer(recipe: LayerRecipe, seed: int = 0, experts: bool = True) -> Layer:
    """Draw one layer.  experts=False leaves the expert arrays empty (for
    router-only work such as bias calibration)."""
    d = recipe.dims
    H, L, E, I, Is = d.hidden, d.latent, d.n_experts, d.expert_inter, d.shared_inter
    if d.router_f32:
        router_w = (_rng(seed, _T_ROUTER).standard_normal((E, H), dtype=np.float32)
                    * np.float32(recipe.router_std))
    else:
        router_w = _normal_bf16(seed, _T_ROUTER, (E, H), recipe.router_std)
    nE = E if experts else 0
    w13_q = np.empty((nE, 2 * I, L // 2), np.uint8)
    w13_s = np.empty((nE, 2 * I, L // 32), np.uint8)
    w2_q = np.empty((nE, L, I // 2), np.uint8)
    w2_s = np.empty((nE, L, I // 32), np.uint8)
    lo, hi = recipe.scale_exp_lo, recipe.scale_exp_hi

    def draw_expert(e: int) -> None:
        w13_q[e] = expert_codes(seed, _T_W13Q, e, (2 * I, L // 2))
        w13_s[e] = expert_scales(seed, _T_W13S, e, (2 * I, L // 32), lo, hi)
        w2_q[e] = expert_codes(seed, _T_W2Q, e, (L, I // 2))
        w2_s[e] = expert_scales(seed, _T_W2S, e, (L, I // 32), lo, hi)

    # Each expert has its own streams, so the draw order does not matter.
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        list(pool.map(draw_expert, range(nE)))
    return Layer(
        dims=d, seed=seed, router_w=router_w, bias=make_bias(recipe, seed),
        lat_down=_normal_bf16(seed, _T_LDOWN, (L, H), recipe.dense_std),
        lat_up=_normal_bf16(seed, _T_LUP, (H, L), recipe.dense_std),
        w13_q=w13_q, w13_s=w13_s, w2_q=w2_q, w2_s=w2_s,
        sh_w13=_normal_bf16(seed, _T_SH13, (2 * Is, H), recipe.dense_std),
        sh_w2=_normal_bf16(seed, _T_SH2, (H, Is), recipe.dense_std),
    )


def make_tokens(dims: LayerDims, seed: int, batch: int, draw: int = 0) -> np.ndarray:
    """Hidden states x ~ N(0, 1) in bf16, shape [batch][H].  `draw` selects an
    independent batch (benchmarks rotate through several)."""
    g = _rng(seed, _T_X, draw)
    return to_bf16_bits(g.standard_normal((batch, dims.hidden), dtype=np.float32))


# Correlation of the hidden states of one sequence's verify window (the
# accepted token and its drafts); the pages give none, 0.8 is a reading.
SPEC_RHO = 0.8


def make_spec_tokens(dims: LayerDims, seed: int, users: int, drafts: int, draw: int = 0,
                     rho: float = SPEC_RHO) -> np.ndarray:
    """A speculative-decoding verify batch: `users` sequences, each with its
    last accepted token and `drafts` draft tokens, in bf16, shape
    [users * (drafts + 1)][H], rows of one user adjacent.  Within a user the
    rows share a base: x = sqrt(rho) base_u + sqrt(1 - rho) noise, so each
    row is N(0, 1) and two rows of one user correlate with coefficient rho
    (their routing overlaps); users are independent."""
    g = _rng(seed, _T_SPEC, draw)
    base = g.standard_normal((users, 1, dims.hidden), dtype=np.float32)
    noise = g.standard_normal((users, drafts + 1, dims.hidden), dtype=np.float32)
    x = np.float32(np.sqrt(rho)) * base + np.float32(np.sqrt(1.0 - rho)) * noise
    return to_bf16_bits(x.reshape(users * (drafts + 1), dims.hidden))


def make_calibration_tokens(dims: LayerDims, seed: int, count: int) -> np.ndarray:
    """Tokens used only to calibrate the Zipf bias; disjoint stream from
    make_tokens."""
    g = _rng(seed, _T_CALIB)
    return to_bf16_bits(g.standard_normal((count, dims.hidden), dtype=np.float32))


def zipf_rank_permutation(n_experts: int, seed: int) -> np.ndarray:
    """rank_of[e]: popularity rank (1 = most popular) of expert e."""
    perm = _rng(seed, _T_ZIPF_RANK).permutation(n_experts)
    rank_of = np.empty(n_experts, np.int64)
    rank_of[perm] = np.arange(1, n_experts + 1)
    return rank_of
