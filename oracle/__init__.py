"""ctypes front end of the binary64 CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only users.  The GPU library neither imports nor
links anything here.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the front end at another build of moe_oracle.c (the
# mutation tests load deliberately broken copies to show the pins catch them).
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("latent", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("expert_inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("router_is_f32", ctypes.c_int32)]


class _Outputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logit", "score", "key", "idx", "weight", "z", "act", "ylat", "ash", "sh",
                 "up", "out")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.oracle_e2m1_value.argtypes = [i32]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [i32]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_bits_rne.argtypes = [ctypes.c_double]
        L.oracle_bf16_bits_rne.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [ctypes.c_double]
        L.oracle_bf16_round.restype = ctypes.c_double
        L.oracle_mxfp4_element.argtypes = [vp, vp, i32]
        L.oracle_mxfp4_element.restype = ctypes.c_double
        L.oracle_topk.argtypes = [vp, i32, i32, vp]
        L.oracle_topk.restype = i32
        L.oracle_router_scores.argtypes = [ctypes.POINTER(_Dims), i32, vp, vp, vp, vp]
        L.oracle_router_scores.restype = i32
        L.oracle_select.argtypes = [ctypes.POINTER(_Dims), i32, vp, vp, vp, vp, vp, vp]
        L.oracle_select.restype = i32
        L.oracle_moe_step.argtypes = [ctypes.POINTER(_Dims), i32] + [vp] * 11 + \
            [i32, vp, ctypes.POINTER(_Outputs)]
        L.oracle_moe_step.restype = i32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: Optional[np.ndarray], dtype) -> Optional[np.ndarray]:
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def dims_struct(d) -> _Dims:
    return _Dims(d.hidden, d.latent, d.n_experts, d.expert_inter, d.shared_inter, d.top_k,
                 1 if d.router_f32 else 0)


# ---- scalar helpers (format definitions) ----

def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e8m0_value(byte: int) -> float:
    return lib().oracle_e8m0_value(byte)


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(bits)


def bf16_bits_rne(v: float) -> int:
    return lib().oracle_bf16_bits_rne(v)


def bf16_round(v: float) -> float:
    return lib().oracle_bf16_round(v)


def mxfp4_element(q_row: np.ndarray, s_row: np.ndarray, j: int) -> float:
    q = _c(q_row, np.uint8)
    s = _c(s_row, np.uint8)
    return lib().oracle_mxfp4_element(_p(q), _p(s), j)


# ---- routing ----

def topk(key: np.ndarray, k: int) -> np.ndarray:
    """The k largest of binary64 keys (full sort, equal keys to the lower
    index), in ascending index."""
    key = _c(key, np.float64)
    out = np.empty(k, np.int32)
    if lib().oracle_topk(_p(key), key.size, k, _p(out)) != 0:
        raise ValueError("oracle_topk: bad arguments")
    return out


def router_scores(dims, x: np.ndarray, router_w: np.ndarray):
    """(logit, score) for tokens x [B][H]; both binary64 [B][E]."""
    x = _c(x, np.uint16)
    B = x.shape[0]
    rw = _c(router_w, np.float32 if dims.router_f32 else np.uint16)
    logit = np.empty((B, dims.n_experts))
    score = np.empty((B, dims.n_experts))
    ds = dims_struct(dims)
    if lib().oracle_router_scores(ctypes.byref(ds), B, _p(x), _p(rw), _p(logit), _p(score)):
        raise RuntimeError("oracle_router_scores failed")
    return logit, score


def select(dims, score: np.ndarray, bias: Optional[np.ndarray], forced_idx=None):
    """(key [B][E], idx [B][k], weight [B][k]) from scores, all binary64
    except idx."""
    score = _c(score, np.float64)
    B = score.shape[0]
    key = np.empty((B, dims.n_experts), np.float64)
    idx = np.empty((B, dims.top_k), np.int32)
    w = np.empty((B, dims.top_k))
    ds = dims_struct(dims)
    rc = lib().oracle_select(ctypes.byref(ds), B, _p(score), _p(_c(bias, np.float32)),
                             _p(_c(forced_idx, np.int32)), _p(key), _p(idx), _p(w))
    if rc:
        raise RuntimeError("oracle_select failed")
    return key, idx, w


# ---- the whole step ----

_ALL = ("logit", "score", "key", "idx", "weight", "z", "act", "ylat", "ash", "sh", "up", "out")


ROUNDING = {"none": 0, "output": 1, "bf16_all": 2}


def moe_step(layer, x: np.ndarray, rounding: str = "output", forced_idx=None,
             want=("idx", "weight", "out")) -> dict:
    """Run the oracle on tokens x [B][H] (bf16 patterns) of a synth.Layer.

    rounding: "output" (intermediates binary64, output rounded to bf16, the
    policy of the GPU library), "bf16_all" (also z, expert activations,
    combined latent and shared activation rounded to bf16) or "none".
    Returns a dict of the requested results (see oracle_outputs in the C
    source); `want="all"` returns every intermediate.
    """
    d = layer.dims
    x = _c(np.atleast_2d(x), np.uint16)
    B = x.shape[0]
    H, L, E, I, Is, k = d.hidden, d.latent, d.n_experts, d.expert_inter, d.shared_inter, d.top_k
    shapes = {"logit": ((B, E), np.float64), "score": ((B, E), np.float64),
              "key": ((B, E), np.float64), "idx": ((B, k), np.int32),
              "weight": ((B, k), np.float64), "z": ((B, L), np.float64),
              "act": ((B, k, I), np.float64), "ylat": ((B, L), np.float64),
              "ash": ((B, Is), np.float64), "sh": ((B, H), np.float64),
              "up": ((B, H), np.float64), "out": ((B, H), np.float64)}
    names = _ALL if want == "all" else tuple(want)
    res = {n: np.empty(*shapes[n]) for n in names}
    outs = _Outputs(**{n: (_p(res[n]) if n in res else None) for n in _ALL})
    arrs = [_c(layer.router_w, np.float32 if d.router_f32 else np.uint16),
            _c(layer.bias, np.float32), _c(layer.lat_down, np.uint16),
            _c(layer.lat_up, np.uint16), _c(layer.w13_q, np.uint8), _c(layer.w13_s, np.uint8),
            _c(layer.w2_q, np.uint8), _c(layer.w2_s, np.uint8), _c(layer.sh_w13, np.uint16),
            _c(layer.sh_w2, np.uint16)]
    if layer.w13_q.shape[0] != E:
        raise ValueError("layer was generated without experts")
    fi = _c(forced_idx, np.int32)
    ds = dims_struct(d)
    rc = lib().oracle_moe_step(ctypes.byref(ds), B, _p(x), *[_p(a) for a in arrs],
                               ROUNDING[rounding], _p(fi), ctypes.byref(outs))
    if rc:
        raise RuntimeError("oracle_moe_step failed")
    return res


def _is_valid_selection(key64_row: np.ndarray, sel, tau: float) -> bool:
    """min over the selection >= max over the rest - tau."""
    mask = np.zeros(key64_row.size, bool)
    mask[list(sel)] = True
    if mask.all():
        return True
    return bool(key64_row[mask].min() >= key64_row[~mask].max() - tau)


def near_tie_alternatives(key64_row: np.ndarray, k: int, tau: float, limit: int = 200000):
    """Every selection of k experts that a decision on keys within tau / 2 of
    the binary64 keys can produce, for one token.

    A set S is the top-k of some key vector that differs from key64_row by at
    most tau / 2 per element exactly when min_{e in S} key_e >= max_{e not in
    S} key_e - tau (raise S by tau / 2, lower the rest by tau / 2).  Every such
    S contains each expert whose key exceeds the (k+1)-th largest key by more
    than tau, and lies within the experts whose key is at least the k-th
    largest key minus tau; the sets in between are enumerated and filtered by
    the condition.  More than one set qualifies exactly when the k-th and
    (k+1)-th largest keys lie within tau of each other.

    Returns (is_near_tie, list of sorted int32 index arrays).  Raises
    ValueError when more than `limit` sets would be listed.
    """
    import itertools
    from math import comb
    key64_row = np.asarray(key64_row, np.float64)
    E = key64_row.size
    order = np.lexsort((np.arange(E), -key64_row))
    top = np.sort(order[:k]).astype(np.int32)
    if k >= E:
        return False, [top]
    v_k, v_k1 = key64_row[order[k - 1]], key64_row[order[k]]
    if v_k - v_k1 > tau:
        return False, [top]
    must = [int(e) for e in np.nonzero(key64_row > v_k1 + tau)[0]]
    cand = [int(e) for e in np.nonzero((key64_row >= v_k - tau) & (key64_row <= v_k1 + tau))[0]]
    free = k - len(must)
    if comb(len(cand), free) > limit:
        raise ValueError(f"{comb(len(cand), free)} candidate selections")
    alts = []
    for combo in itertools.combinations(cand, free):
        sel = must + list(combo)
        if _is_valid_selection(key64_row, sel, tau):
            alts.append(np.sort(np.array(sel, np.int32)))
    return len(alts) > 1, alts
