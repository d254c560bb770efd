"""Write k3_zipf_bias.txt: a router bias for the K3 layer (seed 0) under which
expert popularity follows Zipf(s = 1.1).

Recipe (an input-generation choice, not part of the method):
  * target inclusion frequency of popularity rank r: f_r = min(1, c r^-1.1), with
    c chosen so that sum_r f_r = k = 16 (a token picks 16 experts);
  * ranks are assigned to experts by a seeded permutation;
  * starting from zero, 300 rounds of  b += 0.02 sign(f_tgt - f) min(1, |ln(f_tgt/f)|)
    where f is the measured inclusion frequency over 4,096 calibration tokens
    drawn from a stream disjoint from every test/benchmark token stream.

All routing arithmetic (scores, selection) is the CPU oracle's; nothing here
touches the GPU library.  Run from the repository root:
    python tests/golden/make_zipf_bias.py
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sparse_moe_decode_router_amd import synth  # noqa: E402

N_CALIB, ROUNDS, STEP, ZIPF_S = 4096, 300, 0.02, 1.1


def zipf_targets(E: int, k: int, s: float) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    lo, hi = 0.0, float(k)
    for _ in range(200):                       # bisection for c
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * r ** -s).sum() < k:
            lo = c
        else:
            hi = c
    return np.minimum(1.0, hi * r ** -s)


def main() -> None:
    recipe = synth.K3
    d = recipe.dims
    layer = synth.make_layer(recipe, seed=0, experts=False)
    xc = synth.make_calibration_tokens(d, seed=0, count=N_CALIB)

    chunks = np.array_split(np.arange(N_CALIB), 16)

    def scores_of(ix):
        return oracle.router_scores(d, xc[ix], layer.router_w)[1]

    with ThreadPoolExecutor(max_workers=os.cpu_count() or 1) as pool:
        score = np.concatenate(list(pool.map(scores_of, chunks)))

    rank_of = synth.zipf_rank_permutation(d.n_experts, seed=0)
    f_by_rank = zipf_targets(d.n_experts, d.top_k, ZIPF_S)
    f_tgt = f_by_rank[rank_of - 1]

    b = np.zeros(d.n_experts)
    for it in range(ROUNDS):
        _, idx, _ = oracle.select(d, score, b.astype(np.float32))
        f = np.bincount(idx.ravel(), minlength=d.n_experts) / N_CALIB
        with np.errstate(divide="ignore"):
            mag = np.minimum(1.0, np.abs(np.log(f_tgt / f)))
        b += STEP * np.sign(f_tgt - f) * mag
        if it % 50 == 0 or it == ROUNDS - 1:
            err = np.abs(f - f_tgt).sum()
            print(f"round {it:3d}: sum|f - f_tgt| = {err:.3f}", flush=True)

    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "k3_zipf_bias.txt")
    with open(out, "w") as fh:
        fh.write("# Router bias (float32, one per expert id) for the K3 layer, seed 0:\n")
        fh.write("# expert popularity ~ Zipf(1.1). Written by make_zipf_bias.py from the\n")
        fh.write("# CPU oracle's routing; see that script for the recipe.\n")
        for v in b.astype(np.float32):
            fh.write(f"{float(v):.9g}\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
