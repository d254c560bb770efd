"""Host checks of the seeded input generators (no GPU): the speculative
verify batches have the stated correlation structure, and routing on them
shares experts within a user (oracle routing)."""
import numpy as np

import oracle
from sparse_moe_decode_router_amd import synth


def test_spec_tokens_structure():
    d = synth.K3.dims
    x = synth.bf16_bits_to_f32(synth.make_spec_tokens(d, 7, users=3, drafts=3)).astype(np.float64)
    assert x.shape == (12, d.hidden)
    np.testing.assert_array_equal(synth.make_spec_tokens(d, 7, 3, 3), synth.make_spec_tokens(d, 7, 3, 3))
    assert not np.array_equal(synth.make_spec_tokens(d, 7, 3, 3, draw=1),
                              synth.make_spec_tokens(d, 7, 3, 3))
    c = np.corrcoef(x)
    # Rows of one user correlate with coefficient rho; users are independent
    # (7168 samples: standard error of a correlation about 0.012).
    for u in range(3):
        for i in range(4):
            assert abs(x[4 * u + i].std() - 1.0) < 0.03
            for j in range(4):
                if i != j:
                    assert abs(c[4 * u + i, 4 * u + j] - synth.SPEC_RHO) < 0.05
    for a in range(12):
        for b in range(12):
            if a // 4 != b // 4:
                assert abs(c[a, b]) < 0.05


def test_spec_tokens_share_experts():
    """Oracle routing of the K3 router: a user's 8 tokens share experts (a
    correlated batch touches far fewer than 8 x 16), independent tokens much
    less so."""
    layer = synth.make_layer(synth.K3, 0, experts=False)
    spec = synth.make_spec_tokens(layer.dims, 3, users=1, drafts=7)
    flat = synth.make_tokens(layer.dims, 3, 8)
    def distinct(x):
        _, score = oracle.router_scores(layer.dims, x, layer.router_w)
        return len(np.unique(oracle.select(layer.dims, score, layer.bias)[1]))
    ds, df = distinct(spec), distinct(flat)
    assert ds < 0.75 * 128 and ds < df
