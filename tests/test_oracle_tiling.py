"""P5: the online (tiled) recurrence equals the plain definition for every split.

Brute force over tiny inputs: N in 1..8, d in 1..3, every pair of tile sizes
(B_r, B_c) in 1..N+1, causal on and off, in both loop orders -- the
FlashAttention-1 order (K/V tiles outer, O/l/m written back every step) and
the FlashAttention-2 order (Q tiles outer, unnormalised accumulator).  The
pages call the merge exact up to floating-point ordering, so the bar is 1e-12.
A slip in the rescale factors (e.g. the inverse that the printed pseudocode
puts on them), a dropped ragged tile or a mask applied at tile rather than
element granularity breaks it.
"""
import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("N", range(1, 9))
@pytest.mark.parametrize("d", [1, 2, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_dense(N, d, causal):
    rng = np.random.default_rng(100 * N + 10 * d + causal)
    q, k, v = (rng.standard_normal((N, d)) * 2 for _ in range(3))
    scale = 0.7
    o_ref, l_ref = oracle.attention(torch.from_numpy(q[None, None]), torch.from_numpy(k[None, None]),
                                    torch.from_numpy(v[None, None]), scale, causal)
    o_ref, l_ref = o_ref[0, 0], l_ref[0, 0]
    for Br in range(1, N + 2):
        for Bc in range(1, N + 2):
            for fn in (oracle.tiled_fa1, oracle.tiled_fa2):
                o, l = fn(q, k, v, scale, causal, Br, Bc)
                assert np.allclose(o, o_ref, rtol=0, atol=1e-12), (fn.__name__, Br, Bc)
                assert np.allclose(l, l_ref, rtol=0, atol=1e-12), (fn.__name__, Br, Bc)


def test_tiled_sharp_scores_stay_finite():
    # scores spanning ~1e3 would overflow a softmax without the running max
    rng = np.random.default_rng(7)
    N, d = 8, 2
    q, k, v = rng.standard_normal((N, d)) * 30, rng.standard_normal((N, d)) * 30, \
        rng.standard_normal((N, d))
    o_ref, l_ref = oracle.attention(torch.from_numpy(q[None, None]), torch.from_numpy(k[None, None]),
                                    torch.from_numpy(v[None, None]), 1.0, False)
    assert np.all(np.isfinite(o_ref)) and np.all(np.isfinite(l_ref))
    for fn in (oracle.tiled_fa1, oracle.tiled_fa2):
        o, l = fn(q, k, v, 1.0, False, 3, 2)
        assert np.allclose(o, o_ref[0, 0], atol=1e-12)
        assert np.allclose(l, l_ref[0, 0], rtol=1e-14, atol=1e-12)
