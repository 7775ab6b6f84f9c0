"""Pins of the dense-attention oracle against facts that do not come from it.

Each test fixes the oracle to something other than itself: closed forms
derived by hand from the definition, identities the pages state (shift
invariance, exact merge), special cases that reduce to a library routine
(scipy's softmax / logsumexp, numpy's and torch's float conversions), and
brute force.  A plausible mistake -- a dropped key, a sign, an off-by-one in
the causal mask, a transposed operand, log base 2 instead of e, the scale in
the wrong place -- fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rnd(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape)


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# --------------------------------------------------------------------------
# exact widening of the storage types
# --------------------------------------------------------------------------

def test_widen_fp16_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.widen(torch.from_numpy(bits.view(np.int16)).view(torch.float16))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_widen_bf16_every_bit_pattern():
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    b = bits.view(torch.bfloat16)
    ref = b.to(torch.float64).numpy()
    got = oracle.widen(b)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_widen_fp32_exact():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.widen(x), x.astype(np.float64))


# --------------------------------------------------------------------------
# closed forms worked by hand
# --------------------------------------------------------------------------

def _hand_inputs():
    # d = 1, scale = 1: s_ij = q_i * k_j with k = (ln 1, ln 2, ln 4)
    q = np.array([1.0, 2.0, 0.0]).reshape(1, 1, 3, 1)
    k = np.array([0.0, math.log(2.0), math.log(4.0)]).reshape(1, 1, 3, 1)
    v = np.array([3.0, -5.0, 7.0]).reshape(1, 1, 3, 1)
    return q, k, v


def test_hand_example_noncausal():
    # row 0: e^s = 1, 2, 4 -> /7; row 1: 1, 4, 16 -> /21; row 2: uniform
    q, k, v = _hand_inputs()
    o, lse = oracle.attention(t64(q), t64(k), t64(v), 1.0, False)
    exp_o = [(3 - 10 + 28) / 7, (3 - 20 + 112) / 21, (3 - 5 + 7) / 3]
    exp_l = [math.log(7), math.log(21), math.log(3)]
    assert np.allclose(o.ravel(), exp_o, rtol=0, atol=1e-14)
    assert np.allclose(lse.ravel(), exp_l, rtol=0, atol=1e-14)


def test_hand_example_causal():
    # row 0 sees key 0 only; row 1 keys 0,1 (e^s = 1, 4); row 2 keys 0..2 (uniform)
    q, k, v = _hand_inputs()
    o, lse = oracle.attention(t64(q), t64(k), t64(v), 1.0, True)
    exp_o = [3.0, (3 - 20) / 5, (3 - 5 + 7) / 3]
    exp_l = [0.0, math.log(5), math.log(3)]
    assert np.allclose(o.ravel(), exp_o, rtol=0, atol=1e-14)
    assert np.allclose(lse.ravel(), exp_l, rtol=0, atol=1e-14)


def test_hand_example_scale_multiplies_scores():
    # scale 0.5 on row 1 (q = 2): s = ln(1), ln(2), ln(4) again -> /7
    q, k, v = _hand_inputs()
    o, lse = oracle.attention(t64(q), t64(k), t64(v), 0.5, False)
    assert abs(o[0, 0, 1, 0] - (3 - 10 + 28) / 7) < 1e-14
    assert abs(lse[0, 0, 1] - math.log(7)) < 1e-14


# --------------------------------------------------------------------------
# library special case: scipy softmax / logsumexp on explicit score matrices
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 3), (5, 4), (17, 8), (40, 16)])
def test_matches_scipy_softmax(N, d, causal):
    q, k, v = rnd(1, (2, 3, N, d)), rnd(2, (2, 3, N, d)), rnd(3, (2, 3, N, d))
    scale = 0.37
    o, lse = oracle.attention(t64(q), t64(k), t64(v), scale, causal)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = scipy.special.softmax(s, axis=-1)
    assert np.allclose(o, p @ v, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-12, atol=1e-12)
    P = oracle.probs(t64(q), t64(k), scale, causal)
    assert np.allclose(P, p, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# the pages' invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_P1_rows_of_P_sum_to_one(causal):
    N, d = 23, 8
    q, k = rnd(4, (1, 2, N, d)) * 3, rnd(5, (1, 2, N, d)) * 3
    P = oracle.probs(t64(q), t64(k), 0.5, causal)
    assert np.all(P >= 0)
    assert np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    if causal:
        assert np.all(P[..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_P2_shift_invariance(causal):
    # k[:, d-1] = 1 makes q[i, d-1] add a constant to every score of row i
    N, d, scale, delta = 19, 6, 0.8, 2.0
    q, k, v = rnd(6, (1, 1, N, d)), rnd(7, (1, 1, N, d)), rnd(8, (1, 1, N, d))
    k[..., d - 1] = 1.0
    o1, l1 = oracle.attention(t64(q), t64(k), t64(v), scale, causal)
    q2 = q.copy()
    q2[..., d - 1] += delta
    o2, l2 = oracle.attention(t64(q2), t64(k), t64(v), scale, causal)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)
    assert np.allclose(l2 - l1, scale * delta, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_P3_one_hot_v_exposes_P(causal):
    N, d = 12, 16
    q, k = rnd(9, (1, 1, N, d)), rnd(10, (1, 1, N, d))
    v = np.zeros((1, 1, N, d))
    v[0, 0, np.arange(N), np.arange(N)] = 1.0
    o, _ = oracle.attention(t64(q), t64(k), t64(v), 0.3, causal)
    s = 0.3 * q[0, 0] @ k[0, 0].T
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = scipy.special.softmax(s, axis=-1)
    assert np.allclose(o[0, 0, :, :N], p, rtol=0, atol=1e-14)
    assert np.all(o[0, 0, :, N:] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_P4_constant_keys_average_values(causal):
    N, d, scale = 31, 5, 0.9
    q, v = rnd(11, (1, 1, N, d)), rnd(12, (1, 1, N, d))
    k = np.broadcast_to(rnd(13, (d,)), (1, 1, N, d)).copy()
    o, lse = oracle.attention(t64(q), t64(k), t64(v), scale, causal)
    for i in range(N):
        n = i + 1 if causal else N
        assert np.allclose(o[0, 0, i], v[0, 0, :n].mean(0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - (scale * q[0, 0, i] @ k[0, 0, 0] + math.log(n))) < 1e-12


def test_P7_causal_first_row_is_first_value():
    N, d, scale = 9, 4, 0.6
    q, k, v = rnd(14, (2, 2, N, d)), rnd(15, (2, 2, N, d)), rnd(16, (2, 2, N, d))
    o, lse = oracle.attention(t64(q), t64(k), t64(v), scale, True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.allclose(lse[:, :, 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], -1), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_P8_zero_scale_is_mean(causal):
    N, d = 14, 3
    q, k, v = rnd(17, (1, 1, N, d)), rnd(18, (1, 1, N, d)), rnd(19, (1, 1, N, d))
    o, lse = oracle.attention(t64(q), t64(k), t64(v), 0.0, causal)
    for i in range(N):
        n = i + 1 if causal else N
        assert np.allclose(o[0, 0, i], v[0, 0, :n].mean(0), atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(n)) < 1e-14


def test_P9_joint_key_value_permutation():
    N, d = 27, 7
    q, k, v = rnd(20, (1, 2, N, d)), rnd(21, (1, 2, N, d)), rnd(22, (1, 2, N, d))
    perm = np.random.default_rng(23).permutation(N)
    o1, l1 = oracle.attention(t64(q), t64(k), t64(v), 0.4, False)
    o2, l2 = oracle.attention(t64(q), t64(k[:, :, perm]), t64(v[:, :, perm]), 0.4, False)
    assert np.allclose(o1, o2, atol=1e-13)
    assert np.allclose(l1, l2, atol=1e-13)


def test_P9_causal_is_not_permutation_invariant():
    # guard against a causal mask that is silently ignored
    N, d = 8, 4
    q, k, v = rnd(24, (1, 1, N, d)), rnd(25, (1, 1, N, d)), rnd(26, (1, 1, N, d))
    oc, _ = oracle.attention(t64(q), t64(k), t64(v), 0.5, True)
    on, _ = oracle.attention(t64(q), t64(k), t64(v), 0.5, False)
    assert np.allclose(oc[0, 0, N - 1], on[0, 0, N - 1], atol=1e-14)  # last row sees all
    assert not np.allclose(oc[0, 0, : N - 1], on[0, 0, : N - 1])


@pytest.mark.parametrize("Hkv", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_kv_heads_equal_repeated_kv(Hkv, causal):
    # grouped query heads (k, v with Hkv heads) are multi-head attention on
    # k, v repeated so that query head h sees kv head h // (H // Hkv)
    B, H, N, d = 2, 4, 9, 5
    q = t64(rnd(41, (B, H, N, d)))
    k = t64(rnd(42, (B, Hkv, N, d)))
    v = t64(rnd(43, (B, Hkv, N, d)))
    o, lse = oracle.attention(q, k, v, 0.4, causal)
    kr = torch.repeat_interleave(k, H // Hkv, dim=1)
    vr = torch.repeat_interleave(v, H // Hkv, dim=1)
    o2, lse2 = oracle.attention(q, kr, vr, 0.4, causal)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # query heads of one group with equal queries give equal rows
    q2 = q.clone()
    q2[:, 1] = q2[:, 0]
    o3, _ = oracle.attention(q2, k, v, 0.4, causal)
    if Hkv == 1 or H // Hkv >= 2:
        assert np.array_equal(o3[:, 0], o3[:, 1])


def test_P12_single_token():
    q, k, v = rnd(27, (3, 2, 1, 16)), rnd(28, (3, 2, 1, 16)), rnd(29, (3, 2, 1, 16))
    for causal in (False, True):
        o, lse = oracle.attention(t64(q), t64(k), t64(v), 0.25, causal)
        assert np.array_equal(o, v)
        assert np.allclose(lse[..., 0], 0.25 * np.sum(q[..., 0, :] * k[..., 0, :], -1),
                           atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_P13_convexity(causal):
    N, d = 33, 9
    q, k, v = rnd(30, (1, 1, N, d)) * 4, rnd(31, (1, 1, N, d)) * 4, rnd(32, (1, 1, N, d))
    o, _ = oracle.attention(t64(q), t64(k), t64(v), 1.0, causal)
    for i in range(N):
        n = i + 1 if causal else N
        assert np.all(o[0, 0, i] >= v[0, 0, :n].min(0) - 1e-14)
        assert np.all(o[0, 0, i] <= v[0, 0, :n].max(0) + 1e-14)


# --------------------------------------------------------------------------
# storage types, sampled rows, argument checks
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_storage_types_read_exactly(dtype):
    shape = (2, 2, 21, 8)
    q, k, v = [torch.from_numpy(rnd(s, shape).astype(np.float32)).to(dtype) for s in (33, 34, 35)]
    o1, l1 = oracle.attention(q, k, v, 0.35, True)
    o2, l2 = oracle.attention(q.double(), k.double(), v.double(), 0.35, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sampled_rows_match_full():
    shape = (2, 3, 50, 8)
    q, k, v = [t64(rnd(s, shape)) for s in (36, 37, 38)]
    rows = [0, 1, 17, 48, 49]
    of, lf = oracle.attention(q, k, v, 0.5, True)
    orow, lrow = oracle.attention(q, k, v, 0.5, True, rows=rows)
    assert np.array_equal(of[:, :, rows], orow)
    assert np.array_equal(lf[:, :, rows], lrow)


def test_bad_arguments_rejected():
    q = t64(rnd(39, (1, 1, 4, 2)))
    with pytest.raises(ValueError):
        oracle.attention(q, q, q, 1.0, False, rows=[4])
    with pytest.raises(ValueError):
        oracle.attention(q, q, t64(rnd(40, (1, 1, 5, 2))), 1.0, False)
