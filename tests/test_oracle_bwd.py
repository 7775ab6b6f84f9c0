"""Pins of the backward oracle (dQ, dK, dV) against facts that do not come from it.

The backward oracle is the chain rule of the forward definition.  It is
pinned to: central finite differences of the pinned forward oracle
(L = sum(O * dO), so dL/dO = dO); torch's fp64 autograd through its math
attention on the CPU (a library routine of the same definition); closed
forms for one token and for constant values; the softmax-Jacobian identity
sum_j dS_ij = 0 (hence sum_j dK_j = 0); D_i = dO_i . O_i with O from the
forward oracle; and exact agreement of sampled rows and keys with the full
result.  A dropped term, a sign, a transposed operand, a missing scale or
a wrong kv-head mapping fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rnd(seed, shape, scale=1.0):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape) * scale)


def inputs(seed, B, H, Hkv, N, d):
    return (rnd(seed, (B, H, N, d)), rnd(seed + 1, (B, Hkv, N, d)),
            rnd(seed + 2, (B, Hkv, N, d)), rnd(seed + 3, (B, H, N, d)))


def loss(q, k, v, dout, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(o * dout.numpy()))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2)])
def test_finite_differences(causal, H, Hkv):
    """Every gradient entry against a central difference of the forward oracle."""
    B, N, d, scale, h = 1, 5, 3, 0.8, 1e-5
    q, k, v, dout = inputs(11, B, H, Hkv, N, d)
    g = oracle.attention_bwd(q, k, v, dout, scale, causal)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = np.empty(x.shape)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            args_p = dict(q=q, k=k, v=v)
            args_m = dict(q=q, k=k, v=v)
            args_p[name[1]] = xp
            args_m[name[1]] = xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"], dout, scale, causal) -
                       loss(args_m["q"], args_m["k"], args_m["v"], dout, scale, causal)) / (2 * h)
        np.testing.assert_allclose(g[name], fd, rtol=0, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv,N,d", [(3, 3, 37, 16), (4, 1, 29, 8), (6, 2, 64, 32)])
def test_matches_torch_fp64_autograd(causal, H, Hkv, N, d):
    """torch's CPU math attention in fp64, differentiated by autograd."""
    B, scale = 2, 0.3
    q, k, v, dout = inputs(5, B, H, Hkv, N, d)
    g = oracle.attention_bwd(q, k, v, dout, scale, causal)
    qq, kk, vv = (t.clone().requires_grad_() for t in (q, k, v))
    rep = H // Hkv
    s = scale * torch.matmul(qq, kk.repeat_interleave(rep, 1).transpose(-1, -2).contiguous())
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, -1), vv.repeat_interleave(rep, 1))
    o.backward(dout)
    np.testing.assert_allclose(g["dq"], qq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dk"], kk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dv"], vv.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_single_token(causal):
    """N = 1: P = 1, so dV = dO (summed over the group), dQ = dK = 0."""
    q, k, v, dout = inputs(2, 2, 4, 2, 1, 8)
    g = oracle.attention_bwd(q, k, v, dout, 1.3, causal)
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    want = dout.numpy().reshape(2, 2, 2, 1, 8).sum(axis=2)
    np.testing.assert_allclose(g["dv"], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_no_score_gradient(causal):
    """Equal value rows make O independent of P: dS = 0, so dQ = dK = 0 and
    dV_j = sum_i P_ij dO_i sums to sum_i dO_i over the keys."""
    q, k, v, dout = inputs(3, 1, 2, 2, 9, 4)
    v = v[:, :, :1, :].expand(-1, -1, 9, -1).contiguous()
    g = oracle.attention_bwd(q, k, v, dout, 0.9, causal)
    assert np.abs(g["dq"]).max() < 1e-14 and np.abs(g["dk"]).max() < 1e-14
    np.testing.assert_allclose(g["dv"].sum(axis=2), dout.numpy().sum(axis=2), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    """sum_j dS_ij = D_i - D_i = 0 for every row, so sum_j dK_j = 0."""
    q, k, v, dout = inputs(4, 2, 4, 2, 23, 8)
    g = oracle.attention_bwd(q, k, v, dout, 0.6, causal)
    assert np.abs(g["dk"].sum(axis=2)).max() < 1e-12
    assert np.abs(g["dk"]).max() > 1e-2


def test_causal_boundary_rows():
    """Causal: row 0 sees key 0 only (dQ_0 = 0); the last key is seen by the
    last row only, with P = exp(s - lse)."""
    B, H, N, d, scale = 1, 2, 7, 4, 0.7
    q, k, v, dout = inputs(8, B, H, H, N, d)
    g = oracle.attention_bwd(q, k, v, dout, scale, True)
    assert np.all(g["dq"][:, :, 0] == 0)
    _, lse = oracle.attention(q, k, v, scale, True)
    s_last = scale * (q[:, :, N - 1] * k[:, :, N - 1]).sum(-1).numpy()
    p = np.exp(s_last - lse[:, :, N - 1])
    np.testing.assert_allclose(g["dv"][:, :, N - 1], p[..., None] * dout[:, :, N - 1].numpy(),
                               rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_D_is_dO_dot_O(causal):
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i with O from the forward oracle."""
    q, k, v, dout = inputs(9, 1, 4, 2, 31, 16)
    g = oracle.attention_bwd(q, k, v, dout, 0.4, causal)
    o, _ = oracle.attention(q, k, v, 0.4, causal)
    np.testing.assert_allclose(g["D"], (o * dout.numpy()).sum(-1), rtol=1e-12, atol=1e-13)


def test_scale_zero():
    """scale = 0: P is uniform over admissible keys and dQ = dK = 0."""
    q, k, v, dout = inputs(10, 1, 2, 2, 6, 4)
    g = oracle.attention_bwd(q, k, v, dout, 0.0, False)
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_allclose(g["dv"], np.broadcast_to(dout.numpy().mean(axis=2, keepdims=True),
                                                        g["dv"].shape), rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_keys_match_full(causal):
    q, k, v, dout = inputs(12, 2, 4, 2, 40, 8)
    full = oracle.attention_bwd(q, k, v, dout, 0.5, causal)
    rows, keys = [39, 0, 17], [5, 39, 0]
    part = oracle.attention_bwd(q, k, v, dout, 0.5, causal, rows=rows, keys=keys)
    assert np.array_equal(part["dq"], full["dq"][:, :, rows])
    assert np.array_equal(part["dk"], full["dk"][:, :, keys])
    assert np.array_equal(part["dv"], full["dv"][:, :, keys])
    only_q = oracle.attention_bwd(q, k, v, dout, 0.5, causal, rows=rows, keys=[])
    assert np.array_equal(only_q["dq"], full["dq"][:, :, rows])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_storage_types_read_exactly(dtype):
    q, k, v, dout = (t.to(dtype) for t in inputs(13, 1, 2, 1, 11, 8))
    a = oracle.attention_bwd(q, k, v, dout, 0.5, True)
    b = oracle.attention_bwd(*(t.to(torch.float64) for t in (q, k, v, dout)), 0.5, True)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(a[name], b[name])


def test_bad_arguments_rejected():
    q, k, v, dout = inputs(14, 1, 3, 2, 4, 4)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, k, v, dout, 1.0, False)
    q, k, v, dout = inputs(14, 1, 2, 2, 4, 4)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, k, v, dout, 1.0, False, rows=[4])
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, k, v, dout, 1.0, False, keys=[-1])
