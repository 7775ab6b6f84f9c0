"""Pins of the general-mask attention oracle (rectangular, windowed, boolean mask).

Pinned to torch's fp64 math attention on the CPU with an explicit boolean
mask (a library routine of the same definition) for rectangular causal
masks aligned to the bottom-right corner, sliding windows and random masks;
to closed forms (a zero-width window returns one value row; an all-true mask
is the unmasked result); and to the convention for rows with no admissible
key.
"""
import numpy as np
import pytest
import torch

import oracle


def rnd(seed, shape):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape))


def explicit_mask(Nq, Nk, causal, wl, wr):
    i = torch.arange(Nq)[:, None]
    j = torch.arange(Nk)[None, :]
    off = Nk - Nq
    m = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        m &= j <= i + off
    if wl >= 0:
        m &= j >= i + off - wl
    if wr >= 0:
        m &= j <= i + off + wr
    return m


def torch_ref(q, k, v, scale, mask):
    rep = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(rep, 1)
    vv = v.repeat_interleave(rep, 1)
    s = scale * torch.matmul(q, kk.transpose(-1, -2).contiguous())
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, -1)
    o = torch.matmul(torch.softmax(s, -1), vv)
    return o.numpy(), lse.numpy()


CASES = [  # Nq, Nk, causal, wl, wr
    (7, 19, True, -1, -1), (19, 19, True, -1, -1), (12, 30, False, 5, 3), (30, 30, True, 6, -1),
    (16, 40, False, 0, 0), (25, 25, False, -1, 4), (9, 33, True, 4, 2)]


@pytest.mark.parametrize("Nq,Nk,causal,wl,wr", CASES)
def test_windows_and_rectangles_match_torch(Nq, Nk, causal, wl, wr):
    B, H, Hkv, d, scale = 2, 4, 2, 8, 0.37
    q, k, v = rnd(1, (B, H, Nq, d)), rnd(2, (B, Hkv, Nk, d)), rnd(3, (B, Hkv, Nk, d))
    m = explicit_mask(Nq, Nk, causal, wl, wr)
    o, lse = oracle.attention_ext(q, k, v, scale, causal, (wl, wr))
    ro, rl = torch_ref(q, k, v, scale, m.expand(B, H, Nq, Nk))
    ok = m.any(-1).numpy()  # rows with an admissible key (the others are NaN in torch)
    np.testing.assert_allclose(o[:, :, ok], ro[:, :, ok], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, ok], rl[:, :, ok], rtol=0, atol=1e-12)
    assert np.all(o[:, :, ~ok] == 0) and np.all(lse[:, :, ~ok] == -np.inf)


@pytest.mark.parametrize("shape", [(1, 1), (2, 1), (1, 3), (2, 3)])
def test_boolean_mask_matches_torch(shape):
    B, H, Nq, Nk, d, scale = 2, 3, 11, 23, 8, 0.5
    q, k, v = rnd(4, (B, H, Nq, d)), rnd(5, (B, H, Nk, d)), rnd(6, (B, H, Nk, d))
    g = np.random.default_rng(7)
    m = torch.from_numpy(g.random(shape + (Nq, Nk)) < 0.6)
    m[..., 3, :] = False  # a row with no admissible key
    o, lse = oracle.attention_ext(q, k, v, scale, False, (-1, -1), mask=m)
    mm = m.expand(B, H, Nq, Nk)
    ro, rl = torch_ref(q, k, v, scale, mm)
    ok = mm.any(-1).numpy()
    np.testing.assert_allclose(o[ok], ro[ok], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[ok], rl[ok], rtol=0, atol=1e-12)
    assert np.all(o[~ok] == 0) and np.all(lse[~ok] == -np.inf)
    assert (~ok).sum() >= B * H


def test_mask_combines_with_causal_and_window():
    B, H, Nq, Nk, d = 1, 2, 10, 26, 4
    q, k, v = rnd(8, (B, H, Nq, d)), rnd(9, (B, H, Nk, d)), rnd(10, (B, H, Nk, d))
    m = torch.from_numpy(np.random.default_rng(11).random((Nq, Nk)) < 0.7)
    o, lse = oracle.attention_ext(q, k, v, 0.8, True, (7, -1), mask=m)
    full = m & explicit_mask(Nq, Nk, True, 7, -1)
    o2, l2 = oracle.attention_ext(q, k, v, 0.8, False, (-1, -1), mask=full)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_zero_width_window_is_one_value_row():
    Nq, Nk = 6, 15
    q, k, v = rnd(12, (1, 2, Nq, 4)), rnd(13, (1, 2, Nk, 4)), rnd(14, (1, 2, Nk, 4))
    o, lse = oracle.attention_ext(q, k, v, 1.0, False, (0, 0))
    off = Nk - Nq
    np.testing.assert_allclose(o, v[:, :, off:].numpy(), rtol=0, atol=1e-15)
    s = (q * k[:, :, off:]).sum(-1).numpy()
    np.testing.assert_allclose(lse, s, rtol=1e-14, atol=1e-14)


def test_square_causal_equals_dense_oracle():
    q, k, v = rnd(15, (2, 2, 33, 8)), rnd(16, (2, 2, 33, 8)), rnd(17, (2, 2, 33, 8))
    a = oracle.attention_ext(q, k, v, 0.3, True)
    b = oracle.attention(q, k, v, 0.3, True)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-14)


def test_all_true_mask_is_unmasked():
    q, k, v = rnd(18, (1, 2, 9, 4)), rnd(19, (1, 2, 21, 4)), rnd(20, (1, 2, 21, 4))
    a = oracle.attention_ext(q, k, v, 0.6, False, mask=torch.ones(9, 21, dtype=torch.bool))
    b = oracle.attention_ext(q, k, v, 0.6, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sampled_rows_match_full():
    q, k, v = rnd(21, (2, 2, 40, 8)), rnd(22, (2, 2, 70, 8)), rnd(23, (2, 2, 70, 8))
    m = torch.from_numpy(np.random.default_rng(24).random((40, 70)) < 0.5)
    full = oracle.attention_ext(q, k, v, 0.4, True, (9, -1), mask=m)
    rows = [39, 0, 17]
    part = oracle.attention_ext(q, k, v, 0.4, True, (9, -1), mask=m, rows=rows)
    assert np.array_equal(part[0], full[0][:, :, rows]) and np.array_equal(part[1], full[1][:, :, rows])
