"""GPU parity of the forward kernels' lazy reference max, through the C ABI.

The forward kernels exponentiate each key tile against a reference max set on
the first tile and move the reference only when some probability taken
against it would exceed a bound (2^14 for the 16-bit and fp32 kernels, 2^8
for the FP8 kernel).  Moving it recomputes the tile's scores, rescales the
accumulator and both row sums by e^(scale*(m_old - m_new)), and
exponentiates again (shift invariance: "FlashAttention: GPU 메모리 계층을
활용한 어텐션 최적화 분석", youngju.dev, section 6.3; "Flash Attention",
suniverse77.github.io, Eq. (2)-(3)).  With iid N(0, 1) inputs that branch
runs rarely, so these inputs are built to take it on every tile.

Construction: head dimension 0 carries a ramp.  For the rows that ramp, q[i, 0]
= A, and k[j, 0] = L * (j // G) for key groups of G = 32 keys (the smallest
tile of any kernel), so the scaled score rises by scale * A * L >= 12.7 per
group while the other dimensions (N(0, 1) * 0.5) move it by about +-1.  Before
running anything each test checks, in fp64 on its own inputs, that for every
ramping row and every key tile after the first, the tile holds a key whose
scaled score exceeds every earlier score of the row by more than ln(bound) +
0.5.  The reference is always the row max of some earlier keys, so that key's
probability against it exceeds the bound and the branch must run on that
tile, in the kernel's wave-uniform branch, for every wave holding such a
row.  The other rows (q[i, 0] = 0) move their reference in the same branch
with their own, ordinary, row max.  Outputs are compared with the fp64
oracle at the forward's usual bar.

The FP8 case spreads the ramp over every head dimension (q[i, c] = A s_c +
noise, k[j, c] = L (j // G) s_c + noise with a fixed sign pattern s): the
FP8 matrix instruction sums its products in groups of 8 and truncates those
far below the largest one of a group, so a score carried by one dimension
would test that truncation rather than the rebase.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
import oracle
from exact_attention_12_amd import inputs
from gpu_util import FP8_TOL, TOL, errors, progress

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
GROUP = 32  # keys per ramp step: the smallest key tile of any forward kernel


@pytest.fixture(autouse=True)
def _announce(request):
    progress("start " + request.node.nodeid)
    yield


def ramp_inputs(cid, B, H, Nq, Nk, d, dtype, A=8.0, L=18.0, every=2, spread=False, noise=0.5):
    """q [B, H, Nq, d], k and v [B, H, Nk, d]: rows i with i % every == 0 ramp.

    spread=False: head dimension 0 carries the ramp (q[i, 0] = A, k[j, 0] =
    L * (j // GROUP)).  spread=True: every dimension carries it with a fixed
    sign pattern (q[i, c] += A s_c, k[j, c] += L (j // GROUP) s_c), so that no
    single product dominates a score (the FP8 matrix instruction truncates
    products far below the largest one of its group of 8)."""
    q = inputs.normal(1000 * cid + 0, (B, H, Nq, d), noise, torch.float32)
    k = inputs.normal(1000 * cid + 1, (B, H, Nk, d), noise, torch.float32)
    v = inputs.normal(1000 * cid + 2, (B, H, Nk, d), 1.0, torch.float32)
    ramp_rows = (torch.arange(Nq) % every) == 0
    level = L * (torch.arange(Nk) // GROUP).float()
    if spread:
        sign = torch.from_numpy(np.where(np.random.default_rng(1000 * cid + 9).random(d) < 0.5, -1.0, 1.0)).float()
        q += torch.where(ramp_rows, torch.tensor(A), torch.tensor(0.0))[:, None] * sign
        k += level[:, None] * sign
    else:
        q[:, :, :, 0] = torch.where(ramp_rows, torch.tensor(A), torch.tensor(0.0))
        k[:, :, :, 0] = level
    return q.to(dtype), k.to(dtype), v.to(dtype), ramp_rows.numpy()


def visible(Nq, Nk, causal, window=(-1, -1)):
    """[Nq, Nk] admissible pairs: diagonal aligned bottom-right (j <= i + Nk - Nq if causal)."""
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    off = Nk - Nq
    ok = np.ones((Nq, Nk), dtype=bool)
    wl, wr = window
    if causal:
        wr = 0 if wr < 0 else min(wr, 0)
    if wr >= 0:
        ok &= j <= i + off + wr
    if wl >= 0:
        ok &= j >= i + off - wl
    return ok


def assert_rebase_every_tile(s, ok, ramp_rows, tile, bound):
    """s: scaled scores [B, H, Nq, Nk] fp64; ok: admissible pairs [Nq, Nk].

    For every ramping row and every key tile after the row's first visible
    one: some visible key of the tile beats every earlier visible score by
    more than ln(bound) + 0.5."""
    need = math.log(bound) + 0.5
    Nk = s.shape[-1]
    checked = 0
    for i in np.nonzero(ramp_rows)[0]:
        cols = np.nonzero(ok[i])[0]
        if len(cols) == 0:
            continue
        tiles = np.unique(cols // tile)
        for t in tiles[1:]:
            cur = cols[(cols // tile) == t]
            prev = cols[(cols // tile) < t]
            gap = s[:, :, i, cur].max(-1) - s[:, :, i, prev].max(-1)
            assert gap.min() > need, (i, t, gap.min(), need)
            checked += 1
    assert checked > 0, "the construction forces no rebase"
    return checked


def scaled_scores(q, k, scale):
    qd, kd = q.double().numpy(), k.double().numpy()
    return scale * np.einsum("bhid,bhjd->bhij", qd, kd)


def compare(o, lse, ro, rl, dtype, label):
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    empty = np.isneginf(rl)
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty])), label
    okr = ~empty
    assert np.all(np.isfinite(og[okr])) and np.all(np.isfinite(lg[okr])), label
    tol = TOL[dtype]
    omax, omean = errors(og[okr], ro[okr])
    lmax, _ = errors(lg[okr], rl[okr])
    progress("%s max|dO|=%.3g mean|dO|=%.3g max|dlse|=%.3g" % (label, omax, omean, lmax))
    assert omax <= tol["o_max"] and omean <= tol["o_mean"] and lmax <= tol["lse_max"], (
        label, omax, omean, lmax)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fa_fwd_rebase_every_tile(gpu, fa_lib, dt, d, causal):
    B, H, N = 1, 2, 333
    dtype = DT[dt]
    q, k, v, ramp = ramp_inputs(120 + d // 64, B, H, N, N, d, dtype)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    tile = 32 if dt == "f32" else 64
    n = assert_rebase_every_tile(scaled_scores(q, k, scale), visible(N, N, causal), ramp, tile, 2.0 ** 14)
    label = "fa_fwd rebase %s d%d causal%d (%d forced)" % (dt, d, causal, n)
    progress(label)
    o, lse = fa.forward(q.to(gpu), k.to(gpu), v.to(gpu), scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, scale, causal)
    compare(o, lse, ro, rl, dtype, label)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fa_fwd_gqa_rebase_every_tile(gpu, fa_lib, dt):
    B, H, Hkv, N, d = 1, 4, 2, 300, 128
    dtype = DT[dt]
    q, k, v, ramp = ramp_inputs(123, B, H, N, N, d, dtype)
    k, v = k[:, :Hkv].contiguous(), v[:, :Hkv].contiguous()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    kk = k.repeat_interleave(H // Hkv, dim=1)
    assert_rebase_every_tile(scaled_scores(q, kk, scale), visible(N, N, True), ramp,
                             32 if dt == "f32" else 64, 2.0 ** 14)
    label = "fa_fwd_gqa rebase %s" % dt
    progress(label)
    o, lse = fa.forward(q.to(gpu), k.to(gpu), v.to(gpu), scale=scale, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, scale, True)
    compare(o, lse, ro, rl, dtype, label)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", ["window", "mask", "rect", "mask_map"])
def test_fa_fwd_ext_rebase_every_tile(gpu, fa_lib, dt, case):
    B, H, d = 1, 2, 128
    Nq, Nk = (200, 333) if case == "rect" else (333, 333)
    dtype = DT[dt]
    q, k, v, ramp = ramp_inputs(125, B, H, Nq, Nk, d, dtype)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    causal = case != "mask"
    window = (150, -1) if case == "window" else (-1, -1)
    mask = None
    ok = visible(Nq, Nk, causal, window)
    if case in ("mask", "mask_map"):
        # drop every third 16-key run of each row (whole tiles stay visible)
        keep = ((np.arange(Nk)[None, :] // 16 + np.arange(Nq)[:, None]) % 3) != 0
        keep[:, :16] = True
        mask = torch.from_numpy(keep)
        ok = ok & keep
    tile = 32 if dt == "f32" else 64
    n = assert_rebase_every_tile(scaled_scores(q, k, scale), ok, ramp, tile, 2.0 ** 14)
    label = "fa_fwd_ext rebase %s %s (%d forced)" % (dt, case, n)
    progress(label)
    md = None if mask is None else mask.to(gpu)
    o, lse = fa.forward_ext(q.to(gpu), k.to(gpu), v.to(gpu), scale=scale, causal=causal, window=window,
                            mask=md, block_map=True if case == "mask_map" else None)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_ext(q, k, v, scale, causal, window, mask)
    compare(o, lse, ro, rl, dtype, label)


@pytest.mark.parametrize("causal", [False, True])
def test_fa_fwd_fp8_rebase_every_tile(gpu, fa_lib, causal):
    # the FP8 kernel's bound is 2^8; its key tiles are 64 keys.  The ramp is
    # spread over every head dimension: the rise per 32 keys is scale * A * L * d
    B, H, N, d = 1, 2, 333, 128
    q, k, v, ramp = ramp_inputs(127, B, H, N, N, d, torch.bfloat16, A=1.0, L=0.75, spread=True, noise=0.1)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    deq = []
    for t, layout in ((q, 0), (k, 0), (v, 1)):
        c, e = oracle.quant_fp8(t, layout)
        deq.append(torch.from_numpy(oracle.dequant_fp8(c, e, B, H, N, d, layout)))
    n = assert_rebase_every_tile(scaled_scores(deq[0], deq[1], scale), visible(N, N, causal), ramp, 64,
                                 2.0 ** 8)
    label = "fa_fwd_fp8 rebase causal%d (%d forced)" % (causal, n)
    progress(label)
    q8, qe = fa.quant_fp8(q.to(gpu), 0)
    k8, ke = fa.quant_fp8(k.to(gpu), 0)
    v8, ve = fa.quant_fp8(v.to(gpu), 1)
    o, lse = fa.forward_fp8(q8, k8, v8, qe, ke, ve, B, H, H, N, d, scale, causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(deq[0], deq[1], deq[2], scale, causal)
    ra, _ = oracle.attention(deq[0], deq[1], deq[2].abs(), scale, causal)
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    ratio = float((np.abs(og - ro) / (FP8_TOL["rel"] * ra + FP8_TOL["abs"])).max())
    lmax = float(np.abs(lg - rl).max())
    progress("%s max |dO|/bound=%.3f max|dlse|=%.3g" % (label, ratio, lmax))
    assert ratio <= 1.0 and lmax <= FP8_TOL["lse_max"], (label, ratio, lmax)
