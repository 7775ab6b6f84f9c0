"""GPU parity of fa_fwd_ext (rectangular, windowed, boolean-masked) against the
fp64 oracle, through the C ABI.

Rows that see no key must come back as o = 0 and lse = -inf exactly; the
others meet the forward's bar for their input type.  Full comparison on
ragged shapes; at B=2 H=32 N=8192 d=128 (bf16) a causal sliding window and a
broadcast boolean mask on 256 sampled rows per head.  The mask's block map
(fa_mask_blocks) must equal the oracle's bit for bit.  A forward given the map
meets the same bar against the oracle, and stays within MAP_DIFF of the same
forward without the map: the map only removes tiles that change nothing, but
the tiles left over may run in the other of the loop body's two compiled
copies (one per LDS buffer), which can round the reference's products in the
last bit (observed: 2.4e-7 in O, two ulp in lse).
"""
import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
import oracle
from exact_attention_12_amd import inputs
from gpu_util import TOL, errors, gather_rows, oracle_per_head, progress

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
MAP_DIFF = 1e-5  # largest |difference| of o and of finite lse with and without the block map


@pytest.fixture(autouse=True)
def _announce(request):
    progress("start " + request.node.nodeid)
    yield


def ext_inputs(cid, B, H, Hkv, Nq, Nk, d, dtype):
    q = inputs.normal(1000 * cid + 0, (B, H, Nq, d), 1.0, dtype)
    k = inputs.normal(1000 * cid + 1, (B, Hkv, Nk, d), 1.0, dtype)
    v = inputs.normal(1000 * cid + 2, (B, Hkv, Nk, d), 1.0, dtype)
    return q, k, v


def check(q, k, v, causal, window, mask, dev, label, rows=None, block_map=False):
    B, H, Nq, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d)))
    progress("fa_fwd_ext %s Nq=%d Nk=%d causal=%d window=%s mask=%s map=%d" % (
        label, Nq, k.shape[2], causal, window, None if mask is None else tuple(mask.shape),
        block_map))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    md = None if mask is None else mask.to(dev)
    o, lse = fa.forward_ext(qd, kd, vd, scale=scale, causal=causal, window=window, mask=md,
                            block_map=True if block_map else None)
    if block_map:
        o2, lse2 = fa.forward_ext(qd, kd, vd, scale=scale, causal=causal, window=window, mask=md)
        torch.cuda.synchronize()
        # the same rows see no key with and without the map
        assert torch.equal(torch.isneginf(lse), torch.isneginf(lse2)), label
        fin = torch.isfinite(lse2)
        dmax = (o - o2).abs().max().item() if o.numel() else 0.0
        lmax = (lse[fin] - lse2[fin]).abs().max().item() if fin.any() else 0.0
        progress("%s map vs no map: max|dO|=%.3g max|dlse|=%.3g" % (label, dmax, lmax))
        assert dmax <= MAP_DIFF and lmax <= MAP_DIFF, (label, dmax, lmax)
    torch.cuda.synchronize()
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    if rows is None:
        ro, rl = oracle.attention_ext(q, k, v, scale, causal, window, mask)
    else:
        # rows [B * H, R]: each head's own sampled rows; the mask here is one
        # [Nq, Nk] matrix broadcast over batch and heads
        ro, rl = oracle_per_head(oracle.attention_ext, q, k, v, rows, scale, causal, window, mask)
        og, lg = gather_rows(og, rows), gather_rows(lg, rows)
    empty = np.isneginf(rl)
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty])), label
    ok = ~empty
    assert np.all(np.isfinite(og[ok])) and np.all(np.isfinite(lg[ok])), label
    tol = TOL[q.dtype]
    omax, omean = errors(og[ok], ro[ok])
    lmax, _ = errors(lg[ok], rl[ok])
    progress("%s rows=%d empty=%d max|dO|=%.3g mean|dO|=%.3g max|dlse|=%.3g" % (
        label, ok.sum(), empty.sum(), omax, omean, lmax))
    assert omax <= tol["o_max"] and omean <= tol["o_mean"] and lmax <= tol["lse_max"], (
        label, omax, omean, lmax)


WINDOWS = [  # Nq, Nk, causal, window
    (100, 1000, True, (-1, -1)),    # chunked prefill: new rows at the end of a context
    (333, 333, True, (-1, -1)),     # square: fa_fwd's causal mask
    (300, 100, True, (-1, -1)),     # more queries than keys: the first 200 rows see nothing
    (1000, 1000, True, (128, -1)),  # causal sliding window
    (700, 700, False, (64, 64)),    # symmetric window
    (257, 513, False, (0, 0)),      # one key per row
    (190, 190, False, (-1, 30)),    # right window only
]


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("Nq,Nk,causal,window", WINDOWS)
def test_windows(gpu, fa_lib, dt, Nq, Nk, causal, window):
    d = 64 if dt == "f32" else 128
    q, k, v = ext_inputs(60, 1, 4, 2, Nq, Nk, d, DT[dt])
    check(q, k, v, causal, window, None, gpu, "%s %s" % (dt, window))


MASKS = [  # mask shape prefix, Nq, Nk, causal, window, density
    ((), 200, 301, False, (-1, -1), 0.5),   # broadcast, Nk not a multiple of 4
    ((4,), 129, 256, False, (-1, -1), 0.3),  # per head
    ((2, 1), 150, 150, True, (-1, -1), 0.7),  # per batch, with causal
    ((2, 4), 64, 640, False, (100, 50), 0.9),  # per (b, h), with a window
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("prefix,Nq,Nk,causal,window,density", MASKS)
def test_boolean_masks(gpu, fa_lib, dt, prefix, Nq, Nk, causal, window, density):
    d = 128 if dt == "bf16" else 64
    q, k, v = ext_inputs(61, 2, 4, 4, Nq, Nk, d, DT[dt])
    g = np.random.default_rng(62 + Nq)
    m = torch.from_numpy(g.random(prefix + (Nq, Nk)) < density)
    m[..., 5, :] = False  # a row with no admissible key
    if len(prefix) == 0:
        m[:, 64:128] = False  # a fully masked key tile
    check(q, k, v, causal, window, m, gpu, "%s mask%s" % (dt, prefix))


def test_tril_mask_equals_causal(gpu, fa_lib):
    """The pages' example: attn_mask = tril(ones) gives the causal result."""
    q, k, v = ext_inputs(63, 1, 2, 2, 300, 300, 128, torch.bfloat16)
    m = torch.ones(300, 300, dtype=torch.bool).tril()
    dev = gpu
    a = fa.forward_ext(q.to(dev), k.to(dev), v.to(dev), causal=False, mask=m.to(dev))
    b = fa.forward(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    assert (a[0] - b[0]).abs().max().item() <= 1e-2 and (a[1] - b[1]).abs().max().item() <= 1e-3
    check(q, k, v, False, (-1, -1), m, dev, "tril")


def test_headline_sliding_window_sampled(gpu, fa_lib):
    cfg = inputs.FWD_CAUSAL_N8192
    q, k, v = inputs.fwd_inputs(cfg)
    rows = inputs.sample_rows_per_head(cfg.N, cfg.B * cfg.H, 256, seed=1000 * cfg.cid + 5)
    check(q, k, v, True, (1024, -1), None, gpu, "B2 H32 N8192 window 1024", rows=rows)


def test_headline_boolean_mask_sampled(gpu, fa_lib):
    cfg = inputs.FWD_CAUSAL_N8192
    q, k, v = inputs.fwd_inputs(cfg)
    N = cfg.N
    # block-sparse causal pattern: each 64-key block is kept with probability 1/2
    keep = torch.from_numpy(np.random.default_rng(64).random((N // 128, N // 64)) < 0.5)
    m = keep.repeat_interleave(128, 0).repeat_interleave(64, 1) & torch.ones(N, N, dtype=torch.bool).tril()
    m[:, 0] = True
    rows = inputs.sample_rows_per_head(N, cfg.B * cfg.H, 256, seed=1000 * cfg.cid + 5)
    check(q, k, v, False, (-1, -1), m, gpu, "B2 H32 N8192 block-sparse mask", rows=rows)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("use_map", [False, True])
def test_zero_scale_rows_without_keys(gpu, fa_lib, dt, use_map):
    # scale 0: every visible key has probability 1/n, so o is the mean of the
    # visible values and lse = ln n; rows that see no key (fully masked rows,
    # and the first Nq - Nk rows of a bottom-right causal rectangle) must
    # still give o = 0 and lse = -inf exactly, not NaN from 0 * (-inf)
    Nq, Nk = 300, 200
    d = 128 if dt == "bf16" else 64
    q, k, v = ext_inputs(67, 1, 2, 2, Nq, Nk, d, DT[dt])
    m = torch.from_numpy(np.random.default_rng(68).random((Nq, Nk)) < 0.6)
    m[150:160] = False
    progress("fa_fwd_ext scale 0 %s map=%d" % (dt, use_map))
    o, lse = fa.forward_ext(q.to(gpu), k.to(gpu), v.to(gpu), scale=0.0, causal=True, mask=m.to(gpu),
                            block_map=True if use_map else None)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_ext(q, k, v, 0.0, True, (-1, -1), m)
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    empty = np.isneginf(rl)
    assert empty[:, :, :100].all() and empty[:, :, 150:160].all()
    assert not np.isnan(lg).any(), "NaN lse"
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty]))
    tol = TOL[q.dtype]
    assert np.abs(og[~empty] - ro[~empty]).max() <= tol["o_max"]
    assert np.abs(lg[~empty] - rl[~empty]).max() <= tol["lse_max"]


# ---- block map of the mask --------------------------------------------------

def map_words(mp):
    """uint32 view of a map tensor, shaped as the oracle's."""
    return mp.cpu().numpy().view(np.uint32)


MAP_CASES = [  # mask prefix, Nq, Nk, kind
    ((), 1, 1, "ones"),
    ((), 300, 5000, "sparse"),       # 79 key blocks over 3 words
    ((), 129, 2049, "tril"),         # ragged query and key blocks
    ((3,), 1000, 1000, "blocks"),    # per head
    ((2, 1), 257, 700, "zeros"),     # per batch
    ((2, 3), 640, 130, "dense"),     # per (b, h)
]


def make_mask(prefix, Nq, Nk, kind, seed):
    g = np.random.default_rng(seed)
    shape = prefix + (Nq, Nk)
    if kind == "ones":
        m = np.ones(shape, bool)
    elif kind == "zeros":
        m = np.zeros(shape, bool)
    elif kind == "sparse":
        m = g.random(shape) < 0.0005
    elif kind == "tril":
        m = np.broadcast_to(np.tril(np.ones((Nq, Nk), bool), Nk - Nq), shape).copy()
    elif kind == "dense":
        m = g.random(shape) < 0.999
    else:  # "blocks": whole 128 x 64 blocks kept at random, then some single bytes flipped
        keep = g.random(prefix + ((Nq + 127) // 128, (Nk + 63) // 64)) < 0.4
        m = np.repeat(np.repeat(keep, 128, -2), 64, -1)[..., :Nq, :Nk].copy()
        flip = g.random(shape) < 0.0002
        m ^= flip
    return torch.from_numpy(m)


@pytest.mark.parametrize("prefix,Nq,Nk,kind", MAP_CASES)
def test_mask_block_map_exact(gpu, fa_lib, prefix, Nq, Nk, kind):
    m = make_mask(prefix, Nq, Nk, kind, 70 + Nq)
    B, H = 2, 3
    progress("fa_mask_blocks %s Nq=%d Nk=%d %s" % (prefix, Nq, Nk, kind))
    mp = fa.mask_block_map(m.to(gpu), B, H, Nq, Nk)
    torch.cuda.synchronize()
    ref = oracle.mask_blocks(m)
    assert mp.numel() == ref.size
    assert (map_words(mp).reshape(ref.shape) == ref).all(), kind


def test_mask_block_map_ignores_row_padding(gpu, fa_lib):
    """Bytes between Nk and the row stride are not part of the mask."""
    Nq, Nk, ldm = 200, 70, 96
    m = make_mask((), Nq, Nk, "blocks", 75)
    buf = torch.full((Nq, ldm), 255, dtype=torch.uint8)
    buf[:, :Nk] = m.to(torch.uint8) * 3
    bd = buf.to(gpu)
    words = fa.fa_mask_blocks_words(1, 1, Nq, Nk, 0, 0)
    mp = torch.full((words,), -1, dtype=torch.int32, device=gpu)
    fa.fa_mask_blocks(bd, 1, 1, Nq, Nk, 0, 0, ldm, mp)
    torch.cuda.synchronize()
    ref = oracle.mask_blocks(m)
    assert (map_words(mp).reshape(ref.shape) == ref).all()


MAPPED = [  # dtype, prefix, Nq, Nk, causal, window, kind
    ("bf16", (), 1000, 1000, True, (-1, -1), "blocks"),
    ("f16", (4,), 333, 1200, False, (-1, -1), "blocks"),
    ("f32", (), 700, 700, True, (-1, -1), "blocks"),          # 32-key tiles: two per block
    ("bf16", (2, 1), 300, 5000, False, (-1, -1), "sparse"),   # long runs of empty blocks
    ("bf16", (), 500, 2100, False, (300, 200), "blocks"),     # with a window
    ("f32", (2, 4), 129, 2049, False, (-1, -1), "tril"),
    ("bf16", (), 640, 640, False, (-1, -1), "zeros"),         # nothing visible
    ("f16", (), 384, 384, False, (-1, -1), "ones"),           # everything visible
]


@pytest.mark.parametrize("dt,prefix,Nq,Nk,causal,window,kind", MAPPED)
def test_boolean_masks_with_block_map(gpu, fa_lib, dt, prefix, Nq, Nk, causal, window, kind):
    d = 64 if dt == "f32" else 128
    q, k, v = ext_inputs(66, 2, 4, 2, Nq, Nk, d, DT[dt])
    m = make_mask(prefix, Nq, Nk, kind, 80 + Nq)
    check(q, k, v, causal, window, m, gpu, "%s map %s %s" % (dt, kind, prefix), block_map=True)


def test_headline_block_sparse_mask_with_map_sampled(gpu, fa_lib):
    cfg = inputs.FWD_CAUSAL_N8192
    q, k, v = inputs.fwd_inputs(cfg)
    N = cfg.N
    keep = torch.from_numpy(np.random.default_rng(64).random((N // 128, N // 64)) < 0.5)
    m = keep.repeat_interleave(128, 0).repeat_interleave(64, 1) & torch.ones(N, N, dtype=torch.bool).tril()
    m[:, 0] = True
    rows = inputs.sample_rows_per_head(N, cfg.B * cfg.H, 256, seed=1000 * cfg.cid + 5)
    check(q, k, v, False, (-1, -1), m, gpu, "B2 H32 N8192 block-sparse mask, map", rows=rows,
          block_map=True)
