"""Pins of the oracle's block map of a boolean mask (oracle.mask_blocks).

The map summarises the boolean attn_mask of "FlashAttention: GPU 메모리
계층을 활용한 어텐션 최적화 분석" (youngju.dev), section 11.3, per block of
128 query rows x 64 keys.  Its definition is plain; the pins fix it against
closed forms (constant masks, the lower-triangular mask), single-byte
perturbations that must flip exactly one bit, ragged edges, the broadcast
layout, and a block-by-block reduction with numpy on random masks.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def bits(words, nbits):
    """Bits 0..nbits-1 of a little-endian word array as a bool vector."""
    w = np.asarray(words, dtype=np.uint64)
    return np.array([(int(w[i // 32]) >> (i % 32)) & 1 for i in range(nbits)], dtype=bool)


def as_blocks(mp, Nq, Nk):
    """(any, full) bool arrays [Bm, Hm, nqb, nkb] decoded from a map."""
    Bm, Hm, nqb, _, nkw = mp.shape
    nkb = (Nk + 63) // 64
    anyb = np.zeros((Bm, Hm, nqb, nkb), bool)
    full = np.zeros((Bm, Hm, nqb, nkb), bool)
    for b in range(Bm):
        for h in range(Hm):
            for qb in range(nqb):
                anyb[b, h, qb] = bits(mp[b, h, qb, 0], nkb)
                full[b, h, qb] = bits(mp[b, h, qb, 1], nkb)
    return anyb, full


def test_shape_and_zero_mask():
    mp = oracle.mask_blocks(np.zeros((300, 5000), np.uint8))
    assert mp.shape == (1, 1, 3, 2, 3)
    assert not mp.any()


def test_ones_mask_ragged_edges():
    # 79 key blocks (the last one holds keys 4992..4999 only); padding never counts
    mp = oracle.mask_blocks(np.ones((300, 5000), bool))
    for qb in range(3):
        for half in range(2):
            assert list(mp[0, 0, qb, half]) == [0xFFFFFFFF, 0xFFFFFFFF, (1 << 15) - 1]


@pytest.mark.parametrize("N", [300, 777, 1024])
def test_lower_triangular_closed_form(N):
    # row i sees keys j <= i: block (qb, kb) has a visible pair iff its first
    # key is <= its last row, and no masked pair iff its last key is <= its
    # first row
    anyb, full = as_blocks(oracle.mask_blocks(np.tril(np.ones((N, N), np.uint8))), N, N)
    for qb in range(anyb.shape[2]):
        first_row, last_row = qb * 128, min(qb * 128 + 127, N - 1)
        for kb in range(anyb.shape[3]):
            first_key, last_key = kb * 64, min(kb * 64 + 63, N - 1)
            assert anyb[0, 0, qb, kb] == (first_key <= last_row), (qb, kb)
            assert full[0, 0, qb, kb] == (last_key <= first_row), (qb, kb)


def test_single_visible_byte_sets_one_bit():
    rng = np.random.default_rng(1)
    Nq, Nk = 400, 3000
    for _ in range(6):
        i, j = int(rng.integers(Nq)), int(rng.integers(Nk))
        m = np.zeros((Nq, Nk), np.uint8)
        m[i, j] = 200
        anyb, full = as_blocks(oracle.mask_blocks(m), Nq, Nk)
        want = np.zeros_like(anyb)
        want[0, 0, i // 128, j // 64] = True
        assert (anyb == want).all(), (i, j)
        assert not full.any()


def test_single_masked_byte_clears_one_bit():
    rng = np.random.default_rng(2)
    Nq, Nk = 260, 2100
    for _ in range(6):
        i, j = int(rng.integers(Nq)), int(rng.integers(Nk))
        m = np.ones((Nq, Nk), np.uint8)
        m[i, j] = 0
        anyb, full = as_blocks(oracle.mask_blocks(m), Nq, Nk)
        assert anyb.all()
        want = np.ones_like(full)
        want[0, 0, i // 128, j // 64] = False
        assert (full == want).all(), (i, j)


@pytest.mark.parametrize("i,j", [(0, 0), (127, 0), (0, 63), (127, 63), (128, 64), (255, 127),
                                 (128, 63), (127, 64), (299, 1999)])
def test_block_corners(i, j):
    # the first and last row and key of a block belong to it, and not to its
    # neighbours
    Nq, Nk = 300, 2000
    m = np.zeros((Nq, Nk), np.uint8)
    m[i, j] = 1
    anyb, full = as_blocks(oracle.mask_blocks(m), Nq, Nk)
    want = np.zeros_like(anyb)
    want[0, 0, i // 128, j // 64] = True
    assert (anyb == want).all() and not full.any()
    anyb, full = as_blocks(oracle.mask_blocks(1 - m), Nq, Nk)
    assert anyb.all() and (full == ~want).all()


def test_tiny_block_is_full_or_empty():
    assert oracle.mask_blocks(np.ones((1, 1), np.uint8)).ravel().tolist() == [1, 1]
    assert oracle.mask_blocks(np.zeros((1, 1), np.uint8)).ravel().tolist() == [0, 0]


def test_broadcast_slices_are_independent():
    rng = np.random.default_rng(3)
    m = rng.random((2, 3, 200, 700)) < 0.02
    mp = oracle.mask_blocks(m)
    assert mp.shape == (2, 3, 2, 2, 1)
    for b in range(2):
        for h in range(3):
            assert (mp[b, h] == oracle.mask_blocks(m[b, h])[0, 0]).all()


@pytest.mark.parametrize("shape,p", [((333, 1500), 0.001), ((128, 64), 0.5), ((500, 2200), 0.9995)])
def test_numpy_block_reduction(shape, p):
    rng = np.random.default_rng(4)
    m = rng.random(shape) < p
    Nq, Nk = shape
    anyb, full = as_blocks(oracle.mask_blocks(m), Nq, Nk)
    nqb, nkb = anyb.shape[2:]
    # numpy slices stop at the array's edge: a ragged block holds only the
    # rows and keys inside the range
    for qb in range(nqb):
        for kb in range(nkb):
            blk = m[qb * 128:(qb + 1) * 128, kb * 64:(kb + 1) * 64]
            assert anyb[0, 0, qb, kb] == blk.any()
            assert full[0, 0, qb, kb] == blk.all()
