"""Pins of the block-scaled FP8 (E4M3) quantisation in the oracle.

The encoder and decoder are pinned to torch's float8_e4m3fn conversion (a
library implementation of the OCP E4M3FN format, round to nearest even) over
every code and over dense sweeps of values; the block exponent to numpy's
frexp; the codes to torch's conversion of the exactly scaled values; the
dequantised values to the format's error bound; and the V tile layout to the
row-major layout by a transpose.
"""
import numpy as np
import pytest
import torch

import oracle

F8 = torch.float8_e4m3fn


def torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(F8).view(torch.uint8).numpy()


def test_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(F8).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_encode_every_code_and_midpoint():
    """Every finite code round-trips; midpoints between neighbours round to even."""
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals)]
    assert np.array_equal(oracle.e4m3_encode(fin), torch_codes(fin))
    pos = np.unique(fin[fin >= 0])
    mid = (pos[:-1] + pos[1:]) / 2
    assert np.array_equal(oracle.e4m3_encode(mid), torch_codes(mid))
    assert np.array_equal(oracle.e4m3_encode(-mid), torch_codes(-mid))


def test_encode_dense_sweep():
    """All fp16 values of magnitude <= 448 and random doubles spanning the range."""
    h = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    h = h[np.isfinite(h) & (np.abs(h) <= 448)]
    assert np.array_equal(oracle.e4m3_encode(h), torch_codes(h))
    r = np.random.default_rng(0)
    x = r.uniform(-1, 1, 200000) * np.exp2(r.uniform(-14, 8.8, 200000))
    assert np.array_equal(oracle.e4m3_encode(x), torch_codes(x))


def blocks(seed, shape, dtype):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))
    # spread the magnitudes over many binades, block by block
    N = shape[2]
    f = torch.from_numpy(np.exp2(np.random.default_rng(seed + 1).integers(-20, 12, size=(shape[0], shape[1], (N + 127) // 128)))).float()
    f = f.repeat_interleave(128, dim=2)[:, :, :N, None]
    return (x * f).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_block_exponents_and_codes(dtype):
    B, H, N, d = 2, 3, 300, 16
    x = blocks(3, (B, H, N, d), dtype)
    codes, exps = oracle.quant_fp8(x, 0)
    xa = x.double().numpy()
    for b in range(B):
        for h in range(H):
            for blk in range((N + 127) // 128):
                sl = xa[b, h, blk * 128:(blk + 1) * 128]
                amax = np.abs(sl).max()
                e = int(np.frexp(amax)[1]) - 1 - 7
                assert exps[b, h, blk] == e
                assert 128 <= amax * 2.0 ** -e < 256
                assert np.array_equal(codes[b, h, blk * 128:(blk + 1) * 128], torch_codes(np.ldexp(sl, -e)))


def test_zero_block_and_tiny_values():
    x = torch.zeros(1, 1, 200, 8)
    x[0, 0, 150:] = 2.0 ** -140  # fp32 subnormal-range block
    x[0, 0, 150, 0] = 3 * 2.0 ** -141
    codes, exps = oracle.quant_fp8(x, 0)
    assert exps[0, 0, 0] == 0 and np.all(codes[0, 0, :128] == 0)
    assert exps[0, 0, 1] == -140 - 7
    deq = oracle.dequant_fp8(codes, exps, 1, 1, 200, 8, 0)
    assert np.array_equal(deq, x.double().numpy())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dequantised_error_bound(dtype):
    """|value - x| <= 2^-4 |x| in the normal range, <= 2^(e-10) below it."""
    B, H, N, d = 1, 2, 257, 32
    x = blocks(5, (B, H, N, d), dtype)
    codes, exps = oracle.quant_fp8(x, 0)
    deq = oracle.dequant_fp8(codes, exps, B, H, N, d, 0)
    xa = x.double().numpy()
    e = np.broadcast_to(np.repeat(exps, 128, axis=2)[:, :, :N, None], xa.shape).astype(np.float64)
    err = np.abs(deq - xa)
    normal = np.abs(xa) >= np.exp2(e - 6)
    assert np.all(err[normal] <= np.abs(xa[normal]) * 2.0 ** -4)
    assert np.all(err[~normal] <= np.exp2(e - 10)[~normal])
    assert np.abs(deq).max() > 0


def test_representable_inputs_round_trip():
    r = np.random.default_rng(7)
    # codes of magnitude < 256 (exponent field <= 14), any sign and mantissa
    sign = r.integers(0, 2, size=(1, 2, 130, 8)) << 7
    ef = r.integers(0, 15, size=(1, 2, 130, 8)) << 3
    codes = (sign | ef | r.integers(0, 8, size=(1, 2, 130, 8))).astype(np.uint8)
    v = oracle.e4m3_decode(codes)
    # force each block's largest magnitude into [128, 256) so e = 0 and values round-trip
    v[:, :, :, 0] = 192.0  # an E4M3 value in [128, 256)
    x = torch.from_numpy(v)
    c2, e2 = oracle.quant_fp8(x, 0)
    assert np.all(e2 == 0)
    assert np.array_equal(oracle.dequant_fp8(c2, e2, 1, 2, 130, 8, 0), v)


@pytest.mark.parametrize("N", [64, 100, 129])
def test_tile_layout_is_transposed_row_layout(N):
    B, H, d = 2, 2, 16
    x = blocks(11, (B, H, N, d), torch.bfloat16)
    c0, e0 = oracle.quant_fp8(x, 0)
    c1, e1 = oracle.quant_fp8(x, 1)
    assert np.array_equal(e0, e1)
    T = (N + 63) // 64
    pad = np.zeros((B, H, T * 64, d), dtype=np.uint8)
    pad[:, :, :N] = c0
    assert np.array_equal(c1, pad.reshape(B, H, T, 64, d).transpose(0, 1, 2, 4, 3))
    assert np.array_equal(oracle.dequant_fp8(c1, e1, B, H, N, d, 1),
                          oracle.dequant_fp8(c0, e0, B, H, N, d, 0))
