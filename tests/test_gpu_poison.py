"""The LDS-poisoning debug build against the product build, through the C ABI.

libfa_poison.so is libfa.so compiled with FA_DEBUG_POISON: every kernel fills
its LDS with 0xff bytes (NaN as fp32, bf16 and fp16) before first use.  A
kernel that reads an LDS slot its launch never wrote -- a missing load, a
wrong stage, a pad row or a tail that was assumed to hold finite leftovers --
then produces NaN or a different value.  Each entry point runs on the same
seeded inputs through both libraries (small shapes with ragged tails and
several tiles); the outputs must be finite and bitwise equal.  The product
build's own agreement with the oracle is what the other GPU tests check.
"""
import contextlib
import os

import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
from exact_attention_12_amd import build as fa_build
from exact_attention_12_amd import inputs
from gpu_util import progress

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    progress("start " + request.node.nodeid)
    yield


@pytest.fixture(scope="module")
def poison_lib(fa_lib):
    if not os.path.exists(fa_build.LIB_POISON):
        raise RuntimeError("libfa_poison.so is not built: `python -m exact_attention_12_amd.build`")
    return fa.load_debug_library(fa_build.LIB_POISON)


@contextlib.contextmanager
def using(lib):
    saved = fa._LIB
    fa._LIB = lib
    try:
        yield
    finally:
        fa._LIB = saved


def both(fa_lib, poison_lib, fn):
    """fn() under the product library, then under the poisoning one; both results (tuples of tensors)."""
    with using(fa_lib):
        a = fn()
        torch.cuda.synchronize()
    with using(poison_lib):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def same(a, b, label):
    for i, (x, y) in enumerate(zip(a, b)):
        assert x.shape == y.shape
        if x.dtype.is_floating_point:
            assert torch.isfinite(y).all(), "%s output %d: non-finite values in the poisoned build" % (label, i)
        assert torch.equal(x, y), "%s output %d differs: max |d| %.3g" % (
            label, i, (x.double() - y.double()).abs().max().item())
    progress("%s: %d outputs bitwise equal" % (label, len(a)))


@pytest.mark.parametrize("dt,d,causal,N,H,Hkv", [
    ("bf16", 128, True, 333, 4, 2), ("bf16", 128, False, 200, 2, 2), ("f16", 64, True, 257, 2, 1),
    ("f32", 128, False, 97, 2, 2), ("f32", 64, True, 150, 2, 2)])
def test_forward(gpu, fa_lib, poison_lib, dt, d, causal, N, H, Hkv):
    dtype = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    cfg = inputs.FwdConfig(90, 1, H, N, d, dtype, causal, 1.0, "", Hkv=Hkv)
    q, k, v = (t.to(gpu) for t in inputs.fwd_inputs(cfg))
    a, b = both(fa_lib, poison_lib, lambda: fa.forward(q, k, v, causal=causal))
    same(a, b, "fa_fwd %s d%d causal%d N%d H%d Hkv%d" % (dt, d, causal, N, H, Hkv))


@pytest.mark.parametrize("map_first", [False, True])
def test_forward_ext_mask_window(gpu, fa_lib, poison_lib, map_first):
    cfg = inputs.FwdConfig(91, 1, 2, 300, 128, torch.bfloat16, False, 1.0, "")
    q, k, v = (t.to(gpu) for t in inputs.fwd_inputs(cfg))
    mask = (inputs.normal(92, (1, 1, 300, 300)) > -0.5).to(torch.uint8).to(gpu)
    mask[..., 128:256, 64:192] = 0  # empty blocks
    mask[..., :64, :] = 1           # full blocks
    a, b = both(fa_lib, poison_lib, lambda: fa.forward_ext(q, k, v, causal=True, window=(150, 10), mask=mask,
                                                           block_map=True if map_first else None))
    same(a, b, "fa_fwd_ext mask+window map=%d" % map_first)


def test_forward_ext_rectangular(gpu, fa_lib, poison_lib):
    qc = inputs.FwdConfig(93, 1, 2, 77, 64, torch.float16, False, 1.0, "")
    kc = inputs.FwdConfig(94, 1, 2, 301, 64, torch.float16, False, 1.0, "")
    q = inputs.fwd_inputs(qc)[0].to(gpu)
    _, k, v = (t.to(gpu) for t in inputs.fwd_inputs(kc))
    a, b = both(fa_lib, poison_lib, lambda: fa.forward_ext(q, k, v, causal=True))
    same(a, b, "fa_fwd_ext Nq77 Nk301 bottom-right causal")


def on(gpu, d):
    return {k_: (t.to(gpu) if torch.is_tensor(t) else t) for k_, t in d.items()}


def _decode_case(gpu, cid, Hkv):
    cfg = inputs.DecodeConfig(cid=cid, num_seqs=5, num_heads=8, num_kv_heads=Hkv, head_size=128, block_size=16,
                              num_blocks=200, ctx_lo=1, ctx_hi=700, dtype=torch.float16)
    d = inputs.decode_inputs(cfg)
    return cfg, on(gpu, d)


@pytest.mark.parametrize("Hkv", [8, 2])
def test_paged_decode(gpu, fa_lib, poison_lib, Hkv):
    cfg, d = _decode_case(gpu, 95, Hkv)
    maxctx = int(d["context_lens"].max())
    a, b = both(fa_lib, poison_lib, lambda: (fa.paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                                             d["context_lens"], maxctx, scale=cfg.scale),))
    same(a, b, "fa_paged_decode Hkv%d" % Hkv)


def test_paged_prefill(gpu, fa_lib, poison_lib):
    cfg = inputs.DecodeConfig(cid=96, num_seqs=3, num_heads=4, num_kv_heads=2, head_size=128, block_size=16,
                              num_blocks=200, ctx_lo=200, ctx_hi=600, dtype=torch.bfloat16)
    d = on(gpu, inputs.decode_inputs(cfg))
    q = inputs.prefill_queries(cfg, 70).to(gpu)
    a, b = both(fa_lib, poison_lib, lambda: fa.forward_paged(q, d["k_cache"], d["v_cache"], d["block_tables"],
                                                             d["context_lens"], scale=cfg.scale, causal=True))
    same(a, b, "fa_fwd_paged")


@pytest.mark.parametrize("dt,d,causal,N,Hkv", [("bf16", 128, True, 333, 2), ("f16", 64, False, 191, 1),
                                               ("bf16", 64, True, 64, 2)])
def test_backward(gpu, fa_lib, poison_lib, dt, d, causal, N, Hkv):
    dtype = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    cfg = inputs.FwdConfig(97, 1, 2, N, d, dtype, causal, 1.0, "", Hkv=Hkv)
    q, k, v = (t.to(gpu) for t in inputs.fwd_inputs(cfg))
    dout = inputs.bwd_dout(cfg).to(gpu)
    with using(fa_lib):
        o, lse = fa.forward(q, k, v, causal=causal)
    a, b = both(fa_lib, poison_lib, lambda: fa.backward(q, k, v, o, lse, dout, causal=causal))
    same(a, b, "fa_bwd %s d%d causal%d N%d Hkv%d" % (dt, d, causal, N, Hkv))


@pytest.mark.parametrize("causal", [True, False])
def test_fp8(gpu, fa_lib, poison_lib, causal):
    cfg = inputs.FwdConfig(98, 1, 2, 300, 128, torch.bfloat16, causal, 1.0, "")
    q, k, v = (t.to(gpu) for t in inputs.fwd_inputs(cfg))

    def run():
        q8, qe = fa.quant_fp8(q, 0)
        k8, ke = fa.quant_fp8(k, 0)
        v8, ve = fa.quant_fp8(v, 1)
        o, lse = fa.forward_fp8(q8, k8, v8, qe, ke, ve, 1, 2, 2, 300, 128, scale=float(np.float32(cfg.scale)),
                                causal=causal)
        return q8, qe, v8, ve, o, lse

    a, b = both(fa_lib, poison_lib, run)
    same(a, b, "fa_quant_fp8 + fa_fwd_fp8 causal%d" % causal)
