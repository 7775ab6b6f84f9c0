"""GPU parity of fa_bwd (dQ, dK, dV) against the fp64 backward oracle, through the C ABI.

The backward pass reads the forward pass's o and lse, so every case runs
fa_fwd (or fa_fwd_gqa) and then fa_bwd on the device, and compares the three
gradients with the oracle's, computed from the same rounded q, k, v, dO.
Full comparison on ragged shapes that span several tiles; at the headline
size (B=2, H=32, N=8192, d=128, causal, the configuration the benchmark
times) the whole backward pass runs and sampled heads, rows and keys are
compared.
"""
import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
import oracle
from exact_attention_12_amd import inputs
from gpu_util import BWD_TOL, assert_bwd_close, progress

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(autouse=True)
def _announce(request):
    progress("start " + request.node.nodeid)
    yield


def run_bwd(q, k, v, dout, scale, causal, dev):
    qd, kd, vd, gd = q.to(dev), k.to(dev), v.to(dev), dout.to(dev)
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, gd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check_full(cfg, dev, label):
    progress("fa_bwd %s B=%d H=%d Hkv=%d N=%d d=%d causal=%d" % (
        label, cfg.B, cfg.H, cfg.kv_heads, cfg.N, cfg.d, cfg.causal))
    q, k, v = inputs.fwd_inputs(cfg)
    dout = inputs.bwd_dout(cfg)
    scale = float(np.float32(cfg.scale))
    dq, dk, dv = run_bwd(q, k, v, dout, scale, cfg.causal, dev)
    ref = oracle.attention_bwd(q, k, v, dout, scale, cfg.causal)
    assert_bwd_close(dq.double().numpy(), dk.double().numpy(), dv.double().numpy(), ref,
                     cfg.dtype, label)


SHAPES = [  # (dtype, d, B, H, Hkv, N, causal)
    ("bf16", 128, 1, 2, 2, 333, True),
    ("bf16", 128, 1, 2, 2, 333, False),
    ("f16", 128, 2, 2, 2, 200, True),
    ("bf16", 64, 2, 3, 3, 257, True),
    ("f16", 64, 1, 2, 2, 191, False),
    ("bf16", 128, 1, 1, 1, 1, True),
    ("bf16", 128, 1, 1, 1, 1, False),
    ("f16", 64, 1, 2, 2, 31, True),
    ("bf16", 128, 1, 2, 2, 64, True),
    ("bf16", 128, 1, 2, 2, 65, False),
    ("bf16", 128, 1, 1, 1, 512, True),
    ("f16", 128, 1, 1, 1, 384, False),
]


@pytest.mark.parametrize("dt,d,B,H,Hkv,N,causal", SHAPES)
def test_shapes(gpu, fa_lib, dt, d, B, H, Hkv, N, causal):
    cfg = inputs.FwdConfig(80, B, H, N, d, DT[dt], causal, 1.0, "", Hkv=Hkv)
    check_full(cfg, gpu, "%s d%d B%d H%d N%d causal%d" % (dt, d, B, H, N, causal))


@pytest.mark.parametrize("dt,d,H,Hkv,causal", [
    ("bf16", 128, 8, 2, True), ("bf16", 128, 8, 1, False), ("f16", 64, 6, 3, True),
    ("f16", 128, 4, 2, False)])
def test_grouped_kv_heads(gpu, fa_lib, dt, d, H, Hkv, causal):
    cfg = inputs.FwdConfig(81, 2, H, 333, d, DT[dt], causal, 1.0, "", Hkv=Hkv)
    check_full(cfg, gpu, "gqa %s d%d H%d Hkv%d causal%d" % (dt, d, H, Hkv, causal))


def test_scale_zero(gpu, fa_lib):
    """scale 0: uniform P, dQ = dK = 0 exactly."""
    cfg = inputs.FwdConfig(82, 1, 2, 150, 64, torch.bfloat16, True, 1.0, "")
    q, k, v = inputs.fwd_inputs(cfg)
    dout = inputs.bwd_dout(cfg)
    dq, dk, dv = run_bwd(q, k, v, dout, 0.0, True, gpu)
    assert torch.all(dq == 0) and torch.all(dk == 0)
    ref = oracle.attention_bwd(q, k, v, dout, 0.0, True)
    assert_bwd_close(dq.double().numpy(), dk.double().numpy(), dv.double().numpy(), ref,
                     cfg.dtype, "scale0")


def test_deterministic(gpu, fa_lib):
    cfg = inputs.FwdConfig(83, 1, 4, 700, 128, torch.bfloat16, True, 1.0, "", Hkv=2)
    q, k, v = inputs.fwd_inputs(cfg)
    dout = inputs.bwd_dout(cfg)
    a = run_bwd(q, k, v, dout, cfg.scale, True, gpu)
    b = run_bwd(q, k, v, dout, cfg.scale, True, gpu)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def check_sampled(cfg, dev, heads):
    """Whole backward pass at cfg's size on the device; the oracle on the
    kv-head groups in `heads` ((b, kv head) pairs), 256 sampled rows (dQ) and
    256 sampled keys (dK, dV) of each group's own."""
    progress("fa_bwd sampled %s" % cfg.name)
    q, k, v = inputs.fwd_inputs(cfg)
    dout = inputs.bwd_dout(cfg)
    scale = float(np.float32(cfg.scale))
    dq, dk, dv = run_bwd(q, k, v, dout, scale, cfg.causal, dev)
    # rows and keys drawn independently for every (b, kv head) group,
    # stratified over the 128-row tiles
    all_rows = inputs.sample_rows_per_head(cfg.N, cfg.B * cfg.kv_heads, 256, seed=1000 * cfg.cid + 5)
    all_keys = inputs.sample_rows_per_head(cfg.N, cfg.B * cfg.kv_heads, 256, seed=1000 * cfg.cid + 8)
    G = cfg.H // cfg.kv_heads
    for b, g in heads:
        rows, keys = all_rows[b * cfg.kv_heads + g], all_keys[b * cfg.kv_heads + g]
        hs = slice(g * G, (g + 1) * G)
        sl = lambda t, s: t[b:b + 1, s].contiguous()
        ref = oracle.attention_bwd(sl(q, hs), sl(k, slice(g, g + 1)), sl(v, slice(g, g + 1)),
                                   sl(dout, hs), scale, cfg.causal, rows=rows, keys=keys)
        got_q = dq[b:b + 1, hs][:, :, rows].double().numpy()
        got_k = dk[b:b + 1, g:g + 1][:, :, keys].double().numpy()
        got_v = dv[b:b + 1, g:g + 1][:, :, keys].double().numpy()
        assert_bwd_close(got_q, got_k, got_v, ref, cfg.dtype, "%s b%d g%d" % (cfg.name, b, g))


def test_headline_sampled(gpu, fa_lib):
    check_sampled(inputs.FWD_CAUSAL_N8192, gpu, [(0, 0), (1, 31)])


def test_gqa_headline_sampled(gpu, fa_lib):
    check_sampled(inputs.FWD_GQA_CONFIG, gpu, [(1, 5)])
