"""GPU parity of fa_fwd_paged (chunked prefill over the paged cache) against
the fp64 oracle, through the C ABI.

The caches come from the decode generator: unused pool blocks, unused table
entries and the slots past each context's end are NaN, so a read outside a
context poisons the result.  Rows that see no token must return o = 0 and
lse = -inf exactly; the others meet the forward's bar for their type.
Contexts shorter than Nq, ragged block tails, grouped kv heads, causal or
not, bf16 and fp16; the benchmark's workload on sampled sequences.
"""
import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
import oracle
from exact_attention_12_amd import inputs
from gpu_util import TOL, errors, progress

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    progress("start " + request.node.nodeid)
    yield


def run_case(dev, cfg, ctx, Nq, causal, label, seqs=None):
    d = inputs.decode_inputs(cfg, context_lens=ctx)
    q = inputs.prefill_queries(cfg, Nq)
    scale = float(np.float32(cfg.scale))
    progress("fa_fwd_paged %s S=%d H=%d Hkv=%d Nq=%d ctx=%s causal=%d" % (
        label, cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, Nq, list(ctx)[:8], causal))
    o, lse = fa.forward_paged(q.to(dev), d["k_cache"].to(dev), d["v_cache"].to(dev),
                              d["block_tables"].to(dev), d["context_lens"].to(dev), scale=scale,
                              causal=causal)
    torch.cuda.synchronize()
    sel = list(range(cfg.num_seqs)) if seqs is None else list(seqs)
    ro, rl = oracle.paged_prefill(q[sel], d["k_cache"], d["v_cache"], d["block_tables"][sel],
                                  d["context_lens"][sel], scale, causal)
    og, lg = o.cpu().double().numpy()[sel], lse.cpu().double().numpy()[sel]
    empty = np.isneginf(rl)
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty])), label
    ok = ~empty
    assert np.all(np.isfinite(og[ok])) and np.all(np.isfinite(lg[ok])), label
    tol = TOL[cfg.dtype]
    omax, omean = errors(og[ok], ro[ok])
    lmax, _ = errors(lg[ok], rl[ok])
    progress("%s rows=%d empty=%d max|dO|=%.3g mean|dO|=%.3g max|dlse|=%.3g" % (
        label, ok.sum(), empty.sum(), omax, omean, lmax))
    assert omax <= tol["o_max"] and omean <= tol["o_mean"] and lmax <= tol["lse_max"], (
        label, omax, omean, lmax)
    return o, lse


CASES = [  # Hkv, Nq, context lengths
    (4, 1, [1, 16, 17, 300]),
    (4, 17, [17, 40, 129, 500]),
    (2, 128, [100, 128, 129, 1000]),    # a context shorter than Nq: its first rows see nothing
    (1, 200, [0, 200, 777, 1024]),      # an empty context
    (2, 300, [301, 512, 1500, 2049]),
]


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hkv,Nq,ctx", CASES)
def test_paged_prefill(gpu, fa_lib, dt, causal, Hkv, Nq, ctx):
    cfg = inputs.DecodeConfig(cid=90, num_seqs=4, num_heads=4, num_kv_heads=Hkv, num_blocks=600,
                              ctx_lo=1, ctx_hi=max(ctx), dtype=dt)
    run_case(gpu, cfg, ctx, Nq, causal, "%s Hkv=%d Nq=%d" % (str(dt)[6:], Hkv, Nq))


def test_paged_prefill_deterministic(gpu, fa_lib):
    cfg = inputs.DecodeConfig(cid=91, num_seqs=3, num_heads=8, num_kv_heads=2, num_blocks=300,
                              ctx_lo=1, ctx_hi=1200, dtype=torch.bfloat16)
    d = inputs.decode_inputs(cfg, context_lens=[300, 700, 1200])
    q = inputs.prefill_queries(cfg, 256).to(gpu)
    args = [d[n].to(gpu) for n in ("k_cache", "v_cache", "block_tables", "context_lens")]
    a = fa.forward_paged(q, *args)
    b = fa.forward_paged(q, *args)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_paged_prefill_equals_contiguous_ext(gpu, fa_lib):
    """The same attention through fa_fwd_ext on K, V gathered to contiguous rows."""
    cfg = inputs.DecodeConfig(cid=92, num_seqs=1, num_heads=4, num_kv_heads=4, num_blocks=100,
                              ctx_lo=1, ctx_hi=1000, dtype=torch.bfloat16)
    d = inputs.decode_inputs(cfg, context_lens=[1000])
    q = inputs.prefill_queries(cfg, 333)
    kc, vc, bt = d["k_cache"], d["v_cache"], d["block_tables"][0]
    nb = (1000 + 15) // 16
    K = kc[bt[:nb].long()].permute(1, 0, 3, 2, 4).reshape(4, nb * 16, 128)[:, :1000]
    V = vc[bt[:nb].long()].permute(1, 0, 3, 2).reshape(4, nb * 16, 128)[:, :1000]
    o1, l1 = fa.forward_paged(q.to(gpu), kc.to(gpu), vc.to(gpu), d["block_tables"].to(gpu),
                              d["context_lens"].to(gpu))
    o2, l2 = fa.forward_ext(q.to(gpu), K[None].contiguous().to(gpu), V[None].contiguous().to(gpu),
                            causal=True)
    torch.cuda.synchronize()
    # same tiles, same arithmetic order
    assert (o1 - o2).abs().max().item() <= 1e-5 and (l1 - l2).abs().max().item() <= 1e-5


def test_full_prefill_equals_square_causal_forward(gpu, fa_lib):
    """Nq = context length: the whole context is new, the mask is fa_fwd's square causal one."""
    n = 1000
    cfg = inputs.DecodeConfig(cid=93, num_seqs=2, num_heads=8, num_kv_heads=8, num_blocks=200,
                              ctx_lo=1, ctx_hi=n, dtype=torch.bfloat16)
    o1, l1 = run_case(gpu, cfg, [n, n], n, True, "full prefill")
    d = inputs.decode_inputs(cfg, context_lens=[n, n])
    q = inputs.prefill_queries(cfg, n)
    nb = (n + 15) // 16
    Ks, Vs = [], []
    for s in range(2):
        bt = d["block_tables"][s, :nb].long()
        Ks.append(d["k_cache"][bt].permute(1, 0, 3, 2, 4).reshape(8, nb * 16, 128)[:, :n])
        Vs.append(d["v_cache"][bt].permute(1, 0, 3, 2).reshape(8, nb * 16, 128)[:, :n])
    o2, l2 = fa.forward(q.to(gpu), torch.stack(Ks).contiguous().to(gpu), torch.stack(Vs).contiguous().to(gpu),
                        causal=True)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 1e-5 and (l1 - l2).abs().max().item() <= 1e-5


def test_multi_query_prefill(gpu, fa_lib):
    cfg = inputs.DecodeConfig(cid=95, num_seqs=3, num_heads=32, num_kv_heads=1, num_blocks=300,
                              ctx_lo=1, ctx_hi=1500, dtype=torch.float16)
    run_case(gpu, cfg, [129, 700, 1500], 129, True, "multi-query 32/1")


def test_headline_paged_prefill_sampled(gpu, fa_lib):
    cfg = inputs.PREFILL_CONFIG
    rng = np.random.default_rng(1000 * cfg.cid + 3)
    ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=cfg.num_seqs)
    run_case(gpu, cfg, ctx, inputs.PREFILL_NQ, True, "16 seqs x 512 new tokens", seqs=[0, 7, 15])


def test_prefill_equal_context_lengths(gpu, fa_lib):
    # workgroups go longest sequence first; equal lengths must still give every
    # (sequence, head, query tile) exactly one workgroup
    cfg = inputs.DecodeConfig(cid=96, num_seqs=8, num_heads=4, num_kv_heads=2, num_blocks=300,
                              ctx_lo=1, ctx_hi=1000, dtype=torch.bfloat16)
    run_case(gpu, cfg, [300, 300, 17, 300, 17, 1000, 1000, 20], 20, True, "equal lengths")


@pytest.mark.parametrize("S,Hkv", [(64, 1), (72, 1), (70, 2)])
def test_prefill_many_sequences(gpu, fa_lib, S, Hkv):
    # as many sequences as one wave ranks (64), and more (kept in order), with
    # and without 8 | S * Hkv
    cfg = inputs.DecodeConfig(cid=97, num_seqs=S, num_heads=2, num_kv_heads=Hkv, num_blocks=1200,
                              ctx_lo=1, ctx_hi=200, dtype=torch.float16)
    ctx = np.random.default_rng(97 + S).integers(1, 201, size=S)
    run_case(gpu, cfg, ctx, 5, True, "S=%d Hkv=%d" % (S, Hkv))
