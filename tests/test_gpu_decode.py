"""GPU parity of fa_paged_decode against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
import oracle
from exact_attention_12_amd import inputs
from gpu_util import DECODE_TOL, errors, progress

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    progress("start " + request.node.nodeid)
    yield


def run_decode(d, cfg, dev, workspace=None):
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    out = fa.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                          t["context_lens"], t["max_context_len"],
                          scale=float(np.float32(cfg.scale)), workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu()


def check(d, cfg, dev, label):
    progress("fa_paged_decode %s S=%d H=%d Hkv=%d max_ctx=%d" % (
        label, cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, d["max_context_len"]))
    out = run_decode(d, cfg, dev)
    ref, _ = oracle.paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                 d["context_lens"], float(np.float32(cfg.scale)))
    got = out.double().numpy()
    assert np.all(np.isfinite(got)), label
    omax, omean = errors(got, ref)
    progress("%s max|dO|=%.3g mean|dO|=%.3g" % (label, omax, omean))
    assert omax <= DECODE_TOL["o_max"] and omean <= DECODE_TOL["o_mean"], (label, omax, omean)
    return out


def test_decode_64x32_full(gpu, fa_lib):
    cfg = inputs.DECODE_CONFIG
    check(inputs.decode_inputs(cfg), cfg, gpu, "64 seqs x 32 heads")


def test_decode_gqa_64x32_over_8_full(gpu, fa_lib):
    # the grouped-query decode as the benchmark runs it: 4 query heads per kv
    # head (one workgroup per kv head and partition), every row against the oracle
    cfg = inputs.DECODE_GQA_CONFIG
    check(inputs.decode_inputs(cfg), cfg, gpu, "64 seqs x 32 heads over 8 kv heads")


EDGE_CTX = [0, 1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1000, 2049, 4096]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("Hkv", [8, 2])
def test_edge_context_lengths(gpu, fa_lib, dt, Hkv):
    cfg = inputs.DecodeConfig(cid=90, num_seqs=len(EDGE_CTX), num_heads=8, num_kv_heads=Hkv,
                              num_blocks=1200, ctx_lo=0, ctx_hi=4096,
                              dtype=torch.float16 if dt == "f16" else torch.bfloat16)
    d = inputs.decode_inputs(cfg, context_lens=EDGE_CTX)
    out = check(d, cfg, gpu, "edge %s Hkv%d" % (dt, Hkv))
    assert torch.all(out[0] == 0)  # empty context


# more than 16 partitions of 256 tokens: the merge combines its chunks of 16
# partitions online (4097 -> 17 partitions, 8192 -> 32, 8193 -> 33, 65553 -> 257)
LONG_CTX = [4097, 4352, 8191, 8192, 8193, 20000, 65553]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("Hkv", [4, 2])
def test_long_contexts_many_partitions(gpu, fa_lib, dt, Hkv):
    cfg = inputs.DecodeConfig(cid=94, num_seqs=len(LONG_CTX), num_heads=4, num_kv_heads=Hkv,
                              num_blocks=7600, ctx_lo=1, ctx_hi=max(LONG_CTX),
                              dtype=torch.float16 if dt == "f16" else torch.bfloat16)
    d = inputs.decode_inputs(cfg, context_lens=LONG_CTX)
    check(d, cfg, gpu, "long contexts %s Hkv%d" % (dt, Hkv))


@pytest.mark.parametrize("H,Hkv", [(12, 4), (8, 1), (32, 2), (16, 8)],
                         ids=["G3", "MQA-G8", "G16", "G2"])
def test_grouped_query_heads(gpu, fa_lib, H, Hkv):
    # query heads sharing a kv head are served by one workgroup (groups of up
    # to 8; G = 16 needs two workgroups per kv head)
    cfg = inputs.DecodeConfig(cid=95, num_seqs=6, num_heads=H, num_kv_heads=Hkv, num_blocks=1600,
                              ctx_lo=1, ctx_hi=3000)
    d = inputs.decode_inputs(cfg, context_lens=[1, 17, 256, 700, 2049, 3000])
    check(d, cfg, gpu, "gqa H%d Hkv%d" % (H, Hkv))


def test_all_contexts_empty(gpu, fa_lib):
    cfg = inputs.DecodeConfig(cid=91, num_seqs=3, num_heads=4, num_kv_heads=4, num_blocks=8,
                              ctx_lo=0, ctx_hi=16)
    d = inputs.decode_inputs(cfg, context_lens=[0, 0, 0])
    out = run_decode(d, cfg, gpu)
    assert torch.all(out == 0)


def test_P10_paging_invariance_bitwise(gpu, fa_lib):
    # the same logical K/V under two block permutations gives identical bits
    cfg = inputs.DecodeConfig(cid=92, num_seqs=6, num_heads=8, num_kv_heads=8, num_blocks=700,
                              ctx_lo=100, ctx_hi=1500)
    d1 = inputs.decode_inputs(cfg)
    d2 = inputs.decode_inputs(cfg.replace(cid=93), context_lens=d1["context_lens"].numpy())
    # rebuild d2's caches so that its blocks hold d1's logical content
    k2, v2 = torch.full_like(d1["k_cache"], float("nan")), torch.full_like(d1["v_cache"], float("nan"))
    S, BS = cfg.num_seqs, cfg.block_size
    for s in range(S):
        n = (int(d1["context_lens"][s]) + BS - 1) // BS
        src, dst = d1["block_tables"][s, :n].long(), d2["block_tables"][s, :n].long()
        k2[dst] = d1["k_cache"][src]
        v2[dst] = d1["v_cache"][src]
    d2.update(k_cache=k2, v_cache=v2, q=d1["q"])
    o1 = run_decode(d1, cfg, gpu)
    o2 = run_decode(d2, cfg, gpu)
    assert torch.equal(o1, o2)


def test_workspace_reuse_and_determinism(gpu, fa_lib):
    cfg = inputs.DecodeConfig(cid=94, num_seqs=5, num_heads=8, num_kv_heads=8, num_blocks=600,
                              ctx_lo=200, ctx_hi=2000)
    d = inputs.decode_inputs(cfg)
    nbytes = fa.fa_paged_decode_workspace_size(cfg.num_seqs, cfg.num_heads, 128, 2000)
    ws = torch.full((nbytes // 4,), float("nan"), device=gpu)
    o1 = run_decode(d, cfg, gpu, workspace=ws)
    # a second, different problem through the same workspace
    d_b = inputs.decode_inputs(cfg.replace(cid=95))
    ob = run_decode(d_b, cfg, gpu, workspace=ws)
    ref_b, _ = oracle.paged_decode(d_b["q"], d_b["k_cache"], d_b["v_cache"], d_b["block_tables"],
                                   d_b["context_lens"], float(np.float32(cfg.scale)))
    assert errors(ob.double().numpy(), ref_b)[0] <= DECODE_TOL["o_max"]
    o2 = run_decode(d, cfg, gpu, workspace=ws)
    assert torch.equal(o1, o2)


def test_invalid_decode_launches_nothing(gpu, fa_lib):
    q = torch.zeros(2, 4, 128, dtype=torch.float16, device=gpu)
    kc = torch.zeros(4, 4, 16, 16, 8, dtype=torch.float16, device=gpu)
    vc = torch.zeros(4, 4, 128, 16, dtype=torch.float16, device=gpu)
    bt = torch.zeros(2, 2, dtype=torch.int32, device=gpu)
    cl = torch.tensor([5, 7], dtype=torch.int32, device=gpu)
    out = torch.full_like(q, 3.0)
    ws = torch.empty(16, dtype=torch.uint8, device=gpu)  # too small
    with pytest.raises(fa.FAError) as e:
        fa.fa_paged_decode(q, kc, vc, bt, cl, out, 2, 4, 4, 128, 16, 2, 7, 0.1, ws)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
