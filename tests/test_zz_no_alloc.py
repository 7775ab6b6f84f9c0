"""fa_paged_decode_noalloc (the decode for callers that cannot allocate) against
fa_paged_decode, through the C ABI.

Both entry points run the same kernels with the same reduction order; only
where the per-partition partials live differs (the library's per-device
scratch array, or the caller's workspace), so the outputs must be bitwise
equal.  Two calls in a row, the second on a smaller problem, check that a
call reads nothing the previous one left in the scratch; sizes past the
scratch's limit must be refused without launching anything.
"""
import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
from exact_attention_12_amd import inputs
from gpu_util import DECODE_TOL, progress

pytestmark = pytest.mark.gpu

FA_ERR_SCRATCH = -6


def _dev(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def both(d, cfg, dev):
    """(out of fa_paged_decode with a workspace, out of fa_paged_decode_noalloc)."""
    t = _dev(d, dev)
    S, H, D = t["q"].shape
    Hkv, BS, MB = t["k_cache"].shape[1], t["k_cache"].shape[3], t["block_tables"].shape[1]
    scale = float(np.float32(cfg.scale))
    ref = fa.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                          t["max_context_len"], scale=scale)
    out = torch.full_like(t["q"], float("nan"))
    fa.fa_paged_decode_noalloc(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                               out, S, H, Hkv, D, BS, MB, t["max_context_len"], scale)
    torch.cuda.synchronize()
    return ref.cpu(), out.cpu()


def test_noalloc_equals_workspace_decode_two_calls(gpu, fa_lib):
    # first the 64-sequence x 32-head workload (16 partitions), then a smaller
    # grouped-query problem with other context lengths
    big = inputs.DECODE_CONFIG
    small = inputs.DecodeConfig(cid=91, num_seqs=9, num_heads=8, num_kv_heads=2, num_blocks=600,
                                ctx_lo=0, ctx_hi=1500)
    for cfg, ctx in ((big, None), (small, [0, 1, 17, 256, 257, 700, 1000, 1499, 1500])):
        d = inputs.decode_inputs(cfg, context_lens=ctx)
        need = fa.fa_paged_decode_workspace_size(cfg.num_seqs, cfg.num_heads, cfg.head_size,
                                                 d["max_context_len"])
        assert need <= fa.FA_DECODE_NOALLOC_SCRATCH_BYTES
        progress("noalloc S=%d H=%d Hkv=%d max_ctx=%d scratch %d bytes" % (
            cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, d["max_context_len"], need))
        ref, out = both(d, cfg, gpu)
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref), float((out.double() - ref.double()).abs().max())
        err = (out.double() - ref.double()).abs()
        assert err.max() <= DECODE_TOL["o_max"] and err.mean() <= DECODE_TOL["o_mean"]


def test_noalloc_refuses_sizes_past_the_scratch(gpu, fa_lib):
    S, H, D = 64, 32, 128
    max_ctx = 64 * 256  # 64 partitions: 64*32*64 partials of 520 bytes > 32 MiB
    assert fa.fa_paged_decode_workspace_size(S, H, D, max_ctx) > fa.FA_DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(S, H, D, dtype=torch.float16, device=gpu)
    kc = torch.zeros(8, H, D // 8, 16, 8, dtype=torch.float16, device=gpu)
    vc = torch.zeros(8, H, D, 16, dtype=torch.float16, device=gpu)
    bt = torch.zeros(S, max_ctx // 16, dtype=torch.int32, device=gpu)
    cl = torch.zeros(S, dtype=torch.int32, device=gpu)
    out = torch.full((S, H, D), 7.0, dtype=torch.float16, device=gpu)
    with pytest.raises(fa.FAError) as e:
        fa.fa_paged_decode_noalloc(q, kc, vc, bt, cl, out, S, H, H, D, 16, max_ctx // 16, max_ctx,
                                   0.088)
    assert e.value.status == FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (out == 7.0).all()
