"""Every entry point runs on the stream it is given and can be captured in a
HIP graph.

The library allocates nothing, synchronises nothing and issues no memset: a
call only enqueues kernels on its stream.  Two checks, on small shapes:
  - each entry point on a second stream (ordered after the inputs' stream)
    returns the same bits as on the current stream;
  - one captured graph of the forward, the backward, the FP8 quantiser and
    forward, a masked forward with its block map, the paged decode and the
    chunked prefill over the paged cache,
    replayed three times with new inputs written eagerly between replays,
    returns on every replay the same bits as the eager calls on those inputs.
The kernels use no atomics, so equal inputs give equal bits.
"""
import numpy as np
import pytest
import torch

import exact_attention_12_amd as fa
from exact_attention_12_amd import inputs
from gpu_util import progress

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 4, 300, 128
NK = 450  # keys of the masked forward


class Case:
    """Inputs and preallocated outputs of every entry point, on one device."""

    def __init__(self, dev, seed):
        self.dev = dev
        bf = torch.bfloat16
        self.q = inputs.normal(seed, (B, H, N, D), 1.0, bf).to(dev)
        self.k = inputs.normal(seed + 1, (B, H, N, D), 1.0, bf).to(dev)
        self.v = inputs.normal(seed + 2, (B, H, N, D), 1.0, bf).to(dev)
        self.dout = inputs.normal(seed + 3, (B, H, N, D), 1.0, bf).to(dev)
        self.kx = inputs.normal(seed + 4, (B, H, NK, D), 1.0, bf).to(dev)
        self.vx = inputs.normal(seed + 5, (B, H, NK, D), 1.0, bf).to(dev)
        keep = np.random.default_rng(seed + 6).random((3, 8)) < 0.5
        m = np.repeat(np.repeat(keep, 128, 0), 64, 1)[:N, :NK] & np.tri(N, NK, NK - N, dtype=bool)
        m[:, 0] = True
        self.ldm = (NK + 15) // 16 * 16
        mask = np.zeros((N, self.ldm), np.uint8)
        mask[:, :NK] = m
        self.mask = torch.from_numpy(mask).to(dev)
        self.mwords = fa.fa_mask_blocks_words(B, H, N, NK, 0, 0)
        dc = inputs.DecodeConfig(cid=9, num_seqs=3, num_heads=4, num_kv_heads=2, num_blocks=64,
                                 ctx_lo=1, ctx_hi=400)
        d = inputs.decode_inputs(dc, context_lens=[1, 250, 400])
        self.dec = {n: d[n].to(dev) for n in ("q", "k_cache", "v_cache", "block_tables", "context_lens")}
        self.dec_max = d["max_context_len"]
        self.pre_q = inputs.normal(seed + 7, (3, 4, 64, D), 1.0, d["q"].dtype).to(dev)
        self.dec_scale = float(np.float32(dc.scale))
        self.scale = float(np.float32(1.0 / np.sqrt(D)))
        f32 = torch.float32
        z = lambda *s, dt=f32: torch.zeros(s, dtype=dt, device=dev)
        self.out = dict(o=z(B, H, N, D), lse=z(B, H, N), dq=z(B, H, N, D), dk=z(B, H, N, D),
                        dv=z(B, H, N, D), o8=z(B, H, N, D), lse8=z(B, H, N), ox=z(B, H, N, D),
                        lx=z(B, H, N), mblk=z(self.mwords, dt=torch.int32),
                        dout_dec=torch.zeros_like(self.dec["q"]), opre=z(3, 4, 64, D), lpre=z(3, 4, 64))
        self.bws = z(fa.fa_bwd_workspace_size(B, H, N), dt=torch.uint8)
        self.dws = z(fa.fa_paged_decode_workspace_size(3, 4, D, self.dec_max), dt=torch.uint8)
        nb = lambda lay: fa.fa_fp8_codes_bytes(B, H, N, D, lay)
        self.codes = [z(nb(0), dt=torch.uint8), z(nb(0), dt=torch.uint8), z(nb(1), dt=torch.uint8)]
        self.exps = [z(B, H, (N + 127) // 128, dt=torch.int32) for _ in range(3)]

    def refill(self, seed):
        """Write new q, k, v, dout and decode queries in place (eager work)."""
        bf = torch.bfloat16
        for i, t in enumerate((self.q, self.k, self.v, self.dout)):
            t.copy_(inputs.normal(seed + i, tuple(t.shape), 1.0, bf).to(self.dev))
        self.dec["q"].copy_(inputs.normal(seed + 9, tuple(self.dec["q"].shape), 1.0,
                                          self.dec["q"].dtype).to(self.dev))
        self.pre_q.copy_(inputs.normal(seed + 10, tuple(self.pre_q.shape), 1.0,
                                       self.pre_q.dtype).to(self.dev))

    def run(self, stream=None):
        """Enqueue every entry point on stream (None: torch's current stream)."""
        o = self.out
        fa.fa_fwd(self.q, self.k, self.v, o["o"], o["lse"], B, H, N, D, self.scale, True, stream=stream)
        fa.fa_bwd(self.q, self.k, self.v, o["o"], o["lse"], self.dout, o["dq"], o["dk"], o["dv"], B, H, H,
                  N, D, self.scale, True, self.bws, stream=stream)
        for x, lay, c, e in ((self.q, 0, self.codes[0], self.exps[0]), (self.k, 0, self.codes[1], self.exps[1]),
                             (self.v, 1, self.codes[2], self.exps[2])):
            fa.fa_quant_fp8(x, B, H, N, D, lay, c, e, stream=stream)
        fa.fa_fwd_fp8(*self.codes, *self.exps, o["o8"], o["lse8"], B, H, H, N, D, self.scale, True,
                      stream=stream)
        fa.fa_mask_blocks(self.mask, B, H, N, NK, 0, 0, self.ldm, o["mblk"], self.mwords, stream=stream)
        fa.fa_fwd_ext(self.q, self.kx, self.vx, o["ox"], o["lx"], B, H, H, N, NK, D, self.scale, False,
                      -1, -1, self.mask, 0, 0, self.ldm, mask_blocks=o["mblk"], stream=stream)
        dd = self.dec
        fa.fa_paged_decode(dd["q"], dd["k_cache"], dd["v_cache"], dd["block_tables"], dd["context_lens"],
                           o["dout_dec"], 3, 4, 2, D, 16, dd["block_tables"].shape[1], self.dec_max,
                           self.dec_scale, self.dws, stream=stream)
        fa.fa_fwd_paged(self.pre_q, dd["k_cache"], dd["v_cache"], dd["block_tables"], dd["context_lens"],
                        o["opre"], o["lpre"], 3, 4, 2, 64, D, 16, dd["k_cache"].shape[0],
                        dd["block_tables"].shape[1], self.dec_scale, True, stream=stream)

    def snapshot(self):
        return {n: t.clone() for n, t in self.out.items()}


def assert_same(a, b, label):
    for n in a:
        assert torch.equal(a[n], b[n]), (label, n)


def test_side_stream(gpu, fa_lib):
    c = Case(gpu, 9100)
    progress("streams: current stream")
    c.run()
    torch.cuda.synchronize()
    ref = c.snapshot()
    for t in c.out.values():
        t.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    progress("streams: side stream")
    c.run(stream=side)
    side.synchronize()
    assert_same(ref, c.snapshot(), "side stream")


def test_graph_replay(gpu, fa_lib):
    c = Case(gpu, 9200)
    c.run()  # first launches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    progress("graph: capture")
    with torch.cuda.graph(g, stream=cap):
        c.run()
    torch.cuda.synchronize()
    for rep in range(3):
        c.refill(9300 + 10 * rep)
        torch.cuda.synchronize()
        c.run()  # eager, on the current stream
        torch.cuda.synchronize()
        want = c.snapshot()
        for t in c.out.values():
            t.zero_()
        torch.cuda.synchronize()
        progress("graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        got = c.snapshot()
        assert all(torch.isfinite(t.float()).all() for n, t in got.items()
                   if n not in ("lse", "lx", "lse8", "lpre")), rep
        assert_same(want, got, "replay %d" % rep)
