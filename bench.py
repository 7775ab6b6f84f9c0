#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. fa_fwd on the headline forward workload: B=2, H=32, N=8192, d=128, bf16,
     causal, scale 1/sqrt(128), Q/K/V iid N(0,1);
  2. fa_paged_decode on the decode workload: 64 sequences x 32 heads, head
     size 128, fp16, block size 16, context lengths uniform in [512, 4096],
     a 20000-block pool addressed through a random permutation;
  3. fa_paged_decode on the grouped-query variant: the same shape with 8 kv
     heads (4 query heads per kv head);
  4. fa_fwd_gqa on the forward workload with 8 kv heads (fwd_gqa);
  5. fa_bwd on the forward workload (bwd): dQ, dK, dV for a seeded N(0,1)
     upstream gradient, from step 1's o and lse;
  6. fa_fwd_fp8 on the forward workload quantised to block-scaled E4M3
     (fwd_fp8), and fa_quant_fp8 of its q, k, v (quant_fp8);
  7. fa_fwd_ext on the forward workload with a causal sliding window of 1024
     keys (fwd_window) and with a block-sparse causal boolean mask
     (fwd_mask: each (128-query, 64-key) block kept with probability 1/2),
     and the same mask through its block map (fwd_mask_map: fa_mask_blocks
     + fa_fwd_ext, the map rebuilt every step);
  8. fa_fwd_paged, chunked prefill over the paged cache (fwd_paged): 16
     sequences, 512 new tokens each at the end of a context of U[1024, 4096]
     tokens, 32 query heads over 8 kv heads, bf16, block 16.
Inputs are generated on the host with fixed seeds and copied to HBM before
the timed region.  The timed region runs K steps between two device
synchronisations; each kernel call is bracketed by HIP events recorded on the
stream the kernels run on (torch's current stream).

Prints ONE JSON line.  `value` is the forward pass's throughput in TFLOP/s
(4*B*H*N^2*d / 2 for causal, per second of fa_fwd time); the decode's HBM
bandwidth (algorithmic bytes per second of fa_paged_decode time) is reported
under "decode".  `cpu_baseline` times the fp64 CPU oracle on a bounded sample
of the forward workload (every query row of the first few heads).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak (published)
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak (published)
PEAK_CLOCK_GHZ = 2.4       # the shader clock the published peaks assume
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_attention_12_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they are current."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _clk_sources(kind="sclk"):
    """sysfs files that report a current GPU clock: pp_dpm_sclk (shader) or
    pp_dpm_mclk (memory), whose starred line is the current frequency."""
    import glob
    return sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_%s" % kind))


def _read_sclk_ghz(path):
    with open(path) as fh:
        for line in fh:
            if line.rstrip().endswith("*"):
                mhz = line.split(":", 1)[1].strip().rstrip("*").strip()
                return float(mhz.lower().replace("mhz", "")) / 1e3
    return None


class ClockSampler:
    """Samples a GPU clock (kind "sclk" or "mclk") from sysfs every few
    milliseconds on a host thread while the GPU runs; reports the median in GHz
    (None if unreadable).  With several cards visible, the one whose clock
    moves most is taken."""

    def __init__(self, period_s=0.002, kind="sclk"):
        import threading
        self.period = period_s
        self.files = _clk_sources(kind)
        self.samples = {f: [] for f in self.files}
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            for f in self.files:
                try:
                    g = _read_sclk_ghz(f)
                except (OSError, ValueError, IndexError):
                    g = None
                if g is not None:
                    self.samples[f].append(g)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.files:
            self._t.start()
        return self

    def __exit__(self, *exc):
        if self.files:
            self._stop.set()
            self._t.join()

    def result(self):
        best = None
        for f, xs in self.samples.items():
            if len(xs) >= 5:
                spread = max(xs) - min(xs)
                if best is None or spread > best[0]:
                    best = (spread, f, xs)
        if best is None:
            return None
        xs = best[2]
        return dict(ghz_median=round(median(xs), 3), ghz_min=round(min(xs), 3), ghz_max=round(max(xs), 3),
                    samples=len(xs), source=best[1])


def cpu_baseline(q, k, v, scale, causal, target_s=12.0):
    """Time the oracle on the first heads of batch 0 of the forward workload.

    A short probe (64 evenly spaced rows of one head) sizes the sample; the
    timed sample is then every query row of the first `nh` heads, with nh
    chosen so that it takes about target_s seconds.
    """
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    H, N, d = q.shape[1], q.shape[2], q.shape[3]

    def run(nh, rows):
        qh, kh, vh = (t[:1, :nh].contiguous() for t in (q, k, v))
        t0 = time.perf_counter()
        oracle.attention(qh, kh, vh, scale, causal, rows=rows, nthreads=threads)
        dt = time.perf_counter() - t0
        r = np.arange(N, dtype=np.int64) if rows is None else rows
        keys = (r + 1).sum() if causal else len(r) * N
        return dt, 4.0 * d * float(keys) * nh

    probe = np.unique(np.linspace(0, N - 1, 64).round().astype(np.int64))
    dt, fl = run(1, probe)
    full_head = 4.0 * d * (N * (N + 1) / 2.0 if causal else float(N) * N)
    nh = int(min(H, max(1, round(target_s / max(dt * full_head / fl, 1e-3)))))
    dt, fl = run(nh, None)
    return dict(value=fl / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                seconds=round(dt, 3), cpu_model=cpu_model(),
                sample="fp64 oracle on heads 0..%d of batch 0 of the forward workload "
                       "(all %d query rows each, causal): %.3g flop" % (nh - 1, N, fl))


def cpu_long_context_sample(rows_per_head=256):
    """The oracle on the long-context forward workload (B=1 H=8 N=65536 d=128
    causal): rows_per_head sampled rows of every head, and the full problem
    extrapolated from them by the ratio of per-row work sum(i + 1)."""
    import numpy as np
    import oracle
    from exact_attention_12_amd import inputs
    cfg = inputs.FWD_CAUSAL_N65536
    q, k, v = inputs.fwd_inputs(cfg)
    threads = oracle.default_threads()
    rows = inputs.sample_rows(cfg.N, rows_per_head, seed=1000 * cfg.cid + 5)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, float(np.float32(cfg.scale)), True, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    work_sample = float((rows + 1).sum())
    work_full = cfg.N * (cfg.N + 1) / 2.0
    flop = 4.0 * cfg.d * work_sample * cfg.B * cfg.H
    return dict(workload=cfg.name, rows_per_head=rows_per_head, heads=cfg.B * cfg.H,
                seconds=round(dt, 3), tflops=flop / dt / 1e12, cores=threads,
                full_seconds_extrapolated=round(dt * work_full / work_sample, 1),
                note="full-problem time extrapolated by the ratio of per-row work sum(i+1)")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timing (e.g. under a profiler)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 plain device copies of MIB MiB "
                         "(reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 5}), flush=True)
        return

    import exact_attention_12_amd as fa
    from exact_attention_12_amd import inputs

    if not os.path.exists(fa.lib_path()):
        from exact_attention_12_amd import build as fa_build
        fa_build.build()
    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------- inputs (host, seeded) -> HBM
    fcfg = inputs.FWD_CAUSAL_N8192
    log("generating forward inputs: " + fcfg.name)
    q, k, v = inputs.fwd_inputs(fcfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, H, N, d = qd.shape
    fscale = float(np.float32(fcfg.scale))
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    dcfg = inputs.DECODE_CONFIG
    log("generating decode inputs: " + dcfg.name)
    dec = inputs.decode_inputs(dcfg)
    dq, dk, dv = dec["q"].to(dev), dec["k_cache"].to(dev), dec["v_cache"].to(dev)
    dbt, dcl = dec["block_tables"].to(dev), dec["context_lens"].to(dev)
    maxctx = dec["max_context_len"]
    S, Hq, D = dq.shape
    Hkv, BS = dk.shape[1], dk.shape[3]
    MB = dbt.shape[1]
    dscale = float(np.float32(dcfg.scale))
    dout = torch.empty_like(dq)
    ws_bytes = fa.fa_paged_decode_workspace_size(S, Hq, D, maxctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    del dec["k_cache"], dec["v_cache"]

    qcfg = inputs.FWD_GQA_CONFIG
    log("generating grouped-query forward inputs: " + qcfg.name)
    gfq, gfk, gfv = (t.to(dev) for t in inputs.fwd_inputs(qcfg))
    gHkv_f = gfk.shape[1]
    go = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    glse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    gcfg = inputs.DECODE_GQA_CONFIG
    log("generating grouped-query decode inputs: " + gcfg.name)
    gdec = inputs.decode_inputs(gcfg)
    gq, gk, gv = gdec["q"].to(dev), gdec["k_cache"].to(dev), gdec["v_cache"].to(dev)
    gbt, gcl = gdec["block_tables"].to(dev), gdec["context_lens"].to(dev)
    gmaxctx = gdec["max_context_len"]
    gHkv, gMB = gk.shape[1], gbt.shape[1]
    gout = torch.empty_like(gq)
    gws = torch.empty(fa.fa_paged_decode_workspace_size(S, Hq, D, gmaxctx), dtype=torch.uint8,
                      device=dev)
    del gdec["k_cache"], gdec["v_cache"]

    pcfg = inputs.PREFILL_CONFIG
    log("generating chunked-prefill inputs: " + pcfg.name)
    pdec = inputs.decode_inputs(pcfg)
    pq = inputs.prefill_queries(pcfg, inputs.PREFILL_NQ).to(dev)
    pk, pv = pdec["k_cache"].to(dev), pdec["v_cache"].to(dev)
    pbt, pcl = pdec["block_tables"].to(dev), pdec["context_lens"].to(dev)
    pctx = pdec["context_lens"].numpy().astype(np.int64)
    pS, pH, pNq, pD = pq.shape
    pHkv, pNB = pk.shape[1], pk.shape[0]
    po = torch.empty((pS, pH, pNq, pD), dtype=torch.float32, device=dev)
    pl = torch.empty((pS, pH, pNq), dtype=torch.float32, device=dev)
    del pdec["k_cache"], pdec["v_cache"]

    log("generating the upstream gradient of the backward pass")
    gdo = inputs.bwd_dout(fcfg).to(dev)
    bdq = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    bdk = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    bdv = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    bws = torch.empty(fa.fa_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=dev)

    log("quantising the forward inputs to block-scaled E4M3")
    q8, qe8 = fa.quant_fp8(qd, 0)
    k8, ke8 = fa.quant_fp8(kd, 0)
    v8, ve8 = fa.quant_fp8(vd, 1)
    o8 = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lse8 = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    log("building the block-sparse mask")
    win = 1024
    keep = np.random.default_rng(64).random((N // 128, N // 64)) < 0.5
    mask_h = np.repeat(np.repeat(keep, 128, 0), 64, 1) & np.tri(N, N, dtype=bool)
    mask_h[:, 0] = True
    mask_d = torch.from_numpy(mask_h.astype(np.uint8)).to(dev)
    mask_pairs = int(mask_h.sum())
    del mask_h
    map_words = fa.fa_mask_blocks_words(B, H, N, N, 0, 0)
    mask_map = torch.empty(map_words, dtype=torch.int32, device=dev)
    omb = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lmb = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ow = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lw = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    om = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lm = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.fa_fwd(qd, kd, vd, o, lse, B, H, N, d, fscale, True, stream=stream)
        if evs:
            evs[1].record(stream)
        fa.fa_paged_decode(dq, dk, dv, dbt, dcl, dout, S, Hq, Hkv, D, BS, MB, maxctx, dscale, ws,
                           stream=stream)
        if evs:
            evs[2].record(stream)
        fa.fa_paged_decode(gq, gk, gv, gbt, gcl, gout, S, Hq, gHkv, D, BS, gMB, gmaxctx, dscale, gws,
                           stream=stream)
        if evs:
            evs[3].record(stream)
        fa.fa_fwd_gqa(gfq, gfk, gfv, go, glse, B, H, gHkv_f, N, d, fscale, True, stream=stream)
        if evs:
            evs[4].record(stream)
        fa.fa_bwd(qd, kd, vd, o, lse, gdo, bdq, bdk, bdv, B, H, H, N, d, fscale, True, bws,
                  stream=stream)
        if evs:
            evs[5].record(stream)
        fa.fa_fwd_fp8(q8, k8, v8, qe8, ke8, ve8, o8, lse8, B, H, H, N, d, fscale, True, stream=stream)
        if evs:
            evs[6].record(stream)
        fa.fa_quant_fp8(qd, B, H, N, d, 0, q8, qe8, stream=stream)
        fa.fa_quant_fp8(kd, B, H, N, d, 0, k8, ke8, stream=stream)
        fa.fa_quant_fp8(vd, B, H, N, d, 1, v8, ve8, stream=stream)
        if evs:
            evs[7].record(stream)
        fa.fa_fwd_ext(qd, kd, vd, ow, lw, B, H, H, N, N, d, fscale, True, win, -1, stream=stream)
        if evs:
            evs[8].record(stream)
        fa.fa_fwd_ext(qd, kd, vd, om, lm, B, H, H, N, N, d, fscale, True, -1, -1, mask_d, 0, 0,
                      stream=stream)
        if evs:
            evs[9].record(stream)
        # the same mask through its block map: the map is built every step
        fa.fa_mask_blocks(mask_d, B, H, N, N, 0, 0, N, mask_map, map_words, stream=stream)
        if evs:
            evs[10].record(stream)
        fa.fa_fwd_ext(qd, kd, vd, omb, lmb, B, H, H, N, N, d, fscale, True, -1, -1, mask_d, 0, 0,
                      mask_blocks=mask_map, stream=stream)
        if evs:
            evs[11].record(stream)
        fa.fa_fwd_paged(pq, pk, pv, pbt, pcl, po, pl, pS, pH, pHkv, pNq, pD, 16, pNB, pbt.shape[1],
                        float(np.float32(pcfg.scale)), True, stream=stream)
        if evs:
            evs[12].record(stream)

    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(13)] for _ in range(args.steps)]
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the shader clock under the forward alone: back-to-back fa_fwd calls
    # while a host thread samples the clock (outside the timed steps)
    log("sampling the shader and memory clocks under the forward")
    with ClockSampler() as clk, ClockSampler(kind="mclk") as mclk:
        ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ce0.record(stream)
        for _ in range(40):
            fa.fa_fwd(qd, kd, vd, o, lse, B, H, N, d, fscale, True, stream=stream)
        ce1.record(stream)
        torch.cuda.synchronize()
    clock = clk.result()
    mem_clock = mclk.result()
    clock_fwd_ms = ce0.elapsed_time(ce1) / 40
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    gqa_ms = [e[2].elapsed_time(e[3]) for e in evs]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    gqa_avg = sum(gqa_ms) / len(gqa_ms)
    fgqa_ms = [e[3].elapsed_time(e[4]) for e in evs]
    fgqa_avg = sum(fgqa_ms) / len(fgqa_ms)
    bwd_ms = [e[4].elapsed_time(e[5]) for e in evs]
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    # backward flop: five N x N x d products per head (S recomputed, dP, dV,
    # dK, dQ), 2.5 times the forward's two
    bwd_flops = 2.5 * fcfg.flops()
    bwd_tflops = bwd_flops / (bwd_avg * 1e-3) / 1e12
    f8_ms = [e[5].elapsed_time(e[6]) for e in evs]
    f8_avg = sum(f8_ms) / len(f8_ms)
    f8_tflops = fcfg.flops() / (f8_avg * 1e-3) / 1e12
    qz_ms = [e[6].elapsed_time(e[7]) for e in evs]
    qz_avg = sum(qz_ms) / len(qz_ms)
    nel = B * H * N * d
    qz_bytes = 3 * nel * qd.element_size() + 2 * nel + fa.fa_fp8_codes_bytes(B, H, N, d, 1) \
        + 3 * B * H * ((N + 127) // 128) * 4
    qz_gbs = qz_bytes / (qz_avg * 1e-3) / 1e9
    # flop over the visible (query, key) pairs only
    win_pairs = sum(min(i + 1, win + 1) for i in range(N))
    win_flops = 4.0 * B * H * d * win_pairs
    mk_flops = 4.0 * B * H * d * mask_pairs
    win_ms = [e[7].elapsed_time(e[8]) for e in evs]
    mk_ms = [e[8].elapsed_time(e[9]) for e in evs]
    win_avg, mk_avg = sum(win_ms) / len(win_ms), sum(mk_ms) / len(mk_ms)
    win_tf = win_flops / (win_avg * 1e-3) / 1e12
    mk_tf = mk_flops / (mk_avg * 1e-3) / 1e12
    map_ms = [e[9].elapsed_time(e[10]) for e in evs]
    mkb_ms = [e[10].elapsed_time(e[11]) for e in evs]
    map_avg, mkb_avg = sum(map_ms) / len(map_ms), sum(mkb_ms) / len(mkb_ms)
    mkb_tf = mk_flops / (mkb_avg * 1e-3) / 1e12
    mkb_all_tf = mk_flops / ((map_avg + mkb_avg) * 1e-3) / 1e12
    map_gbs = N * N / (map_avg * 1e-3) / 1e9  # the mask's bytes, read once
    pg_ms = [e[11].elapsed_time(e[12]) for e in evs]
    pg_avg = sum(pg_ms) / len(pg_ms)
    # visible pairs: row i of a context of c tokens sees min(i + c - Nq + 1, c) of them
    pg_pairs = sum(int(np.clip(np.arange(pNq) + c - pNq + 1, 0, c).sum()) for c in pctx)
    pg_flops = 4.0 * pH * pD * pg_pairs
    pg_tf = pg_flops / (pg_avg * 1e-3) / 1e12

    # quick sanity of the last step's results (full parity lives in the tests)
    finite = bool(torch.isfinite(o).all().item() and torch.isfinite(dout).all().item()
                  and torch.isfinite(gout).all().item() and torch.isfinite(go).all().item()
                  and all(torch.isfinite(t).all().item() for t in (bdq, bdk, bdv, o8, ow, om))
                  and (om - omb).abs().max().item() <= 1e-5 and torch.isfinite(po).all().item())

    flops = fcfg.flops()
    tflops = flops / (fwd_avg * 1e-3) / 1e12
    ctx = dec["context_lens"].numpy().astype(np.int64)
    esz = dq.element_size()
    dec_bytes = (int(ctx.sum()) * Hkv * D * esz * 2          # K and V of every context token
                 + S * Hq * D * esz * 2                      # q read, out written
                 + int(((ctx + BS - 1) // BS).sum()) * 4 + S * 4)  # table entries, lengths
    dec_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9
    gctx = gdec["context_lens"].numpy().astype(np.int64)
    gqa_bytes = (int(gctx.sum()) * gHkv * D * esz * 2            # K and V once per kv head
                 + S * Hq * D * esz * 2
                 + int(((gctx + BS - 1) // BS).sum()) * 4 + S * 4)
    gqa_gbs = gqa_bytes / (gqa_avg * 1e-3) / 1e9

    fwd_hash = source_hash("fa_fwd.hip", "fa_device.h", "fa_tile.h", "fa_sizes.h")
    bwd_hash = source_hash("fa_bwd.hip", "fa_device.h", "fa_tile.h", "fa_sizes.h")
    dec_hash = source_hash("fa_decode.hip", "fa_device.h", "fa_tile.h", "fa_sizes.h")
    fwd_traffic = measured_traffic("fa_fwd_kernel", fwd_hash)
    dec_traffic = measured_traffic("fa_decode_partition_kernel", dec_hash)
    bwd_traffic = measured_traffic("fa_bwd", bwd_hash)
    f8_traffic = measured_traffic("fa_fwd_fp8_kernel", source_hash("fa_fp8.hip", "fa_device.h", "fa_tile.h"))

    result = {
        "metric": "attn fwd TFLOP/s + % bf16 MFMA peak (N=8192,d=128,causal); decode HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "attention forward B=2 H=32 N=8192 d=128 bf16 causal (fp32 O, lse) "
                        "+ paged decode 64 seqs x 32 heads x 128, fp16, block 16, "
                        "ctx U[512,4096], 20000-block pool",
            "fwd": {"B": B, "H": H, "N": N, "d": d, "causal": True, "flop": flops,
                    "kernel_ms_avg": round(fwd_avg, 4), "kernel_ms_median": round(median(fwd_ms), 4),
                    "kernel_ms_min": round(min(fwd_ms), 4),
                    "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
                    "clock": clock, "memory_clock": mem_clock, "clock_loop_ms_per_call": round(clock_fwd_ms, 4),
                    "pct_bf16_peak_at_observed_clock":
                        round(100.0 * flops / (clock_fwd_ms * 1e-3) / 1e12
                              / (PEAK_BF16_TFLOPS * clock["ghz_median"] / PEAK_CLOCK_GHZ), 2)
                        if clock else None},
            "decode": {"num_seqs": S, "num_heads": Hq, "num_kv_heads": Hkv, "head_size": D,
                       "block_size": BS, "sum_ctx": int(ctx.sum()), "max_ctx": maxctx,
                       "algorithmic_bytes": dec_bytes, "ms_avg": round(dec_avg, 4),
                       "ms_median": round(median(dec_ms), 4), "ms_min": round(min(dec_ms), 4)},
            "outputs_finite": finite,
        },
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": fwd_traffic, "kernel": "fa_fwd_kernel<bf16,128,causal>",
                     "algorithmic_per_launch": flops},
        "decode": {"metric": "paged decode HBM bandwidth", "value": round(dec_gbs, 1),
                   "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                                "traffic": dec_traffic,
                                "kernel": "fa_decode_partition_kernel + fa_decode_merge_kernel",
                                "algorithmic_per_launch": dec_bytes}},
        "fwd_gqa": {"metric": "attention forward TFLOP/s, 4 query heads per kv head",
                    "value": round(qcfg.flops() / (fgqa_avg * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                    "workload": qcfg.name, "kernel_ms_avg": round(fgqa_avg, 4), "ms_median": round(median(fgqa_ms), 4),
                    "kernel_ms_min": round(min(fgqa_ms), 4),
                    "roofline": {"bound": "mfma",
                                 "achieved": round(qcfg.flops() / (fgqa_avg * 1e-3) / 1e12, 2),
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(qcfg.flops() / (fgqa_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                 "kernel": "fa_fwd_kernel<bf16,128,causal> (grouped kv heads)",
                                 "algorithmic_per_launch": qcfg.flops()}},
        "bwd": {"metric": "attention backward TFLOP/s (dQ, dK, dV; 5 products of 2*N^2*d "
                          "per head, halved for causal)",
                "value": round(bwd_tflops, 2), "unit": "TFLOP/s", "workload": fcfg.name,
                "ms_avg": round(bwd_avg, 4), "ms_median": round(median(bwd_ms), 4), "ms_min": round(min(bwd_ms), 4),
                "roofline": {"bound": "mfma", "achieved": round(bwd_tflops, 2),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                             "traffic": bwd_traffic,
                             "kernel": "fa_bwd_prep_kernel + fa_bwd_dkdv_kernel + fa_bwd_dq_kernel "
                                       "(bf16, d=128, causal)",
                             "algorithmic_per_launch": bwd_flops}},
        "fwd_fp8": {"metric": "attention forward TFLOP/s on block-scaled E4M3 inputs",
                    "value": round(f8_tflops, 2), "unit": "TFLOP/s", "workload": fcfg.name + ", E4M3",
                    "kernel_ms_avg": round(f8_avg, 4), "ms_median": round(median(f8_ms), 4), "kernel_ms_min": round(min(f8_ms), 4),
                    "speedup_vs_bf16": round(fwd_avg / f8_avg, 3),
                    "roofline": {"bound": "mfma", "achieved": round(f8_tflops, 2),
                                 "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(f8_tflops / PEAK_FP8_TFLOPS, 4),
                                 "traffic": f8_traffic,
                                 "kernel": "fa_fwd_fp8_kernel<causal>",
                                 "algorithmic_per_launch": fcfg.flops()}},
        "quant_fp8": {"metric": "block-scaled E4M3 quantisation of q, k, v (HBM GB/s)",
                      "value": round(qz_gbs, 1), "unit": "GB/s", "ms_avg": round(qz_avg, 4),
                      "roofline": {"bound": "hbm", "achieved": round(qz_gbs, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(qz_gbs / PEAK_HBM_GBS, 4),
                                   "kernel": "fa_quant_fp8_kernel (q, k) + fa_quant_fp8_vt_kernel (v)",
                                   "algorithmic_per_launch": qz_bytes}},
        "fwd_window": {"metric": "attention forward TFLOP/s over visible pairs, causal sliding window",
                       "value": round(win_tf, 2), "unit": "TFLOP/s",
                       "workload": fcfg.name + ", window 1024 keys", "kernel_ms_avg": round(win_avg, 4),
                       "roofline": {"bound": "mfma", "achieved": round(win_tf, 2),
                                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                    "frac": round(win_tf / PEAK_BF16_TFLOPS, 4),
                                    "kernel": "fa_fwd_kernel<bf16,128,ext>",
                                    "algorithmic_per_launch": win_flops}},
        "fwd_mask": {"metric": "attention forward TFLOP/s over visible pairs, boolean mask",
                     "value": round(mk_tf, 2), "unit": "TFLOP/s",
                     "workload": fcfg.name + ", block-sparse causal uint8 mask (" +
                                 "%.3f of the causal pairs)" % (mask_pairs / (N * (N + 1) / 2)),
                     "kernel_ms_avg": round(mk_avg, 4),
                     "roofline": {"bound": "mfma", "achieved": round(mk_tf, 2),
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(mk_tf / PEAK_BF16_TFLOPS, 4),
                                  "kernel": "fa_fwd_kernel<bf16,128,ext+mask>",
                                  "algorithmic_per_launch": mk_flops}},
        "fwd_mask_map": {"metric": "attention forward TFLOP/s over visible pairs, boolean mask "
                                   "with its block map (fa_mask_blocks + fa_fwd_ext)",
                         "value": round(mkb_all_tf, 2), "unit": "TFLOP/s",
                         "workload": "the fwd_mask workload, map built every step",
                         "map_ms_avg": round(map_avg, 4), "map_read_gbs": round(map_gbs, 1),
                         "kernel_ms_avg": round(mkb_avg, 4),
                         "roofline": {"bound": "mfma", "achieved": round(mkb_tf, 2),
                                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(mkb_tf / PEAK_BF16_TFLOPS, 4),
                                      "kernel": "fa_fwd_kernel<bf16,128,ext+mask> with the map",
                                      "algorithmic_per_launch": mk_flops}},
        "fwd_paged": {"metric": "chunked prefill over the paged cache, TFLOP/s over visible pairs",
                      "value": round(pg_tf, 2), "unit": "TFLOP/s", "workload": pcfg.name,
                      "new_tokens_per_seq": pNq, "sum_ctx": int(pctx.sum()),
                      "kernel_ms_avg": round(pg_avg, 4),
                      "roofline": {"bound": "mfma", "achieved": round(pg_tf, 2),
                                   "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(pg_tf / PEAK_BF16_TFLOPS, 4),
                                   "kernel": "fa_fwd_kernel<bf16,128,ext paged>",
                                   "algorithmic_per_launch": pg_flops}},
        "decode_gqa": {"metric": "paged decode HBM bandwidth, 4 query heads per kv head",
                       "value": round(gqa_gbs, 1), "unit": "GB/s",
                       "workload": gcfg.name, "sum_ctx": int(gctx.sum()),
                       "ms_avg": round(gqa_avg, 4), "ms_median": round(median(gqa_ms), 4), "ms_min": round(min(gqa_ms), 4),
                       "roofline": {"bound": "hbm", "achieved": round(gqa_gbs, 1),
                                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(gqa_gbs / PEAK_HBM_GBS, 4),
                                    "kernel": "fa_decode_gqa_partition_kernel + fa_decode_merge_kernel",
                                    "algorithmic_per_launch": gqa_bytes}},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(q, k, v, fscale, True)
        log("timing the CPU oracle on the long-context workload's sampled rows")
        result["cpu_baseline"]["long_context_sample"] = cpu_long_context_sample()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
