"""Shared helpers of the GPU parity tests: tolerances, comparisons, progress lines."""
import os

import numpy as np
import torch

# Tolerances (absolute), per input element type, against the fp64 oracle run
# on the same rounded inputs:
#   fp32 inputs: max |dO| <= 1e-4 and max |dlse| <= 1e-4;
#   bf16/fp16 inputs (fp32 accumulation): max |dO| <= 1e-2, mean |dO| <= 1e-3,
#   max |dlse| <= 1e-3.
TOL = {
    torch.float32: dict(o_max=1e-4, o_mean=1e-4, lse_max=1e-4),
    torch.bfloat16: dict(o_max=1e-2, o_mean=1e-3, lse_max=1e-3),
    torch.float16: dict(o_max=1e-2, o_mean=1e-3, lse_max=1e-3),
}
DECODE_TOL = dict(o_max=1e-2, o_mean=1e-3)
# Backward (16-bit inputs, fp32 outputs): per gradient tensor, the largest
# error against the largest reference magnitude, and the mean error against
# the mean reference magnitude, each with a small absolute floor for
# gradients that are exactly zero in the reference (N = 1).  The kernel
# rounds two fp32 intermediates to the input type before a matrix product
# -- P (recomputed from lse) for dV = P^T dO and dS = P o (dP - D) for
# dQ = dS K and dK = dS^T Q -- and accumulates the exact 16-bit products in
# fp32, so the error is a sum of terms each carrying one relative rounding
# of at most u (2^-8 for bf16, 2^-11 for fp16).  Measured over the shapes of
# test_gpu_bwd.py (ragged, d 64/128, grouped kv heads, full-size rows): the
# largest max ratio is 0.78 u and the largest mean ratio 0.45 u, for both
# types.  The bars are 2 u and 1.25 u, about 2.7 times those.
_U = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
BWD_TOL = {dt: dict(max_rel=2.0 * u, mean_rel=1.25 * u, floor=1e-5) for dt, u in _U.items()}
# Block-scaled FP8 forward, against the oracle on the dequantised inputs.
# The only rounding beyond fp32 accumulation is that of each probability to
# E4M3 before the P.V product: |P^ - P~| <= 2^-4 P~ in the normal range and
# <= 2^-10 below it, and O is normalised by the unrounded sum.  Hence, per
# element, |dO_ic| <= 2^-4 sum_j w_ij |v_jc| + (subnormal terms), with w the
# exact softmax weights: the test computes sum_j w_ij |v_jc| with the oracle
# (attention applied to |V|) and allows 2^-4 of it plus 2^-8.  lse uses the
# unrounded sum, as in the 16-bit forward.
FP8_TOL = dict(rel=2.0 ** -4, abs=2.0 ** -8, lse_max=1e-3)


_LOG = os.environ.get("FA_PROGRESS_LOG") or os.path.join(
    os.path.dirname(os.path.dirname(os.path.abspath(__file__))), ".test_progress", "gpu_progress.log")


def progress(msg):
    """Append a progress line (test case, shape, errors) to a log file, flushed at once.

    pytest captures the test's own stdout/stderr; the file keeps the record of
    which case ran last even if the process dies."""
    try:
        os.makedirs(os.path.dirname(_LOG), exist_ok=True)
        with open(_LOG, "a") as f:
            f.write("[gpu] %s\n" % msg)
    except OSError:
        pass


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    e = np.abs(got - ref)
    return float(e.max()) if e.size else 0.0, float(e.mean()) if e.size else 0.0


def assert_fwd_close(o, lse, o_ref, lse_ref, dtype, label=""):
    """o, lse: GPU results (numpy fp64) at the oracle's rows; refs from the oracle."""
    assert np.all(np.isfinite(o)), "non-finite O " + label
    assert np.all(np.isfinite(lse)), "non-finite lse " + label
    tol = TOL[dtype]
    omax, omean = errors(o, o_ref)
    lmax, _ = errors(lse, lse_ref)
    progress("%s max|dO|=%.3g mean|dO|=%.3g max|dlse|=%.3g" % (label, omax, omean, lmax))
    assert omax <= tol["o_max"], (label, omax)
    assert omean <= tol["o_mean"], (label, omean)
    assert lmax <= tol["lse_max"], (label, lmax)
    return omax, omean, lmax


def assert_bwd_close(dq, dk, dv, ref, dtype, label=""):
    """dq, dk, dv: GPU gradients (numpy fp64) at the oracle's rows / keys."""
    out = {}
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        r = ref[name]
        if r.size == 0:
            continue
        assert np.all(np.isfinite(got)), "non-finite %s %s" % (name, label)
        emax, emean = errors(got, r)
        rmax, rmean = float(np.abs(r).max()), float(np.abs(r).mean())
        out[name] = (emax, emean, rmax, rmean)
        progress("%s %s max|err|=%.3g mean|err|=%.3g max|ref|=%.3g mean|ref|=%.3g" % (
            label, name, emax, emean, rmax, rmean))
    tol = BWD_TOL[dtype]
    for name, (emax, emean, rmax, rmean) in out.items():
        assert emax <= tol["max_rel"] * rmax + tol["floor"], (label, name, emax, rmax)
        assert emean <= tol["mean_rel"] * rmean + tol["floor"], (label, name, emean, rmean)
    return out


def oracle_per_head(fn, q, k, v, rows, *args, **kw):
    """Run an oracle routine head by head, each (b, h) on its own query rows.

    fn(q, k, v, *args, rows=..., **kw) -> (o, lse) is oracle.attention or
    oracle.attention_ext; q [B, H, N, d], k and v [B, Hkv, Nk, d]; rows
    [B * H, R] (inputs.sample_rows_per_head).  Query head h reads kv head
    h // (H // Hkv).  Returns (o [B, H, R, d], lse [B, H, R]) in fp64.
    """
    B, H = q.shape[0], q.shape[1]
    g = H // k.shape[1]
    R = rows.shape[1]
    o = np.empty((B, H, R, q.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kvh = h // g
            o1, l1 = fn(q[b:b + 1, h:h + 1], k[b:b + 1, kvh:kvh + 1], v[b:b + 1, kvh:kvh + 1], *args,
                        rows=rows[b * H + h], **kw)
            o[b, h], lse[b, h] = o1[0, 0], l1[0, 0]
    return o, lse


def gather_rows(x, rows):
    """x [B, H, N, ...] (numpy) at each head's own rows [B * H, R] -> [B, H, R, ...]."""
    B, H = x.shape[0], x.shape[1]
    idx = rows.reshape(B, H, -1)
    return np.take_along_axis(x, idx.reshape(idx.shape + (1,) * (x.ndim - 3)), axis=2)
