"""The exact-attention ORACLE (fp64, CPU) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU
baseline leg may import this package.  The GPU library and its Python binding
never import it, and it shares no code with them.

``oracle.c`` holds the arithmetic (plain loops, fp64, libm exp/log, sums in
ascending index order); this module builds it with gcc and wraps it with
ctypes.  Inputs are read in their storage type (fp32 / bf16 / fp16 / fp64)
and widened exactly inside the C code.

Functions (each cites the page passages it follows in ``oracle.c``):
  attention(q, k, v, scale, causal, rows=None)        dense definition
  attention_ext(q, k, v, scale, causal, window, mask)  rectangular, windowed, masked
  mask_blocks(mask)                                   block map of a boolean mask
  probs(q, k, scale, causal)                          the full P matrix
  tiled_fa1 / tiled_fa2(q, k, v, scale, causal, Br, Bc)
                                                      the online recurrence in
                                                      both loop orders
  attention_bwd(q, k, v, dout, scale, causal, rows=None, keys=None)
                                                      gradients dQ, dK, dV
  e4m3_encode / e4m3_decode, quant_fp8, dequant_fp8  block-scaled FP8 (E4M3)
  paged_decode(...), paged_decode_partitioned(...)    single-query decode
  paged_prefill(...)                                  Nq new queries over the paged cache
  widen(x)                                            exact fp64 view
"""
import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_TEST_SOURCE names a modified copy of oracle.c to build and load
# instead (the mutation tests plant a mistake there and expect a pin to fail).
_SRC_OVERRIDE = os.environ.get("ORACLE_TEST_SOURCE")
SRC = _SRC_OVERRIDE or os.path.join(_HERE, "oracle.c")
LIB = (os.path.splitext(_SRC_OVERRIDE)[0] + ".so") if _SRC_OVERRIDE else os.path.join(_HERE, "liboracle.so")
_lib = None

OR_F32, OR_BF16, OR_F16, OR_F64 = 0, 1, 2, 3
_CODES = {torch.float32: OR_F32, torch.bfloat16: OR_BF16, torch.float16: OR_F16,
          torch.float64: OR_F64}


def build() -> str:
    """Compile liboracle.so with gcc (no -ffast-math) and return its path.

    ORACLE_EXTRA_CFLAGS (space-separated) adds flags, e.g. the sanitizer
    build of the host-sanitizer test."""
    tmp = LIB + ".tmp%d" % os.getpid()
    extra = os.environ.get("ORACLE_EXTRA_CFLAGS", "").split()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"] + extra + \
          [SRC, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    vp, i, d, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
    lib.oracle_widen.argtypes = [vp, i, i64, vp]
    lib.oracle_attention.argtypes = [vp, vp, vp, i, i, i, i, i, i, d, i, vp, i64, vp, vp, i]
    lib.oracle_probs.argtypes = [vp, vp, i, i, i, i, i, d, i, vp]
    lib.oracle_tiled_fa1.argtypes = [vp, vp, vp, i, i, d, i, i, i, vp, vp]
    lib.oracle_tiled_fa2.argtypes = [vp, vp, vp, i, i, d, i, i, i, vp, vp]
    lib.oracle_paged_decode.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, i, d, vp, vp, i]
    lib.oracle_paged_decode_partitioned.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, i, d, i,
                                                    vp, vp, vp, vp, vp, i]
    lib.oracle_attention_bwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, d, i, vp, i64, vp, i64,
                                         vp, vp, vp, vp, i]
    lib.oracle_attention_ext.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, d, i, i, i, vp, i64, i64,
                                         vp, i64, vp, vp, i]
    lib.oracle_attention_ext.restype = i
    lib.oracle_mask_blocks.argtypes = [vp, i, i, i, i, i64, i64, i64, vp]
    lib.oracle_mask_blocks.restype = i
    lib.oracle_paged_prefill.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, i, i, d, i, vp, vp, i]
    lib.oracle_paged_prefill.restype = i
    lib.oracle_e4m3_encode.argtypes = [vp, i64, vp]
    lib.oracle_e4m3_decode.argtypes = [vp, i64, vp]
    lib.oracle_fp8_codes_len.argtypes = [i, i, i, i, i]
    lib.oracle_fp8_codes_len.restype = i64
    lib.oracle_quant_fp8.argtypes = [vp, i, i, i, i, i, i, vp, vp]
    lib.oracle_dequant_fp8.argtypes = [vp, vp, i, i, i, i, i, vp]
    for name in ("oracle_e4m3_encode", "oracle_e4m3_decode", "oracle_quant_fp8", "oracle_dequant_fp8"):
        getattr(lib, name).restype = i
    for name in ("oracle_widen", "oracle_attention", "oracle_probs", "oracle_tiled_fa1",
                 "oracle_tiled_fa2", "oracle_paged_decode", "oracle_paged_decode_partitioned",
                 "oracle_attention_bwd"):
        getattr(lib, name).restype = i
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def _host(x):
    """(contiguous CPU tensor, dtype code) for a torch tensor or numpy array."""
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    if not isinstance(x, torch.Tensor):
        raise TypeError("expected a tensor or array")
    x = x.detach().cpu().contiguous()
    if x.dtype not in _CODES:
        raise TypeError("unsupported dtype %s" % x.dtype)
    return x, _CODES[x.dtype]


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if isinstance(t, torch.Tensor) else \
        ctypes.c_void_p(t.ctypes.data)


def _check(st, name):
    if st != 0:
        raise ValueError("%s rejected its arguments or ran out of memory" % name)


def widen(x) -> np.ndarray:
    """Exact fp64 values of x (decoded from its storage type by the oracle)."""
    t, code = _host(x)
    out = np.empty(t.numel(), dtype=np.float64)
    _check(_load().oracle_widen(_p(t), code, t.numel(), _p(out)), "oracle_widen")
    return out.reshape(tuple(t.shape))


def attention(q, k, v, scale, causal, rows=None, nthreads=None):
    """Dense attention on q [B, H, N, d] and k, v [B, Hkv, N, d] (Hkv divides H;
    query head h uses kv head h // (H // Hkv)).

    Returns (o [B, H, R, d], lse [B, H, R]) in fp64, R = len(rows) or N.
    """
    qt, code = _host(q)
    kt, c2 = _host(k)
    vt, c3 = _host(v)
    if not (code == c2 == c3) or qt.dim() != 4 or kt.shape != vt.shape or kt.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape, one dtype")
    B, H, N, d = qt.shape
    Hkv = kt.shape[1]
    if (kt.shape[0], kt.shape[2], kt.shape[3]) != (B, N, d) or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")
    if rows is None:
        rarr, R = None, N
    else:
        rarr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = len(rarr)
    o = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    st = _load().oracle_attention(_p(qt), _p(kt), _p(vt), code, B, H, Hkv, N, d, float(scale),
                                  int(bool(causal)),
                                  None if rarr is None else _p(rarr), R, _p(o), _p(lse),
                                  nthreads or default_threads())
    _check(st, "oracle_attention")
    return o, lse


def attention_ext(q, k, v, scale, causal=False, window=(-1, -1), mask=None, rows=None,
                  nthreads=None):
    """Attention of q [B, H, Nq, d] over k, v [B, Hkv, Nk, d] with a bottom-right aligned
    causal mask, a (left, right) window around the diagonal i + Nk - Nq (-1 = unbounded)
    and an optional boolean mask broadcastable to [B, H, Nq, Nk] (True = admissible).

    Returns (o [B, H, R, d], lse [B, H, R]) fp64 for the R selected rows (all Nq if
    rows is None); rows with no admissible key get o = 0 and lse = -inf.
    """
    qt, code = _host(q)
    kt, c2 = _host(k)
    vt, c3 = _host(v)
    if not (code == c2 == c3) or qt.dim() != 4 or kt.shape != vt.shape or kt.dim() != 4:
        raise ValueError("q [B, H, Nq, d] and k, v one [B, Hkv, Nk, d] shape, one dtype")
    B, H, Nq, d = qt.shape
    Hkv, Nk = kt.shape[1], kt.shape[2]
    if kt.shape[0] != B or kt.shape[3] != d or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, Nk, d] with Hkv dividing H")
    m, sb, sh = None, 0, 0
    if mask is not None:
        mt = torch.as_tensor(mask).detach().cpu().to(torch.uint8)
        while mt.dim() < 4:
            mt = mt.unsqueeze(0)
        Bm, Hm = mt.shape[0], mt.shape[1]   # 1 (broadcast) or B / H
        if mt.shape[2:] != (Nq, Nk) or Bm not in (1, B) or Hm not in (1, H):
            raise ValueError("mask must broadcast to [B, H, Nq, Nk]")
        m = mt.contiguous()
        sb = 0 if Bm == 1 else Hm * Nq * Nk
        sh = 0 if Hm == 1 else Nq * Nk
    if rows is None:
        rarr, R = None, Nq
    else:
        rarr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = len(rarr)
    o = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    st = _load().oracle_attention_ext(_p(qt), _p(kt), _p(vt), code, B, H, Hkv, Nq, Nk, d,
                                      float(scale), int(bool(causal)), int(window[0]),
                                      int(window[1]), None if m is None else _p(m), sb, sh,
                                      None if rarr is None else _p(rarr), R,
                                      _p(o), _p(lse), nthreads or default_threads())
    _check(st, "oracle_attention_ext")
    return o, lse


def mask_blocks(mask) -> np.ndarray:
    """Block map of a boolean / uint8 mask [Bm, Hm, Nq, Nk] (fewer leading dims are
    broadcast as 1): uint32 [Bm, Hm, ceil(Nq/128), 2, nkw], nkw = ceil(ceil(Nk/64)/32);
    [.., 0, w] bit i: key block 32w+i of that query block holds a nonzero byte,
    [.., 1, w] bit i: it holds no zero byte."""
    m = np.asarray(mask.cpu() if isinstance(mask, torch.Tensor) else mask)
    while m.ndim < 4:
        m = m[None]
    Bm, Hm, Nq, Nk = m.shape
    # rows padded with a nonzero byte past Nk: padding must not count
    ld = (Nk + 15) // 16 * 16 + 16
    buf = np.full((Bm, Hm, Nq, ld), 7, dtype=np.uint8)
    buf[..., :Nk] = (m != 0).astype(np.uint8) * np.where(np.arange(Nk) % 3 == 0, 1, 255).astype(np.uint8)
    buf = np.ascontiguousarray(buf)
    nqb, nkw = (Nq + 127) // 128, ((Nk + 63) // 64 + 31) // 32
    out = np.zeros((Bm, Hm, nqb, 2, nkw), dtype=np.uint32)
    lib = _load()
    _check(lib.oracle_mask_blocks(buf.ctypes.data, Bm, Hm, Nq, Nk, Hm * Nq * ld, Nq * ld, ld,
                                  out.ctypes.data), "oracle_mask_blocks")
    return out


def attention_bwd(q, k, v, dout, scale, causal, rows=None, keys=None, nthreads=None):
    """Gradients of dense attention for upstream gradient dout [B, H, N, d].

    q, dout [B, H, N, d]; k, v [B, Hkv, N, d] (one storage dtype).  rows
    selects the query rows whose dQ is returned (None: all N; an empty list
    skips dQ), keys the key rows whose dK, dV are returned (None: all N).

    Returns dict(dq [B, H, R, d], dk [B, Hkv, K, d], dv [B, Hkv, K, d],
    D [B, H, N]) in fp64; D_i = sum_j P_ij dP_ij, NaN where no pass needed
    row i.
    """
    qt, code = _host(q)
    kt, c2 = _host(k)
    vt, c3 = _host(v)
    dt, c4 = _host(dout)
    if not (code == c2 == c3 == c4) or qt.dim() != 4 or kt.dim() != 4:
        raise ValueError("q, dout [B, H, N, d] and k, v [B, Hkv, N, d] of one dtype")
    if dt.shape != qt.shape or kt.shape != vt.shape:
        raise ValueError("dout must match q and v must match k")
    B, H, N, d = qt.shape
    Hkv = kt.shape[1]
    if (kt.shape[0], kt.shape[2], kt.shape[3]) != (B, N, d) or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")

    def sel(x):
        if x is None:
            return None, N
        a = np.ascontiguousarray(np.asarray(x, dtype=np.int64).reshape(-1))
        return a, len(a)

    rarr, R = sel(rows)
    karr, K = sel(keys)
    dq = np.empty((B, H, R, d), dtype=np.float64)
    dk = np.empty((B, Hkv, K, d), dtype=np.float64)
    dv = np.empty((B, Hkv, K, d), dtype=np.float64)
    D = np.full((B, H, N), np.nan, dtype=np.float64)
    dummy = np.empty(1, dtype=np.int64)
    st = _load().oracle_attention_bwd(
        _p(qt), _p(kt), _p(vt), _p(dt), code, B, H, Hkv, N, d, float(scale), int(bool(causal)),
        None if rarr is None else _p(rarr if R else dummy), R,
        None if karr is None else _p(karr if K else dummy), K,
        _p(dq) if R else None, _p(dk) if K else None, _p(dv) if K else None, _p(D),
        nthreads or default_threads())
    _check(st, "oracle_attention_bwd")
    return dict(dq=dq, dk=dk, dv=dv, D=D)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 (OCP E4M3FN) codes of fp64 values, round to nearest even, saturating at 448."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint8)
    _check(_load().oracle_e4m3_encode(_p(a), a.size, _p(out)), "oracle_e4m3_encode")
    return out


def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes (NaN for S.1111.111)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    _check(_load().oracle_e4m3_decode(_p(c), c.size, _p(out)), "oracle_e4m3_decode")
    return out


def fp8_codes_shape(layout, B, H, N, d):
    """Shape of the code tensor: [B, H, N, d] (layout 0) or [B, H, ceil(N/64), d, 64] (layout 1)."""
    return (B, H, N, d) if layout == 0 else (B, H, (N + 63) // 64, d, 64)


def quant_fp8(x, layout):
    """Block-scaled E4M3 quantisation of x [B, H, N, d] (128-row blocks, power-of-two scales).

    Returns (codes uint8 of fp8_codes_shape(layout, ...), exps int32 [B, H, ceil(N/128)]).
    """
    t, code = _host(x)
    if t.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = t.shape
    codes = np.empty(fp8_codes_shape(layout, B, H, N, d), dtype=np.uint8)
    exps = np.empty((B, H, (N + 127) // 128), dtype=np.int32)
    _check(_load().oracle_quant_fp8(_p(t), code, B, H, N, d, int(layout), _p(codes), _p(exps)),
           "oracle_quant_fp8")
    return codes, exps


def dequant_fp8(codes, exps, B, H, N, d, layout) -> np.ndarray:
    """fp64 values [B, H, N, d] of block-scaled E4M3 codes (value(code) * 2^e)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    e = np.ascontiguousarray(np.asarray(exps, dtype=np.int32))
    if c.shape != fp8_codes_shape(layout, B, H, N, d) or e.shape != (B, H, (N + 127) // 128):
        raise ValueError("codes / exps shape mismatch")
    out = np.empty((B, H, N, d), dtype=np.float64)
    _check(_load().oracle_dequant_fp8(_p(c), _p(e), B, H, N, d, int(layout), _p(out)),
           "oracle_dequant_fp8")
    return out


def probs(q, k, scale, causal):
    """Full P = softmax(scale Q K^T [+mask]) [B, H, N, N] fp64 (tiny inputs only)."""
    qt, code = _host(q)
    kt, c2 = _host(k)
    if code != c2 or qt.shape != kt.shape or qt.dim() != 4:
        raise ValueError("q, k must share one [B, H, N, d] shape and dtype")
    B, H, N, d = qt.shape
    P = np.empty((B, H, N, N), dtype=np.float64)
    _check(_load().oracle_probs(_p(qt), _p(kt), code, B, H, N, d, float(scale),
                                int(bool(causal)), _p(P)), "oracle_probs")
    return P


def _tiled(fn, q, k, v, scale, causal, Br, Bc):
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    N, d = q.shape
    o = np.empty((N, d), dtype=np.float64)
    lse = np.empty(N, dtype=np.float64)
    _check(fn(_p(q), _p(k), _p(v), N, d, float(scale), int(bool(causal)), int(Br), int(Bc),
              _p(o), _p(lse)), "oracle_tiled")
    return o, lse


def tiled_fa1(q, k, v, scale, causal, Br, Bc):
    """FlashAttention-1 order (KV tiles outer) on one head: (o [N,d], lse [N])."""
    return _tiled(_load().oracle_tiled_fa1, q, k, v, scale, causal, Br, Bc)


def tiled_fa2(q, k, v, scale, causal, Br, Bc):
    """FlashAttention-2 order (Q tiles outer, deferred normalisation) on one head."""
    return _tiled(_load().oracle_tiled_fa2, q, k, v, scale, causal, Br, Bc)


def _dec_args(q, k_cache, v_cache, block_tables, context_lens):
    qt, code = _host(q)
    kt, c2 = _host(k_cache)
    vt, c3 = _host(v_cache)
    if not (code == c2 == c3):
        raise ValueError("q and caches must share a dtype")
    bt = np.ascontiguousarray(torch.as_tensor(block_tables).cpu().numpy().astype(np.int32))
    cl = np.ascontiguousarray(torch.as_tensor(context_lens).cpu().numpy().astype(np.int32))
    S, H, D = qt.shape
    Hkv, BS = kt.shape[1], kt.shape[3]
    return qt, kt, vt, code, bt, cl, S, H, Hkv, D, BS, bt.shape[1]


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale, nthreads=None):
    """Unsplit paged decode: (out [S, H, D], lse [S, H]) fp64."""
    qt, kt, vt, code, bt, cl, S, H, Hkv, D, BS, MB = _dec_args(q, k_cache, v_cache, block_tables,
                                                               context_lens)
    out = np.empty((S, H, D), dtype=np.float64)
    lse = np.empty((S, H), dtype=np.float64)
    st = _load().oracle_paged_decode(_p(qt), _p(kt), _p(vt), code, _p(bt), _p(cl), S, H, Hkv, D,
                                     BS, MB, float(scale), _p(out), _p(lse),
                                     nthreads or default_threads())
    _check(st, "oracle_paged_decode")
    return out, lse


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, scale, causal, nthreads=None):
    """Nq new queries per sequence (q [S, H, Nq, D], the last Nq tokens of each context)
    over the paged cache, bottom-right causal or not: (o [S, H, Nq, D], lse [S, H, Nq]) fp64."""
    qt, code = _host(q)
    kt, c2 = _host(k_cache)
    vt, c3 = _host(v_cache)
    if not (code == c2 == c3):
        raise ValueError("q and caches must share a dtype")
    bt = np.ascontiguousarray(torch.as_tensor(block_tables).cpu().numpy().astype(np.int32))
    cl = np.ascontiguousarray(torch.as_tensor(context_lens).cpu().numpy().astype(np.int32))
    S, H, Nq, D = qt.shape
    Hkv, BS = kt.shape[1], kt.shape[3]
    o = np.empty((S, H, Nq, D), dtype=np.float64)
    lse = np.empty((S, H, Nq), dtype=np.float64)
    st = _load().oracle_paged_prefill(_p(qt), _p(kt), _p(vt), code, _p(bt), _p(cl), S, H, Hkv, Nq, D,
                                      BS, bt.shape[1], float(scale), int(bool(causal)), _p(o), _p(lse),
                                      nthreads or default_threads())
    _check(st, "oracle_paged_prefill")
    return o, lse


def paged_decode_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale, part_tokens,
                             nthreads=None):
    """Partitioned paged decode merged by Eq. (4).

    Returns dict(out, lse, part_m, part_l, part_o) in fp64.
    """
    qt, kt, vt, code, bt, cl, S, H, Hkv, D, BS, MB = _dec_args(q, k_cache, v_cache, block_tables,
                                                               context_lens)
    P = (MB * BS + part_tokens - 1) // part_tokens
    out = np.empty((S, H, D), dtype=np.float64)
    lse = np.empty((S, H), dtype=np.float64)
    pm = np.empty((S, H, P), dtype=np.float64)
    pl = np.empty((S, H, P), dtype=np.float64)
    po = np.empty((S, H, P, D), dtype=np.float64)
    st = _load().oracle_paged_decode_partitioned(
        _p(qt), _p(kt), _p(vt), code, _p(bt), _p(cl), S, H, Hkv, D, BS, MB, float(scale),
        int(part_tokens), _p(out), _p(lse), _p(pm), _p(pl), _p(po), nthreads or default_threads())
    _check(st, "oracle_paged_decode_partitioned")
    return dict(out=out, lse=lse, part_m=pm, part_l=pl, part_o=po)
