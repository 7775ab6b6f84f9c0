"""exact_attention_12_amd -- exact attention on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libfa.so`` (C ABI in ``include/fa.h``).  The
functions named like the C entry points (``fa_fwd``, ``fa_fwd_gqa``,
``fa_bwd``, ``fa_bwd_workspace_size``, ``fa_paged_decode``,
``fa_paged_decode_workspace_size``, ``fa_strerror``) only marshal arguments:
every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and streams.  ``forward``, ``backward`` and
``paged_decode`` are conveniences that allocate the outputs and call those
entry points.

There is no fallback: if ``libfa.so`` is missing or fails to load, every call
raises.
"""
import ctypes
import math
import os

import torch

__all__ = [
    "FA_F32", "FA_BF16", "FA_F16", "FA_DECODE_PARTITION_TOKENS", "FAError", "fa_fwd_gqa",
    "fa_fwd", "fa_fwd_ext", "forward_ext", "fa_bwd", "fa_bwd_workspace_size", "fa_fp8_codes_bytes", "fa_quant_fp8",
    "fa_fwd_fp8", "fa_paged_decode", "fa_paged_decode_workspace_size", "fa_strerror", "forward",
    "backward", "quant_fp8", "forward_fp8", "paged_decode", "lib_path", "load_library",
    "FA_FP8_BLOCK_ROWS", "FA_MASK_BLOCK_ROWS", "FA_MASK_BLOCK_COLS", "fa_mask_blocks_words",
    "fa_mask_blocks", "mask_block_map", "fa_fwd_paged", "forward_paged", "fa_paged_decode_noalloc",
    "FA_DECODE_NOALLOC_SCRATCH_BYTES",
]

FA_F32, FA_BF16, FA_F16 = 0, 1, 2
FA_DECODE_PARTITION_TOKENS = 256  # must match include/fa.h
FA_MASK_BLOCK_ROWS, FA_MASK_BLOCK_COLS = 128, 64  # must match include/fa.h
FA_FP8_BLOCK_ROWS = 128           # must match include/fa.h
FA_DECODE_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # must match include/fa.h

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_DTYPE_CODE = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.float16: FA_F16}


class FAError(RuntimeError):
    """A non-zero status returned by libfa.so."""

    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, fa_strerror(status), status))


def lib_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def load_debug_library(path):
    """Bind another build of the C ABI (the LDS-poisoning debug build); returns
    the handle without replacing the product library."""
    import ctypes
    return _bind(ctypes.CDLL(path))


def load_library():
    """Load libfa.so once; raise if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            "libfa.so is not built (expected at %s); build it with "
            "`python -m exact_attention_12_amd.build`" % path)
    _LIB = _bind(ctypes.CDLL(path))
    return _LIB


def _bind(lib):
    """Declare the argument and result types of every entry point on a loaded library."""
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_gqa.restype = i
    i64 = ctypes.c_int64
    lib.fa_fwd_ext.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, i64, i64, i64, vp,
                               i, vp]
    lib.fa_fwd_ext.restype = i
    lib.fa_mask_blocks_words.argtypes = [i, i, i, i, i64, i64]
    lib.fa_mask_blocks_words.restype = sz
    lib.fa_mask_blocks.argtypes = [vp, i, i, i, i, i64, i64, i64, vp, sz, vp]
    lib.fa_mask_blocks.restype = i
    lib.fa_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_paged.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_fp8_codes_bytes.argtypes = [i, i, i, i, i]
    lib.fa_fp8_codes_bytes.restype = sz
    lib.fa_quant_fp8.argtypes = [vp, i, i, i, i, i, i, vp, vp, vp]
    lib.fa_quant_fp8.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_paged_decode_workspace_size.argtypes = [i, i, i, i]
    lib.fa_paged_decode_workspace_size.restype = sz
    lib.fa_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_paged_decode.restype = i
    lib.fa_paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_paged_decode_noalloc.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(dtype):
    try:
        return _DTYPE_CODE[dtype]
    except KeyError:
        raise TypeError("unsupported element type %s" % dtype) from None


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype=None, stream=None):
    """C entry point ``fa_fwd``: enqueue the forward pass on ``stream``.

    q, k, v: [B, H, N, d] device tensors (or raw device addresses) of one
    element type; o: [B, H, N, d] fp32; lse: [B, H, N] fp32.  ``dtype``
    defaults to q's element type.
    """
    if dtype is None:
        dtype = _dtype_code(q.dtype)
    st = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                               int(N), int(d), float(scale), int(bool(causal)), int(dtype),
                               _stream(stream))
    if st != 0:
        raise FAError(st, "fa_fwd")


def fa_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, dtype=None, stream=None):
    """C entry point ``fa_fwd_gqa``: fa_fwd with k, v of Hkv heads ([B, Hkv, N, d])."""
    if dtype is None:
        dtype = _dtype_code(q.dtype)
    st = load_library().fa_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                   int(Hkv), int(N), int(d), float(scale), int(bool(causal)),
                                   int(dtype), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_fwd_gqa")


def fa_fwd_ext(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window_left=-1,
               window_right=-1, mask=None, mask_stride_b=0, mask_stride_h=0, mask_ld=None,
               mask_blocks=None, dtype=None, stream=None):
    """C entry point ``fa_fwd_ext``: rectangular / windowed / boolean-masked forward
    (``mask_blocks``: the mask's block map from ``fa_mask_blocks``, or None)."""
    if dtype is None:
        dtype = _dtype_code(q.dtype)
    st = load_library().fa_fwd_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                   int(Hkv), int(Nq), int(Nk), int(d), float(scale),
                                   int(bool(causal)), int(window_left), int(window_right),
                                   _ptr(mask), int(mask_stride_b), int(mask_stride_h),
                                   int(Nk if mask_ld is None else mask_ld), _ptr(mask_blocks),
                                   int(dtype), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_fwd_ext")


def fa_fwd_paged(q, k_cache, v_cache, block_tables, context_lens, o, lse, num_seqs, num_heads,
                 num_kv_heads, Nq, head_size, block_size, num_blocks, max_blocks_per_seq, scale,
                 causal, dtype=None, stream=None):
    """C entry point ``fa_fwd_paged``: Nq new queries per sequence over the paged cache."""
    if dtype is None:
        dtype = _dtype_code(q.dtype)
    st = load_library().fa_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                     _ptr(context_lens), _ptr(o), _ptr(lse), int(num_seqs),
                                     int(num_heads), int(num_kv_heads), int(Nq), int(head_size),
                                     int(block_size), int(num_blocks), int(max_blocks_per_seq),
                                     float(scale), int(bool(causal)), int(dtype), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_fwd_paged")


def fa_mask_blocks_words(B, H, Nq, Nk, mask_stride_b, mask_stride_h) -> int:
    """C entry point ``fa_mask_blocks_words`` (uint32 words of the map; 0 if invalid)."""
    return int(load_library().fa_mask_blocks_words(int(B), int(H), int(Nq), int(Nk),
                                                   int(mask_stride_b), int(mask_stride_h)))


def fa_mask_blocks(mask, B, H, Nq, Nk, mask_stride_b, mask_stride_h, mask_ld, blocks,
                   blocks_words=None, stream=None):
    """C entry point ``fa_mask_blocks``: the block map of a uint8 mask into ``blocks``."""
    if blocks_words is None:
        blocks_words = blocks.numel() if isinstance(blocks, torch.Tensor) else 0
    st = load_library().fa_mask_blocks(_ptr(mask), int(B), int(H), int(Nq), int(Nk),
                                       int(mask_stride_b), int(mask_stride_h), int(mask_ld),
                                       _ptr(blocks), int(blocks_words), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_mask_blocks")


def fa_bwd_workspace_size(B, H, N) -> int:
    """C entry point ``fa_bwd_workspace_size`` (bytes; 0 if invalid)."""
    return int(load_library().fa_bwd_workspace_size(int(B), int(H), int(N)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, scale, causal, workspace,
           workspace_bytes=None, dtype=None, stream=None):
    """C entry point ``fa_bwd``: enqueue the backward pass on ``stream``.

    q, dout [B, H, N, d] and k, v [B, Hkv, N, d] of one 16-bit element type;
    o [B, H, N, d] and lse [B, H, N] fp32 from the forward pass; dq, dk, dv
    fp32 outputs shaped like q, k, v.
    """
    if dtype is None:
        dtype = _dtype_code(q.dtype)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load_library().fa_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        int(B), int(H), int(Hkv), int(N), int(d), float(scale), int(bool(causal)), int(dtype),
        _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_bwd")


def fa_fp8_codes_bytes(B, H, N, d, layout) -> int:
    """C entry point ``fa_fp8_codes_bytes`` (bytes; 0 if invalid)."""
    return int(load_library().fa_fp8_codes_bytes(int(B), int(H), int(N), int(d), int(layout)))


def fa_quant_fp8(x, B, H, N, d, layout, codes, exps, dtype=None, stream=None):
    """C entry point ``fa_quant_fp8``: block-scaled E4M3 codes and exponents of x."""
    if dtype is None:
        dtype = _dtype_code(x.dtype)
    st = load_library().fa_quant_fp8(_ptr(x), int(dtype), int(B), int(H), int(N), int(d),
                                     int(layout), _ptr(codes), _ptr(exps), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_quant_fp8")


def fa_fwd_fp8(q8, k8, v8, q_exp, k_exp, v_exp, o, lse, B, H, Hkv, N, d, scale, causal,
               stream=None):
    """C entry point ``fa_fwd_fp8``: the forward pass on block-scaled E4M3 inputs."""
    st = load_library().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_exp), _ptr(k_exp),
                                   _ptr(v_exp), _ptr(o), _ptr(lse), int(B), int(H), int(Hkv),
                                   int(N), int(d), float(scale), int(bool(causal)), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_fwd_fp8")


def fa_paged_decode_workspace_size(num_seqs, num_heads, head_size, max_context_len) -> int:
    """C entry point ``fa_paged_decode_workspace_size`` (bytes; 0 if invalid)."""
    return int(load_library().fa_paged_decode_workspace_size(
        int(num_seqs), int(num_heads), int(head_size), int(max_context_len)))


def fa_paged_decode(q, k_cache, v_cache, block_tables, context_lens, out, num_seqs, num_heads,
                    num_kv_heads, head_size, block_size, max_blocks_per_seq, max_context_len,
                    scale, workspace, workspace_bytes=None, dtype=None, stream=None):
    """C entry point ``fa_paged_decode``: enqueue the paged decode on ``stream``."""
    if dtype is None:
        dtype = _dtype_code(q.dtype)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load_library().fa_paged_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(out),
        int(num_seqs), int(num_heads), int(num_kv_heads), int(head_size), int(block_size),
        int(max_blocks_per_seq), int(max_context_len), float(scale), int(dtype),
        _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_paged_decode")


def fa_paged_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, out, num_seqs,
                            num_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                            max_context_len, scale, dtype=None, stream=None):
    """C entry point ``fa_paged_decode_noalloc``: the paged decode without a workspace
    (its partials go to the library's own per-device scratch); allocates nothing."""
    if dtype is None:
        dtype = _dtype_code(q.dtype)
    st = load_library().fa_paged_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(out),
        int(num_seqs), int(num_heads), int(num_kv_heads), int(head_size), int(block_size),
        int(max_blocks_per_seq), int(max_context_len), float(scale), int(dtype), _stream(stream))
    if st != 0:
        raise FAError(st, "fa_paged_decode_noalloc")


def _check_dev(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def forward(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """Allocate o (fp32) and lse (fp32) and run ``fa_fwd`` (``fa_fwd_gqa`` when
    k and v have fewer heads than q); returns (o, lse)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d) or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_dev("out", out, torch.float32)
    _check_dev("lse", lse, torch.float32)
    if Hkv == H:
        fa_fwd(q, k, v, out, lse, B, H, N, d, scale, causal, stream=stream)
    else:
        fa_fwd_gqa(q, k, v, out, lse, B, H, Hkv, N, d, scale, causal, stream=stream)
    return out, lse


def _padded_mask(mask, B, H, Nq, Nk):
    """A boolean / uint8 mask broadcastable to [B, H, Nq, Nk] as the C ABI takes it:
    uint8 rows padded to a multiple of 16 bytes.  Returns (mask, stride_b, stride_h, ld)."""
    m = mask
    while m.dim() < 4:
        m = m.unsqueeze(0)
    if m.shape[2:] != (Nq, Nk) or m.shape[0] not in (1, B) or m.shape[1] not in (1, H):
        raise ValueError("mask must broadcast to [B, H, Nq, Nk]")
    # rows padded to a multiple of 16 bytes, as the kernel streams 16-byte chunks
    ldm = (Nk + 15) // 16 * 16
    padded = torch.zeros(m.shape[:3] + (ldm,), dtype=torch.uint8, device=m.device)
    padded[..., :Nk] = m.to(torch.uint8)
    sb = 0 if m.shape[0] == 1 else m.shape[1] * Nq * ldm
    sh = 0 if m.shape[1] == 1 else Nq * ldm
    _check_dev("mask", padded, torch.uint8)
    return padded, sb, sh, ldm


def mask_block_map(mask, B, H, Nq, Nk, stream=None):
    """Block map (``fa_mask_blocks``) of a boolean / uint8 mask broadcastable to
    [B, H, Nq, Nk], as an int32 tensor to pass to ``forward_ext(block_map=...)``."""
    padded, sb, sh, ldm = _padded_mask(mask, B, H, Nq, Nk)
    words = fa_mask_blocks_words(B, H, Nq, Nk, sb, sh)
    blocks = torch.empty(words, dtype=torch.int32, device=padded.device)
    fa_mask_blocks(padded, B, H, Nq, Nk, sb, sh, ldm, blocks, words, stream=stream)
    return blocks


def forward_ext(q, k, v, scale=None, causal=False, window=(-1, -1), mask=None, block_map=None,
                stream=None):
    """Allocate o, lse and run ``fa_fwd_ext``: q [B, H, Nq, d], k, v [B, Hkv, Nk, d], a
    bottom-right aligned causal mask, a (left, right) window (-1 = unbounded) and an
    optional boolean / uint8 mask broadcastable to [B, H, Nq, Nk] (True = takes part).
    block_map: None, True (compute the mask's block map first) or the tensor that
    ``mask_block_map`` returned for this mask."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, Nk, d] with Hkv dividing H")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sb = sh = 0
    ldm = None
    blocks = None
    if mask is not None:
        mask, sb, sh, ldm = _padded_mask(mask, B, H, Nq, Nk)
        if block_map is True:
            blocks = torch.empty(fa_mask_blocks_words(B, H, Nq, Nk, sb, sh), dtype=torch.int32,
                                 device=mask.device)
            fa_mask_blocks(mask, B, H, Nq, Nk, sb, sh, ldm, blocks, stream=stream)
        elif block_map is not None:
            blocks = block_map
            if blocks.numel() < fa_mask_blocks_words(B, H, Nq, Nk, sb, sh):
                raise ValueError("block_map is smaller than the map of this mask")
            _check_dev("block_map", blocks, torch.int32)
    elif block_map is not None:
        raise ValueError("block_map needs a mask")
    o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_ext(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window[0], window[1], mask,
               sb, sh, ldm, mask_blocks=blocks, stream=stream)
    return o, lse


def forward_paged(q, k_cache, v_cache, block_tables, context_lens, scale=None, causal=True,
                  stream=None):
    """Allocate o, lse and run ``fa_fwd_paged``: q [S, H, Nq, D] (the last Nq tokens of
    each context), caches as for ``paged_decode``; returns (o, lse)."""
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_dev(n, t, q.dtype)
    _check_dev("block_tables", block_tables, torch.int32)
    _check_dev("context_lens", context_lens, torch.int32)
    if q.dim() != 4 or k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("q must be [S, H, Nq, D], k_cache [blocks, Hkv, D/x, BS, x], "
                         "v_cache [blocks, Hkv, D, BS]")
    S, H, Nq, D = q.shape
    NB, Hkv, BS = k_cache.shape[0], k_cache.shape[1], k_cache.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((S, H, Nq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((S, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_paged(q, k_cache, v_cache, block_tables, context_lens, o, lse, S, H, Hkv, Nq, D, BS, NB,
                 block_tables.shape[1], scale, causal, stream=stream)
    return o, lse


def backward(q, k, v, o, lse, dout, scale=None, causal=False, workspace=None, stream=None):
    """Allocate dq, dk, dv (fp32) and the workspace and run ``fa_bwd``;
    returns (dq, dk, dv).  o and lse are ``forward``'s outputs."""
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_dev(n, t, q.dtype)
    _check_dev("o", o, torch.float32)
    _check_dev("lse", lse, torch.float32)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or dout.shape != q.shape:
        raise ValueError("q, dout must be [B, H, N, d] and k, v one [B, Hkv, N, d] shape")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d) or H % Hkv != 0:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")
    if o.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("o must be [B, H, N, d] and lse [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_size(B, H, N), 256), dtype=torch.uint8,
                                device=q.device)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, scale, causal, workspace,
           stream=stream)
    return dq, dk, dv


def quant_fp8(x, layout, stream=None):
    """Allocate and fill the E4M3 codes (uint8, flat) and block exponents (int32
    [B, H, ceil(N/128)]) of x [B, H, N, d]; layout 0 for q and k, 1 for v."""
    _check_dev("x", x)
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    codes = torch.empty(max(fa_fp8_codes_bytes(B, H, N, d, layout), 16), dtype=torch.uint8,
                        device=x.device)
    exps = torch.empty((B, H, (N + FA_FP8_BLOCK_ROWS - 1) // FA_FP8_BLOCK_ROWS),
                       dtype=torch.int32, device=x.device)
    fa_quant_fp8(x, B, H, N, d, layout, codes, exps, stream=stream)
    return codes, exps


def forward_fp8(q8, k8, v8, q_exp, k_exp, v_exp, B, H, Hkv, N, d=128, scale=None, causal=False,
                stream=None):
    """Allocate o (fp32) and lse (fp32) and run ``fa_fwd_fp8``; returns (o, lse)."""
    for n, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check_dev(n, t, torch.uint8)
    for n, t in (("q_exp", q_exp), ("k_exp", k_exp), ("v_exp", v_exp)):
        _check_dev(n, t, torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v8, q_exp, k_exp, v_exp, o, lse, B, H, Hkv, N, d, scale, causal,
               stream=stream)
    return o, lse


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale=None,
                 out=None, workspace=None, stream=None):
    """Allocate out and the workspace and run ``fa_paged_decode``; returns out."""
    _check_dev("q", q)
    _check_dev("k_cache", k_cache, q.dtype)
    _check_dev("v_cache", v_cache, q.dtype)
    _check_dev("block_tables", block_tables, torch.int32)
    _check_dev("context_lens", context_lens, torch.int32)
    S, H, D = q.shape
    num_kv_heads = k_cache.shape[1]
    block_size = k_cache.shape[3]
    mbs = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = fa_paged_decode_workspace_size(S, H, D, max_context_len)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    fa_paged_decode(q, k_cache, v_cache, block_tables, context_lens, out, S, H, num_kv_heads, D,
                    block_size, mbs, max_context_len, scale, workspace, stream=stream)
    return out
