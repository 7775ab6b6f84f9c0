"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic, so the GPU path and the CPU oracle can both read what
it produces.

Recipe (every tensor on the host first, so both sides see identical values):
  seed = 1000 * config_id + t, with t = 0 for Q, 1 for K, 2 for V, 3 for the
  context lengths, 4 for the block permutation, 5 for sampled rows, 6 for the
  decode query, 7 for the upstream gradient dO of the backward pass, 8 for
  sampled keys;
  numpy PCG64 ``standard_normal`` in fp32, times the config's factor, then one
  round-to-nearest-even cast to the element type (``torch.Tensor.to``).
"""
import math
from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["FwdConfig", "FWD_CONFIGS", "FWD_FP32_N256", "FWD_BF16_N2048", "FWD_CAUSAL_N8192",
           "FWD_CAUSAL_N65536", "DecodeConfig", "DECODE_CONFIG", "normal",
           "fwd_inputs", "bwd_dout", "sample_rows", "sample_rows_per_head", "decode_inputs",
           "prefill_queries",
           "PREFILL_CONFIG", "PREFILL_NQ"]


@dataclass(frozen=True)
class FwdConfig:
    """One forward workload: [B, H, N, d] tensors of one element type."""
    cid: int
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    causal: bool
    qk_factor: float = 1.0  # Q and K are drawn N(0,1) * qk_factor
    name: str = ""
    Hkv: int = 0            # kv heads of K and V (0: H, i.e. multi-head)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Matmul flop count 4*B*H*N^2*d, halved for causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def replace(self, **kw) -> "FwdConfig":
        args = dict(cid=self.cid, B=self.B, H=self.H, N=self.N, d=self.d, dtype=self.dtype,
                    causal=self.causal, qk_factor=self.qk_factor, name=self.name, Hkv=self.Hkv)
        args.update(kw)
        return FwdConfig(**args)


# the forward workloads, named by what they are (the first field seeds the inputs)
FWD_FP32_N256 = FwdConfig(1, 1, 1, 256, 64, torch.float32, False, 1.0, "B1 H1 N256 d64 fp32")
FWD_BF16_N2048 = FwdConfig(2, 4, 16, 2048, 64, torch.bfloat16, False, 1.0, "B4 H16 N2048 d64 bf16")
FWD_CAUSAL_N8192 = FwdConfig(3, 2, 32, 8192, 128, torch.bfloat16, True, 1.0,
                             "B2 H32 N8192 d128 bf16 causal")  # the benchmark's forward workload
FWD_CAUSAL_N65536 = FwdConfig(4, 1, 8, 65536, 128, torch.bfloat16, True, 2.0,
                              "B1 H8 N65536 d128 bf16 causal, Q,K x2")
FWD_CONFIGS = {c.cid: c for c in (FWD_FP32_N256, FWD_BF16_N2048, FWD_CAUSAL_N8192, FWD_CAUSAL_N65536)}
# grouped-query forward: the causal N=8192 workload with 8 kv heads (4 query heads per kv head)
FWD_GQA_CONFIG = FwdConfig(7, 2, 32, 8192, 128, torch.bfloat16, True, 1.0,
                           "B2 H32 Hkv8 N8192 d128 bf16 causal", Hkv=8)


def normal(seed: int, shape, factor: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """N(0,1) * factor drawn in fp32 from PCG64(seed), cast (RNE) to dtype; CPU tensor."""
    x = np.random.default_rng(seed).standard_normal(size=tuple(shape), dtype=np.float32)
    if factor != 1.0:
        x *= np.float32(factor)
    return torch.from_numpy(x).to(dtype)


def fwd_inputs(cfg: FwdConfig):
    """(q, k, v) CPU tensors of cfg.dtype: q [B, H, N, d], k and v [B, Hkv, N, d]."""
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    kv_shape = (cfg.B, cfg.kv_heads, cfg.N, cfg.d)
    base = 1000 * cfg.cid
    q = normal(base + 0, shape, cfg.qk_factor, cfg.dtype)
    k = normal(base + 1, kv_shape, cfg.qk_factor, cfg.dtype)
    v = normal(base + 2, kv_shape, 1.0, cfg.dtype)
    return q, k, v


def bwd_dout(cfg: FwdConfig) -> torch.Tensor:
    """Upstream gradient dO [B, H, N, d] of cfg.dtype, N(0,1); CPU tensor."""
    return normal(1000 * cfg.cid + 7, (cfg.B, cfg.H, cfg.N, cfg.d), 1.0, cfg.dtype)


def sample_rows(N: int, count: int = 256, seed: int = 5) -> np.ndarray:
    """Sorted query rows: {0, 1, 127, 128, N-1} (where < N) plus random distinct rows."""
    fixed = sorted({r for r in (0, 1, 127, 128, N - 1) if 0 <= r < N})
    if count >= N:
        return np.arange(N, dtype=np.int64)
    rest = np.setdiff1d(np.arange(N, dtype=np.int64), np.array(fixed, dtype=np.int64))
    extra = np.random.default_rng(seed).choice(rest, size=count - len(fixed), replace=False)
    return np.sort(np.concatenate([np.array(fixed, dtype=np.int64), extra]))


def sample_rows_per_head(N: int, heads: int, count: int, seed: int, tile: int = 128) -> np.ndarray:
    """Sorted query rows drawn independently for each of `heads` heads: [heads, count].

    Every head gets {0, 1, 127, 128, N-1} (where < N) and the rest stratified
    over the `tile`-row query tiles: each tile contributes the same number of
    distinct rows (tiles drawn at random for the remainder), so with count >=
    ceil(N / tile) every tile of every head is checked.  Head x draws from
    PCG64([seed, x]).
    """
    if count >= N:
        return np.tile(np.arange(N, dtype=np.int64), (heads, 1))
    fixed = sorted({r for r in (0, 1, 127, 128, N - 1) if 0 <= r < N})
    ntiles = (N + tile - 1) // tile
    out = np.empty((heads, count), dtype=np.int64)
    for x in range(heads):
        rng = np.random.default_rng([seed, x])
        chosen = set(fixed)
        need = count - len(chosen)
        per, extra = divmod(need, ntiles)
        bonus = set(rng.choice(ntiles, size=extra, replace=False).tolist()) if extra else set()
        short = 0
        for t in range(ntiles):
            lo, hi = t * tile, min(N, (t + 1) * tile)
            free = np.setdiff1d(np.arange(lo, hi, dtype=np.int64), np.array(sorted(chosen), dtype=np.int64))
            want = per + (1 if t in bonus else 0)
            take = min(want, len(free))
            short += want - take
            if take:
                chosen.update(rng.choice(free, size=take, replace=False).tolist())
        if short:  # a tile had fewer free rows than its share: fill from the rest
            free = np.setdiff1d(np.arange(N, dtype=np.int64), np.array(sorted(chosen), dtype=np.int64))
            chosen.update(rng.choice(free, size=short, replace=False).tolist())
        out[x] = np.sort(np.fromiter(chosen, dtype=np.int64))
    return out


@dataclass(frozen=True)
class DecodeConfig:
    """Paged single-query decode workload."""
    cid: int = 5
    num_seqs: int = 64
    num_heads: int = 32
    num_kv_heads: int = 32
    head_size: int = 128
    block_size: int = 16
    num_blocks: int = 20000
    ctx_lo: int = 512
    ctx_hi: int = 4096
    dtype: torch.dtype = torch.float16
    name: str = "64 seqs, 32 heads, head 128, fp16, block 16, ctx U[512,4096], 20000-block pool"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_size)

    @property
    def max_blocks_per_seq(self) -> int:
        return (self.ctx_hi + self.block_size - 1) // self.block_size

    def replace(self, **kw) -> "DecodeConfig":
        args = {f: getattr(self, f) for f in self.__dataclass_fields__}
        args.update(kw)
        return DecodeConfig(**args)


DECODE_CONFIG = DecodeConfig()
# grouped-query variant: 4 query heads per kv head
DECODE_GQA_CONFIG = DecodeConfig(cid=6, num_kv_heads=8,
                                 name="64 seqs, 32 query heads / 8 kv heads, head 128, fp16, block 16, "
                                      "ctx U[512,4096], 20000-block pool")


# chunked prefill over the paged cache: 16 sequences, 512 new tokens each at
# the end of a context of U[1024, 4096] tokens, 32 query heads over 8 kv heads
PREFILL_CONFIG = DecodeConfig(cid=10, num_seqs=16, num_heads=32, num_kv_heads=8, ctx_lo=1024,
                              ctx_hi=4096, dtype=torch.bfloat16,
                              name="16 seqs x 512 new tokens, 32 query heads / 8 kv heads, head 128, "
                                   "bf16, block 16, ctx U[1024,4096], 20000-block pool")
PREFILL_NQ = 512


def prefill_queries(cfg: DecodeConfig, Nq: int) -> torch.Tensor:
    """Queries [S, H, Nq, D] of a chunked prefill over the cache of decode_inputs(cfg):
    the last Nq tokens of each sequence's context, N(0,1) in cfg.dtype (CPU)."""
    return normal(1000 * cfg.cid + 7, (cfg.num_seqs, cfg.num_heads, Nq, cfg.head_size), 1.0, cfg.dtype)


def decode_inputs(cfg: DecodeConfig = DECODE_CONFIG, context_lens=None):
    """Paged-cache inputs as CPU tensors.

    Returns dict(q [S,H,D], k_cache [NB,Hkv,D/x,BS,x], v_cache [NB,Hkv,D,BS],
    block_tables [S, max_blocks] int32, context_lens [S] int32, max_context_len).
    Context lengths are integers uniform in [ctx_lo, ctx_hi] (both inclusive)
    unless given.  One seeded permutation of the pool hands each sequence its
    next ceil(ctx/BS) blocks in order.  Every pool element that no context
    token uses -- whole unused blocks and the slots past the end of a
    sequence's last block -- is NaN, and unused table entries point at an
    all-NaN block, so any read outside the context poisons the output.
    """
    S, H, Hkv, D, BS, NB = (cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size,
                            cfg.block_size, cfg.num_blocks)
    esize = torch.empty((), dtype=cfg.dtype).element_size()
    x = 16 // esize
    base = 1000 * cfg.cid
    if context_lens is None:
        ctx = np.random.default_rng(base + 3).integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=S)
    else:
        ctx = np.asarray(context_lens, dtype=np.int64)
    mb = max(1, cfg.max_blocks_per_seq, int((ctx.max() + BS - 1) // BS) if len(ctx) else 1)
    nblk = (ctx + BS - 1) // BS
    total = int(nblk.sum())
    if total >= NB:
        raise ValueError("pool of %d blocks cannot hold %d used blocks plus a NaN block"
                         % (NB, total))
    perm = np.random.default_rng(base + 4).permutation(NB)
    nan_block = int(perm[-1])
    tables = np.full((S, mb), nan_block, dtype=np.int32)
    pos = 0
    for s in range(S):
        n = int(nblk[s])
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    used = torch.from_numpy(perm[:total].astype(np.int64))

    k_cache = torch.full((NB, Hkv, D // x, BS, x), float("nan"), dtype=cfg.dtype)
    v_cache = torch.full((NB, Hkv, D, BS), float("nan"), dtype=cfg.dtype)
    if total:
        k_cache[used] = normal(base + 1, (total, Hkv, D // x, BS, x), 1.0, cfg.dtype)
        v_cache[used] = normal(base + 2, (total, Hkv, D, BS), 1.0, cfg.dtype)
    # NaN the slots past each context's end inside its last block
    for s in range(S):
        n, c = int(nblk[s]), int(ctx[s])
        if n and c % BS:
            blk = int(tables[s, n - 1])
            k_cache[blk, :, :, c % BS:, :] = float("nan")
            v_cache[blk, :, :, c % BS:] = float("nan")
    q = normal(base + 6, (S, H, D), 1.0, cfg.dtype)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=torch.from_numpy(tables),
                context_lens=torch.from_numpy(ctx.astype(np.int32)),
                max_context_len=int(ctx.max()) if len(ctx) else 0)
