"""Pins of the paged-decode oracle.

- The cache layouts and the block-table addressing are checked against the
  page's worked numbers (tests/golden/paged_layout.json) and against an
  independent gather written with numpy reshapes/transposes, whose result is
  fed to the dense oracle (P11: decode equals dense attention on the gathered
  keys and values with one query and no mask).
- Coordinate-encoded caches: with scale 0 the output is the plain mean of the
  value vectors of the context, and with a one-hot query and a dominant key it
  is that key's value vector -- both closed forms over values that name their
  own (block, head, element, slot), so a transposed or mis-strided index shows.
- P6: the partitioned decode merged with Eq. (4) equals the unsplit one for
  every partition size, empty partitions included.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_12_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_layout.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def gather(k_cache, v_cache, table, ctx, kvh):
    """Dense K, V [ctx, D] of one (sequence, kv head), built with reshapes."""
    kc = k_cache[:, kvh]                         # [NB, D/x, BS, x]
    NB, Dx, BS, x = kc.shape
    kt = kc.permute(0, 2, 1, 3).reshape(NB, BS, Dx * x)   # token-major rows
    vt = v_cache[:, kvh].permute(0, 2, 1)        # [NB, BS, D]
    nblk = (ctx + BS - 1) // BS
    ks = torch.cat([kt[int(b)] for b in table[:nblk]], 0)[:ctx] if ctx else kt[:0, 0]
    vs = torch.cat([vt[int(b)] for b in table[:nblk]], 0)[:ctx] if ctx else vt[:0, 0]
    return ks, vs


def small_cfg(**kw):
    base = dict(cid=55, num_seqs=5, num_heads=4, num_kv_heads=4, head_size=128, block_size=16,
                num_blocks=64, ctx_lo=1, ctx_hi=70, dtype=torch.float16)
    base.update(kw)
    return inputs.DecodeConfig(**base)


def test_golden_layout_numbers():
    g = golden()
    fp16 = g["fp16"]
    assert fp16["VEC_SIZE"] * fp16["thread_group_size"] * fp16["element_bytes"] == g["vec_bytes"]
    assert fp16["V_VEC_SIZE"] * fp16["element_bytes"] == g["vec_bytes"]
    assert fp16["x"] == g["vec_bytes"] // fp16["element_bytes"]
    te = g["thread_group_example"]
    for t, els in enumerate(te["elements_of_thread"]):
        assert els == list(range(t, te["head_size"], te["thread_group_size"]))
    be = g["block_example"]
    assert be["block_size"] * be["head_size"] == be["elements_per_block_per_head"]
    qe = g["query_vec_example"]
    assert qe["head_size"] // qe["VEC_SIZE"] == qe["vecs"]
    wb = g["warp_block_example"]
    assert [list(range(w, wb["blocks"], wb["warps"])) for w in range(wb["warps"])] == \
        wb["blocks_of_warp"]
    ve = g["value_example"]
    assert ve["warp_size"] * ve["V_VEC_SIZE"] == ve["elements_per_inner_iteration"]
    assert ve["head_size"] * ve["block_size"] // ve["elements_per_inner_iteration"] == \
        ve["inner_iterations"]


@pytest.mark.parametrize("t0,i0", [(0, 0), (5, 9), (15, 127), (10, 64), (3, 71)])
def test_golden_layout_addresses_pin_oracle(t0, i0):
    # The page's cache layouts, placed element by element from the golden
    # file's shapes and x: K(token t, element i) of kv head h in block b at
    # k_cache[b, h, i // x, t, i % x], V(t, i) at v_cache[b, h, i, t].  A
    # one-hot query on element i0 and a dominant K(t0, i0) (all other keys 0)
    # make the softmax one-hot at t0, so the oracle's output must be the V row
    # stored for token t0, each element naming its own (t, i).
    g = golden()
    assert g["k_cache_shape"] == "[num_blocks, num_kv_heads, head_size/x, block_size, x]"
    assert g["v_cache_shape"] == "[num_blocks, num_kv_heads, head_size, block_size]"
    x = g["fp16"]["x"]
    D, BS = g["block_example"]["head_size"], g["block_example"]["block_size"]
    NB, Hkv, blk, h = 3, 2, 1, 1
    kc = torch.zeros((NB, Hkv, D // x, BS, x), dtype=torch.float16)
    vc = torch.zeros((NB, Hkv, D, BS), dtype=torch.float16)
    for t in range(BS):
        for i in range(D):
            vc[blk, h, i, t] = (t * D + i) / 4.0  # exact in fp16 (at most 11 significant bits)
    kc[blk, h, i0 // x, t0, i0 % x] = 60.0
    q = torch.zeros((1, Hkv, D), dtype=torch.float16)
    q[0, h, i0] = 1.0
    tables = torch.tensor([[blk]], dtype=torch.int32)
    lens = torch.tensor([BS], dtype=torch.int32)
    out, lse = oracle.paged_decode(q, kc, vc, tables, lens, 1.0)
    want = (t0 * D + np.arange(D)) / 4.0
    # the other 15 keys score 0 against 60: relative weight 15 e^-60
    assert np.allclose(out[0, h], want, rtol=0, atol=1e-20 + 600 * 15 * math.exp(-60))
    assert abs(lse[0, h] - (60.0 + math.log1p(15 * math.exp(-60)))) < 1e-12


def test_generator_layout_matches_page():
    g = golden()
    cfg = small_cfg()
    d = inputs.decode_inputs(cfg)
    x = g["fp16"]["x"]
    assert tuple(d["k_cache"].shape) == (cfg.num_blocks, cfg.num_kv_heads, cfg.head_size // x,
                                         cfg.block_size, x)
    assert tuple(d["v_cache"].shape) == (cfg.num_blocks, cfg.num_kv_heads, cfg.head_size,
                                         cfg.block_size)
    assert d["k_cache"][0, 0].numel() == g["block_example"]["elements_per_block_per_head"]


@pytest.mark.parametrize("Hkv", [4, 2, 1])
def test_P11_decode_equals_dense_on_gathered_kv(Hkv):
    cfg = small_cfg(num_kv_heads=Hkv)
    d = inputs.decode_inputs(cfg)
    out, lse = oracle.paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["context_lens"], cfg.scale)
    for s in range(cfg.num_seqs):
        ctx = int(d["context_lens"][s])
        for h in range(cfg.num_heads):
            kvh = h // (cfg.num_heads // Hkv)
            ks, vs = gather(d["k_cache"], d["v_cache"], d["block_tables"][s], ctx, kvh)
            assert not torch.isnan(ks).any() and not torch.isnan(vs).any()
            # one query against ctx keys: repeat it as ctx identical rows
            qq = d["q"][s, h].expand(ctx, -1).contiguous()
            o, l = oracle.attention(qq[None, None], ks[None, None].contiguous(),
                                    vs[None, None].contiguous(), cfg.scale, False, rows=[0])
            assert np.allclose(out[s, h], o[0, 0, 0], rtol=0, atol=1e-13)
            assert abs(lse[s, h] - l[0, 0, 0]) < 1e-12


def _coord_caches(NB, Hkv, D, BS, x):
    """fp64 caches whose every element encodes (block, head, element, slot)."""
    b = torch.arange(NB, dtype=torch.float64).view(NB, 1, 1, 1)
    hh = torch.arange(Hkv, dtype=torch.float64).view(1, Hkv, 1, 1)
    e = torch.arange(D, dtype=torch.float64).view(1, 1, D, 1)
    o = torch.arange(BS, dtype=torch.float64).view(1, 1, 1, BS)
    v = 1000.0 * b + 100.0 * hh + e / 4.0 + o / 64.0          # [NB, Hkv, D, BS]
    k = torch.zeros(NB, Hkv, D // x, BS, x, dtype=torch.float64)
    return k, v


def _v_code(b, hh, e, o):
    return 1000.0 * b + 100.0 * hh + e / 4.0 + o / 64.0


def test_value_addressing_closed_form():
    # scale 0: out = mean over the context of V_t, with V_t[e] = code(block, head, e, slot)
    NB, H, Hkv, D, BS, x = 40, 4, 2, 16, 4, 2   # fp64: x = 16 B / 8 B
    k, v = _coord_caches(NB, Hkv, D, BS, x)
    ctx = [1, 4, 5, 13]
    perm = np.random.default_rng(3).permutation(NB)
    tables = np.zeros((len(ctx), 5), dtype=np.int32)
    pos = 0
    for s, c in enumerate(ctx):
        n = (c + BS - 1) // BS
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    q = torch.ones(len(ctx), H, D, dtype=torch.float64)
    out, lse = oracle.paged_decode(q, k, v, tables, ctx, 0.0)
    for s, c in enumerate(ctx):
        for h in range(H):
            kvh = h // (H // Hkv)
            for e in range(D):
                want = np.mean([_v_code(tables[s, t // BS], kvh, e, t % BS) for t in range(c)])
                assert abs(out[s, h, e] - want) < 1e-9
            assert abs(lse[s, h] - math.log(c)) < 1e-12


def test_key_addressing_one_hot():
    # q = e_c; only token t* has K[c] = 1 (all other keys 0): with a large scale
    # the softmax puts all weight on t*, so out = V_{t*}.  fp64 storage: a
    # 16-byte vector holds x = 2 elements.
    NB, H, Hkv, D, BS, x = 12, 2, 2, 16, 4, 2
    _, v = _coord_caches(NB, Hkv, D, BS, x)
    tables = np.array([[7, 2, 9, 4]], dtype=np.int32)
    ctx = [15]
    rng = np.random.default_rng(11)
    for trial in range(20):
        c = int(rng.integers(D))
        ts = int(rng.integers(ctx[0]))
        h = int(rng.integers(H))
        k = torch.zeros(NB, Hkv, D // x, BS, x, dtype=torch.float64)
        blk, off = int(tables[0, ts // BS]), ts % BS
        k[blk, h, c // x, off, c % x] = 1.0          # page layout, element c of token ts
        q = torch.zeros(1, H, D, dtype=torch.float64)
        q[0, h, c] = 1.0
        out, _ = oracle.paged_decode(q, k, v, tables, ctx, 200.0)
        want = torch.tensor([_v_code(blk, h, e, off) for e in range(D)], dtype=torch.float64)
        assert np.allclose(out[0, h], want.numpy(), rtol=0, atol=1e-9), (c, ts, h)


@pytest.mark.parametrize("part", [1, 7, 16, 33, 64, 1000])
def test_P6_partition_merge_equals_unsplit(part):
    cfg = small_cfg(num_seqs=6, ctx_hi=90)
    d = inputs.decode_inputs(cfg, context_lens=[0, 1, 16, 17, 64, 90])
    ref, lref = oracle.paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                    d["context_lens"], cfg.scale)
    r = oracle.paged_decode_partitioned(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                        d["context_lens"], cfg.scale, part)
    assert np.allclose(r["out"], ref, rtol=0, atol=1e-13)
    ok = np.isfinite(lref)
    assert np.allclose(r["lse"][ok], lref[ok], rtol=0, atol=1e-12)
    ctx = d["context_lens"].numpy()
    for s in range(cfg.num_seqs):
        nparts = (int(ctx[s]) + part - 1) // part
        assert np.all(r["part_l"][s, :, :nparts] >= 1.0)   # the max term contributes e^0
        assert np.all(r["part_m"][s, :, nparts:] == -np.inf)
        assert np.all(r["part_l"][s, :, nparts:] == 0.0)


def test_empty_context_is_zero():
    cfg = small_cfg(num_seqs=3)
    d = inputs.decode_inputs(cfg, context_lens=[0, 5, 0])
    out, lse = oracle.paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["context_lens"], cfg.scale)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(out[1]))


def test_out_of_context_slots_never_read():
    # the generator NaN-fills every element no context token uses
    cfg = small_cfg()
    d = inputs.decode_inputs(cfg)
    out, _ = oracle.paged_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                 d["context_lens"], cfg.scale)
    assert np.all(np.isfinite(out))
