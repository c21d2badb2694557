"""Seeded sweeps over shapes and options of every attention entry point, against the fp64 oracle.

Each case draws its configuration from a seeded generator (batch, heads and group size up to 64
query heads per KV head, lengths that are not tile multiples, head dim, window, position offset,
output dtype, key mode, split count, block size, per-sequence chunk starts, one of them sometimes
out of range) and checks the HIP result with the bf16 bars; the per-sequence sweep also appends
each sequence's next token and decodes it.  The configuration is printed before each launch.
"""

import numpy as np
import pytest
import torch

import oracle
from conftest import assert_bf16_parity, banner, to_np
from transformer_self_attention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_self_attention_amd import lib as L
    return L


def _heads(rng):
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 8, 16, 20, 32, 48, 64]))
    return Hkv * G, Hkv


@pytest.mark.parametrize("seed", range(40))
def test_prefill_sweep(lib, seed):
    rng = np.random.default_rng(1000 + seed)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 3))
    S = int(rng.integers(1, 600))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.8)
    W = int(rng.integers(0, S + 40)) if causal and rng.random() < 0.5 else None
    pos0 = int(rng.integers(0, 3000))
    mode = str(rng.choice(["workspace", "fused", "norope"]))
    out_dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    banner(f"prefill sweep seed={seed}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} W={W} "
           f"pos0={pos0} mode={mode} out={out_dtype}")
    wl = inputs.Workload("s", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=2000 + seed, kind="prefill")
    p = inputs.make_prefill(wl)
    rope = mode != "norope"
    tab = lib.make_rope_table(pos0 + S, D) if rope else None
    ws = None
    if mode == "workspace":
        ws = torch.empty(lib.prefill_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    o = lib.prefill(p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda"), tab, causal=causal,
                    pos0=pos0 if rope else 0, window=W, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(p.q.f64(), p.k.f64(), p.v.f64(), causal=causal, rope_base=10000.0 if rope else None,
                              pos0=pos0 if rope else 0, window=W)
    assert_bf16_parity(to_np(o), ref, "o")


@pytest.mark.parametrize("seed", range(40))
def test_decode_sweep(lib, seed):
    rng = np.random.default_rng(3000 + seed)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 6))
    S = int(rng.integers(1, 3000))
    D = int(rng.choice([64, 128]))
    lens = rng.integers(0, S + 1, size=B).astype(np.int32)
    qpos = (lens + rng.integers(0, 5, size=B)).astype(np.int32)
    W = int(rng.integers(0, S + 10)) if rng.random() < 0.4 else None
    n_split = int(rng.choice([0, 0, 1, 2, 5]))
    paged = bool(rng.random() < 0.5)
    bs = int(rng.choice([16, 32, 64]))
    banner(f"decode sweep seed={seed}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} lens={lens.tolist()} W={W} "
           f"n_split={n_split} paged={paged} bs={bs}")
    wl = inputs.Workload("d", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=4000 + seed, kind="decode")
    tab = lib.make_rope_table(int(qpos.max()) + 1, D)
    cl = torch.from_numpy(lens).cuda()
    qp = torch.from_numpy(qpos).cuda()
    if paged:
        pd = inputs.make_paged_decode(wl, block_size=bs, cache_len=lens, q_pos=qpos)
        o = lib.decode_paged(pd.q.torch("cuda"), pd.k_pages.torch("cuda"), pd.v_pages.torch("cuda"),
                             torch.from_numpy(pd.block_table).cuda(), cl, qp, tab, n_split=n_split, window=W,
                             out_dtype=torch.float32)
        d = pd.contiguous
    else:
        d = inputs.make_decode(wl, cache_len=lens, q_pos=qpos)
        o = lib.decode(d.q.torch("cuda"), d.k_cache.torch("cuda"), d.v_cache.torch("cuda"), cl, qp, tab,
                       n_split=n_split, window=W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(d.q.f64(), d.k_cache.f32, d.v_cache.f32, lens, qpos, window=W)
    got = to_np(o)
    empty = np.isneginf(ref_lse)
    assert np.all(got[empty] == 0.0)
    assert_bf16_parity(got, ref, "o")


@pytest.mark.parametrize("seed", range(24))
def test_chunk_sweep(lib, seed):
    rng = np.random.default_rng(5000 + seed)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 3))
    Sq = int(rng.integers(1, 400))
    pos0 = int(rng.integers(0, 900))
    S_max = pos0 + Sq + int(rng.integers(0, 50))
    D = int(rng.choice([64, 128]))
    W = int(rng.integers(0, pos0 + Sq + 10)) if rng.random() < 0.4 else None
    rope = bool(rng.random() < 0.8)
    banner(f"chunk sweep seed={seed}: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} pos0={pos0} S_max={S_max} D={D} "
           f"W={W} rope={rope}")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=6000 + seed, kind="chunk",
                         pos0=pos0, S_max=S_max)
    c = inputs.make_chunk(wl)
    tab = lib.make_rope_table(S_max, D) if rope else None
    kc, vc = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    o = lib.prefill_chunk(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"), kc, vc, pos0, tab,
                          window=W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    base = 10000.0 if rope else None
    ref_k, ref_v = oracle.append_to_cache(c.k_cache.f64(), c.v_cache.f64(), c.k_new.f64(), c.v_new.f64(), pos0,
                                          rope_base=base)
    ref, _ = oracle.attention_with_cache(c.q.f64(), ref_k, ref_v, pos0, rope_base=base, window=W)
    assert_bf16_parity(to_np(o), ref, "o")


@pytest.mark.parametrize("seed", range(16))
def test_paged_chunk_sweep(lib, seed):
    rng = np.random.default_rng(7000 + seed)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 3))
    Sq = int(rng.integers(1, 300))
    pos0 = int(rng.integers(0, 700))
    S_max = pos0 + Sq + int(rng.integers(0, 50))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64, 256]))
    W = int(rng.integers(0, pos0 + Sq + 10)) if rng.random() < 0.4 else None
    rope = bool(rng.random() < 0.8)
    banner(f"paged chunk sweep seed={seed}: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} pos0={pos0} S_max={S_max} D={D} "
           f"bs={bs} W={W} rope={rope}")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=8000 + seed, kind="chunk",
                         pos0=pos0, S_max=S_max)
    p = inputs.make_paged_chunk(wl, block_size=bs)
    c = p.chunk
    tab = lib.make_rope_table(S_max, D) if rope else None
    o = lib.prefill_chunk_paged(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"),
                                p.k_pages.torch("cuda"), p.v_pages.torch("cuda"), torch.from_numpy(p.block_table).cuda(),
                                pos0, tab, window=W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    base = 10000.0 if rope else None
    rk, rv = oracle.append_to_cache_paged(p.k_pages.f64(), p.v_pages.f64(), p.block_table, c.k_new.f64(),
                                          c.v_new.f64(), pos0, rope_base=base)
    ck, cv = oracle.gather_pages(rk, rv, p.block_table, pos0 + Sq)
    ref, _ = oracle.attention_with_cache(c.q.f64(), ck, cv, pos0, rope_base=base, window=W)
    assert_bf16_parity(to_np(o), ref, "o")


@pytest.mark.parametrize("seed", range(16))
def test_varpos_chunk_sweep(lib, seed):
    """Chunks at per-sequence starts (contiguous or paged), then one append + decode step per
    sequence at its next position; every sequence against the oracle run on it alone."""
    rng = np.random.default_rng(9000 + seed)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 5))
    Sq = int(rng.integers(1, 300))
    S_max = Sq + int(rng.integers(1, 700))
    pos0_max = S_max - Sq - 1          # room for the decode token after the chunk
    starts = [int(rng.integers(0, pos0_max + 1)) for _ in range(B)]
    if B > 1 and rng.random() < 0.3:
        starts[int(rng.integers(0, B))] = pos0_max + 1 + int(rng.integers(0, 5))   # out of range: NaN rows
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64]))
    W = int(rng.integers(0, S_max)) if rng.random() < 0.4 else None
    rope = bool(rng.random() < 0.8)
    paged = bool(rng.random() < 0.5)
    banner(f"varpos sweep seed={seed}: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} S_max={S_max} starts={starts} "
           f"pos0_max={pos0_max} D={D} bs={bs} W={W} rope={rope} paged={paged}")
    wl = inputs.Workload("v", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=10000 + seed, kind="chunk",
                         pos0=0, S_max=S_max)
    pc = inputs.make_paged_chunk(wl, block_size=bs)
    c = pc.chunk
    tab = lib.make_rope_table(S_max, D) if rope else None
    p0 = torch.tensor(starts, dtype=torch.int32, device="cuda")
    q, kn, vn = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    if paged:
        kc, vc = pc.k_pages.torch("cuda"), pc.v_pages.torch("cuda")
        bt = torch.from_numpy(pc.block_table).cuda()
        o = lib.prefill_chunk_paged_varpos(q, kn, vn, kc, vc, bt, p0, pos0_max, tab, window=W,
                                           out_dtype=torch.float32)
    else:
        kc, vc = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
        o = lib.prefill_chunk_varpos(q, kn, vn, kc, vc, p0, pos0_max, tab, window=W, out_dtype=torch.float32)
    # one decode step at each valid sequence's next position: append its token, then attend
    grng = np.random.Generator(np.random.PCG64(11000 + seed))
    q1 = inputs.Tensor(grng.standard_normal((B, Hq, 1, D)).astype(np.float32), "bf16")
    k1 = inputs.Tensor(grng.standard_normal((B, Hkv, 1, D)).astype(np.float32), "bf16")
    v1 = inputs.Tensor(grng.standard_normal((B, Hkv, 1, D)).astype(np.float32), "bf16")
    nxt = np.array([p + Sq if p <= pos0_max else 0 for p in starts], dtype=np.int32)
    nxt_t = torch.from_numpy(nxt).cuda()
    if paged:
        lib.cache_append_paged(k1.torch("cuda"), v1.torch("cuda"), kc, vc, bt, nxt_t, tab)
        od = lib.decode_paged(q1.torch("cuda"), kc, vc, bt, nxt_t + 1, nxt_t, tab, window=W, out_dtype=torch.float32)
    else:
        lib.cache_append(k1.torch("cuda"), v1.torch("cuda"), kc, vc, nxt_t, tab)
        od = lib.decode(q1.torch("cuda"), kc, vc, nxt_t + 1, nxt_t, tab, window=W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    base = 10000.0 if rope else None
    for b, p in enumerate(starts):
        if p > pos0_max:
            assert torch.isnan(o[b]).all(), f"seq {b}: start {p} out of range, output not NaN"
            continue
        sl = slice(b, b + 1)
        rk, rv = oracle.append_to_cache(c.k_cache.f64()[sl], c.v_cache.f64()[sl], c.k_new.f64()[sl],
                                        c.v_new.f64()[sl], p, rope_base=base)
        ref, _ = oracle.attention_with_cache(c.q.f64()[sl], rk, rv, p, rope_base=base, window=W)
        assert_bf16_parity(to_np(o)[sl], ref, f"seq {b} chunk at {p}")
        rk, rv = oracle.append_to_cache(rk, rv, k1.f64()[sl], v1.f64()[sl], p + Sq, rope_base=base)
        ref1, _ = oracle.attention_with_cache(q1.f64()[sl], rk, rv, p + Sq, rope_base=base, window=W)
        assert_bf16_parity(to_np(od)[sl], ref1, f"seq {b} decode at {p + Sq}")
