"""Tensors of more than 2^31 elements on the GPU, checked against the fp64 oracle:
  * the prefill (keys rotated into a workspace, and the one-call form with the rotation fused
    into the tile loads) and rope_apply over a query tensor of 66 x 256 x 1024 x 128 bf16 values
    (4.4 GiB), on sampled rows: the first, the last, and rows whose element offsets lie just
    past 2^31, where 32-bit element arithmetic would wrap;
  * decode with query groups of 8 against a contiguous cache and a paged pool of over 2^32
    elements each, reading rows past 2^31 and 2^32 (the oracle sees exactly the rows each
    sequence attends to).

The tensors are drawn N(0, 1) on the device from a seeded torch generator (the host generator
would take minutes at this size); the sampled rows are copied back and fed to the oracle as the
exact bf16 values the kernels read.
"""

import numpy as np
import pytest
import torch

import oracle
from conftest import assert_bf16_parity, banner, err_stats, to_np

pytestmark = pytest.mark.gpu

B, HQ, HKV, S, D = 66, 256, 2, 1024, 128


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_self_attention_amd import lib as L
    return L


@pytest.fixture(scope="module")
def big():
    assert B * HQ * S * D > 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(2024)
    q = torch.randn((B, HQ, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((B, HKV, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((B, HKV, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
    yield q, k, v
    del q, k, v
    torch.cuda.empty_cache()


def _samples():
    """(b, h, row) triples: the corners, and the rows holding element 2^31 and just after."""
    out = [(0, 0, 0), (0, 0, S - 1), (B - 1, HQ - 1, S - 1), (B - 1, HQ - 1, 0)]
    for e in (2 ** 31 - D, 2 ** 31, 2 ** 31 + 5 * D, 2 ** 32 // 2 + S * D):
        r = e // D
        out.append((r // (HQ * S), (r // S) % HQ, r % S))
    return out


def _oracle_row(q, k, v, b, h, r):
    kv = h // (HQ // HKV)
    qh = to_np(q[b, h])[None, None]
    kh = to_np(k[b, kv])[None, None]
    vh = to_np(v[b, kv])[None, None]
    o, lse = oracle.attention(qh, kh, vh, rows=np.array([[r]]))
    return o[0, 0, 0], lse[0, 0, 0]


def test_prefill_over_2p31_elements(lib, big):
    q, k, v = big
    banner(f"prefill over 2^31 elements: B={B} Hq={HQ} Hkv={HKV} S={S} D={D}")
    tab = lib.make_rope_table(S, D)
    ws = torch.empty(lib.prefill_workspace_bytes(B, HKV, S, D), dtype=torch.uint8, device="cuda")
    lse = torch.empty((B, HQ, S), dtype=torch.float32, device="cuda")
    o = lib.prefill(q, k, v, tab, workspace=ws, lse=lse)
    torch.cuda.synchronize()
    got, ref, got_l, ref_l = [], [], [], []
    for b, h, r in _samples():
        ro, rl = _oracle_row(q, k, v, b, h, r)
        got.append(to_np(o[b, h, r]))
        ref.append(ro)
        got_l.append(float(lse[b, h, r]))
        ref_l.append(rl)
    assert_bf16_parity(np.stack(got), np.stack(ref), "prefill o, sampled rows")
    assert err_stats(np.array(got_l), np.array(ref_l))[0] < 2e-2
    del o, ws
    # the one-call form (rotation fused into the K tile loads), same rows
    o2 = lib.prefill(q, k, v, tab)
    torch.cuda.synchronize()
    got2 = [to_np(o2[b, h, r]) for b, h, r in _samples()]
    assert_bf16_parity(np.stack(got2), np.stack(ref), "prefill o (fused rotation), sampled rows")


def test_rope_apply_over_2p31_elements(lib, big):
    q, _, _ = big
    banner(f"rope_apply over 2^31 elements: [{B}, {HQ}, {S}, {D}] bf16, pos0 = 3")
    tab = lib.make_rope_table(S + 3, D)
    out = lib.rope_apply(q, tab, pos0=3)
    torch.cuda.synchronize()
    for b, h, r in _samples():
        x = to_np(q[b, h, r])[None, None, None]
        ref = oracle.rope(x, np.array([3 + r]))[0, 0, 0]
        got = to_np(out[b, h, r])
        # one bf16 rounding of the fp32 result
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6), (b, h, r)


# ---- decode, query groups of 8 (the narrow decode kernel), caches over 2^32 elements ----
DB, DHQ, DHKV = 2, 64, 8


def _decode_oracle_rows(q, kr, vr, q_pos):
    """Oracle decode of each sequence against exactly the rows it sees (kr, vr: lists of
    [Hkv, n_b, D] tensors), the query rotated at its true position."""
    outs = []
    for b in range(len(kr)):
        o, _ = oracle.decode(to_np(q[b:b + 1]), to_np(kr[b])[None], to_np(vr[b])[None], [kr[b].shape[1]],
                             [q_pos[b]])
        outs.append(o[0])
    return np.stack(outs)


def test_decode_cache_over_2p32_elements_window(lib):
    """A contiguous cache [2, 8, 2^21 + 64, 128] bf16 (8.6 GB per tensor): with a window of 300
    each sequence reads only rows just below its cache length, at element offsets past 2^31
    and, for the last KV head, past 2^32."""
    S_max = 2 ** 21 + 64
    assert DB * DHKV * S_max * D > 2 ** 32
    banner(f"decode, cache over 2^32 elements: B={DB} Hq={DHQ} Hkv={DHKV} S_max={S_max} window 300")
    g = torch.Generator(device="cuda").manual_seed(2025)
    kc = torch.randn((DB, DHKV, S_max, D), generator=g, device="cuda", dtype=torch.bfloat16)
    vc = torch.randn((DB, DHKV, S_max, D), generator=g, device="cuda", dtype=torch.bfloat16)
    q = torch.randn((DB, DHQ, 1, D), generator=g, device="cuda", dtype=torch.bfloat16)
    lens = [S_max, S_max - 1000]
    W = 300
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    tab = lib.make_rope_table(S_max + 1, D)
    o = lib.decode(q, kc, vc, cl, cl.clone(), tab, window=W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # visible rows: positions q_pos - W .. cache_len - 1 (q_pos = cache_len)
    kr = [kc[b, :, lens[b] - W:lens[b]] for b in range(DB)]
    vr = [vc[b, :, lens[b] - W:lens[b]] for b in range(DB)]
    ref = _decode_oracle_rows(q, kr, vr, lens)
    assert_bf16_parity(to_np(o), ref, "decode o (cache over 2^32 elements)")
    del kc, vc
    torch.cuda.empty_cache()


def test_paged_decode_pool_over_2p32_elements(lib):
    """A paged pool [262656, 8, 16, 128] bf16 (8.6 GB per pool) with every block of the two
    sequences near its far end, in shuffled order: pool offsets past 2^32 elements."""
    bs, nb = 16, 2 ** 18 + 512
    assert nb * DHKV * bs * D > 2 ** 32
    banner(f"paged decode, pool over 2^32 elements: B={DB} Hq={DHQ} Hkv={DHKV} blocks={nb} bs={bs}")
    g = torch.Generator(device="cuda").manual_seed(2026)
    kp = torch.randn((nb, DHKV, bs, D), generator=g, device="cuda", dtype=torch.bfloat16)
    vp = torch.randn((nb, DHKV, bs, D), generator=g, device="cuda", dtype=torch.bfloat16)
    q = torch.randn((DB, DHQ, 1, D), generator=g, device="cuda", dtype=torch.bfloat16)
    lens = [777, 500]
    mb = -(-max(lens) // bs)
    rng = np.random.default_rng(7)
    ids = nb - 1 - rng.permutation(DB * mb)                 # the last DB * mb blocks, shuffled
    table = ids.reshape(DB, mb).astype(np.int32)
    bt = torch.from_numpy(table).cuda()
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    tab = lib.make_rope_table(max(lens) + 1, D)
    o = lib.decode_paged(q, kp, vp, bt, cl, cl.clone(), tab, out_dtype=torch.float32)
    torch.cuda.synchronize()
    idx = [torch.from_numpy(table[b]).long().cuda() for b in range(DB)]
    kr = [kp[idx[b]].permute(1, 0, 2, 3).reshape(DHKV, mb * bs, D)[:, :lens[b]] for b in range(DB)]
    vr = [vp[idx[b]].permute(1, 0, 2, 3).reshape(DHKV, mb * bs, D)[:, :lens[b]] for b in range(DB)]
    ref = _decode_oracle_rows(q, kr, vr, lens)
    assert_bf16_parity(to_np(o), ref, "paged decode o (pool over 2^32 elements)")
    del kp, vp
    torch.cuda.empty_cache()
