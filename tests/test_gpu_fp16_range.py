"""Inputs whose rotated Q or K rows leave the fp16 range, through every path with fp16 Q.K^T operands.

The kernels round rotated queries and keys to IEEE half for the score products.  A row whose
largest magnitude reaches 2^15 is first scaled by 2^-e (e >= 0, the smallest that brings it
below 2^15; exact) and its scores are scaled back by 2^e in fp32.  These tests put such rows
into prefill (rotation in a workspace and fused into the K tile loads, D = 128 and 64), the
two-stage prefill, the chunk against a contiguous cache and the chunk against a paged cache,
and compare every output element with the fp64 oracle at the bf16 bars.

Construction (exact scores whatever the magnitude): every query has one RoPE pair (2p, 2p+1)
set to zero and chosen key rows carry +-A in that pair; RoPE rotates each pair within itself,
so those keys' large components meet only zeros and the exact scores stay O(1).  Queries are
planted the same way in another pair that every key has zeroed.  A key row at 1e5 in fp16
without its exponent is inf (the score inf * 0 = NaN); with a wrong exponent, a wrong lane or a
wrong sign its scores are off by a power of two, far outside the bars.  Amplitudes: 3.5e4 and
1e5 for keys (rotated pairs of norm 1.25 A: e = 0 or 1 at 3.5e4, 2 or 3 at 1e5); 1e5 and 1e6 for
queries, which are scaled by log2(e)/sqrt(D) before the test (qa = 0 at 1e5, 2 or 3 at 1e6).

A last case lets large keys meet the queries fully: scores of order 1e4 whose fp16 rounding
error (about 2^-10 of sum |q_i k_i| / sqrt(D), some tens) is far above the bars.  There every
output must be finite, and the rows whose exact softmax is decided by a margin above 300 (in
score units; the worst-case error of one score is about 115 there) must match the oracle at
the bars.
"""

import numpy as np
import pytest
import torch

import oracle
from conftest import assert_bf16_parity, banner, err_stats, to_np
from transformer_self_attention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_self_attention_amd import lib as L
    return L


def _bf16(x32):
    return inputs.Tensor(np.ascontiguousarray(x32, dtype=np.float32), "bf16")


def _big_rows(rng, n_rows, count, lead=(0,)):
    """count distinct rows of [0, n_rows), always holding `lead` and the last row."""
    fixed = sorted({r for r in lead if 0 <= r < n_rows} | {n_rows - 1})
    pool = np.setdiff1d(np.arange(n_rows), fixed)
    extra = rng.choice(pool, size=max(0, min(count - len(fixed), pool.size)), replace=False)
    return np.sort(np.concatenate([fixed, extra])).astype(np.int64)


def _plant(x, rows_per_bh, pair, amp, zero_pair=None):
    """x [B, H, S, D] float32 (copied): rows of each (b, h) get (amp, -0.75 amp) in `pair`;
    `zero_pair` is cleared in every row first."""
    x = x.copy()
    if zero_pair is not None:
        x[..., 2 * zero_pair:2 * zero_pair + 2] = 0.0
    if amp:
        for (b, h), rows in rows_per_bh.items():
            x[b, h, rows, 2 * pair] = amp
            x[b, h, rows, 2 * pair + 1] = -0.75 * amp
    return x


def _rows_map(rng, B, H, S, count, lead=(0,)):
    return {(b, h): _big_rows(rng, S, count, lead) for b in range(B) for h in range(H)}


def planted_prefill(B, Hq, Hkv, S, D, amp_k, amp_q, seed):
    """Seeded prefill inputs with key pair kp planted at amp_k (zero in every query) and query
    pair qp planted at amp_q (zero in every key)."""
    wl = inputs.Workload("r", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=seed, kind="prefill")
    p = inputs.make_prefill(wl)
    rng = np.random.Generator(np.random.PCG64(seed + 77))
    kp, qp = D // 2 - 3, 5
    krows = _rows_map(rng, B, Hkv, S, 6)
    qrows = _rows_map(rng, B, Hq, S, 6, lead=(0, 1, 64, 127))
    k32 = _plant(p.k.f32, krows, kp, amp_k, zero_pair=qp)
    q32 = _plant(p.q.f32, qrows, qp, amp_q, zero_pair=kp)
    p.q, p.k = _bf16(q32), _bf16(k32)
    return p, krows


CASES = [(3.5e4, 0.0), (1e5, 0.0), (0.0, 1e5), (0.0, 1e6), (1e5, 1e6), (3.5e4, 1e5)]


@pytest.mark.parametrize("amp_k,amp_q", CASES)
@pytest.mark.parametrize("mode", ["workspace", "fused"])
def test_prefill_large_rows(lib, amp_k, amp_q, mode):
    B, Hq, Hkv, S, D = 2, 8, 2, 333, 128
    banner(f"prefill fp16 range mode={mode} |k|={amp_k:g} |q|={amp_q:g} B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    p, _ = planted_prefill(B, Hq, Hkv, S, D, amp_k, amp_q, seed=int(amp_k) + 3 * int(amp_q) + 11)
    tab = lib.make_rope_table(S, D)
    q, k, v = p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda")
    ws = None
    if mode == "workspace":
        ws = torch.empty(lib.prefill_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o = lib.prefill(q, k, v, tab, out_dtype=torch.float32, lse=lse, workspace=ws)
    ob = lib.prefill(q, k, v, tab, workspace=ws)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(p.q.f64(), p.k.f64(), p.v.f64(), causal=True, rope_base=10000.0)
    assert_bf16_parity(to_np(o), ref, "o fp32")
    assert_bf16_parity(to_np(ob), ref, "o bf16")
    assert err_stats(to_np(lse), ref_lse)[0] < 2e-2


@pytest.mark.parametrize("amp_k,amp_q", [(1e5, 1e6), (3.5e4, 0.0)])
@pytest.mark.parametrize("mode", ["workspace", "fused"])
def test_prefill_large_rows_d64(lib, amp_k, amp_q, mode):
    B, Hq, Hkv, S, D = 1, 4, 4, 200, 64
    banner(f"prefill fp16 range D=64 mode={mode} |k|={amp_k:g} |q|={amp_q:g}")
    p, _ = planted_prefill(B, Hq, Hkv, S, D, amp_k, amp_q, seed=501)
    tab = lib.make_rope_table(S, D)
    ws = None
    if mode == "workspace":
        ws = torch.empty(lib.prefill_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    o = lib.prefill(p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda"), tab, out_dtype=torch.float32,
                    workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(p.q.f64(), p.k.f64(), p.v.f64(), causal=True, rope_base=10000.0)
    assert_bf16_parity(to_np(o), ref, "o")


def test_two_stage_exponents_and_keys(lib):
    """The rotated-key buffer: planted rows carry exponent e > 0 with 2^e * key within one fp16
    rounding of the oracle's rotation, every other row e = 0; the second stage equals one call."""
    B, Hq, Hkv, S, D = 2, 8, 2, 333, 128
    banner("two-stage prefill with key rows at 1e5 and query rows at 1e6")
    p, krows = planted_prefill(B, Hq, Hkv, S, D, 1e5, 1e6, seed=91)
    tab = lib.make_rope_table(S + 5, D)
    q, k, v = p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda")
    krot = lib.rotate_keys_f16(k, tab, pos0=5)
    o2 = lib.prefill_prerotated(q, krot, v, tab, pos0=5)
    ws = torch.empty(lib.prefill_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    o1 = lib.prefill(q, k, v, tab, pos0=5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    keys, exps = lib.rotated_keys_view(krot, B, Hkv, S, D)
    e = exps.cpu().numpy().astype(np.int64)
    want = np.zeros((B, Hkv, S), dtype=bool)
    for (b, h), rows in krows.items():
        want[b, h, rows] = True
    assert np.all(e[~want] == 0), "an unplanted key row was scaled"
    assert np.all(e[want] > 0), "a planted key row (|x| >= 2^15 after rotation) kept exponent 0"
    ref_k = oracle.rope(p.k.f64(), 5 + np.arange(S))
    got = to_np(keys) * np.exp2(e)[..., None]
    assert np.all(np.abs(to_np(keys)) <= 2.0 ** 15)
    assert np.all(np.abs(got - ref_k) <= np.abs(ref_k) * 2.0 ** -10 + 1e-6 * np.exp2(e)[..., None])
    # the largest element of every scaled row sits in [2^14, 2^15) once scaled: e is the smallest
    m = np.abs(to_np(keys)).max(axis=-1)
    assert np.all(m[want] >= 2.0 ** 14)
    ref, _ = oracle.attention(p.q.f64(), p.k.f64(), p.v.f64(), causal=True, rope_base=10000.0, pos0=5)
    assert_bf16_parity(to_np(o2), ref, "o")


def _chunk_planted(B, Hq, Hkv, Sq, S_max, D, pos0, amp_k, amp_q, seed):
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=seed, kind="chunk",
                         pos0=pos0, S_max=S_max)
    c = inputs.make_chunk(wl)
    rng = np.random.Generator(np.random.PCG64(seed + 77))
    kp, qp = D // 2 - 3, 5
    cached = _rows_map(rng, B, Hkv, pos0, 6)     # rows of the cache before the chunk
    new = _rows_map(rng, B, Hkv, Sq, 4)
    c.k_cache = _bf16(_plant(c.k_cache.f32, cached, kp, amp_k, zero_pair=qp))
    c.k_new = _bf16(_plant(c.k_new.f32, new, kp, amp_k, zero_pair=qp))
    c.q = _bf16(_plant(c.q.f32, _rows_map(rng, B, Hq, Sq, 5), qp, amp_q, zero_pair=kp))
    return c, wl


@pytest.mark.parametrize("amp_k,amp_q", [(1e5, 0.0), (3.5e4, 1e6)])
def test_chunk_large_rows(lib, amp_k, amp_q):
    B, Hq, Hkv, Sq, S_max, D, pos0 = 2, 8, 2, 150, 400, 128, 181
    banner(f"chunk fp16 range |k|={amp_k:g} |q|={amp_q:g} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} pos0={pos0}")
    c, wl = _chunk_planted(B, Hq, Hkv, Sq, S_max, D, pos0, amp_k, amp_q, seed=300 + int(amp_q) % 97)
    tab = lib.make_rope_table(S_max, D)
    kc, vc = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    o = lib.prefill_chunk(c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda"), kc, vc, pos0, tab,
                          out_dtype=torch.float32, lse=lse)
    torch.cuda.synchronize()
    rk, rv = oracle.append_to_cache(c.k_cache.f64(), c.v_cache.f64(), c.k_new.f64(), c.v_new.f64(), pos0,
                                    rope_base=10000.0)
    ref, ref_lse = oracle.attention_with_cache(c.q.f64(), rk, rv, pos0, rope_base=10000.0)
    assert_bf16_parity(to_np(o), ref, "chunk o")
    assert err_stats(to_np(lse), ref_lse)[0] < 2e-2


def test_paged_chunk_large_rows(lib):
    B, Hq, Hkv, Sq, S_max, D, pos0, bs = 2, 8, 2, 100, 300, 128, 137, 16
    banner(f"paged chunk fp16 range |k|=1e5 |q|=1e6 B={B} Sq={Sq} pos0={pos0} bs={bs}")
    c, wl = _chunk_planted(B, Hq, Hkv, Sq, S_max, D, pos0, 1e5, 1e6, seed=433)
    nb = -(-S_max // bs)
    rng = np.random.Generator(np.random.PCG64(434))
    perm = rng.permutation(B * nb + 3)
    table = perm[:B * nb].reshape(B, nb).astype(np.int32)

    def scatter(bits):
        pool = np.full((B * nb + 3, Hkv, bs, D), inputs.BF16_NAN_BITS, dtype=np.uint16)
        for b in range(B):
            for t in range(S_max):
                pool[table[b, t // bs], :, t % bs] = bits[b, :, t]
        return torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).cuda()

    kp, vp = scatter(c.k_cache.bits), scatter(c.v_cache.bits)
    tab = lib.make_rope_table(S_max, D)
    q, kn, vn = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    o = lib.prefill_chunk_paged(q, kn, vn, kp, vp, torch.from_numpy(table).cuda(), pos0, tab,
                                out_dtype=torch.float32)
    kc, vc = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    oc = lib.prefill_chunk(q, kn, vn, kc, vc, pos0, tab, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, oc), "paged and contiguous chunk outputs differ"
    rk, rv = oracle.append_to_cache(c.k_cache.f64(), c.v_cache.f64(), c.k_new.f64(), c.v_new.f64(), pos0,
                                    rope_base=10000.0)
    ref, _ = oracle.attention_with_cache(c.q.f64(), rk, rv, pos0, rope_base=10000.0)
    assert_bf16_parity(to_np(o), ref, "paged chunk o")


@pytest.mark.parametrize("mode", ["workspace", "fused"])
def test_large_keys_meeting_queries(lib, mode):
    """Key rows x 2^14 (bf16-exact, |k| up to ~1e5 after rotation) against ordinary queries."""
    B, Hq, Hkv, S, D = 1, 4, 2, 320, 128
    banner(f"large keys meeting queries mode={mode}")
    wl = inputs.Workload("r", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=808, kind="prefill")
    p = inputs.make_prefill(wl)
    rng = np.random.Generator(np.random.PCG64(809))
    k32 = p.k.f32.copy()
    for h in range(Hkv):
        rows = _big_rows(rng, S, 12, lead=(0, 70, 200))
        k32[0, h, rows] *= np.float32(2.0 ** 14)
    p.k = _bf16(k32)
    tab = lib.make_rope_table(S, D)
    ws = None
    if mode == "workspace":
        ws = torch.empty(lib.prefill_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    o = lib.prefill(p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda"), tab, out_dtype=torch.float32,
                    workspace=ws)
    torch.cuda.synchronize()
    got = to_np(o)
    assert np.all(np.isfinite(got)), "non-finite output with large keys"
    ref, _ = oracle.attention(p.q.f64(), p.k.f64(), p.v.f64(), causal=True, rope_base=10000.0)
    # the exact scores decide which rows have a margin that the fp16 rounding cannot close
    qr = oracle.rope(p.q.f64(), np.arange(S))
    kr = oracle.rope(p.k.f64(), np.arange(S))
    G = Hq // Hkv
    decided = np.zeros((B, Hq, S), dtype=bool)
    for h in range(Hq):
        s = qr[0, h] @ kr[0, h // G].T / np.sqrt(D)
        s[np.triu_indices(S, 1)] = -np.inf
        top2 = -np.sort(-s, axis=1)[:, :2]
        decided[0, h] = top2[:, 0] - top2[:, 1] > 300.0
        # rows whose visible large keys all score far below the row's best ordinary key also
        # follow the ordinary keys exactly (the large ones get weight 0)
        big = np.abs(kr[0, h // G]).max(axis=1) > 1e3
        sb = np.where(big[None, :], s, -np.inf).max(axis=1)
        so = np.where(~big[None, :], s, -np.inf).max(axis=1)
        decided[0, h] |= (so - sb > 300.0) & np.isfinite(so)
    n = int(decided.sum())
    print(f"    rows decided by a margin > 300: {n} of {decided.size}", flush=True)
    assert n > decided.size // 2
    assert_bf16_parity(got[decided], ref[decided], "decided rows")
