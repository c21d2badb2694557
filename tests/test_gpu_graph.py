"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point enqueues kernels on the caller's stream and does nothing else on the host side
(no allocation, synchronisation or memset), so a step can be captured once and replayed.  Each
case captures one step on preallocated buffers, then replays it several times; before each
replay new inputs are copied into the captured buffers eagerly and the stream is synchronised,
and each replay must equal, bit for bit, the same call made eagerly on the same inputs.  Cases:
the prefill step (key rotation into a workspace + attention), a decode split over the cache with
its merge pass, the multi-query decode (wide kernel + merge), a serving step against a paged
pool (a chunk appended into its blocks and attended, then a split decode against the pool), and
a paged chunk with per-sequence starts whose starts change between replays (they are read from
device memory, so one capture serves every step).
"""

import pytest
import torch

from conftest import banner
from transformer_self_attention_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_self_attention_amd import lib as L
    return L


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # one eager call on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(g, load, out, eager, n=4):
    """Replay n times; before each, load() writes new inputs eagerly; compare with eager()."""
    for i in range(n):
        load(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = eager()
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"replay {i} differs from the eager call"


def test_graph_prefill_step(lib):
    banner("HIP graph: prefill step (key rotation + attention), 4 replays")
    B, Hq, Hkv, S, D = 1, 16, 4, 1000, 128
    g0 = torch.Generator(device="cuda").manual_seed(31)
    q = torch.randn((B, Hq, S, D), generator=g0, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, S, D), generator=g0, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, S, D), generator=g0, device="cuda").to(torch.bfloat16)
    tab = lib.make_rope_table(S, D)
    ws = torch.empty(lib.prefill_workspace_bytes(B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    g = _capture(lambda: lib.prefill(q, k, v, tab, workspace=ws, out=out))

    def load(i):
        gi = torch.Generator(device="cuda").manual_seed(100 + i)
        q.copy_(torch.randn(q.shape, generator=gi, device="cuda").to(torch.bfloat16))
        k.copy_(torch.randn(k.shape, generator=gi, device="cuda").to(torch.bfloat16))

    ws2 = torch.empty_like(ws)
    _replays(g, load, out, lambda: lib.prefill(q, k, v, tab, workspace=ws2))


@pytest.mark.parametrize("Hq,Hkv,n_split", [(16, 2, 4), (64, 1, 0)])
def test_graph_decode_with_merge(lib, Hq, Hkv, n_split):
    B, S, D = 4, 2048, 128
    banner(f"HIP graph: decode B={B} Hq={Hq} Hkv={Hkv} S={S} n_split={n_split or 'auto'} (+ merge), 4 replays")
    wl = inputs.Workload("g", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=33, kind="decode")
    d = inputs.make_decode(wl)
    q, kc, vc = d.q.torch("cuda"), d.k_cache.torch("cuda"), d.v_cache.torch("cuda")
    cl = torch.tensor([S, 1500, 77, 1], dtype=torch.int32, device="cuda")
    qp = cl.clone()
    tab = lib.make_rope_table(S + 1, D)
    assert lib.decode_num_splits(B, Hq, Hkv, S, D, n_split) > 1, "the case must take the merge pass"
    ws = torch.empty(lib.decode_workspace_bytes(B, Hq, Hkv, S, D, n_split), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    g = _capture(lambda: lib.decode(q, kc, vc, cl, qp, tab, n_split=n_split, out=out, workspace=ws))

    def load(i):
        gi = torch.Generator(device="cuda").manual_seed(200 + i)
        q.copy_(torch.randn(q.shape, generator=gi, device="cuda").to(torch.bfloat16))
        cl.copy_(torch.tensor([S - i, 1500 + 3 * i, 77, 1 + i], dtype=torch.int32, device="cuda"))
        qp.copy_(cl)

    ws2 = torch.empty_like(ws)
    _replays(g, load, out, lambda: lib.decode(q, kc, vc, cl, qp, tab, n_split=n_split, workspace=ws2))


def test_graph_serving_step_paged(lib):
    """One serving step in one graph: a 100-token chunk at pos0 = 300 appended into a shuffled
    16-token block pool and attended (three launches), then the next token's decode against the
    pool (split + merge).  Each replay must match the eager step in both outputs and in every
    byte of the pools."""
    B, Hq, Hkv, D, bs = 2, 16, 4, 128, 16
    S_max, pos0, Sq = 512, 300, 100
    banner(f"HIP graph: serving step, chunk Sq={Sq} at pos0={pos0} into a paged pool + paged decode, 4 replays")
    max_blocks = S_max // bs
    num_blocks = B * max_blocks + 3
    g0 = torch.Generator(device="cuda").manual_seed(41)

    def rnd(shape, g=g0):
        return torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)

    k_pages, v_pages = rnd((num_blocks, Hkv, bs, D)), rnd((num_blocks, Hkv, bs, D))
    perm = torch.randperm(num_blocks, generator=torch.Generator().manual_seed(5))[:B * max_blocks]
    block_table = perm.view(B, max_blocks).to(torch.int32).cuda()
    q_chunk, k_chunk, v_chunk = rnd((B, Hq, Sq, D)), rnd((B, Hkv, Sq, D)), rnd((B, Hkv, Sq, D))
    q1 = rnd((B, Hq, 1, D))
    cache_len = torch.full((B,), pos0 + Sq, dtype=torch.int32, device="cuda")
    q_pos = cache_len.clone()
    tab = lib.make_rope_table(S_max + 1, D)
    assert lib.decode_num_splits(B, Hq, Hkv, max_blocks * bs, D) > 1, "the decode must take the merge pass"

    def buffers():
        return (torch.empty(lib.prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D), dtype=torch.uint8,
                            device="cuda"),
                torch.empty(lib.decode_workspace_bytes(B, Hq, Hkv, max_blocks * bs, D), dtype=torch.uint8,
                            device="cuda"),
                torch.empty_like(q_chunk), torch.empty_like(q1))

    def step(ws_c, ws_d, o_c, o_d):
        lib.prefill_chunk_paged(q_chunk, k_chunk, v_chunk, k_pages, v_pages, block_table, pos0, tab, out=o_c,
                                workspace=ws_c)
        lib.decode_paged(q1, k_pages, v_pages, block_table, cache_len, q_pos, tab, out=o_d, workspace=ws_d)

    cap = buffers()
    g = _capture(lambda: step(*cap))
    eager = buffers()
    for i in range(4):
        gi = torch.Generator(device="cuda").manual_seed(300 + i)
        for t in (q_chunk, k_chunk, v_chunk, q1):
            t.copy_(rnd(t.shape, gi))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_c, got_d = cap[2].clone(), cap[3].clone()
        kp, vp = k_pages.clone(), v_pages.clone()
        step(*eager)   # appends the same rows again: the pools must not change
        torch.cuda.synchronize()
        assert torch.equal(got_c, eager[2]), f"replay {i}: chunk output differs from the eager call"
        assert torch.equal(got_d, eager[3]), f"replay {i}: decode output differs from the eager call"
        assert torch.equal(kp, k_pages) and torch.equal(vp, v_pages), f"replay {i}: pools differ"
        assert torch.isfinite(got_c.float()).all() and torch.isfinite(got_d.float()).all()


def test_graph_varpos_chunk_new_starts_each_replay(lib):
    """A chunk append + attention with per-sequence starts (attn_prefill_chunk_paged_varpos)
    captured once: the starts live in device memory, so each replay can take new ones.  Each
    replay must match the eager call on the same starts, outputs and pools bit for bit."""
    B, Hq, Hkv, D, bs, Sq, S_max, pos0_max = 3, 8, 2, 128, 16, 64, 512, 448
    banner(f"HIP graph: paged chunk with per-sequence starts, new starts on each of 4 replays")
    max_blocks = S_max // bs
    num_blocks = B * max_blocks + 2
    g0 = torch.Generator(device="cuda").manual_seed(43)

    def rnd(shape, g=g0):
        return torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)

    k_pages, v_pages = rnd((num_blocks, Hkv, bs, D)), rnd((num_blocks, Hkv, bs, D))
    perm = torch.randperm(num_blocks, generator=torch.Generator().manual_seed(6))[:B * max_blocks]
    block_table = perm.view(B, max_blocks).to(torch.int32).cuda()
    q, kn, vn = rnd((B, Hq, Sq, D)), rnd((B, Hkv, Sq, D)), rnd((B, Hkv, Sq, D))
    starts = torch.tensor([0, 100, 300], dtype=torch.int32, device="cuda")
    tab = lib.make_rope_table(S_max, D)
    ws_bytes = lib.prefill_chunk_paged_workspace_bytes(B, Hkv, pos0_max, Sq, D)

    def step(ws, o, kp, vp):
        lib.prefill_chunk_paged_varpos(q, kn, vn, kp, vp, block_table, starts, pos0_max, tab, out=o, workspace=ws)

    ws, out = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda"), torch.empty_like(q)
    g = _capture(lambda: step(ws, out, k_pages, v_pages))
    ws2, out2 = torch.empty_like(ws), torch.empty_like(q)
    for i, st in enumerate(([7, 448, 33], [448, 0, 250], [64, 64, 64], [1, 200, 447])):
        starts.copy_(torch.tensor(st, dtype=torch.int32, device="cuda"))
        gi = torch.Generator(device="cuda").manual_seed(400 + i)
        for t in (q, kn, vn):
            t.copy_(rnd(t.shape, gi))
        kp_e, vp_e = k_pages.clone(), v_pages.clone()   # the pools as the replay will find them
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(ws2, out2, kp_e, vp_e)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), f"replay {i} (starts {st}): output differs from the eager call"
        assert torch.equal(k_pages, kp_e) and torch.equal(v_pages, vp_e), f"replay {i}: pools differ"
        assert torch.isfinite(out.float()).all()
