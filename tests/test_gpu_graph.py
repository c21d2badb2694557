"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point enqueues kernels on the caller's stream and does nothing else on the host side
(no allocation, synchronisation or memset), so a step can be captured once and replayed.  Each
case captures one step on preallocated buffers, then replays it several times; before each
replay new inputs are copied into the captured buffers eagerly and the stream is synchronised,
and each replay must equal, bit for bit, the same call made eagerly on the same inputs.  Cases:
the prefill step (key rotation into a workspace + attention), a decode split over the cache with
its merge pass, and the multi-query decode (wide kernel + merge).
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
