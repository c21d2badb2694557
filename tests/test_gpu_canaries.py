"""Canaries around every buffer the library writes.

Each output, LSE, workspace and KV cache handed to an entry point is a view into a larger device
buffer whose bytes before and after the view hold a fixed pattern.  After the call the pattern
must be intact, and the results must equal those of the same call on ordinary tensors, bit for
bit.  Covered: prefill (workspace, fused and no-RoPE modes; bf16 and fp32 output), the
two-stage prefill (rotated-key buffer), decode (the narrow kernel with and without a merge pass,
the wide kernel with and without one, the paged cache, the allocation-free entry point), the
chunk against a contiguous cache (cache rows outside [pos0, pos0 + Sq) unchanged, the cache
tensor's neighbours untouched) and against a paged cache, and RoPE apply.
"""

import math

import numpy as np
import pytest
import torch

from conftest import banner
from transformer_self_attention_amd import inputs

pytestmark = pytest.mark.gpu

PAD = 4096   # canary elements on each side (8-16 KiB: keeps every view 16-byte aligned)
FILL = {torch.bfloat16: -3.0, torch.float32: -1234.5, torch.uint8: 0xA5, torch.int32: -7}


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_self_attention_amd import lib as L
    return L


class Fenced:
    """A view of `shape` in the middle of a device buffer whose other elements hold FILL[dtype]
    (or, with `like`, a copy of that tensor's contents in the view)."""

    def __init__(self, shape, dtype, like=None):
        self.n = math.prod(shape)
        self.dtype = dtype
        self.buf = torch.full((PAD + self.n + PAD,), FILL[dtype], dtype=dtype, device="cuda")
        self.view = self.buf[PAD:PAD + self.n].view(shape)
        if like is not None:
            self.view.copy_(like)

    def assert_intact(self, what):
        torch.cuda.synchronize()
        ref = torch.full((PAD,), FILL[self.dtype], dtype=self.dtype, device="cuda")
        assert torch.equal(self.buf[:PAD], ref), f"{what}: written before the buffer"
        assert torch.equal(self.buf[PAD + self.n:], ref), f"{what}: written past the buffer"


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("mode", ["workspace", "fused", "norope"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_canaries(lib, mode, out_dtype):
    B, Hq, Hkv, S, D = 2, 8, 2, 333, 128
    banner(f"canaries: prefill mode={mode} out={out_dtype}")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=8100, kind="prefill")
    p = inputs.make_prefill(wl)
    q, k, v = p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda")
    tab = lib.make_rope_table(S, D) if mode != "norope" else None
    o = Fenced((B, Hq, S, D), out_dtype)
    lse = Fenced((B, Hq, S), torch.float32)
    ws = Fenced((lib.prefill_workspace_bytes(B, Hkv, S, D),), torch.uint8) if mode == "workspace" else None
    lib.prefill(q, k, v, tab, out=o.view, lse=lse.view, workspace=ws.view if ws else None)
    o.assert_intact("o")
    lse.assert_intact("lse")
    if ws:
        ws.assert_intact("workspace")
    plain_lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    plain = lib.prefill(q, k, v, tab, out_dtype=out_dtype, lse=plain_lse,
                        workspace=torch.empty_like(ws.view) if ws else None)
    torch.cuda.synchronize()
    assert _bits_equal(o.view, plain) and _bits_equal(lse.view, plain_lse)


def test_two_stage_canaries(lib):
    B, Hq, Hkv, S, D = 1, 8, 4, 200, 64
    banner("canaries: rotate_keys_f16 + prefill_prerotated")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=8101, kind="prefill")
    p = inputs.make_prefill(wl)
    q, k, v = p.q.torch("cuda"), p.k.torch("cuda"), p.v.torch("cuda")
    tab = lib.make_rope_table(S + 3, D)
    krot = Fenced((lib.prefill_workspace_bytes(B, Hkv, S, D),), torch.uint8)
    lib.rotate_keys_f16(k, tab, pos0=3, out=krot.view)
    krot.assert_intact("rotated keys")
    o = Fenced((B, Hq, S, D), torch.bfloat16)
    lse = Fenced((B, Hq, S), torch.float32)
    lib.prefill_prerotated(q, krot.view, v, tab, pos0=3, out=o.view, lse=lse.view)
    o.assert_intact("o")
    lse.assert_intact("lse")
    assert _bits_equal(o.view, lib.prefill(q, k, v, tab, pos0=3, workspace=torch.empty_like(krot.view)))


DECODE_CASES = [
    # B, Hq, Hkv, S, n_split: narrow kernel (<= 16 query heads per KV head) and wide kernel, with
    # one split (o written by the attention kernel) and several (merge pass)
    (4, 8, 2, 1000, 1),
    (4, 8, 2, 1000, 0),
    (3, 64, 1, 1500, 1),
    (3, 64, 1, 1500, 0),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,n_split", DECODE_CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_decode_canaries(lib, B, Hq, Hkv, S, n_split, out_dtype):
    D = 128
    banner(f"canaries: decode B={B} Hq={Hq} Hkv={Hkv} S={S} n_split={n_split} out={out_dtype}")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=8200 + Hq, kind="decode")
    d = inputs.make_decode(wl, cache_len=np.array([S, S // 2, 1, 0][:B], dtype=np.int32))
    args = (d.q.torch("cuda"), d.k_cache.torch("cuda"), d.v_cache.torch("cuda"),
            torch.from_numpy(d.cache_len).cuda(), torch.from_numpy(d.q_pos).cuda(),
            lib.make_rope_table(S + 1, D))
    o = Fenced((B, Hq, 1, D), out_dtype)
    lse = Fenced((B, Hq), torch.float32)
    ws = Fenced((lib.decode_workspace_bytes(B, Hq, Hkv, S, D, n_split),), torch.uint8)
    lib.decode(*args, n_split=n_split, out=o.view, lse=lse.view, workspace=ws.view)
    o.assert_intact("o")
    lse.assert_intact("lse")
    ws.assert_intact("workspace")
    plain_lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    plain = lib.decode(*args, n_split=n_split, out_dtype=out_dtype, lse=plain_lse)
    torch.cuda.synchronize()
    assert _bits_equal(o.view, plain) and _bits_equal(lse.view, plain_lse)
    # the allocation-free entry point: same results, same canaries
    o2 = Fenced((B, Hq, 1, D), out_dtype)
    lse2 = Fenced((B, Hq), torch.float32)
    lib.decode_noalloc(*args, n_split=n_split, out=o2.view, lse=lse2.view)
    o2.assert_intact("o (noalloc)")
    lse2.assert_intact("lse (noalloc)")
    assert _bits_equal(o2.view, plain) and _bits_equal(lse2.view, plain_lse)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (64, 1)])
def test_decode_paged_canaries(lib, Hq, Hkv):
    B, S, D, bs = 3, 700, 128, 16
    banner(f"canaries: paged decode B={B} Hq={Hq} Hkv={Hkv} S={S} block={bs}")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16", seed=8300 + Hq, kind="decode")
    p = inputs.make_paged_decode(wl, block_size=bs)
    kp, vp = p.k_pages.torch("cuda"), p.v_pages.torch("cuda")
    bt = torch.from_numpy(p.block_table).cuda()
    cl = torch.from_numpy(p.cache_len).cuda()
    qp = torch.from_numpy(p.q_pos).cuda()
    q = p.q.torch("cuda")
    tab = lib.make_rope_table(S + 1, D)
    o = Fenced((B, Hq, 1, D), torch.float32)
    lse = Fenced((B, Hq), torch.float32)
    mb = p.block_table.shape[1]
    ws = Fenced((lib.decode_workspace_bytes(B, Hq, Hkv, mb * bs, D, 0),), torch.uint8)
    lib.decode_paged(q, kp, vp, bt, cl, qp, tab, out=o.view, lse=lse.view, workspace=ws.view)
    o.assert_intact("o")
    lse.assert_intact("lse")
    ws.assert_intact("workspace")
    assert _bits_equal(o.view, lib.decode_paged(q, kp, vp, bt, cl, qp, tab, out_dtype=torch.float32))


def test_chunk_canaries(lib):
    B, Hq, Hkv, Sq, S_max, D, pos0 = 2, 8, 2, 77, 300, 128, 100
    banner(f"canaries: chunk B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} S_max={S_max} pos0={pos0}")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=8400, kind="chunk",
                         pos0=pos0, S_max=S_max)
    c = inputs.make_chunk(wl)
    q, kn, vn = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    tab = lib.make_rope_table(S_max, D)
    kc = Fenced((B, Hkv, S_max, D), torch.bfloat16, like=c.k_cache.torch("cuda"))
    vc = Fenced((B, Hkv, S_max, D), torch.bfloat16, like=c.v_cache.torch("cuda"))
    o = Fenced((B, Hq, Sq, D), torch.bfloat16)
    lse = Fenced((B, Hq, Sq), torch.float32)
    ws = Fenced((lib.prefill_workspace_bytes(B, Hkv, pos0 + Sq, D),), torch.uint8)
    lib.prefill_chunk(q, kn, vn, kc.view, vc.view, pos0, tab, out=o.view, lse=lse.view, workspace=ws.view)
    for f, what in ((kc, "k_cache"), (vc, "v_cache"), (o, "o"), (lse, "lse"), (ws, "workspace")):
        f.assert_intact(what)
    outside = np.r_[0:pos0, pos0 + Sq:S_max]
    for f, t in ((kc, c.k_cache), (vc, c.v_cache)):
        got = f.view.cpu().view(torch.int16).numpy()
        assert np.array_equal(got[:, :, outside], t.bits.view(np.int16)[:, :, outside]), "cache rows outside the chunk"
    kc2, vc2 = c.k_cache.torch("cuda"), c.v_cache.torch("cuda")
    plain = lib.prefill_chunk(q, kn, vn, kc2, vc2, pos0, tab)
    torch.cuda.synchronize()
    assert _bits_equal(o.view, plain) and _bits_equal(kc.view, kc2) and _bits_equal(vc.view, vc2)


def test_chunk_paged_canaries(lib):
    B, Hq, Hkv, Sq, S_max, D, pos0, bs = 2, 8, 2, 100, 150, 128, 37, 16
    banner(f"canaries: paged chunk B={B} Sq={Sq} pos0={pos0} block={bs}")
    wl = inputs.Workload("c", B=B, Hq=Hq, Hkv=Hkv, S=Sq, D=D, dtype="bf16", seed=8500, kind="chunk",
                         pos0=pos0, S_max=S_max)
    p = inputs.make_paged_chunk(wl, block_size=bs)
    c = p.chunk
    q, kn, vn = c.q.torch("cuda"), c.k_new.torch("cuda"), c.v_new.torch("cuda")
    tab = lib.make_rope_table(S_max, D)
    shape = tuple(p.k_pages.shape)
    kp = Fenced(shape, torch.bfloat16, like=p.k_pages.torch("cuda"))
    vp = Fenced(shape, torch.bfloat16, like=p.v_pages.torch("cuda"))
    bt = torch.from_numpy(p.block_table).cuda()
    o = Fenced((B, Hq, Sq, D), torch.float32)
    lse = Fenced((B, Hq, Sq), torch.float32)
    ws = Fenced((lib.prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D),), torch.uint8)
    lib.prefill_chunk_paged(q, kn, vn, kp.view, vp.view, bt, pos0, tab, out=o.view, lse=lse.view,
                            workspace=ws.view)
    for f, what in ((kp, "k_pages"), (vp, "v_pages"), (o, "o"), (lse, "lse"), (ws, "workspace")):
        f.assert_intact(what)
    kp2, vp2 = p.k_pages.torch("cuda"), p.v_pages.torch("cuda")
    plain = lib.prefill_chunk_paged(q, kn, vn, kp2, vp2, bt, pos0, tab, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert _bits_equal(o.view, plain) and _bits_equal(kp.view, kp2) and _bits_equal(vp.view, vp2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_apply_canaries(lib, dtype):
    B, H, S, D = 2, 3, 37, 128
    banner(f"canaries: rope_apply {dtype}")
    x = torch.randn((B, H, S, D), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda").to(dtype)
    tab = lib.make_rope_table(S + 9, D)
    out = Fenced((B, H, S, D), dtype)
    lib.rope_apply(x, tab, pos0=9, out=out.view)
    out.assert_intact("out")
    inplace = Fenced((B, H, S, D), dtype, like=x)
    lib.rope_apply(inplace.view, tab, pos0=9, out=inplace.view)
    inplace.assert_intact("in place")
    assert _bits_equal(out.view, inplace.view)
