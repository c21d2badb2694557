"""The Python binding's own argument checks, on the CPU.

The C ABI sees raw pointers and the sizes it is given, so a tensor smaller than those sizes (an
output, an lse vector, a cache, a RoPE table of another head dim) would be read or written past
its end on the device.  The binding compares every tensor with the shapes it passes, and raises
ValueError / TypeError before anything is enqueued.  Here the C library is replaced by a stub that
records calls, and CPU tensors stand in for device ones, so each rejection is checked to happen
before any call reaches the ABI.
"""

import pytest
import torch

from transformer_self_attention_amd import lib


class _Stub:
    """Every attribute is an ABI function that records its call and returns ATTN_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            # size queries are host arithmetic (they enqueue nothing), so only launches are kept
            if not (name.endswith("_bytes") or name.endswith("_num_splits")):
                self.calls.append((name, args))
            return 1 << 20 if name.endswith("_bytes") else lib.ATTN_OK
        return fn


@pytest.fixture
def stub(monkeypatch):
    s = _Stub()

    def need(t, name, device=None):  # the real check minus "is a GPU tensor"
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if device is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}")

    monkeypatch.setattr(lib, "_lib", s)
    monkeypatch.setattr(lib, "_need", need)
    monkeypatch.setattr(lib, "_stream", lambda stream=None: None)
    return s


bf, f32 = torch.bfloat16, torch.float32


def T(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def table(max_pos, D):
    return torch.zeros((max_pos, D // 2, 2), dtype=f32)


# ---- prefill -------------------------------------------------------------------------------

def _pf(**kw):
    a = dict(q=T(1, 8, 64, 128), k=T(1, 2, 64, 128), v=T(1, 2, 64, 128), table=table(64, 128))
    a.update(kw)
    return lib.prefill(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("table"), **a)


def test_prefill_accepts_matching_shapes(stub):
    _pf()
    _pf(out=T(1, 8, 64, 128, dtype=f32), lse=T(1, 8, 64, dtype=f32))
    assert [c[0] for c in stub.calls] == ["attn_prefill", "attn_prefill"]


@pytest.mark.parametrize("kw", [
    dict(out=T(1, 8, 63, 128)),                     # undersized output
    dict(out=T(1, 8, 64, 64)),
    dict(out=T(1, 8, 64, 128), out_dtype=f32),      # out and out_dtype disagree
    dict(lse=T(1, 8, 63, dtype=f32)),               # lse one row short
    dict(lse=T(1, 8, 64)),                          # lse not float32
    dict(table=table(64, 64)),                      # table of another head dim
    dict(table=table(64, 128).to(torch.float64)),
    dict(table=table(64, 128).reshape(64, 128)),
    dict(k=T(1, 2, 63, 128)),                       # keys shorter than the queries
    dict(v=T(1, 2, 64, 64)),
    dict(v=T(1, 2, 128, 64).transpose(2, 3)),       # non-contiguous
])
def test_prefill_rejects_before_launch(stub, kw):
    with pytest.raises(ValueError):
        _pf(**kw)
    assert stub.calls == []


def test_prerotated_and_rotation_reject_before_launch(stub):
    q, v = T(1, 8, 64, 128), T(1, 2, 64, 128)
    need = lib.prefill_workspace_bytes(1, 2, 64, 128)       # the stub answers 1 MiB
    kr = T(need, dtype=torch.uint8)
    tab = table(64, 128)
    for kw in (dict(out=T(1, 8, 64, 127)), dict(lse=T(3, dtype=f32)), dict()):
        with pytest.raises(ValueError):
            lib.prefill_prerotated(q, kr, v, tab if kw else table(64, 64), **kw)
    with pytest.raises(ValueError):                          # keys buffer one byte short
        lib.prefill_prerotated(q, T(need - 1, dtype=torch.uint8), v, tab)
    with pytest.raises(ValueError):                          # not a byte buffer
        lib.prefill_prerotated(q, T(1, 2, 64, 128, dtype=torch.float16), v, tab)
    with pytest.raises(ValueError):
        lib.rotate_keys_f16(v, tab, out=T(1, 2, 64, 128))               # out must be uint8
    with pytest.raises(ValueError):
        lib.rotate_keys_f16(v, tab, out=T(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError):
        lib.rope_apply(q, tab, out=T(1, 8, 64, 64))
    with pytest.raises(ValueError):
        lib.rope_apply(q, table(64, 64))
    assert stub.calls == []
    lib.rope_apply(q, tab, out=q)
    lib.rotate_keys_f16(v, tab)
    assert [c[0] for c in stub.calls] == ["attn_rope_apply", "attn_rotate_keys_f16"]


# ---- chunk ---------------------------------------------------------------------------------

def test_chunk_rejects_before_launch(stub):
    q, kn, vn = T(1, 8, 32, 128), T(1, 2, 32, 128), T(1, 2, 32, 128)
    kc, vc = T(1, 2, 256, 128), T(1, 2, 256, 128)
    tab = table(256, 128)
    bad = [
        dict(k_cache=T(1, 2, 256, 64)), dict(v_cache=T(1, 2, 255, 128)), dict(v_cache=T(2, 2, 256, 128)),
        dict(out=T(1, 8, 31, 128)), dict(lse=T(1, 8, 31, dtype=f32)), dict(table=table(256, 64)),
        dict(k_new=T(1, 2, 31, 128)),
    ]
    for b in bad:
        a = dict(k_new=kn, k_cache=kc, v_cache=vc, table=tab)
        a.update(b)
        with pytest.raises(ValueError):
            lib.prefill_chunk(q, a.pop("k_new"), vn, a.pop("k_cache"), a.pop("v_cache"), 100, a.pop("table"), **a)
    assert stub.calls == []
    lib.prefill_chunk(q, kn, vn, kc, vc, 100, tab)
    assert [c[0] for c in stub.calls] == ["attn_prefill_chunk"]


def test_chunk_paged_rejects_before_launch(stub):
    q, kn, vn = T(1, 8, 32, 128), T(1, 2, 32, 128), T(1, 2, 32, 128)
    kp, vp = T(20, 2, 16, 128), T(20, 2, 16, 128)
    bt = torch.zeros((1, 10), dtype=torch.int32)
    for b in (dict(v_pages=T(20, 2, 16, 64)), dict(v_pages=T(19, 2, 16, 128)),
              dict(bt=torch.zeros((2, 10), dtype=torch.int32)), dict(bt=torch.zeros((1, 10), dtype=torch.int64)),
              dict(out=T(1, 8, 32, 64))):
        a = dict(v_pages=vp, bt=bt)
        a.update(b)
        with pytest.raises(ValueError):
            lib.prefill_chunk_paged(q, kn, vn, kp, a.pop("v_pages"), a.pop("bt"), 64, table(256, 128), **a)
    assert stub.calls == []


# ---- decode --------------------------------------------------------------------------------

def _dec(**kw):
    a = dict(q=T(4, 16, 1, 128), kc=T(4, 2, 512, 128), vc=T(4, 2, 512, 128),
             cl=torch.zeros(4, dtype=torch.int32), qp=torch.zeros(4, dtype=torch.int32), table=table(600, 128))
    a.update(kw)
    return lib.decode(a.pop("q"), a.pop("kc"), a.pop("vc"), a.pop("cl"), a.pop("qp"), a.pop("table"), **a)


def test_decode_accepts_matching_shapes(stub):
    _dec(lse=T(4, 16, dtype=f32), out=T(4, 16, 1, 128))
    assert [c[0] for c in stub.calls] == ["attn_decode"]


@pytest.mark.parametrize("kw", [
    dict(out=T(4, 16, 1, 64)), dict(out=T(4, 8, 1, 128)),
    dict(lse=T(4, 15, dtype=f32)), dict(lse=T(4, 16)),
    dict(kc=T(3, 2, 512, 128), vc=T(3, 2, 512, 128)),     # fewer sequences than queries
    dict(kc=T(4, 2, 512, 64), vc=T(4, 2, 512, 64)),       # another head dim
    dict(vc=T(4, 2, 511, 128)),
    dict(cl=torch.zeros(3, dtype=torch.int32)), dict(qp=torch.zeros(4, dtype=torch.int64)),
    dict(table=table(600, 64)),
    dict(q=T(4, 16, 2, 128)),
])
def test_decode_rejects_before_launch(stub, kw):
    with pytest.raises(ValueError):
        _dec(**kw)
    assert stub.calls == []


def test_decode_paged_rejects_before_launch(stub):
    q = T(2, 16, 1, 128)
    kp, vp = T(40, 2, 16, 128), T(40, 2, 16, 128)
    bt = torch.zeros((2, 20), dtype=torch.int32)
    cl = qp = torch.zeros(2, dtype=torch.int32)
    for b in (dict(v_pages=T(40, 2, 16, 64)), dict(bt=torch.zeros((1, 20), dtype=torch.int32)),
              dict(lse=T(2, 15, dtype=f32)), dict(out=T(2, 16, 1, 64)), dict(table=table(400, 64))):
        a = dict(v_pages=vp, bt=bt, table=table(400, 128))
        a.update(b)
        with pytest.raises(ValueError):
            lib.decode_paged(q, kp, a.pop("v_pages"), a.pop("bt"), cl, qp, a.pop("table"), **a)
    assert stub.calls == []
    lib.decode_paged(q, kp, vp, bt, cl, qp, table(400, 128), lse=T(2, 16, dtype=f32))
    assert [c[0] for c in stub.calls] == ["attn_decode_paged"]
