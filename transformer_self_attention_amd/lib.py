"""Thin ctypes binding of libattn.so (the C ABI declared in include/attn.h).

Argument marshalling only: each function takes torch tensors that already live on the GPU,
checks the things ctypes cannot (dtype, contiguity, device), and passes raw pointers, sizes
and the current HIP stream to the same-named C entry point.  Every step of the computation
runs in the library's HIP kernels; there is no fallback path.  Importing this module raises
if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so libattn.so binds to the same one

# ATTN_LIBRARY: another build of the same library to load instead (the host-sanitized build of
# build.build_host_sanitized(), for instance)
_LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTED = (
    "attn_version",
    "attn_status_string",
    "attn_checked_sites",
    "attn_rope_table_bytes",
    "attn_rope_table_init",
    "attn_rope_table_init_scaled",
    "attn_rope_apply",
    "attn_prefill_workspace_bytes",
    "attn_prefill",
    "attn_rotate_keys_f16",
    "attn_prefill_prerotated",
    "attn_prefill_chunk",
    "attn_prefill_chunk_varpos",
    "attn_prefill_chunk_paged_workspace_bytes",
    "attn_prefill_chunk_paged",
    "attn_prefill_chunk_paged_varpos",
    "attn_cache_append",
    "attn_cache_append_paged",
    "attn_decode_workspace_bytes",
    "attn_decode_num_splits",
    "attn_decode",
    "attn_decode_paged",
    "attn_decode_noalloc",
)

NOALLOC_SCRATCH_BYTES = 16 << 20   # ATTN_NOALLOC_SCRATCH_BYTES


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m transformer_self_attention_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    lib.attn_version.restype = i32
    lib.attn_version.argtypes = []
    lib.attn_checked_sites.restype = i32
    lib.attn_checked_sites.argtypes = [vp, i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i32]
    lib.attn_rope_table_bytes.restype = sz
    lib.attn_rope_table_bytes.argtypes = [i32, i32]
    lib.attn_rope_table_init.restype = i32
    lib.attn_rope_table_init.argtypes = [fp, i32, i32, ctypes.c_double, vp]
    lib.attn_rope_table_init_scaled.restype = i32
    lib.attn_rope_table_init_scaled.argtypes = [fp, i32, i32, ctypes.c_double, i32, ctypes.c_double, i32,
                                                ctypes.c_double, ctypes.c_double, vp]
    lib.attn_rope_apply.restype = i32
    lib.attn_rope_apply.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, fp, i32, vp]
    lib.attn_prefill_workspace_bytes.restype = sz
    lib.attn_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_prefill.restype = i32
    lib.attn_prefill.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                 fp, i32, vp, sz, vp]
    lib.attn_rotate_keys_f16.restype = i32
    lib.attn_rotate_keys_f16.argtypes = [vp, vp, i32, i32, i32, i32, i32, fp, i32, vp]
    lib.attn_prefill_prerotated.restype = i32
    lib.attn_prefill_prerotated.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32, i32, i32,
                                            i32, fp, i32, vp]
    lib.attn_prefill_chunk.restype = i32
    lib.attn_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32, i32, i32,
                                       i32, fp, i32, vp, sz, vp]
    lib.attn_prefill_chunk_varpos.restype = i32
    lib.attn_prefill_chunk_varpos.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, fp, i32, i32, i32, i32, i32, i32,
                                              i32, i32, fp, i32, vp, sz, vp]
    lib.attn_prefill_chunk_paged_workspace_bytes.restype = sz
    lib.attn_prefill_chunk_paged_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_prefill_chunk_paged.restype = i32
    lib.attn_prefill_chunk_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, fp, i32, i32, i32, i32,
                                             i32, i32, i32, i32, fp, i32, vp, sz, vp]
    lib.attn_prefill_chunk_paged_varpos.restype = i32
    lib.attn_prefill_chunk_paged_varpos.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, vp, fp, i32,
                                                    i32, i32, i32, i32, i32, i32, fp, i32, vp, sz, vp]
    lib.attn_cache_append.restype = i32
    lib.attn_cache_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, fp, i32, vp]
    lib.attn_cache_append_paged.restype = i32
    lib.attn_cache_append_paged.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32, i32, fp, i32, vp]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.attn_decode_num_splits.restype = i32
    lib.attn_decode_num_splits.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.attn_decode.restype = i32
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32, i32, i32, fp,
                                i32, i32, vp, sz, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32,
                                      i32, fp, i32, i32, vp, sz, vp]
    lib.attn_decode_noalloc.restype = i32
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32, i32, i32, fp,
                                        i32, i32, vp]
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def raw():
    """The ctypes handle itself (for tests of the C ABI)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.attn_status_string(int(status)).decode()


def checked_sites():
    """Checked build only: the words of failed index checks per source file (rope, cache,
    prefill_bf16, prefill_f32, decode, decode_wide; bit i = check site i), cleared by the read;
    None from a normal build.  Blocking: synchronize the device first."""
    words = (ctypes.c_uint * 8)()
    n = int(_lib.attn_checked_sites(words, 8))
    return None if n < 0 else [int(words[i]) for i in range(n)]


def version() -> int:
    return int(_lib.attn_version())


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _win(window) -> int:
    """Python's window=None (no window) as the ABI's negative value."""
    if window is None:
        return -1
    if window < 0:
        raise ValueError("window must be None or >= 0")
    return int(window)


def _need(t: torch.Tensor, name: str, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _shape(t: torch.Tensor, shape, name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _table(table, D: int, device) -> int:
    """Checks a RoPE coefficient table, float32 [max_pos, D/2, 2], and returns max_pos (0 for None:
    no RoPE).  The C ABI receives only the row count, so the inner shape is checked here."""
    if table is None:
        return 0
    _need(table, "table", device)
    if table.dtype != torch.float32 or table.dim() != 3 or tuple(table.shape[1:]) != (D // 2, 2):
        raise ValueError(f"table must be float32 [max_pos, {D // 2}, 2] for head dim {D}, "
                         f"got {table.dtype} {tuple(table.shape)}")
    return int(table.shape[0])


def _out(out, shape, dtype, device):
    """The output tensor: allocated when None, otherwise checked against the shape and device the
    kernels will write (an undersized buffer would be written past its end)."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(out, "out", device)
    _shape(out, shape, "out")
    if dtype is not None and out.dtype != dtype:
        raise ValueError(f"out has dtype {out.dtype}, expected {dtype}")
    return out


def _lse(lse, n: int, device):
    if lse is None:
        return
    _need(lse, "lse", device)
    if lse.dtype != torch.float32 or lse.numel() != n:
        raise ValueError(f"lse must be float32 with {n} elements, got {lse.dtype} with {lse.numel()}")


def _scratch(workspace, nbytes: int, device, stream):
    """A caller's workspace (checked) or a new one.  A new one is tied to the stream the kernels run
    on, so the allocator does not hand its memory out again while they may still use it."""
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        if stream is not None:
            workspace.record_stream(stream)
        return workspace
    _need(workspace, "workspace", device)
    return workspace


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def rope_table_bytes(max_pos: int, D: int) -> int:
    return int(_lib.attn_rope_table_bytes(max_pos, D))


ROPE_SCALINGS = {"pi": 1, "ntk": 2, "yarn": 3}


def rope_table_init(table: torch.Tensor, max_pos: int, D: int, base: float = 10000.0, stream=None, *,
                    scaling: str = None, factor: float = 1.0, original_max_pos: int = 4096,
                    beta_fast: float = 32.0, beta_slow: float = 1.0):
    """Fill float32 table [max_pos, D/2, 2] with (cos, sin) of m * base^(-2i/D); scaling "pi",
    "ntk" or "yarn" (with factor s and, for YaRN, the trained context and ramp ends) stretches
    it for longer contexts (attn_rope_table_init_scaled)."""
    _need(table, "table")
    if table.dtype != torch.float32 or table.numel() * 4 < rope_table_bytes(max_pos, D):
        raise ValueError("table must be float32 with at least rope_table_bytes() bytes")
    if scaling is None:
        _check(_lib.attn_rope_table_init(_ptr(table), max_pos, D, float(base), _stream(stream)),
               "attn_rope_table_init")
        return
    if scaling not in ROPE_SCALINGS:
        raise ValueError(f"scaling must be one of {sorted(ROPE_SCALINGS)}")
    _check(_lib.attn_rope_table_init_scaled(_ptr(table), max_pos, D, float(base), ROPE_SCALINGS[scaling],
                                            float(factor), int(original_max_pos), float(beta_fast),
                                            float(beta_slow), _stream(stream)), "attn_rope_table_init_scaled")


def make_rope_table(max_pos: int, D: int, base: float = 10000.0, device="cuda", stream=None,
                    **scaling) -> torch.Tensor:
    t = torch.empty((max_pos, D // 2, 2), dtype=torch.float32, device=device)
    rope_table_init(t, max_pos, D, base, stream, **scaling)
    return t


def rope_apply(x: torch.Tensor, table: torch.Tensor, pos0: int = 0, out: torch.Tensor = None, stream=None):
    """Rotate x [B, H, S, D] at positions pos0 + s (out=None: new tensor; out=x: in place)."""
    _need(x, "x")
    if x.dim() != 4:
        raise ValueError("x must be [B, H, S, D]")
    B, H, S, D = x.shape
    tmax = _table(table, D, x.device)
    if tmax == 0:
        raise ValueError("rope_apply needs a table")
    out = x if out is x else _out(out, x.shape, x.dtype, x.device)
    _check(_lib.attn_rope_apply(_ptr(x), _ptr(out), _dt(x), B, H, S, D, pos0, _ptr(table), tmax,
                                _stream(stream)), "attn_rope_apply")
    return out


def prefill_workspace_bytes(B, Hkv, S, D) -> int:
    return int(_lib.attn_prefill_workspace_bytes(B, Hkv, S, D))


def _qkv(q, k, v):
    """Shapes of a prefill's q [B, Hq, S, D] and k, v [B, Hkv, S, D], all on q's device."""
    _need(q, "q")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k and v must be [B, H, S, D]")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, q.device)
        _shape(t, (B, Hkv, S, D), n)
    return B, Hq, Hkv, S, D


def prefill(q, k, v, table=None, *, causal=True, pos0=0, window=None, out=None, out_dtype=None, lse=None,
            workspace=None, stream=None):
    """o = softmax(rope(q) rope(k)^T / sqrt(D)) v over [B, H, S, D] tensors (GQA when Hkv < Hq).

    window: None, or W >= 0 (causal only): row i sees keys i - W .. i.

    workspace: optional uint8 GPU tensor of >= prefill_workspace_bytes() bytes; with it the keys
    are rotated once into it (bf16 input with RoPE), without it the rotation is fused per tile."""
    B, Hq, Hkv, S, D = _qkv(q, k, v)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    out = _out(out, (B, Hq, S, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq * S, q.device)
    tmax = _table(table, D, q.device)
    if workspace is not None:
        _need(workspace, "workspace", q.device)
    _check(_lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dt(q), _dt(out), B, Hq,
                             Hkv, S, D, 1 if causal else 0, pos0, _win(window), _ptr(table), tmax,
                             _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "attn_prefill")
    return out


def rotate_keys_f16(k, table, pos0=0, out=None, stream=None):
    """Rotated keys for prefill_prerotated: a uint8 GPU buffer of prefill_workspace_bytes(B, Hkv, S, D)
    bytes holding the rotated rows as fp16 [B, Hkv, S, D] (rows reaching 2^15 scaled by a power of
    two), then one exponent byte per row.  rotated_keys_view() shows the fp16 part."""
    _need(k, "k")
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, S, D]")
    B, Hkv, S, D = k.shape
    if k.dtype != torch.bfloat16:
        raise TypeError("k must be bfloat16")
    tmax = _table(table, D, k.device)
    if tmax == 0:
        raise ValueError("rotate_keys_f16 needs a table")
    need = prefill_workspace_bytes(B, Hkv, S, D)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=k.device)
    _need(out, "out", k.device)
    if out.dtype != torch.uint8 or out.numel() < need:
        raise ValueError(f"out must be a uint8 buffer of at least {need} bytes")
    _check(_lib.attn_rotate_keys_f16(_ptr(k), _ptr(out), B, Hkv, S, D, pos0, _ptr(table), tmax,
                                     _stream(stream)), "attn_rotate_keys_f16")
    return out


def rotated_keys_view(buf, B, Hkv, S, D):
    """The fp16 rows [B, Hkv, S, D] of a rotate_keys_f16 buffer, and its exponent bytes [B, Hkv, S]."""
    n = B * Hkv * S * D * 2
    return buf[:n].view(torch.float16).view(B, Hkv, S, D), buf[n:n + B * Hkv * S].view(B, Hkv, S)


def prefill_prerotated(q, k_rot, v, table, *, causal=True, pos0=0, window=None, out=None, out_dtype=None,
                       lse=None, stream=None):
    """prefill() for keys already rotated by rotate_keys_f16 (same table and pos0); k_rot is its
    uint8 buffer, v gives B, Hkv, S and D."""
    _need(q, "q")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, H, S, D]")
    B, Hq, S, D = q.shape
    Hkv = v.shape[1]
    _need(v, "v", q.device)
    _shape(v, (B, Hkv, S, D), "v")
    _need(k_rot, "k_rot", q.device)
    need = prefill_workspace_bytes(B, Hkv, S, D)
    if k_rot.dtype != torch.uint8 or k_rot.numel() < need:
        raise ValueError(f"k_rot must be the uint8 buffer of rotate_keys_f16 ({need} bytes)")
    if q.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q and v must be bfloat16")
    tmax = _table(table, D, q.device)
    if tmax == 0:
        raise ValueError("prefill_prerotated needs a table")
    out = _out(out, (B, Hq, S, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq * S, q.device)
    _check(_lib.attn_prefill_prerotated(_ptr(q), _ptr(k_rot), _ptr(v), _ptr(out), _ptr(lse), _dt(out), B, Hq,
                                        Hkv, S, D, 1 if causal else 0, pos0, _win(window), _ptr(table),
                                        tmax, _stream(stream)), "attn_prefill_prerotated")
    return out


def _chunk_inputs(q, k_new, v_new):
    """Shapes of a chunk's q [B, Hq, Sq, D] and k_new, v_new [B, Hkv, Sq, D] (all bf16)."""
    _need(q, "q")
    if q.dim() != 4 or k_new.dim() != 4:
        raise ValueError("q, k_new and v_new must be [B, H, Sq, D]")
    B, Hq, Sq, D = q.shape
    Hkv = k_new.shape[1]
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, q.device)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
    _shape(k_new, (B, Hkv, Sq, D), "k_new")
    _shape(v_new, (B, Hkv, Sq, D), "v_new")
    return B, Hq, Hkv, Sq, D


def prefill_chunk(q, k_new, v_new, k_cache, v_cache, pos0, table=None, *, window=None, out=None,
                  out_dtype=None, lse=None, workspace=None, stream=None):
    """Append a chunk (k_new, v_new [B, Hkv, Sq, D]) to the cache [B, Hkv, S_max, D] at rows
    pos0 .. pos0+Sq-1 (keys rotated there), then attend q [B, Hq, Sq, D] to cache rows
    [0, pos0 + Sq) with the causal mask aligned at the bottom right.  All bf16.

    workspace: uint8 GPU tensor of >= prefill_workspace_bytes(B, Hkv, pos0 + Sq, D) bytes, needed
    with RoPE; allocated here when None."""
    B, Hq, Hkv, Sq, D = _chunk_inputs(q, k_new, v_new)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Hkv, S_max, D]")
    S_max = k_cache.shape[2]
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, q.device)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
        _shape(t, (B, Hkv, S_max, D), n)
    out = _out(out, (B, Hq, Sq, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq * Sq, q.device)
    tmax = _table(table, D, q.device)
    if tmax:
        workspace = _scratch(workspace, prefill_workspace_bytes(B, Hkv, pos0 + Sq, D), q.device, stream)
    elif workspace is not None:
        _need(workspace, "workspace", q.device)
    _check(_lib.attn_prefill_chunk(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                   _ptr(lse), _dt(out), B, Hq, Hkv, Sq, S_max, D, pos0, _win(window), _ptr(table),
                                   tmax, _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "attn_prefill_chunk")
    return out


def prefill_chunk_varpos(q, k_new, v_new, k_cache, v_cache, pos0, pos0_max, table=None, *, window=None,
                         out=None, out_dtype=None, lse=None, workspace=None, stream=None):
    """prefill_chunk() with a chunk start per sequence: pos0 is a device int32 [B] tensor (sequence
    b's chunk goes to cache rows pos0[b] .. pos0[b]+Sq-1) and pos0_max a host bound on its values
    (a sequence whose start lies outside [0, pos0_max] gets NaN rows and an untouched cache).
    workspace: uint8 GPU tensor of >= prefill_workspace_bytes(B, Hkv, pos0_max + Sq, D) bytes,
    needed with RoPE; allocated here when None."""
    B, Hq, Hkv, Sq, D = _chunk_inputs(q, k_new, v_new)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Hkv, S_max, D]")
    S_max = k_cache.shape[2]
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, q.device)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
        _shape(t, (B, Hkv, S_max, D), n)
    _need(pos0, "pos0", q.device)
    if pos0.dtype != torch.int32 or pos0.numel() != B:
        raise ValueError(f"pos0 must be int32 [{B}]")
    out = _out(out, (B, Hq, Sq, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq * Sq, q.device)
    tmax = _table(table, D, q.device)
    if tmax:
        workspace = _scratch(workspace, prefill_workspace_bytes(B, Hkv, pos0_max + Sq, D), q.device, stream)
    elif workspace is not None:
        _need(workspace, "workspace", q.device)
    _check(_lib.attn_prefill_chunk_varpos(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(pos0), int(pos0_max), _ptr(out), _ptr(lse), _dt(out), B, Hq, Hkv,
                                          Sq, S_max, D, _win(window), _ptr(table), tmax, _ptr(workspace),
                                          _nbytes(workspace), _stream(stream)),
           "attn_prefill_chunk_varpos")
    return out


def prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D) -> int:
    return int(_lib.attn_prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D))


def _pool(k_pages, v_pages, Hkv, D, device):
    """A paged pool [num_blocks, Hkv, block_size, D] (bf16) for K and V; returns (num_blocks, bs)."""
    if k_pages.dim() != 4:
        raise ValueError("k_pages must be [num_blocks, Hkv, block_size, D]")
    num_blocks, bs = k_pages.shape[0], k_pages.shape[2]
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n, device)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
        _shape(t, (num_blocks, Hkv, bs, D), n)
    return num_blocks, bs


def _block_table(block_table, B, device):
    _need(block_table, "block_table", device)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be int32 [{B}, max_blocks]")
    return int(block_table.shape[1])


def prefill_chunk_paged(q, k_new, v_new, k_pages, v_pages, block_table, pos0, table=None, *, window=None,
                        out=None, out_dtype=None, lse=None, workspace=None, stream=None):
    """prefill_chunk() against a paged cache: pools [num_blocks, Hkv, block_size, D] and an int32
    block table [B, max_blocks] (token t of sequence b in block block_table[b, t // block_size]).
    The chunk's keys and values go into their blocks; workspace: uint8 GPU tensor of
    >= prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D) bytes, allocated here when None."""
    B, Hq, Hkv, Sq, D = _chunk_inputs(q, k_new, v_new)
    num_blocks, bs = _pool(k_pages, v_pages, Hkv, D, q.device)
    max_blocks = _block_table(block_table, B, q.device)
    out = _out(out, (B, Hq, Sq, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq * Sq, q.device)
    tmax = _table(table, D, q.device)
    workspace = _scratch(workspace, prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D), q.device, stream)
    _check(_lib.attn_prefill_chunk_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                         num_blocks, bs, _ptr(block_table), max_blocks, _ptr(out),
                                         _ptr(lse), _dt(out), B, Hq, Hkv, Sq, D, pos0, _win(window), _ptr(table),
                                         tmax, _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "attn_prefill_chunk_paged")
    return out


def prefill_chunk_paged_varpos(q, k_new, v_new, k_pages, v_pages, block_table, pos0, pos0_max, table=None, *,
                               window=None, out=None, out_dtype=None, lse=None, workspace=None, stream=None):
    """prefill_chunk_paged() with a chunk start per sequence: pos0 is a device int32 [B] tensor and
    pos0_max a host bound on its values (a sequence whose start lies outside [0, pos0_max] gets
    NaN rows and none of its slots written).  workspace: uint8 GPU tensor of
    >= prefill_chunk_paged_workspace_bytes(B, Hkv, pos0_max, Sq, D) bytes, allocated here when None."""
    B, Hq, Hkv, Sq, D = _chunk_inputs(q, k_new, v_new)
    num_blocks, bs = _pool(k_pages, v_pages, Hkv, D, q.device)
    max_blocks = _block_table(block_table, B, q.device)
    _need(pos0, "pos0", q.device)
    if pos0.dtype != torch.int32 or pos0.numel() != B:
        raise ValueError(f"pos0 must be int32 [{B}]")
    out = _out(out, (B, Hq, Sq, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq * Sq, q.device)
    tmax = _table(table, D, q.device)
    workspace = _scratch(workspace, prefill_chunk_paged_workspace_bytes(B, Hkv, pos0_max, Sq, D), q.device, stream)
    _check(_lib.attn_prefill_chunk_paged_varpos(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                                num_blocks, bs, _ptr(block_table), max_blocks, _ptr(pos0),
                                                int(pos0_max), _ptr(out), _ptr(lse), _dt(out), B, Hq, Hkv, Sq, D,
                                                _win(window), _ptr(table), tmax, _ptr(workspace),
                                                _nbytes(workspace), _stream(stream)),
           "attn_prefill_chunk_paged_varpos")
    return out


def _append_inputs(k_new, v_new, pos):
    """Shapes of an append's k_new, v_new [B, Hkv, Sq, D] (bf16) and its int32 [B] positions."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n)
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError(f"{n} must be bfloat16 [B, Hkv, Sq, D]")
    if v_new.shape != k_new.shape or v_new.device != k_new.device:
        raise ValueError("v_new must match k_new")
    B, Hkv, Sq, D = k_new.shape
    _need(pos, "pos", k_new.device)
    if pos.dtype != torch.int32 or pos.numel() != B:
        raise ValueError(f"pos must be int32 [{B}]")
    return B, Hkv, Sq, D


def cache_append(k_new, v_new, k_cache, v_cache, pos, table=None, *, stream=None):
    """Write Sq new tokens of every sequence into the cache [B, Hkv, S_max, D] (bf16): sequence b's
    at rows pos[b] .. pos[b]+Sq-1 (pos: device int32 [B]), keys rotated there, values copied; a
    sequence whose rows would leave the cache (or the table) is not written."""
    B, Hkv, Sq, D = _append_inputs(k_new, v_new, pos)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Hkv, S_max, D]")
    S_max = k_cache.shape[2]
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, k_new.device)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
        _shape(t, (B, Hkv, S_max, D), n)
    tmax = _table(table, D, k_new.device)
    _check(_lib.attn_cache_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(pos), B, Hkv, Sq,
                                  S_max, D, _ptr(table), tmax, _stream(stream)),
           "attn_cache_append")


def cache_append_paged(k_new, v_new, k_pages, v_pages, block_table, pos, table=None, *, stream=None):
    """cache_append() into a paged pool [num_blocks, Hkv, block_size, D] with an int32 block table
    [B, max_blocks] (token t of sequence b in block block_table[b, t // block_size])."""
    B, Hkv, Sq, D = _append_inputs(k_new, v_new, pos)
    num_blocks, bs = _pool(k_pages, v_pages, Hkv, D, k_new.device)
    max_blocks = _block_table(block_table, B, k_new.device)
    tmax = _table(table, D, k_new.device)
    _check(_lib.attn_cache_append_paged(_ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), num_blocks, bs,
                                        _ptr(block_table), max_blocks, _ptr(pos), B, Hkv, Sq, D, _ptr(table), tmax,
                                        _stream(stream)),
           "attn_cache_append_paged")


def decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split=0) -> int:
    return int(_lib.attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split))


def decode_num_splits(B, Hq, Hkv, S_max, D, n_split=0) -> int:
    return int(_lib.attn_decode_num_splits(B, Hq, Hkv, S_max, D, n_split))


def _decode_common(q, cache_len, q_pos):
    """Shapes of a decode's q [B, Hq, 1, D] and its per-sequence int32 [B] vectors."""
    _need(q, "q")
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [B, Hq, 1, D]")
    B, Hq, _, D = q.shape
    for t, n in ((cache_len, "cache_len"), (q_pos, "q_pos")):
        if t is None:
            if n == "cache_len":
                raise ValueError("cache_len is required")
            continue
        _need(t, n, q.device)
        if t.dtype != torch.int32 or t.numel() != B:
            raise ValueError(f"{n} must be int32 [{B}]")
    return B, Hq, D


def decode(q, k_cache, v_cache, cache_len, q_pos, table=None, *, n_split=0, window=None, out=None,
           out_dtype=None, lse=None, workspace=None, stream=None):
    """One query per sequence (q [B, Hq, 1, D]) against the cache [B, Hkv, S_max, D].

    window: None, or W >= 0: only cache rows j >= q_pos[b] - W are seen."""
    B, Hq, D = _decode_common(q, cache_len, q_pos)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Hkv, S_max, D]")
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, q.device)
        _shape(t, (B, Hkv, S_max, D), n)
        if t.dtype != q.dtype:
            raise ValueError(f"{n} must have q's dtype")
    out = _out(out, (B, Hq, 1, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq, q.device)
    tmax = _table(table, D, q.device)
    workspace = _scratch(workspace, decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split), q.device, stream)
    _check(_lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(q_pos),
                            _ptr(out), _ptr(lse), _dt(q), _dt(out), B, Hq, Hkv, S_max, D, _win(window),
                            _ptr(table), tmax, n_split, _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "attn_decode")
    return out


def decode_paged(q, k_pages, v_pages, block_table, cache_len, q_pos, table=None, *, n_split=0, window=None,
                 out=None, out_dtype=None, lse=None, workspace=None, stream=None):
    """decode() against a paged cache: pools [num_blocks, Hkv, block_size, D] and an int32 block
    table [B, max_blocks] (token t of sequence b in block block_table[b, t // block_size])."""
    B, Hq, D = _decode_common(q, cache_len, q_pos)
    if k_pages.dim() != 4:
        raise ValueError("k_pages must be [num_blocks, Hkv, block_size, D]")
    Hkv = k_pages.shape[1]
    num_blocks, bs = _pool(k_pages, v_pages, Hkv, D, q.device)
    if k_pages.dtype != q.dtype:
        raise ValueError("k_pages must have q's dtype")
    max_blocks = _block_table(block_table, B, q.device)
    out = _out(out, (B, Hq, 1, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq, q.device)
    tmax = _table(table, D, q.device)
    workspace = _scratch(workspace, decode_workspace_bytes(B, Hq, Hkv, max_blocks * bs, D, n_split), q.device,
                         stream)
    _check(_lib.attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), num_blocks, bs, _ptr(block_table),
                                  max_blocks, _ptr(cache_len), _ptr(q_pos), _ptr(out), _ptr(lse), _dt(q), _dt(out),
                                  B, Hq, Hkv, D, _win(window), _ptr(table), tmax, n_split, _ptr(workspace),
                                  _nbytes(workspace), _stream(stream)),
           "attn_decode_paged")
    return out


def decode_noalloc(q, k_cache, v_cache, cache_len, q_pos, table=None, *, n_split=0, window=None, out=None,
                   out_dtype=None, lse=None, stream=None):
    """decode() through attn_decode_noalloc: the split partials go to the library's static per-GPU
    buffer instead of a workspace, so the C call allocates nothing (out is allocated here when None).
    Calls that can overlap on one GPU race on that buffer."""
    B, Hq, D = _decode_common(q, cache_len, q_pos)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Hkv, S_max, D]")
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, q.device)
        _shape(t, (B, Hkv, S_max, D), n)
        if t.dtype != q.dtype:
            raise ValueError(f"{n} must have q's dtype")
    out = _out(out, (B, Hq, 1, D), out_dtype or (out.dtype if out is not None else q.dtype), q.device)
    _lse(lse, B * Hq, q.device)
    tmax = _table(table, D, q.device)
    _check(_lib.attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(q_pos),
                                    _ptr(out), _ptr(lse), _dt(q), _dt(out), B, Hq, Hkv, S_max, D, _win(window),
                                    _ptr(table), tmax, n_split, _stream(stream)),
           "attn_decode_noalloc")
    return out
