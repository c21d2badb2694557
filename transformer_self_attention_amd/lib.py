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

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTED = (
    "attn_version",
    "attn_status_string",
    "attn_rope_table_bytes",
    "attn_rope_table_init",
    "attn_rope_table_init_scaled",
    "attn_rope_apply",
    "attn_prefill_workspace_bytes",
    "attn_prefill",
    "attn_rotate_keys_f16",
    "attn_prefill_prerotated",
    "attn_prefill_chunk",
    "attn_prefill_chunk_paged_workspace_bytes",
    "attn_prefill_chunk_paged",
    "attn_decode_workspace_bytes",
    "attn_decode_num_splits",
    "attn_decode",
    "attn_decode_paged",
)


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
    lib.attn_prefill_chunk_paged_workspace_bytes.restype = sz
    lib.attn_prefill_chunk_paged_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_prefill_chunk_paged.restype = i32
    lib.attn_prefill_chunk_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, fp, i32, i32, i32, i32,
                                             i32, i32, i32, i32, fp, i32, vp, sz, vp]
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
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def raw():
    """The ctypes handle itself (for tests of the C ABI)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.attn_status_string(int(status)).decode()


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


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


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
    _need(table, "table")
    B, H, S, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out")
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x")
    _check(_lib.attn_rope_apply(_ptr(x), _ptr(out), _dt(x), B, H, S, D, pos0, _ptr(table),
                                table.shape[0], _stream(stream)), "attn_rope_apply")
    return out


def prefill_workspace_bytes(B, Hkv, S, D) -> int:
    return int(_lib.attn_prefill_workspace_bytes(B, Hkv, S, D))


def prefill(q, k, v, table=None, *, causal=True, pos0=0, window=None, out=None, out_dtype=None, lse=None,
            workspace=None, stream=None):
    """o = softmax(rope(q) rope(k)^T / sqrt(D)) v over [B, H, S, D] tensors (GQA when Hkv < Hq).

    window: None, or W >= 0 (causal only): row i sees keys i - W .. i.

    workspace: optional uint8 GPU tensor of >= prefill_workspace_bytes() bytes; with it the keys
    are rotated once into it (bf16 input with RoPE), without it the rotation is fused per tile."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, S, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    if lse is not None:
        _need(lse, "lse")
        if lse.dtype != torch.float32 or lse.numel() != B * Hq * S:
            raise ValueError("lse must be float32 [B, Hq, S]")
    tmax = 0
    if table is not None:
        _need(table, "table")
        tmax = table.shape[0]
    wsb = 0
    if workspace is not None:
        _need(workspace, "workspace")
        wsb = workspace.numel() * workspace.element_size()
    _check(_lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dt(q), _dt(out), B, Hq,
                             Hkv, S, D, 1 if causal else 0, pos0, _win(window), _ptr(table), tmax,
                             _ptr(workspace), wsb, _stream(stream)),
           "attn_prefill")
    return out


def rotate_keys_f16(k, table, pos0=0, out=None, stream=None):
    """Rotated keys as fp16 (a torch.float16 tensor shaped like k), for prefill_prerotated."""
    _need(k, "k")
    _need(table, "table")
    B, Hkv, S, D = k.shape
    if k.dtype != torch.bfloat16:
        raise TypeError("k must be bfloat16")
    if out is None:
        out = torch.empty(k.shape, dtype=torch.float16, device=k.device)
    _need(out, "out")
    if out.dtype != torch.float16 or out.shape != k.shape:
        raise ValueError("out must be float16 shaped like k")
    _check(_lib.attn_rotate_keys_f16(_ptr(k), _ptr(out), B, Hkv, S, D, pos0, _ptr(table), table.shape[0],
                                     _stream(stream)), "attn_rotate_keys_f16")
    return out


def prefill_prerotated(q, k_rot, v, table, *, causal=True, pos0=0, window=None, out=None, out_dtype=None,
                       lse=None, stream=None):
    """prefill() for keys already rotated by rotate_keys_f16 (same table and pos0)."""
    for t, n in ((q, "q"), (k_rot, "k_rot"), (v, "v"), (table, "table")):
        _need(t, n)
    B, Hq, S, D = q.shape
    Hkv = k_rot.shape[1]
    if k_rot.dtype != torch.float16 or q.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, v bfloat16 and k_rot float16 expected")
    if k_rot.shape != (B, Hkv, S, D) or v.shape != k_rot.shape:
        raise ValueError("k_rot and v must be [B, Hkv, S, D] matching q")
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    if lse is not None:
        _need(lse, "lse")
    _check(_lib.attn_prefill_prerotated(_ptr(q), _ptr(k_rot), _ptr(v), _ptr(out), _ptr(lse), _dt(out), B, Hq,
                                        Hkv, S, D, 1 if causal else 0, pos0, _win(window), _ptr(table),
                                        table.shape[0], _stream(stream)), "attn_prefill_prerotated")
    return out


def prefill_chunk(q, k_new, v_new, k_cache, v_cache, pos0, table=None, *, window=None, out=None,
                  out_dtype=None, lse=None, workspace=None, stream=None):
    """Append a chunk (k_new, v_new [B, Hkv, Sq, D]) to the cache [B, Hkv, S_max, D] at rows
    pos0 .. pos0+Sq-1 (keys rotated there), then attend q [B, Hq, Sq, D] to cache rows
    [0, pos0 + Sq) with the causal mask aligned at the bottom right.  All bf16.

    workspace: uint8 GPU tensor of >= prefill_workspace_bytes(B, Hkv, pos0 + Sq, D) bytes, needed
    with RoPE; allocated here when None."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
    B, Hq, Sq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if k_new.shape != (B, Hkv, Sq, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B, Hkv, Sq, D]")
    if k_cache.shape != (B, Hkv, S_max, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [B, Hkv, S_max, D]")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    if lse is not None:
        _need(lse, "lse")
        if lse.dtype != torch.float32 or lse.numel() != B * Hq * Sq:
            raise ValueError("lse must be float32 [B, Hq, Sq]")
    tmax = 0
    if table is not None:
        _need(table, "table")
        tmax = table.shape[0]
        if workspace is None:
            workspace = torch.empty(max(prefill_workspace_bytes(B, Hkv, pos0 + Sq, D), 16), dtype=torch.uint8,
                                    device=q.device)
    wsb = 0
    if workspace is not None:
        _need(workspace, "workspace")
        wsb = workspace.numel() * workspace.element_size()
    _check(_lib.attn_prefill_chunk(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                   _ptr(lse), _dt(out), B, Hq, Hkv, Sq, S_max, D, pos0, _win(window), _ptr(table),
                                   tmax, _ptr(workspace), wsb, _stream(stream)), "attn_prefill_chunk")
    return out


def prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D) -> int:
    return int(_lib.attn_prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D))


def prefill_chunk_paged(q, k_new, v_new, k_pages, v_pages, block_table, pos0, table=None, *, window=None,
                        out=None, out_dtype=None, lse=None, workspace=None, stream=None):
    """prefill_chunk() against a paged cache: pools [num_blocks, Hkv, block_size, D] and an int32
    block table [B, max_blocks] (token t of sequence b in block block_table[b, t // block_size]).
    The chunk's keys and values go into their blocks; workspace: uint8 GPU tensor of
    >= prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D) bytes, allocated here when None."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
    _need(block_table, "block_table")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    B, Hq, Sq, D = q.shape
    num_blocks, Hkv, bs = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if k_new.shape != (B, Hkv, Sq, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B, Hkv, Sq, D]")
    if k_pages.shape != (num_blocks, Hkv, bs, D) or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages must be [num_blocks, Hkv, block_size, D]")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    if lse is not None:
        _need(lse, "lse")
        if lse.dtype != torch.float32 or lse.numel() != B * Hq * Sq:
            raise ValueError("lse must be float32 [B, Hq, Sq]")
    tmax = 0
    if table is not None:
        _need(table, "table")
        tmax = table.shape[0]
    if workspace is None:
        workspace = torch.empty(max(prefill_chunk_paged_workspace_bytes(B, Hkv, pos0, Sq, D), 16),
                                dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace")
    _check(_lib.attn_prefill_chunk_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                         num_blocks, bs, _ptr(block_table), block_table.shape[1], _ptr(out),
                                         _ptr(lse), _dt(out), B, Hq, Hkv, Sq, D, pos0, _win(window), _ptr(table),
                                         tmax, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream)), "attn_prefill_chunk_paged")
    return out


def decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split=0) -> int:
    return int(_lib.attn_decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split))


def decode_num_splits(B, Hq, Hkv, S_max, D, n_split=0) -> int:
    return int(_lib.attn_decode_num_splits(B, Hq, Hkv, S_max, D, n_split))


def decode(q, k_cache, v_cache, cache_len, q_pos, table=None, *, n_split=0, window=None, out=None,
           out_dtype=None, lse=None, workspace=None, stream=None):
    """One query per sequence (q [B, Hq, 1, D]) against the cache [B, Hkv, S_max, D].

    window: None, or W >= 0: only cache rows j >= q_pos[b] - W are seen."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (cache_len, "cache_len")):
        _need(t, n)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B, Hq, 1, D]")
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if cache_len.dtype != torch.int32 or cache_len.numel() != B:
        raise ValueError("cache_len must be int32 [B]")
    if q_pos is not None:
        _need(q_pos, "q_pos")
        if q_pos.dtype != torch.int32 or q_pos.numel() != B:
            raise ValueError("q_pos must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    need = decode_workspace_bytes(B, Hq, Hkv, S_max, D, n_split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace")
    tmax = 0
    if table is not None:
        _need(table, "table")
        tmax = table.shape[0]
    _check(_lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(q_pos),
                            _ptr(out), _ptr(lse), _dt(q), _dt(out), B, Hq, Hkv, S_max, D, _win(window),
                            _ptr(table), tmax, n_split, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)), "attn_decode")
    return out


def decode_paged(q, k_pages, v_pages, block_table, cache_len, q_pos, table=None, *, n_split=0, window=None,
                 out=None, out_dtype=None, lse=None, workspace=None, stream=None):
    """decode() against a paged cache: pools [num_blocks, Hkv, block_size, D] and an int32 block
    table [B, max_blocks] (token t of sequence b in block block_table[b, t // block_size])."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                 (cache_len, "cache_len")):
        _need(t, n)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B, Hq, 1, D]")
    num_blocks, Hkv, bs, _ = k_pages.shape
    if v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages must match")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    max_blocks = block_table.shape[1]
    if cache_len.dtype != torch.int32 or cache_len.numel() != B:
        raise ValueError("cache_len must be int32 [B]")
    if q_pos is not None:
        _need(q_pos, "q_pos")
        if q_pos.dtype != torch.int32 or q_pos.numel() != B:
            raise ValueError("q_pos must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    need = decode_workspace_bytes(B, Hq, Hkv, max_blocks * bs, D, n_split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace")
    tmax = 0
    if table is not None:
        _need(table, "table")
        tmax = table.shape[0]
    _check(_lib.attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), num_blocks, bs, _ptr(block_table),
                                  max_blocks, _ptr(cache_len), _ptr(q_pos), _ptr(out), _ptr(lse), _dt(q), _dt(out),
                                  B, Hq, Hkv, D, _win(window), _ptr(table), tmax, n_split, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "attn_decode_paged")
    return out
