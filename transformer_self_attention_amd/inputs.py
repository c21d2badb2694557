"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark.

This module holds no attention or RoPE arithmetic: it draws numbers, rounds them to
the storage dtype, and picks sampled row indices.  Both the fp64 oracle and the HIP
path consume exactly the arrays produced here.

Recipe (fixed, so every consumer sees the same bits):
  * ``numpy.random.Generator(PCG64(seed))``; ``standard_normal`` in float64, drawn in
    C order of the tensor shape, in the order Q, K, V (then any extra draws);
  * float64 -> float32 (round to nearest) -> bfloat16 (round to nearest even) for the
    bf16 workloads; fp32 workloads stop after the float32 step;
  * the long-context workload then draws, per (batch, kv-head), round(1% * S) distinct
    key positions and multiplies those pre-RoPE key rows by 8 (exact in bf16);
  * sampled query rows are drawn last, per query head, and always include
    0, 1, S-2 and S-1.

Shapes follow the workloads the pages discuss: 2k-token prefill with 32 heads of width
128, 8k-token GQA with 64 query / 8 KV heads, batch-32 decode over an 8k cache, and a
32k-token long context; the chunked prefill is the last 2k chunk of the 8k GQA prompt.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int           # prefill: query and key length; decode: cache length per sequence
    D: int
    dtype: str       # "f32" or "bf16"
    seed: int
    kind: str        # "prefill" or "decode"
    check_rows: int = 0      # 0: every row is checked
    big_key_frac: float = 0.0
    big_key_scale: float = 1.0
    rope_base: float = 10000.0
    pos0: int = 0            # chunk: position of the chunk's first token (cache rows before it are filled)
    S_max: int = 0           # chunk: cache rows per (sequence, KV head)
    window: int = -1         # sliding window W (a query sees the W keys before it); -1: none

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def prefill_flops(self) -> float:
        """Causal half of the two S x S x D contractions: 2*B*Hq*S^2*D.  With a sliding window W
        the (S-W-1)(S-W)/2 query-key pairs before the windows are not counted."""
        pairs = self.S * self.S / 2.0
        if 0 <= self.window < self.S - 1:
            pairs -= (self.S - self.window - 1) * (self.S - self.window) / 2.0
        return 4.0 * self.B * self.Hq * self.D * pairs

    def prefill_bytes(self) -> int:
        """Bytes a prefill must move at least: read Q, K and V once, write O once."""
        esz = 2 if self.dtype == "bf16" else 4
        return (2 * self.B * self.Hq + 2 * self.B * self.Hkv) * self.S * self.D * esz

    def chunk_flops(self) -> float:
        """Chunk of S queries after pos0 cached keys: query i meets pos0 + i + 1 keys, counted as
        4*D per query-key pair with the diagonal half-block, like prefill_flops at pos0 = 0:
        4*B*Hq*D*(pos0*S + S^2/2)."""
        return 4.0 * self.B * self.Hq * self.D * (self.pos0 * self.S + self.S * self.S / 2.0)

    def decode_kv_bytes(self) -> int:
        """K and V cache bytes one decode step must read (query at position S; with a sliding
        window W only the last min(S, W) cache rows are visible)."""
        esz = 2 if self.dtype == "bf16" else 4
        rows = self.S if self.window < 0 else min(self.S, self.window)
        return 2 * self.B * self.Hkv * rows * self.D * esz


WORKLOADS = {
    "tiny": Workload("tiny", B=1, Hq=4, Hkv=4, S=128, D=64, dtype="f32", seed=0, kind="prefill"),
    "mha": Workload("mha", B=4, Hq=32, Hkv=32, S=2048, D=128, dtype="bf16", seed=1, kind="prefill"),
    "gqa": Workload("gqa", B=1, Hq=64, Hkv=8, S=8192, D=128, dtype="bf16", seed=2, kind="prefill",
                    check_rows=256),
    "decode": Workload("decode", B=32, Hq=64, Hkv=8, S=8192, D=128, dtype="bf16", seed=3, kind="decode"),
    "long": Workload("long", B=1, Hq=32, Hkv=8, S=32768, D=128, dtype="bf16", seed=4, kind="prefill",
                     check_rows=128, big_key_frac=0.01, big_key_scale=8.0),
    # the long-context prefill and the decode workload with a 4096-token sliding window
    "swa": Workload("swa", B=1, Hq=32, Hkv=8, S=32768, D=128, dtype="bf16", seed=6, kind="prefill",
                    check_rows=128, window=4096),
    "swa_decode": Workload("swa_decode", B=32, Hq=64, Hkv=8, S=8192, D=128, dtype="bf16", seed=3, kind="decode",
                           window=4096),
    # multi-query decode: one KV head for all 64 query heads
    "mqa_decode": Workload("mqa_decode", B=32, Hq=64, Hkv=1, S=8192, D=128, dtype="bf16", seed=7, kind="decode"),
    # the last 2048-token chunk of an 8192-token GQA prompt, against the 6144 tokens already cached
    "chunk": Workload("chunk", B=1, Hq=64, Hkv=8, S=2048, D=128, dtype="bf16", seed=5, kind="chunk",
                      check_rows=128, pos0=6144, S_max=8192),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """One generated tensor: storage bits plus the exact values they hold (float64)."""

    def __init__(self, values32: np.ndarray, dtype: str):
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = f32_to_bf16_bits(values32)
            self.f32 = bf16_bits_to_f32(self.bits)
        elif dtype == "f32":
            self.bits = None
            self.f32 = np.ascontiguousarray(values32, dtype=np.float32)
        else:
            raise ValueError(dtype)

    @classmethod
    def from_bf16_bits(cls, bits: np.ndarray) -> "Tensor":
        t = cls.__new__(cls)
        t.dtype = "bf16"
        t.bits = np.ascontiguousarray(bits, dtype=np.uint16)
        t.f32 = bf16_bits_to_f32(t.bits)
        return t

    @property
    def shape(self):
        return self.f32.shape

    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)

    def torch(self, device="cpu"):
        import torch
        if self.dtype == "bf16":
            t = torch.from_numpy(self.bits.view(np.int16).copy()).view(torch.bfloat16)
        else:
            t = torch.from_numpy(self.f32.copy())
        return t.to(device)


def _normal32(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """float64 standard normals drawn in C order (chunked; same stream as one draw), cast to float32."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s)
    return out.reshape(shape)


def sample_rows(rng: np.random.Generator, S: int, n: int) -> np.ndarray:
    """n distinct row indices in [0, S), always containing 0, 1, S-2, S-1 (sorted)."""
    if n <= 0 or n >= S:
        return np.arange(S)
    fixed = np.unique(np.array([0, 1, S - 2, S - 1]))
    pool = np.setdiff1d(np.arange(S), fixed)
    extra = rng.choice(pool, size=max(0, n - fixed.size), replace=False)
    return np.sort(np.concatenate([fixed, extra]))


@dataclasses.dataclass
class PrefillInputs:
    wl: Workload
    q: Tensor
    k: Tensor
    v: Tensor
    big_keys: Optional[np.ndarray]     # [B, Hkv, n] positions scaled, or None
    rows: np.ndarray                   # [Hq, n_rows] checked query rows per head


@dataclasses.dataclass
class DecodeInputs:
    wl: Workload
    q: Tensor           # [B, Hq, 1, D]
    k_cache: Tensor     # [B, Hkv, S, D]
    v_cache: Tensor     # [B, Hkv, S, D]
    cache_len: np.ndarray   # [B] int32
    q_pos: np.ndarray       # [B] int32


def make_prefill(wl: Workload, *, S: Optional[int] = None, B: Optional[int] = None,
                 seed: Optional[int] = None) -> PrefillInputs:
    """Draw Q, K, V for a prefill workload (optionally with S, B or seed overridden)."""
    if S is not None or B is not None:
        wl = dataclasses.replace(wl, S=S if S is not None else wl.S, B=B if B is not None else wl.B)
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    qs = (wl.B, wl.Hq, wl.S, wl.D)
    ks = (wl.B, wl.Hkv, wl.S, wl.D)
    q32 = _normal32(rng, qs)
    k32 = _normal32(rng, ks)
    v32 = _normal32(rng, ks)
    q = Tensor(q32, wl.dtype)
    del q32
    k = Tensor(k32, wl.dtype)
    del k32
    v = Tensor(v32, wl.dtype)
    del v32
    big = None
    if wl.big_key_frac > 0:
        nbig = int(round(wl.big_key_frac * wl.S))
        big = np.empty((wl.B, wl.Hkv, nbig), dtype=np.int64)
        kv = k.f32.copy()
        for b in range(wl.B):
            for h in range(wl.Hkv):
                pos = np.sort(rng.choice(wl.S, size=nbig, replace=False))
                big[b, h] = pos
                kv[b, h, pos, :] *= np.float32(wl.big_key_scale)
        k = Tensor(kv, wl.dtype)   # x8 is a power of two: exact after rounding
    rows = np.stack([sample_rows(rng, wl.S, wl.check_rows) for _ in range(wl.Hq)])
    return PrefillInputs(wl, q, k, v, big, rows)


@dataclasses.dataclass
class ChunkInputs:
    wl: Workload
    q: Tensor           # [B, Hq, S, D]   the chunk's queries (not rotated)
    k_new: Tensor       # [B, Hkv, S, D]  the chunk's keys (not rotated)
    v_new: Tensor       # [B, Hkv, S, D]
    k_cache: Tensor     # [B, Hkv, S_max, D] cache before the chunk (rows < pos0 used; keys as stored)
    v_cache: Tensor     # [B, Hkv, S_max, D]
    rows: np.ndarray    # [Hq, n_rows] checked query rows per head


def make_chunk(wl: Workload, *, seed: Optional[int] = None) -> ChunkInputs:
    """Draw a chunk and the cache it is appended to, in the order q, k_new, v_new, k_cache,
    v_cache (every cache row is drawn; rows from pos0 on are overwritten by the append)."""
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    q = Tensor(_normal32(rng, (wl.B, wl.Hq, wl.S, wl.D)), wl.dtype)
    kn = Tensor(_normal32(rng, (wl.B, wl.Hkv, wl.S, wl.D)), wl.dtype)
    vn = Tensor(_normal32(rng, (wl.B, wl.Hkv, wl.S, wl.D)), wl.dtype)
    kc = Tensor(_normal32(rng, (wl.B, wl.Hkv, wl.S_max, wl.D)), wl.dtype)
    vc = Tensor(_normal32(rng, (wl.B, wl.Hkv, wl.S_max, wl.D)), wl.dtype)
    rows = np.stack([sample_rows(rng, wl.S, wl.check_rows) for _ in range(wl.Hq)])
    return ChunkInputs(wl, q, kn, vn, kc, vc, rows)


def make_decode(wl: Workload, *, B: Optional[int] = None, S: Optional[int] = None,
                seed: Optional[int] = None, cache_len=None, q_pos=None) -> DecodeInputs:
    """Draw the query and the (already rotated) K/V cache for a decode workload."""
    if S is not None or B is not None:
        wl = dataclasses.replace(wl, S=S if S is not None else wl.S, B=B if B is not None else wl.B)
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    q = Tensor(_normal32(rng, (wl.B, wl.Hq, 1, wl.D)), wl.dtype)
    kc = Tensor(_normal32(rng, (wl.B, wl.Hkv, wl.S, wl.D)), wl.dtype)
    vc = Tensor(_normal32(rng, (wl.B, wl.Hkv, wl.S, wl.D)), wl.dtype)
    if cache_len is None:
        cache_len = np.full(wl.B, wl.S, dtype=np.int32)
    if q_pos is None:
        q_pos = np.asarray(cache_len, dtype=np.int32).copy()
    return DecodeInputs(wl, q, kc, vc, np.asarray(cache_len, dtype=np.int32), np.asarray(q_pos, dtype=np.int32))


BF16_NAN_BITS = 0x7FC0


@dataclasses.dataclass
class PagedDecodeInputs:
    wl: Workload
    q: Tensor                 # [B, Hq, 1, D]
    k_pages: Tensor           # [num_blocks, Hkv, block_size, D]
    v_pages: Tensor
    block_table: np.ndarray   # int32 [B, max_blocks]
    cache_len: np.ndarray     # int32 [B]
    q_pos: np.ndarray         # int32 [B]
    block_size: int
    contiguous: DecodeInputs  # the same cache, unpaged


def make_paged_decode(wl: Workload, *, block_size: int = 16, spare_blocks: int = 5, seed: Optional[int] = None,
                      cache_len=None, q_pos=None) -> PagedDecodeInputs:
    """The decode inputs of make_decode (same draws), with the cache cut into blocks of
    block_size tokens scattered over a pool in a seeded random order (as blocks allocated on
    demand end up).  Pool blocks that belong to no sequence (spare_blocks of them, plus the
    unused tail of each sequence's last block) hold bf16 NaN, so reading one shows in the result.
    The layout draws come from their own stream (seed + 1000003), after nothing else."""
    d = make_decode(wl, seed=seed, cache_len=cache_len, q_pos=q_pos)
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed + 1000003))
    B, Hkv, S, D = wl.B, wl.Hkv, wl.S, wl.D
    nb = -(-S // block_size)
    num_blocks = B * nb + spare_blocks
    perm = rng.permutation(num_blocks)
    table = perm[:B * nb].reshape(B, nb).astype(np.int32)

    def scatter(bits):
        pool = np.full((num_blocks, Hkv, block_size, D), BF16_NAN_BITS, dtype=np.uint16)
        padded = np.full((B, Hkv, nb * block_size, D), BF16_NAN_BITS, dtype=np.uint16)
        padded[:, :, :S] = bits
        blocks = padded.reshape(B, Hkv, nb, block_size, D).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv,
                                                                                            block_size, D)
        pool[perm[:B * nb]] = blocks
        return Tensor.from_bf16_bits(pool)

    return PagedDecodeInputs(wl, d.q, scatter(d.k_cache.bits), scatter(d.v_cache.bits), table, d.cache_len,
                             d.q_pos, block_size, d)


@dataclasses.dataclass
class PagedChunkInputs:
    wl: Workload
    chunk: ChunkInputs        # the same draws with the cache contiguous
    k_pages: Tensor           # [num_blocks, Hkv, block_size, D]: the cache cut into blocks
    v_pages: Tensor
    block_table: np.ndarray   # int32 [B, max_blocks]
    block_size: int


def make_paged_chunk(wl: Workload, *, block_size: int = 16, spare_blocks: int = 5,
                     seed: Optional[int] = None) -> PagedChunkInputs:
    """The inputs of make_chunk (same draws), with the cache [B, Hkv, S_max, D] cut into blocks of
    block_size tokens scattered over a pool in a seeded random order.  Pool slots of no
    sequence (spare blocks, the tail of each sequence's last block) hold bf16 NaN.  The layout
    draws come from their own stream (seed + 1000003), after nothing else."""
    c = make_chunk(wl, seed=seed)
    seed = wl.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed + 1000003))
    B, Hkv, S, D = wl.B, wl.Hkv, wl.S_max, wl.D
    nb = -(-S // block_size)
    num_blocks = B * nb + spare_blocks
    perm = rng.permutation(num_blocks)
    table = perm[:B * nb].reshape(B, nb).astype(np.int32)

    def scatter(bits):
        pool = np.full((num_blocks, Hkv, block_size, D), BF16_NAN_BITS, dtype=np.uint16)
        padded = np.full((B, Hkv, nb * block_size, D), BF16_NAN_BITS, dtype=np.uint16)
        padded[:, :, :S] = bits
        blocks = padded.reshape(B, Hkv, nb, block_size, D).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv,
                                                                                            block_size, D)
        pool[perm[:B * nb]] = blocks
        return Tensor.from_bf16_bits(pool)

    return PagedChunkInputs(wl, c, scatter(c.k_cache.bits), scatter(c.v_cache.bits), table, block_size)

