"""fp64 CPU oracle for RoPE + causal multi-head / grouped-query attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.  The
library under ``transformer_self_attention_amd/`` never imports it and shares no code
with it; the two meet only on arrays drawn by ``transformer_self_attention_amd/inputs.py``.

What it computes is the plain definition, written out with NumPy in float64:

* RoPE -- "Transformer Architecture & Self-Attention Mechanics" (devthesis.com), section 3
  "Positional Encodings", subsection "Rotary Position Embeddings (RoPE)": a head vector
  is split into adjacent pairs (x_{2i}, x_{2i+1}); at position m pair i is turned
  counter-clockwise by the angle m * theta_i with theta_i = base^(-2i/d).  The NumPy
  example on "Transformer Architecture: FlashAttention & RoPE" (academy.kwas.tech,
  "Simulating Rotary Position Embedding ... in Python") builds the same frequencies.
* Scores, mask, softmax, output -- devthesis section 1, the "Attention(Q,K,V)" equation
  and the row-wise softmax A_ij; the causal mask of "Multi-Head Attention & Rotary
  Position Embeddings (RoPE)" (learnllm.online), the PyTorch listing under "Rotary
  Position Embeddings (RoPE): Relative Angles in 2D Slices" (strictly upper triangle set
  to -inf before the softmax).
* GQA -- "Building Self-Attention and Transformer Engines" (codingpancake.com) section
  6.1 and its comparison table (one KV head per group of query heads).  The grouping
  formula is lost from the page; the reading used is: query head h reads KV head
  floor(h / G), G = Hq / Hkv (consecutive groups).
* Decode -- "Transformer internals: attention without the mysticism"
  (ninaddeshpande.com), "The KV cache and the memory wall": one new query per sequence
  attends to every cached key.  The cache is used as stored (already rotated); the
  query is rotated at its own position.
* Paged KV cache -- "Building Self-Attention and Transformer Engines" (codingpancake.com),
  section 6.2: the cache lives in fixed-size physical blocks (16 tokens on the page) found
  through a per-sequence table, like virtual-memory pages.  Token t of sequence b is in block
  block_table[b][t // block_size], slot t % block_size; decode then proceeds as above.
* RoPE frequency scaling -- "Transformer internals: attention without the mysticism"
  (ninaddeshpande.com), "Rotary positional embeddings (RoPE)", and devthesis Problem 3,
  "Superiority for Context Window Extension": to reach past the trained context, Position
  Interpolation, NTK-aware scaling and YaRN change the rotation frequencies.  The pages give no
  formulas; the published definitions are used (see RopeScaling).
* Sliding window -- "Building Self-Attention and Transformer Engines" (codingpancake.com),
  section 6.4: each token attends only to the W tokens before it (W = 4096 on the page).  The
  reading taken: the query at position p sees the keys at positions p - W .. p (the W preceding
  tokens and itself), on top of the causal mask.  window=None means no window.
* Chunked prefill against a cache -- the same page and section (keys and values of
  earlier tokens are kept and reused), with the chunked prefill named on "Multi-Head
  Attention & Rotary Position Embeddings (RoPE)" (learnllm.online), "Prefill vs Decode
  Latency & Memory Wall Waterfall": a chunk of Sq new tokens at positions pos0 .. pos0+Sq-1
  first appends its rotated keys (stored in bfloat16, the cache's format) and its values to
  the cache, then each new query attends to every cache row up to and including its own
  position (the causal mask aligned at the bottom right of the Sq x (pos0+Sq) score block).

Every score row is materialised in full (no tiling over keys, no running max/sum), so
nothing here mirrors the GPU's online-softmax recurrence.

Pins (tests/test_oracle.py, tests/test_oracle_cache.py): the pages' Problem 1 and Problem 2 numbers, RoPE norm
preservation, the Problem 3 closed form of the rotated inner product, relative-position
invariance, identity at position 0, softmax rows summing to one, causal row 0 == V[0],
zero-Q prefix means, permutation equivariance, torch's CPU
``scaled_dot_product_attention`` in float64, and a scalar brute force on tiny shapes.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["rope_frequencies", "rope", "attention", "decode", "round_bf16", "append_to_cache",
           "attention_with_cache", "decode_paged", "RopeScaling", "rope_angles"]


def rope_frequencies(D: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base^(-2i/D) for i = 0 .. D/2-1 (devthesis section 3, RoPE rotation matrix)."""
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


@dataclasses.dataclass(frozen=True)
class RopeScaling:
    """A RoPE frequency scaling for contexts longer than the trained one (factor s >= 1).

    kind "pi"   Position Interpolation (Chen et al. 2023): positions are divided by s, so the
                angle of pair i at position m is (m / s) theta_i.
    kind "ntk"  NTK-aware scaling: the base grows to base * s^(D / (D - 2)), which keeps the
                highest frequency (i = 0) and divides the lowest (i = D/2 - 1) by exactly s.
    kind "yarn" YaRN (Peng et al. 2023), "NTK-by-parts" with the attention temperature: with
                wavelength lambda_i = 2 pi / theta_i and r_i = original_max_pos / lambda_i, the
                ramp g_i = clip((r_i - beta_slow) / (beta_fast - beta_slow), 0, 1) mixes
                theta_i' = (1 - g_i) theta_i / s + g_i theta_i (long wavelengths interpolated,
                short ones kept), and both q and k are scaled by 0.1 ln(s) + 1 (so the scores
                by its square).
    """
    kind: str
    factor: float
    original_max_pos: int = 4096
    beta_fast: float = 32.0
    beta_slow: float = 1.0


def rope_angles(D: int, positions, base: float = 10000.0, scaling=None):
    """(angles [S, D/2], amplitude): pair i of the row at position m turns by angles[m, i] and is
    scaled by amplitude (1 except for YaRN)."""
    theta = rope_frequencies(D, base)
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    amp = 1.0
    if scaling is not None:
        s = float(scaling.factor)
        if s < 1.0:
            raise ValueError("scaling factor must be >= 1")
        if scaling.kind == "pi":
            pos = pos / s
        elif scaling.kind == "ntk":
            theta = rope_frequencies(D, float(base) * s ** (D / (D - 2.0)))
        elif scaling.kind == "yarn":
            r = scaling.original_max_pos * theta / (2.0 * math.pi)
            g = np.clip((r - scaling.beta_slow) / (scaling.beta_fast - scaling.beta_slow), 0.0, 1.0)
            theta = (1.0 - g) * theta / s + g * theta
            amp = 0.1 * math.log(s) + 1.0
        else:
            raise ValueError(f"unknown RoPE scaling {scaling.kind!r}")
    return pos[:, None] * theta[None, :], amp


def rope(x: np.ndarray, positions, base: float = 10000.0, scaling=None) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of ``x`` (shape [..., S, D]) at ``positions`` [S].

    Pair i of the row at position m becomes
    (x_{2i} cos(m theta_i) - x_{2i+1} sin(m theta_i), x_{2i} sin(m theta_i) + x_{2i+1} cos(m theta_i)),
    the counter-clockwise rotation R_{Theta,m}^{(i)} of devthesis section 3 (angles and an
    amplitude from ``scaling`` when given, see RopeScaling).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    if np.asarray(positions).reshape(-1).size != x.shape[-2]:
        raise ValueError("one position per row")
    ang, amp = rope_angles(D, positions, base, scaling)   # [S, D/2], formed in float64
    c = amp * np.cos(ang)
    s = amp * np.sin(ang)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _check_window(window, causal):
    if window is not None and (window < 0 or not causal):
        raise ValueError("a window is a non-negative key count, used with the causal mask")


def _softmax_rows(scores: np.ndarray):
    """Row-wise softmax of devthesis section 1 with the row max subtracted (exact in real arithmetic).

    Returns (weights, lse).  A row that is entirely -inf (no visible key) gives zero weights and
    lse = -inf.
    """
    m = np.max(scores, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(scores - m_safe)
    l = np.sum(e, axis=-1, keepdims=True)
    w = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return w, lse[..., 0]


def attention(q, k, v, *, causal: bool = True, rope_base=10000.0, pos0: int = 0, rows=None, window=None,
              rope_scaling=None):
    """Prefill attention over [B, H, S, D] tensors, materialising every score row.

    q: [B, Hq, S, D]; k, v: [B, Hkv, S, D] (float64 or anything castable).
    rope_base: None disables RoPE; otherwise Q and K rows are rotated at positions pos0 + s.
    causal: key j is visible to query row i only if j <= i (square mask aligned at the top left).
    window: None, or W >= 0 (causal only): key j is visible to row i only if j >= i - W.
    rows: None for every row, or an int array [Hq, n] of query rows to compute per head.
    Returns (o, lse): o [B, Hq, n, D], lse [B, Hq, n] (natural log of the softmax normaliser of
    the scaled scores).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _check_window(window, causal)
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if rows is None:
        rows = np.broadcast_to(np.arange(S), (Hq, S))
    rows = np.asarray(rows)
    n = rows.shape[1]
    keys = np.arange(S)
    scale = 1.0 / np.sqrt(D)
    o = np.empty((B, Hq, n, D))
    lse = np.empty((B, Hq, n))
    for b in range(B):
        k_rot = [None] * Hkv
        for kv in range(Hkv):
            k_rot[kv] = rope(k[b, kv], pos0 + keys, rope_base, rope_scaling) if rope_base is not None else k[b, kv]
        for h in range(Hq):
            kv = h // G
            r = rows[h]
            qh = q[b, h, r]
            if rope_base is not None:
                qh = rope(qh, pos0 + r, rope_base, rope_scaling)
            s = (qh @ k_rot[kv].T) * scale                  # [n, S] full rows
            if causal:
                s = np.where(keys[None, :] > r[:, None], -np.inf, s)
            if window is not None:
                s = np.where(keys[None, :] < r[:, None] - window, -np.inf, s)
            w, ls = _softmax_rows(s)
            o[b, h] = w @ v[b, kv]
            lse[b, h] = ls
    return o, lse


def decode(q, k_cache, v_cache, cache_len, q_pos, *, rope_base=10000.0, window=None, rope_scaling=None):
    """One query per sequence against a KV cache (keys already rotated; used as stored).

    q: [B, Hq, 1, D]; k_cache, v_cache: [B, Hkv, S_max, D]; cache_len, q_pos: [B] ints.
    Query head h of sequence b is rotated at q_pos[b] and attends to cache rows
    [0, min(cache_len[b], S_max)); cache_len <= 0 gives o = 0 and lse = -inf.  Cache row j holds
    the token at position j; with a window W only rows j >= q_pos[b] - W are visible (none
    visible: o = 0, lse = -inf).
    Returns (o [B, Hq, 1, D], lse [B, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, Hq, _, D = q.shape
    Hkv, S_max = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    o = np.zeros((B, Hq, 1, D))
    lse = np.full((B, Hq), -np.inf)
    _check_window(window, True)
    for b in range(B):
        L = int(min(max(int(cache_len[b]), 0), S_max))
        lo = 0 if window is None else max(0, int(q_pos[b]) - window)
        if lo >= L:
            continue
        qb = q[b, :, 0, :]                                   # [Hq, D]
        if rope_base is not None:
            qb = rope(qb[:, None, :], [int(q_pos[b])], rope_base, rope_scaling)[:, 0, :]
        for kv in range(Hkv):
            qg = qb[kv * G:(kv + 1) * G]                     # [G, D]
            s = (qg @ kc[b, kv, :L].T) * scale               # [G, L]
            s[:, :lo] = -np.inf                              # outside the window
            w, ls = _softmax_rows(s)
            o[b, kv * G:(kv + 1) * G, 0, :] = w @ vc[b, kv, :L]
            lse[b, kv * G:(kv + 1) * G] = ls
    return o, lse


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits, ties to even); float64 result.

    This is the storage format of the KV cache: keys rotated for a chunk are kept in it at this
    precision.  Written from the format's definition: x = m * 2^e with 0.5 <= |m| < 1, so m * 2^8
    is rounded to an integer (numpy rounds halves to even).  Zeros and non-finite values pass
    through; the bfloat16 subnormal range (|x| < 2^-126) is not treated specially.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    nz = np.isfinite(x) & (x != 0.0)
    m, e = np.frexp(x[nz])
    out[nz] = np.ldexp(np.round(m * 256.0), e - 8)
    return out


def append_to_cache(k_cache, v_cache, k_new, v_new, pos0: int, *, rope_base=10000.0, rope_scaling=None):
    """Cache after a chunk of Sq new tokens is written into rows [pos0, pos0 + Sq).

    k_cache, v_cache: [B, Hkv, S_max, D]; k_new, v_new: [B, Hkv, Sq, D].  Key row s is rotated
    at position pos0 + s (unless rope_base is None) and stored rounded to bfloat16; values are
    stored as given.  Rows outside [pos0, pos0 + Sq) are unchanged.  Returns new arrays.
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    Sq = k_new.shape[2]
    if pos0 < 0 or pos0 + Sq > kc.shape[2]:
        raise ValueError("chunk does not fit the cache")
    kr = rope(k_new, pos0 + np.arange(Sq), rope_base, rope_scaling) if rope_base is not None else k_new
    kc[:, :, pos0:pos0 + Sq] = round_bf16(kr)
    vc[:, :, pos0:pos0 + Sq] = v_new
    return kc, vc


def attention_with_cache(q, k_cache, v_cache, pos0: int, *, rope_base=10000.0, rows=None, window=None,
                         rope_scaling=None):
    """A chunk of Sq queries at positions pos0 .. pos0+Sq-1 against the cache rows [0, pos0 + Sq).

    q: [B, Hq, Sq, D] (rotated here at pos0 + i unless rope_base is None); k_cache, v_cache:
    [B, Hkv, S_max, D] used as stored (the chunk's own keys already appended).  Query i sees
    key j only if j <= pos0 + i (and, with a window W, j >= pos0 + i - W).  rows: None for every
    row, or an int array [Hq, n].
    Returns (o [B, Hq, n, D], lse [B, Hq, n]).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    Hkv = kc.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    Sk = pos0 + Sq
    if pos0 < 0 or Sk > kc.shape[2]:
        raise ValueError("chunk does not fit the cache")
    _check_window(window, True)
    G = Hq // Hkv
    if rows is None:
        rows = np.broadcast_to(np.arange(Sq), (Hq, Sq))
    rows = np.asarray(rows)
    n = rows.shape[1]
    keys = np.arange(Sk)
    scale = 1.0 / np.sqrt(D)
    o = np.empty((B, Hq, n, D))
    lse = np.empty((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            r = rows[h]
            qh = q[b, h, r]
            if rope_base is not None:
                qh = rope(qh, pos0 + r, rope_base, rope_scaling)
            s = (qh @ kc[b, kv, :Sk].T) * scale                  # [n, pos0 + Sq] full rows
            s = np.where(keys[None, :] > pos0 + r[:, None], -np.inf, s)
            if window is not None:
                s = np.where(keys[None, :] < pos0 + r[:, None] - window, -np.inf, s)
            w, ls = _softmax_rows(s)
            o[b, h] = w @ vc[b, kv, :Sk]
            lse[b, h] = ls
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, cache_len, q_pos, *, rope_base=10000.0, window=None,
                 rope_scaling=None):
    """Decode against a paged KV cache.

    k_pages, v_pages: [num_blocks, Hkv, block_size, D] physical blocks; block_table: int
    [B, max_blocks]; token t of sequence b is stored in block block_table[b, t // block_size] at
    slot t % block_size.  Sequence b attends to its tokens [0, min(cache_len[b], max_blocks *
    block_size)).  Other arguments and the result as in decode().
    """
    kp = np.asarray(k_pages, dtype=np.float64)
    vp = np.asarray(v_pages, dtype=np.float64)
    bt = np.asarray(block_table)
    B, max_blocks = bt.shape
    _, Hkv, bs, D = kp.shape
    S_max = max_blocks * bs
    kc = np.zeros((B, Hkv, S_max, D))
    vc = np.zeros((B, Hkv, S_max, D))
    for b in range(B):
        L = int(min(max(int(cache_len[b]), 0), S_max))
        for t in range(L):
            blk = int(bt[b, t // bs])
            kc[b, :, t] = kp[blk, :, t % bs]
            vc[b, :, t] = vp[blk, :, t % bs]
    return decode(q, kc, vc, cache_len, q_pos, rope_base=rope_base, window=window, rope_scaling=rope_scaling)


def append_to_cache_paged(k_pages, v_pages, block_table, k_new, v_new, pos0: int, *, rope_base=10000.0,
                          rope_scaling=None):
    """Pools after a chunk of Sq new tokens of every sequence is written into its blocks.

    k_pages, v_pages: [num_blocks, Hkv, block_size, D]; block_table: int [B, max_blocks] (token t
    of sequence b lives in block block_table[b, t // block_size], slot t % block_size,
    codingpancake.com section 6.2); k_new, v_new: [B, Hkv, Sq, D].  Token pos0 + i gets key row
    i rotated at position pos0 + i (unless rope_base is None) and rounded to bfloat16, and value
    row i as given.  Every other slot is unchanged.  Returns new arrays.
    """
    kp = np.array(k_pages, dtype=np.float64, copy=True)
    vp = np.array(v_pages, dtype=np.float64, copy=True)
    bt = np.asarray(block_table)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, _, Sq, _ = k_new.shape
    bs = kp.shape[2]
    if pos0 < 0 or pos0 + Sq > bt.shape[1] * bs:
        raise ValueError("chunk does not fit the block table")
    kr = rope(k_new, pos0 + np.arange(Sq), rope_base, rope_scaling) if rope_base is not None else k_new
    kr = round_bf16(kr)
    for b in range(B):
        for i in range(Sq):
            t = pos0 + i
            blk = int(bt[b, t // bs])
            kp[blk, :, t % bs] = kr[b, :, i]
            vp[blk, :, t % bs] = v_new[b, :, i]
    return kp, vp


def gather_pages(k_pages, v_pages, block_table, n_tokens: int):
    """The first n_tokens tokens of every sequence of a paged cache as contiguous arrays
    [B, Hkv, n_tokens, D] (same placement rule as append_to_cache_paged)."""
    kp = np.asarray(k_pages, dtype=np.float64)
    vp = np.asarray(v_pages, dtype=np.float64)
    bt = np.asarray(block_table)
    B = bt.shape[0]
    _, Hkv, bs, D = kp.shape
    kc = np.empty((B, Hkv, n_tokens, D))
    vc = np.empty((B, Hkv, n_tokens, D))
    for b in range(B):
        for t in range(n_tokens):
            blk = int(bt[b, t // bs])
            kc[b, :, t] = kp[blk, :, t % bs]
            vc[b, :, t] = vp[blk, :, t % bs]
    return kc, vc
