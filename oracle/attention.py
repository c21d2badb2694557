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

Every score row is materialised in full (no tiling over keys, no running max/sum), so
nothing here mirrors the GPU's online-softmax recurrence.

Pins (tests/test_oracle.py): the pages' Problem 1 and Problem 2 numbers, RoPE norm
preservation, the Problem 3 closed form of the rotated inner product, relative-position
invariance, identity at position 0, softmax rows summing to one, causal row 0 == V[0],
zero-Q prefix means, permutation equivariance, torch's CPU
``scaled_dot_product_attention`` in float64, and a scalar brute force on tiny shapes.
"""

from __future__ import annotations

import numpy as np

__all__ = ["rope_frequencies", "rope", "attention", "decode"]


def rope_frequencies(D: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base^(-2i/D) for i = 0 .. D/2-1 (devthesis section 3, RoPE rotation matrix)."""
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


def rope(x: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of ``x`` (shape [..., S, D]) at ``positions`` [S].

    Pair i of the row at position m becomes
    (x_{2i} cos(m theta_i) - x_{2i+1} sin(m theta_i), x_{2i} sin(m theta_i) + x_{2i+1} cos(m theta_i)),
    the counter-clockwise rotation R_{Theta,m}^{(i)} of devthesis section 3.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    theta = rope_frequencies(D, base)
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    if pos.size != x.shape[-2]:
        raise ValueError("one position per row")
    ang = pos[:, None] * theta[None, :]          # [S, D/2], formed in float64
    c = np.cos(ang)
    s = np.sin(ang)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


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


def attention(q, k, v, *, causal: bool = True, rope_base=10000.0, pos0: int = 0, rows=None):
    """Prefill attention over [B, H, S, D] tensors, materialising every score row.

    q: [B, Hq, S, D]; k, v: [B, Hkv, S, D] (float64 or anything castable).
    rope_base: None disables RoPE; otherwise Q and K rows are rotated at positions pos0 + s.
    causal: key j is visible to query row i only if j <= i (square mask aligned at the top left).
    rows: None for every row, or an int array [Hq, n] of query rows to compute per head.
    Returns (o, lse): o [B, Hq, n, D], lse [B, Hq, n] (natural log of the softmax normaliser of
    the scaled scores).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
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
            k_rot[kv] = rope(k[b, kv], pos0 + keys, rope_base) if rope_base is not None else k[b, kv]
        for h in range(Hq):
            kv = h // G
            r = rows[h]
            qh = q[b, h, r]
            if rope_base is not None:
                qh = rope(qh, pos0 + r, rope_base)
            s = (qh @ k_rot[kv].T) * scale                  # [n, S] full rows
            if causal:
                s = np.where(keys[None, :] > r[:, None], -np.inf, s)
            w, ls = _softmax_rows(s)
            o[b, h] = w @ v[b, kv]
            lse[b, h] = ls
    return o, lse


def decode(q, k_cache, v_cache, cache_len, q_pos, *, rope_base=10000.0):
    """One query per sequence against a KV cache (keys already rotated; used as stored).

    q: [B, Hq, 1, D]; k_cache, v_cache: [B, Hkv, S_max, D]; cache_len, q_pos: [B] ints.
    Query head h of sequence b is rotated at q_pos[b] and attends to cache rows
    [0, min(cache_len[b], S_max)); cache_len <= 0 gives o = 0 and lse = -inf.
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
    for b in range(B):
        L = int(min(max(int(cache_len[b]), 0), S_max))
        if L == 0:
            continue
        qb = q[b, :, 0, :]                                   # [Hq, D]
        if rope_base is not None:
            qb = rope(qb[:, None, :], [int(q_pos[b])], rope_base)[:, 0, :]
        for kv in range(Hkv):
            qg = qb[kv * G:(kv + 1) * G]                     # [G, D]
            s = (qg @ kc[b, kv, :L].T) * scale               # [G, L]
            w, ls = _softmax_rows(s)
            o[b, kv * G:(kv + 1) * G, 0, :] = w @ vc[b, kv, :L]
            lse[b, kv * G:(kv + 1) * G] = ls
    return o, lse
