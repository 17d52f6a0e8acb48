"""fp64 reference for the latent KV cache path (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module; the HIP product path never imports it and it imports nothing from
the product path.

Notation (multi-head latent attention, DeepSeek-V2 convention; DeepSeek-V2 is
listed under "Builds on" on the VideoMLA mlsanity.com page and on the
atlas.scime.ai summary):

  B batch, H heads, d_h head dim, d_c latent rank, d_r positional-key width,
  D = model width.  Weights are stored "out x in" as in that paper:
      w_dkv [d_c, D]      c   = w_dkv @ x           (content latent)
      w_kr  [d_r, D]      k_R = RoPE(w_kr @ x)      (head-shared positional key)
      w_uk  [H, d_h, d_c] k_h = w_uk[h] @ c         (per-head key, never cached)
      w_uv  [H, d_h, d_c] v_h = w_uv[h] @ c         (per-head value, never cached)
  The cache holds, per token, the row [c || k_R]: d_c + d_r scalars (VideoMLA
  atlas.scime.ai summary, "Key results": 224 scalars per token per layer at
  d_c = 192, d_r = 32, against 3072 for 12 heads x 128 of dense K and V).

Readings where the pages are silent:
  * 3D-RoPE: the d_r vector is split into contiguous per-axis blocks
    [t | h | w] (default widths 8/12/12); inside a block of width d_a, the
    adjacent pair (2i, 2i+1) is rotated by angle p_a * theta**(-2i/d_a),
    theta = 1e4.
  * The score of query row (b, i, h) against key j is
        scale * ( q[b,i,h] . k_h[j]  +  RoPE(p_i) q_r[b,i,h] . k_R[j] )
    i.e. the content part uses the per-head key reconstructed from the
    latent and the positional part uses the head-shared rotated key, with
    q_r per head (decoupled RoPE as in DeepSeek-V2).
  * Chunk-causal visibility: key j is visible to query i iff
    chunk(j) <= chunk(i) (bidirectional inside a chunk, causal across).
  * bf16 rounding is round-to-nearest-even, applied directly to the fp64
    value (no intermediate fp32 rounding).
"""

from __future__ import annotations

import numpy as np

# Largest finite bfloat16: (2 - 2**-7) * 2**127.
BF16_MAX = float.fromhex("0x1.fe00000000000p+127")

_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_QUANTUM = 2.0 ** -133


def bf16_rne(v) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16, ties to even; return fp64.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and the fp32
    exponent range.  Writing |v| = m * 2**e with 0.5 <= m < 1, the value on the
    bf16 grid is rint(m * 2**8) * 2**(e-8), with numpy's rint rounding halves
    to even.  Below the smallest normal (2**-126) the grid is uniform with
    spacing 2**-133.  Results whose magnitude exceeds BF16_MAX overflow to inf.

    Pinned by tests/test_oracle.py: hand tie cases, agreement with torch's
    fp32 -> bf16 conversion on fp32-exact values, and the double-rounding case
    that distinguishes direct fp64 rounding from fp64 -> fp32 -> bf16.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    normal = np.abs(v) >= _BF16_MIN_NORMAL
    m, e = np.frexp(v[normal])
    out[normal] = np.ldexp(np.rint(m * 256.0), e - 8)
    sub = ~normal
    out[sub] = np.rint(v[sub] / _BF16_SUBNORMAL_QUANTUM) * _BF16_SUBNORMAL_QUANTUM
    over = np.abs(out) > BF16_MAX
    out[over] = np.copysign(np.inf, v[over])
    return out


def bf16_bits(v) -> np.ndarray:
    """Bit patterns (uint16) of values that are already exactly bfloat16.

    A bf16 value is an fp32 value whose low 16 mantissa bits are zero, so the
    pattern is the top half of the fp32 encoding.  Raises if any value is not
    exactly representable (that would be a misuse, not a rounding).
    """
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), v, equal_nan=True):
        raise ValueError("bf16_bits: values are not exactly representable")
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("bf16_bits: values are not exactly bfloat16")
    return (u >> 16).astype(np.uint16)


def rope3d_angles(pos, split=(8, 12, 12), theta: float = 1e4) -> np.ndarray:
    """Rotation angles of 3D-RoPE, one per rotated pair.

    pos: integer array [..., 3] holding (t, h, w).  Returns fp64 [..., d_r/2]
    where d_r = sum(split).  Pair i of axis a (width d_a) turns by
    p_a * theta**(-2i/d_a); pairs are listed axis by axis (t, then h, then w).

    The 3D rotary key is the one the VideoMLA pages name ("decoupled 3D-RoPE
    positional key", arXiv abstract; atlas.scime.ai summary, "Approach"); the
    frequency schedule and axis split are readings (module docstring).
    Pinned by closed-form angles at unit positions in tests/test_oracle.py.
    """
    pos = np.asarray(pos)
    if pos.shape[-1] != 3:
        raise ValueError("pos must end in (t, h, w)")
    parts = []
    for axis, width in enumerate(split):
        if width % 2:
            raise ValueError("every RoPE axis width must be even")
        i = np.arange(width // 2, dtype=np.float64)
        inv_freq = float(theta) ** (-2.0 * i / width)
        parts.append(pos[..., axis: axis + 1].astype(np.float64) * inv_freq)
    return np.concatenate(parts, axis=-1)


def rope3d(v, pos, split=(8, 12, 12), theta: float = 1e4) -> np.ndarray:
    """Apply the 3D rotary embedding to the last axis of v (width d_r).

    Each adjacent pair (x0, x1) = (v[2k], v[2k+1]) becomes
    (x0 cos a - x1 sin a, x0 sin a + x1 cos a) with a = rope3d_angles(pos)[k].
    pos broadcasts against v's leading axes.

    Pinned by: identity at p = 0, norm preservation, agreement with complex
    multiplication by e^{ia}, and the relative-position property (scores
    depend only on position differences), in tests/test_oracle.py.
    """
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] != sum(split):
        raise ValueError("last axis of v must equal sum(split)")
    a = rope3d_angles(pos, split, theta)
    c, s = np.cos(a), np.sin(a)
    x0, x1 = v[..., 0::2], v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape, a.shape[:-1] + (v.shape[-1],)))
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def latent_rows(x, w_dkv, w_kr, pos, split=(8, 12, 12), theta: float = 1e4) -> np.ndarray:
    """Unrounded cache rows [c || k_R] for new tokens, in fp64.

    x [B, n, D]; w_dkv [d_c, D]; w_kr [d_r, D]; pos [n, 3] (shared by the
    batch).  c = w_dkv @ x (content latent), k_R = RoPE(p)(w_kr @ x)
    (head-shared positional key, rotated once, at append time, so the cache
    stores it already rotated).  Returns [B, n, d_c + d_r].

    VideoMLA pages: the latent and the positional key are what each cached
    token keeps (arXiv abstract; atlas.scime.ai summary, "Approach" and
    "Key results", 224 scalars per token).  Pinned by the exact-tier append
    test (integer-valued closed form) and the 224-vs-3072 footprint fixture.
    """
    x = np.asarray(x, dtype=np.float64)
    c = x @ np.asarray(w_dkv, dtype=np.float64).T
    k = x @ np.asarray(w_kr, dtype=np.float64).T
    k = rope3d(k, np.asarray(pos)[None, :, :], split, theta)
    return np.concatenate([c, k], axis=-1)


def cache_append(cache, x, w_dkv, w_kr, pos, offset: int,
                 split=(8, 12, 12), theta: float = 1e4) -> np.ndarray:
    """Return a copy of cache [B, cap, d_c + d_r] with the new rows written.

    Rows for tokens n = 0..n_new-1 go to slots offset + n, each rounded once
    from fp64 to bfloat16 (bf16_rne).  Slots outside [offset, offset+n_new)
    are untouched.
    """
    rows = bf16_rne(latent_rows(x, w_dkv, w_kr, pos, split, theta))
    out = np.array(cache, dtype=np.float64, copy=True)
    n = rows.shape[1]
    if offset < 0 or offset + n > out.shape[1]:
        raise ValueError("append would write outside the cache")
    out[:, offset: offset + n, :] = rows
    return out


def attention_probs(scores, visible=None) -> np.ndarray:
    """Row-wise softmax of fp64 scores [..., Nk] with optional visibility mask.

    Textbook form: subtract the row maximum over visible keys, exponentiate,
    divide by the row sum.  Masked keys get probability exactly 0.
    Pinned by: rows sum to 1, non-negativity, the two-key closed form
    (logit gap ln 3 gives 3/4 and 1/4), in tests/test_oracle.py.
    """
    s = np.array(scores, dtype=np.float64, copy=True)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def _chunk_visibility(q_chunk, k_chunk, n_q, n_k):
    if q_chunk is None and k_chunk is None:
        return None
    qc = np.zeros(n_q, np.int64) if q_chunk is None else np.asarray(q_chunk, np.int64)
    kc = np.zeros(n_k, np.int64) if k_chunk is None else np.asarray(k_chunk, np.int64)
    return kc[None, :] <= qc[:, None]


def _head_qkv(q, q_r_rot, w_uk, w_uv, c, kr, b, h):
    """Non-absorbed per-head Q, K, V for one (batch, head)."""
    k_h = np.concatenate([c[b] @ w_uk[h].T, kr[b]], axis=-1)      # [Nk, d_h + d_r]
    v_h = c[b] @ w_uv[h].T                                          # [Nk, d_h]
    q_h = np.concatenate([q[b, :, h, :], q_r_rot[b, :, h, :]], -1)  # [Nq, d_h + d_r]
    return q_h, k_h, v_h


def _prep(q, q_r, q_pos, w_uk, w_uv, cache, n_k, split, theta):
    q = np.asarray(q, dtype=np.float64)
    q_r = np.asarray(q_r, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    cache = np.asarray(cache, dtype=np.float64)
    d_c = w_uk.shape[-1]
    c = cache[:, :n_k, :d_c]
    kr = cache[:, :n_k, d_c:]
    q_r_rot = rope3d(q_r, np.asarray(q_pos)[None, :, None, :], split, theta)
    return q, q_r_rot, w_uk, w_uv, c, kr


def chunk_attend(q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float,
                 split=(8, 12, 12), theta: float = 1e4,
                 q_chunk=None, k_chunk=None, block_rows: int = 512) -> np.ndarray:
    """Chunk-causal MLA attention in the plain, non-absorbed form.

    q [B, Nq, H, d_h], q_r [B, Nq, H, d_r], q_pos [Nq, 3], w_uk/w_uv
    [H, d_h, d_c], cache [B, cap, d_c + d_r] whose first n_k rows are the
    visible keys (all cached chunks plus the current one).  Per (b, h):
        K_h = [C w_uk[h]^T || K_R],  V_h = C w_uv[h]^T,
        Q_h = [q_h || RoPE(p) q_r,h],
        O_h = softmax(scale * Q_h K_h^T, chunk-causal mask) V_h.
    q_chunk [Nq] / k_chunk [n_k] give chunk indices for the block-causal
    multi-chunk form; both None means every key is visible (one chunk of
    queries that sees every cached chunk and itself).  Returns O [B, Nq, H, d_h].

    Pinned by: brute-force scalar loops on tiny shapes, the algebraic identity
    with the absorbed form, q = 0 giving the plain mean of V, the two-key
    closed form, key-permutation invariance, torch's CPU fp64
    scaled_dot_product_attention on the reconstructed K/V, and multi-chunk
    block-causal == sequential single-chunk steps (tests/test_oracle.py).
    """
    q, q_r_rot, w_uk, w_uv, c, kr = _prep(q, q_r, q_pos, w_uk, w_uv, cache, n_k, split, theta)
    B, n_q, H, d_h = q.shape
    vis = _chunk_visibility(q_chunk, k_chunk, n_q, n_k)
    out = np.empty((B, n_q, H, d_h))
    for b in range(B):
        for h in range(H):
            q_h, k_h, v_h = _head_qkv(q, q_r_rot, w_uk, w_uv, c, kr, b, h)
            for i0 in range(0, n_q, block_rows):
                i1 = min(n_q, i0 + block_rows)
                s = scale * (q_h[i0:i1] @ k_h.T)
                p = attention_probs(s, None if vis is None else vis[i0:i1])
                out[b, i0:i1, h, :] = p @ v_h
    return out


def chunk_attend_rows(rows, q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float,
                      split=(8, 12, 12), theta: float = 1e4,
                      q_chunk=None, k_chunk=None) -> np.ndarray:
    """chunk_attend for a chosen set of output rows only.

    rows: integer array [R, 3] of (b, i, h).  Returns [R, d_h] equal to
    chunk_attend(..., q_chunk, k_chunk)[b, i, h, :] for each row; used at
    full workload sizes where the whole output is too expensive for fp64 on
    the host.
    """
    rows = np.asarray(rows, dtype=np.int64)
    q, q_r_rot, w_uk, w_uv, c, kr = _prep(q, q_r, q_pos, w_uk, w_uv, cache, n_k, split, theta)
    vis = _chunk_visibility(q_chunk, k_chunk, q.shape[1], n_k)
    out = np.empty((rows.shape[0], q.shape[-1]))
    for (b, h) in sorted({(int(r[0]), int(r[2])) for r in rows}):
        sel = np.nonzero((rows[:, 0] == b) & (rows[:, 2] == h))[0]
        q_h, k_h, v_h = _head_qkv(q, q_r_rot, w_uk, w_uv, c, kr, b, h)
        s = scale * (q_h[rows[sel, 1]] @ k_h.T)
        out[sel] = attention_probs(s, None if vis is None else vis[rows[sel, 1]]) @ v_h
    return out


def mha_attend(q, k, v, n_k: int, scale: float, q_chunk=None, k_chunk=None,
               block_rows: int = 512) -> np.ndarray:
    """Standard multi-head attention over per-head keys and values.

    The dense per-head K/V cache that the latent cache replaces (VideoMLA
    atlas.scime.ai summary, "Key results": 2 x H x d_h cached values per
    token).  q [B, Nq, H, d], k and v [B, cap, H, d] (positional encoding, if
    any, already applied); the first n_k key slots are visible, optionally
    restricted by chunk indices as in chunk_attend.  Per (b, h):
        O = softmax(scale * Q K^T, mask) V.
    Returns O [B, Nq, H, d_v].

    Pinned by: brute-force scalar loops, torch's CPU fp64
    scaled_dot_product_attention, q = 0 giving the plain mean of V, and the
    identity with chunk_attend when K, V are the per-head keys and values
    reconstructed from a latent cache (tests/test_oracle.py).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)[:, :n_k]
    v = np.asarray(v, dtype=np.float64)[:, :n_k]
    B, n_q, H, _ = q.shape
    vis = _chunk_visibility(q_chunk, k_chunk, n_q, n_k)
    out = np.empty((B, n_q, H, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, n_q, block_rows):
                i1 = min(n_q, i0 + block_rows)
                s = scale * (q[b, i0:i1, h] @ k[b, :, h].T)
                p = attention_probs(s, None if vis is None else vis[i0:i1])
                out[b, i0:i1, h, :] = p @ v[b, :, h]
    return out


def mha_attend_rows(rows, q, k, v, n_k: int, scale: float) -> np.ndarray:
    """mha_attend for chosen output rows (b, i, h) only: [R, d_v], each equal
    to mha_attend(q, k, v, n_k, scale)[b, i, h]."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], np.shape(v)[-1]))
    for r, (b, i, h) in enumerate(rows):
        qv = np.asarray(q[b, i, h], dtype=np.float64)
        kk = np.asarray(k[b, :n_k, h], dtype=np.float64)
        vv = np.asarray(v[b, :n_k, h], dtype=np.float64)
        out[r] = attention_probs(scale * (kk @ qv)) @ vv
    return out
