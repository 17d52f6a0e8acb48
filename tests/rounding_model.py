"""Rounding model of the bf16 attention paths (TEST INFRASTRUCTURE ONLY).

It derives the parity tolerance of the fp32-output checks (the RMS-normalised
G2 gates): the error that the roundings of a bf16 MFMA evaluation leave
against the exact fp64 attention, on the same seeded inputs as the GPU tests.
It is neither the oracle nor a stand-in for the kernels: it evaluates each
form in fp64 and applies only the roundings the bf16 path makes, where it
makes them.

Absorbed form (the chunk step):
  * q~ = qscale * [W_UK[h]^T q || RoPE3D(p) q_r] rounded once to bf16, with
    qscale = softmax scale * log2 e (the softmax runs in base 2);
  * scores s = q~ . [c || k_R] and every running sum are exact: the fp32
    accumulations add errors far below the bf16 roundings;
  * p = 2^(s - m) is rounded to bf16 for the P.V product; the normaliser l
    sums the unrounded p ("unrounded") or the rounded ones ("rounded");
  * L = sum_j bf16(p_j) c_j / l, merged over the key segments, each with its
    own m;
  * the up-projection sees L as a bf16 hi + lo pair (about 16 significant
    bits).
Non-absorbed form: K_h = [W_UK[h] c || k_R] and V_h = W_UV[h] c are rounded
once to bf16, the rotated query part once; the scale multiplies the scores;
then the same softmax and P.V.  Dense per-head attention: q, k, v are used as
given.

Two choices of the reference m of a key segment:
  "exact"        the true maximum of the segment's visible scores (any
                 exact-max flash schedule);
  "first_block"  the maximum of the segment's first 32-key block, which the
                 fused kernels fix before they stream the rest of the segment
                 (later scores may exceed it; p > 1 is then rounded too).
The key segments are those of the kernels' stream-K work partition, restated
here from its documented rule: units are (row block, key tile) pairs split
evenly over the workgroups, and chunk-causal calls count only the tiles some
row of a block can see.
"""

from __future__ import annotations

import math

import numpy as np

import oracle

ROWS_PER_BLOCK = 256
PARTITION_CUS = 256
MAX_SPLITS = 16
SEGMENT_UNITS = 16     # start-up units per row block of a chunk-causal partition
FIRST_BLOCK = 32
LOG2E = math.log2(math.e)


def latent_tile(d_c: int) -> int:
    """Keys per tile of the latent kernels (64 up to d_c = 192, 128 at 256)."""
    return 64 if d_c <= 192 else 128


def kv_of_rows(n_q: int, H: int, n_k: int, causal) -> np.ndarray:
    """Visible key count of every row r = h * n_q + i of one sample."""
    i = np.tile(np.arange(n_q), H)
    if causal is None:
        return np.full(H * n_q, n_k, np.int64)
    q_start, c = causal
    return np.minimum(n_k, ((q_start + i) // c + 1) * c).astype(np.int64)


def partition_size(tiles_per_rb, spread: bool) -> tuple[int, int]:
    """(U units, G workgroups) of the partition split_units describes."""
    per = np.asarray(tiles_per_rb, np.int64)
    nrb = per.size
    if spread:
        G = PARTITION_CUS
    else:
        rounds = -(-nrb // PARTITION_CUS)
        G = rounds * PARTITION_CUS if nrb / (rounds * PARTITION_CUS) < 0.9 else nrb
    U = int((per + (SEGMENT_UNITS if spread else 0)).sum())
    return U, max(1, min(G, U, nrb * MAX_SPLITS))


def split_units(tiles_per_rb, spread: bool) -> list[list[tuple[int, int]]]:
    """Tile ranges [t0, t1) of every row block's segments.

    tiles_per_rb: key tiles of each row block.  spread: a chunk-causal call
    whose row blocks see different numbers of key tiles.  Its partition always
    spreads over the compute units, and each row block counts SEGMENT_UNITS
    start-up units ahead of its tiles (the cost of loading its queries and
    writing a partial state); a workgroup whose part of a row block is
    start-up units only leaves no segment for it.  Otherwise
    a row block has only its tiles, and the partition spreads only when one
    workgroup per row block would leave more than 10% of the compute units
    idle in the last round."""
    per = np.asarray(tiles_per_rb, np.int64)
    nrb = per.size
    skip = SEGMENT_UNITS if spread else 0
    units = per + skip
    U, G = partition_size(per, spread)
    first = np.concatenate([[0], np.cumsum(units)])
    bounds = [(w * U) // G for w in range(G + 1)]
    out = []
    for rb in range(nrb):
        u0, u1 = int(first[rb]), int(first[rb + 1])
        w0 = max(0, int(np.searchsorted(bounds, u0, side="right")) - 1)
        segs = []
        for w in range(w0, G):
            if bounds[w] >= u1:
                break
            a = max(u0, bounds[w]) - u0 - skip
            b = min(u1, bounds[w + 1]) - u0 - skip
            if b > max(a, 0):
                segs.append((max(a, 0), b))
        out.append(segs)
    return out


def softmax_values(s2, values, segs, bn: int, m_mode: str, l_mode: str) -> np.ndarray:
    """sum_j bf16(p_j) v_j / l for rows of base-2 scores s2 [R, n_k] (-inf =
    not visible) over the given key-tile segments, merged exactly."""
    n_k = s2.shape[1]
    parts = []
    for (t0, t1) in segs:
        k0, k1 = t0 * bn, min(n_k, t1 * bn)
        s = s2[:, k0:k1]
        m = s.max(axis=1) if m_mode == "exact" else s[:, :FIRST_BLOCK].max(axis=1)
        m_use = np.where(np.isfinite(m), m, 0.0)
        with np.errstate(over="raise"):
            p = np.exp2(s - m_use[:, None])
        pb = oracle.bf16_rne(p)
        parts.append((m, (pb if l_mode == "rounded" else p).sum(axis=1), pb @ values[k0:k1]))
    M = np.max([m for m, _, _ in parts], axis=0)
    num = np.zeros((s2.shape[0], values.shape[1]))
    den = np.zeros(s2.shape[0])
    for m, l_seg, acc in parts:
        ok = np.isfinite(m)
        wgt = np.where(ok, np.exp2(np.where(ok, m - M, 0.0)), 0.0)
        num += wgt[:, None] * acc
        den += wgt * l_seg
    return num / den[:, None]


def _rows_of_sample(x):
    """[n_q, H, d] -> rows r = h * n_q + i."""
    return np.asarray(x).transpose(1, 0, 2).reshape(-1, x.shape[-1])


def attend(q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float, split=(8, 12, 12), theta=1e4,
           causal=None, m_mode: str = "first_block", l_mode: str = "unrounded",
           round_q: bool = True, round_p: bool = True, round_l: bool = True) -> np.ndarray:
    """Modelled bf16 evaluation of the absorbed chunk step: [B, n_q, H, d_h].

    round_q / round_p / round_l switch the three roundings off one by one; with
    all three off the function is exact attention (pinned against the oracle)."""
    q, q_r, w_uk, w_uv, cache = (np.asarray(a, np.float64) for a in (q, q_r, w_uk, w_uv, cache))
    B, n_q, H, d_h = q.shape
    d_c = w_uk.shape[-1]
    bn = latent_tile(d_c)
    rnd = oracle.bf16_rne
    qscale = scale * LOG2E
    rot = oracle.rope3d(q_r, np.asarray(q_pos)[None, :, None, :], split, theta)
    qt = qscale * np.concatenate([np.einsum("bihd,hdc->bihc", q, w_uk), rot], axis=-1)
    if round_q:
        qt = rnd(qt)
    kv = kv_of_rows(n_q, H, n_k, causal)
    rows_b = H * n_q
    rb_per_b = -(-rows_b // ROWS_PER_BLOCK)
    per = [-(-int(kv[r * ROWS_PER_BLOCK: (r + 1) * ROWS_PER_BLOCK].max()) // bn) for r in range(rb_per_b)]
    # a chunk-causal call takes the uneven partition only when its row blocks
    # see different numbers of key tiles
    segs = split_units(per * B, spread=causal is not None and any(t != -(-n_k // bn) for t in per))
    keys = np.arange(n_k)
    out = np.empty((B, n_q, H, d_h))
    for b in range(B):
        s2 = _rows_of_sample(qt[b]) @ cache[b, :n_k].T
        s2 = np.where(keys[None, :] < kv[:, None], s2, -np.inf)
        c = cache[b, :n_k, :d_c]
        L = np.empty((rows_b, d_c))
        for rbl in range(rb_per_b):
            r0, r1 = rbl * ROWS_PER_BLOCK, min(rows_b, (rbl + 1) * ROWS_PER_BLOCK)
            sg = segs[b * rb_per_b + rbl]
            if round_p:
                L[r0:r1] = softmax_values(s2[r0:r1], c, sg, bn, m_mode, l_mode)
            else:
                p = np.exp2(s2[r0:r1] - s2[r0:r1].max(axis=1, keepdims=True))
                L[r0:r1] = (p @ c) / p.sum(axis=1, keepdims=True)
        if round_l:
            hi = rnd(L)
            L = hi + rnd(L - hi)
        out[b] = np.einsum("hic,hdc->ihd", L.reshape(H, n_q, d_c), w_uv)
    return out


def _per_head(q_rows_fn, k_fn, v_fn, B, H, n_q, n_k, qscale, m_mode, l_mode):
    """Shared body of the per-head forms: rows of one (batch, head) are padded
    to whole row blocks, so the partition has B*H*ceil(n_q/256) row blocks of
    64-key tiles."""
    bn = 64
    rb = -(-n_q // ROWS_PER_BLOCK)
    segs = split_units([-(-n_k // bn)] * (B * H * rb), spread=False)
    out = np.empty((B, n_q, H, v_fn(0, 0).shape[-1]))
    for b in range(B):
        for h in range(H):
            s2 = qscale * (q_rows_fn(b, h) @ k_fn(b, h).T)
            v = v_fn(b, h)
            for j in range(rb):
                i0, i1 = j * ROWS_PER_BLOCK, min(n_q, (j + 1) * ROWS_PER_BLOCK)
                out[b, i0:i1, h] = softmax_values(s2[i0:i1], v, segs[(b * H + h) * rb + j], bn, m_mode, l_mode)
    return out


def attend_expanded(q, q_r, q_pos, w_uk, w_uv, cache, n_k: int, scale: float, split=(8, 12, 12), theta=1e4,
                    m_mode: str = "first_block", l_mode: str = "unrounded") -> np.ndarray:
    """Modelled bf16 evaluation of the non-absorbed form: [B, n_q, H, d_h]."""
    q, q_r, w_uk, w_uv, cache = (np.asarray(a, np.float64) for a in (q, q_r, w_uk, w_uv, cache))
    B, n_q, H, d_h = q.shape
    d_c = w_uk.shape[-1]
    rnd = oracle.bf16_rne
    rot = rnd(oracle.rope3d(q_r, np.asarray(q_pos)[None, :, None, :], split, theta))
    c, kr = cache[:, :n_k, :d_c], cache[:, :n_k, d_c:]
    return _per_head(lambda b, h: np.concatenate([q[b, :, h], rot[b, :, h]], -1),
                     lambda b, h: rnd(np.concatenate([c[b] @ w_uk[h].T, kr[b]], -1)),
                     lambda b, h: rnd(c[b] @ w_uv[h].T),
                     B, H, n_q, n_k, scale * LOG2E, m_mode, l_mode)


def mha(q, k, v, n_k: int, scale: float, m_mode: str = "first_block", l_mode: str = "unrounded") -> np.ndarray:
    """Modelled bf16 evaluation of dense per-head attention: [B, n_q, H, d_v]."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, n_q, H, _ = q.shape
    return _per_head(lambda b, h: q[b, :, h], lambda b, h: k[b, :n_k, h], lambda b, h: v[b, :n_k, h],
                     B, H, n_q, n_k, scale * LOG2E, m_mode, l_mode)


def normalised_errors(got, want) -> tuple[float, float]:
    """(max, mean) of |got - want| / RMS(want): the G2 metric."""
    d = np.abs(np.asarray(got) - np.asarray(want))
    rms = float(np.sqrt(np.mean(np.square(want))))
    return float(d.max() / rms), float(d.mean() / rms)
