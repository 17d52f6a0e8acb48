"""Seeded synthetic workloads for the latent KV cache path.

This module only draws inputs: shapes, positions and random values.  It holds
none of the method's arithmetic, so both the HIP path and the fp64 oracle can
be fed from it without sharing any computation.

Shapes follow the Wan2.1-T2V-1.3B backbone the VideoMLA pages study
(atlas.scime.ai summary, first paragraph; 12 heads x 128 = 1536 model width),
with the latent rank d_c = 192 and a 32-wide rotary key (atlas.scime.ai
summary, "Key results": 224 cached scalars per token).  No public dataset is
involved: every value is drawn from a Gaussian with a fixed seed.

Value recipe (all fp32 draws from numpy PCG64, then rounded to nearest-even
bf16 when the bf16 dtype is requested):
  attention inputs  c_KV ~ N(0, 1), k_R ~ N(0, 1), q ~ N(0, 1), q_r ~ N(0, 1),
                    W_UK, W_UV ~ N(0, 1/d_c)
  append inputs     x ~ N(0, 1), W_DKV, W_KR ~ N(0, 1/D)
  dense K/V inputs  q, k, v ~ N(0, 1) per head (sample b: PCG64(3000 + b + 7919*seed))
  seeds             weights: PCG64(7 + 7919*seed); batch sample b:
                    PCG64(1000 + b + 7919*seed) (its own cache, q, q_r, x).
Positions: latent token n of a chunk is frame-major then row-major,
n = f*(Hg*Wg) + y*Wg + x, with position triple (t, y, x) where t is the
absolute latent-frame index.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    grid_hw: Tuple[int, int]          # latent tokens per frame = Hg * Wg
    cache_frames: Tuple[int, ...]     # t of every cached latent frame, in slot order
    query_frames: Tuple[int, ...]     # t of the current chunk's latent frames
    n_heads: int = 12
    head_dim: int = 128
    d_c: int = 192
    d_r: int = 32
    rope_split: Tuple[int, int, int] = (8, 12, 12)
    theta: float = 1e4
    d_model: int = 1536
    chunk_tokens: int = 0             # > 0: queries span chunks of this many tokens (block-causal)
    query_tokens: int = 0             # > 0: only the chunk's first query_tokens tokens are queries (one GPU's
                                      # share of a query-sharded step); the keys still hold the whole chunk
    notes: str = field(default="", compare=False)

    @property
    def frame_tokens(self) -> int:
        return self.grid_hw[0] * self.grid_hw[1]

    @property
    def chunk_len_tokens(self) -> int:
        """Tokens of the current chunk's frames (all appended before attention)."""
        return len(self.query_frames) * self.frame_tokens

    @property
    def n_q(self) -> int:
        return self.query_tokens or self.chunk_len_tokens

    @property
    def n_cached(self) -> int:
        return len(self.cache_frames) * self.frame_tokens

    @property
    def n_k(self) -> int:
        return self.n_cached + self.chunk_len_tokens

    def query_positions(self) -> np.ndarray:
        """(t, y, x) of the query tokens, in token order."""
        return chunk_positions(self.query_frames, self.grid_hw)[:self.n_q]

    @property
    def scale(self) -> float:
        # 1/sqrt(d_h + d_r): unit-variance logits under the recipe above.
        return 1.0 / float(np.sqrt(self.head_dim + self.d_r))

    def with_dc(self, d_c: int) -> "Workload":
        return replace(self, d_c=d_c, name=f"{self.name}_dc{d_c}")

    def with_batch(self, batch: int) -> "Workload":
        return replace(self, batch=batch, name=f"{self.name}_b{batch}")

    @property
    def causal(self):
        """(q_start, chunk_len) of a block-causal call, or None (every key visible)."""
        return (self.n_cached, self.chunk_tokens) if self.chunk_tokens else None

    def visible_keys(self) -> int:
        """Sum over the queries of the keys each one sees."""
        if not self.chunk_tokens:
            return self.n_q * self.n_k
        i = np.arange(self.n_q, dtype=np.int64) + self.n_cached
        return int(np.minimum(self.n_k, (i // self.chunk_tokens + 1) * self.chunk_tokens).sum())

    # Algorithmic work of one chunk step (absorbed form, as computed; visible
    # (query, key) pairs only).
    def attend_flops(self) -> float:
        pairs = self.batch * self.n_heads * self.visible_keys()
        rows = self.batch * self.n_q * self.n_heads
        return float(pairs) * (4 * self.d_c + 2 * self.d_r) + float(rows) * 4 * self.head_dim * self.d_c

    def attend_core_flops(self) -> float:
        """Flops of the fused score/softmax/P.V kernel alone."""
        return float(self.batch * self.n_heads * self.visible_keys()) * (4 * self.d_c + 2 * self.d_r)

    def mha_equiv_flops(self) -> float:
        """Flops of standard attention over materialised per-head keys [k_h || k_R] and values."""
        return float(self.batch * self.n_heads * self.visible_keys()) * (4 * self.head_dim + 2 * self.d_r)

    def dense_flops(self) -> float:
        """Flops of standard attention over a dense per-head K/V cache (d_h-wide keys and values)."""
        return float(self.batch * self.n_heads * self.visible_keys()) * 4 * self.head_dim

    def expand_flops(self) -> float:
        """Flops of materialising K_h = W_UK[h] c and V_h = W_UV[h] c for every key."""
        return 4.0 * self.batch * self.n_k * self.n_heads * self.head_dim * self.d_c

    def min_hbm_bytes(self) -> dict:
        """Bytes one step must move at least (every tensor read or written once):
        append reads x and the two weights and writes the new rows; attention reads
        the latent cache, q, q_r, W_UK and W_UV and writes the output (bf16)."""
        w = self.d_c + self.d_r
        append = 2 * (self.batch * self.n_q * self.d_model + self.d_model * w + self.batch * self.n_q * w)
        attend = 2 * (self.batch * self.n_k * w + self.batch * self.n_q * self.n_heads * (2 * self.head_dim + self.d_r)
                      + 2 * self.n_heads * self.head_dim * self.d_c)
        return {"append": append, "attend": attend}

    def append_flops(self) -> float:
        return 2.0 * self.batch * self.n_q * self.d_model * (self.d_c + self.d_r)


def _frames(a, b):
    return tuple(range(a, b))


TINY = Workload("tiny", 1, (4, 6), _frames(0, 6), _frames(6, 8),
                notes="frame 4x6, chunk 2 frames (48 queries), 3 cached chunks")
WAN480P = Workload("wan480p", 1, (30, 52), _frames(0, 18), _frames(18, 21),
                   notes="frame 30x52, chunk 3 frames (4680 queries), 6 cached chunks")
WAN480P_B8 = replace(WAN480P, batch=8, name="wan480p_b8")
WAN480P_SHARD8 = replace(WAN480P, name="wan480p_shard8", query_tokens=4680 // 8,
                         notes="one GPU's share of an 8-way query-sharded 480P step: 585 of the chunk's "
                               "4680 queries against all 32760 keys")
WAN720P_LONG = Workload("wan720p_long", 1, (45, 80),
                        _frames(0, 3) + _frames(219, 237), _frames(237, 240),
                        notes="frame 45x80, chunk 3 frames (10800 queries), "
                              "1 sink chunk + 6 recent chunks")
DC_SWEEP = tuple(WAN480P.with_dc(d) for d in (64, 128, 192, 256))
# Teacher-forcing form: all 21 latent frames of a 480P clip as queries, in 7
# chunks of 3 frames, each chunk seeing itself and the earlier chunks.
WAN480P_TF = Workload("wan480p_tf", 1, (30, 52), (), _frames(0, 21), chunk_tokens=3 * 30 * 52,
                      notes="7 chunks of 4680 queries, block-causal")

WORKLOADS = {w.name: w for w in (TINY, WAN480P, WAN480P_B8, WAN480P_SHARD8, WAN720P_LONG, WAN480P_TF) + DC_SWEEP}


def chunk_positions(frames, grid_hw) -> np.ndarray:
    """(t, y, x) int32 triples for the tokens of the given frames, in token order."""
    hg, wg = grid_hw
    t = np.repeat(np.asarray(frames, np.int32), hg * wg)
    y = np.tile(np.repeat(np.arange(hg, dtype=np.int32), wg), len(frames))
    x = np.tile(np.arange(wg, dtype=np.int32), hg * len(frames))
    return np.stack([t, y, x], axis=-1).astype(np.int32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    # fp32 draw -> requested dtype (bf16: torch rounds to nearest even).
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def attend_inputs(wl: Workload, seed: int = 0, dtype: torch.dtype = torch.bfloat16,
                  capacity: int | None = None) -> dict:
    """Cache, queries and up-projection weights for one chunk step.

    The cache holds n_k rows [c || k_R] per sample (prior chunks plus the
    current chunk), drawn directly; capacity >= n_k adds zero slots after them.
    """
    cap = wl.n_k if capacity is None else capacity
    assert cap >= wl.n_k
    w = _rng(7 + 7919 * seed)
    w_uk = _normal(w, (wl.n_heads, wl.head_dim, wl.d_c), 1.0 / np.sqrt(wl.d_c))
    w_uv = _normal(w, (wl.n_heads, wl.head_dim, wl.d_c), 1.0 / np.sqrt(wl.d_c))
    width = wl.d_c + wl.d_r
    cache = np.zeros((wl.batch, cap, width), np.float32)
    q = np.empty((wl.batch, wl.n_q, wl.n_heads, wl.head_dim), np.float32)
    q_r = np.empty((wl.batch, wl.n_q, wl.n_heads, wl.d_r), np.float32)
    for b in range(wl.batch):
        r = _rng(1000 + b + 7919 * seed)
        cache[b, :wl.n_k] = _normal(r, (wl.n_k, width))
        q[b] = _normal(r, q.shape[1:])
        q_r[b] = _normal(r, q_r.shape[1:])
    return dict(
        cache=_to(cache, dtype), q=_to(q, dtype), q_r=_to(q_r, dtype),
        w_uk=_to(w_uk, dtype), w_uv=_to(w_uv, dtype),
        q_pos=torch.from_numpy(wl.query_positions()),
        n_k=wl.n_k, scale=wl.scale,
    )


def mha_inputs(wl: Workload, seed: int = 0, capacity: int | None = None) -> dict:
    """Queries and a dense per-head K/V cache [B, capacity, H, d_h] for the same
    chunk step (the cache layout the latent replaces); bf16, every value N(0, 1),
    scale 1/sqrt(d_h).  Slots past n_k are zero."""
    cap = wl.n_k if capacity is None else capacity
    assert cap >= wl.n_k
    H, d = wl.n_heads, wl.head_dim
    q = np.empty((wl.batch, wl.n_q, H, d), np.float32)
    k = np.zeros((wl.batch, cap, H, d), np.float32)
    v = np.zeros((wl.batch, cap, H, d), np.float32)
    for b in range(wl.batch):
        r = _rng(3000 + b + 7919 * seed)
        q[b] = _normal(r, q.shape[1:])
        k[b, :wl.n_k] = _normal(r, (wl.n_k, H, d))
        v[b, :wl.n_k] = _normal(r, (wl.n_k, H, d))
    bf = torch.bfloat16
    return dict(q=_to(q, bf), k=_to(k, bf), v=_to(v, bf), n_k=wl.n_k, scale=1.0 / float(np.sqrt(d)))


def append_inputs(wl: Workload, seed: int = 0, dtype: torch.dtype = torch.bfloat16) -> dict:
    """Hidden states and down-projection weights for the current chunk's tokens."""
    w = _rng(7 + 7919 * seed + 1)
    w_dkv = _normal(w, (wl.d_c, wl.d_model), 1.0 / np.sqrt(wl.d_model))
    w_kr = _normal(w, (wl.d_r, wl.d_model), 1.0 / np.sqrt(wl.d_model))
    x = np.empty((wl.batch, wl.n_q, wl.d_model), np.float32)
    for b in range(wl.batch):
        x[b] = _normal(_rng(1000 + b + 7919 * seed + 500000), x.shape[1:])
    return dict(
        x=_to(x, dtype), w_dkv=_to(w_dkv, dtype), w_kr=_to(w_kr, dtype),
        pos=torch.from_numpy(wl.query_positions()),
    )


def append_inputs_exact(wl: Workload, seed: int = 0, dtype: torch.dtype = torch.bfloat16) -> dict:
    """Append inputs on which every partial sum is exact in fp32.

    x in {-1, 0, 1}, weights in {-8, ..., 8} * 2**-6, all positions (0, 0, 0)
    (rotation by angle 0).  Every partial sum is a multiple of 2**-6 of
    magnitude at most D * 8 * 2**-6 (= 192 at D = 1536), far below
    2**24 * 2**-6, so any summation order gives the same fp32 value and the
    bf16 result is fixed by the rounding rule alone.  About one value in ten
    lands above 4, where bf16 spacing (2**-5 and up) forces rounding,
    including exact ties.
    """
    r = _rng(31 + 7919 * seed)
    x = r.integers(-1, 2, size=(wl.batch, wl.n_q, wl.d_model)).astype(np.float32)
    w_dkv = r.integers(-8, 9, size=(wl.d_c, wl.d_model)).astype(np.float32) / 64.0
    w_kr = r.integers(-8, 9, size=(wl.d_r, wl.d_model)).astype(np.float32) / 64.0
    return dict(
        x=_to(x, dtype), w_dkv=_to(w_dkv, dtype), w_kr=_to(w_kr, dtype),
        pos=torch.zeros((wl.n_q, 3), dtype=torch.int32),
    )
