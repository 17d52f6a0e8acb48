"""GPU parity of standard attention over per-head keys and values against the
fp64 oracle.

Two entry points share one attention kernel (attend_mha.hip):
  * mla_mha_attend: the dense per-head K/V cache that the latent cache
    replaces (VideoMLA atlas.scime.ai summary, "Key results"), checked
    against oracle.mha_attend;
  * mla_chunk_attend_expanded: multi-head latent attention in its
    non-absorbed form (DeepSeek-V2, "Builds on" on the VideoMLA pages), with
    per-head K_h, V_h materialised from the latent cache, checked against
    oracle.chunk_attend, the same definition the absorbed path is held to.
Gates as in test_gpu_attend.py.  The non-absorbed form rounds K_h and V_h to
bf16 where the absorbed form rounds q~; both are single roundings of
unit-scale values feeding fp32 accumulations, so the same G2 bound applies.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import assert_g1, assert_g2, assert_g2x, need_gpu, np64

pytestmark = pytest.mark.gpu


def _dense(mla, inp, n_q=None, out_dtype=None):
    q = inp["q"] if n_q is None else inp["q"][:, :n_q].contiguous()
    out = mla.mha_attend(q.cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["n_k"], inp["scale"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return np64(out)


def _dense_oracle(inp, n_q=None):
    q = np64(inp["q"]) if n_q is None else np64(inp["q"])[:, :n_q]
    return oracle.mha_attend(q, np64(inp["k"]), np64(inp["v"]), inp["n_k"], inp["scale"])


# 2 samples, 3 heads, 70 queries (one ragged 256-row block per head), 105
# keys (three 32-key tiles and a 9-key tail) in a 120-slot cache.
DENSE_SMALL = replace(synth.TINY, name="dense_small", batch=2, n_heads=3, grid_hw=(5, 7),
                      cache_frames=(0,), query_frames=(1, 2))


def test_dense_small_bf16_and_f32_out():
    mla = need_gpu()
    inp = synth.mha_inputs(DENSE_SMALL, seed=0, capacity=120)
    assert (DENSE_SMALL.n_q, inp["n_k"]) == (70, 105)
    want = _dense_oracle(inp)
    assert_g1(_dense(mla, inp), want, "bf16 out")
    assert_g2(_dense(mla, inp, out_dtype=torch.float32), want, "f32 out")


@pytest.mark.parametrize("n_q,n_k", [(1, 1), (1, 33), (31, 32), (257, 300), (600, 1000)])
def test_dense_shapes(n_q, n_k):
    """Single key; one key past a tile; exactly one tile; row blocks past 256
    rows; several row blocks per head over a stream-K partition."""
    mla = need_gpu()
    wl = replace(synth.TINY, name="dense_shape", n_heads=4, grid_hw=(1, n_k), cache_frames=(),
                 query_frames=(0,))
    inp = synth.mha_inputs(wl, seed=1)
    got = _dense(mla, inp, n_q=n_q, out_dtype=torch.float32)
    assert_g2(got, _dense_oracle(inp, n_q=n_q), f"n_q={n_q} n_k={n_k}")


@pytest.mark.parametrize("headroom", ["0"])
def test_dense_two_pass_fallback(monkeypatch, headroom):
    mla = need_gpu()
    monkeypatch.setenv("MLA_ATTEND_HEADROOM", headroom)
    inp = synth.mha_inputs(DENSE_SMALL, seed=2)
    assert_g2(_dense(mla, inp, out_dtype=torch.float32), _dense_oracle(inp), "two-pass")


def test_dense_peaked_scores():
    """Scores up to ~40 in log2 units: the first-block reference max is far
    below later maxima, which the single pass must survive or redo."""
    mla = need_gpu()
    inp = synth.mha_inputs(DENSE_SMALL, seed=3)
    inp = dict(inp, scale=3.0)
    assert_g2(_dense(mla, inp, out_dtype=torch.float32), _dense_oracle(inp), "peaked")


def test_dense_480p_sampled_rows():
    """The 480P chunk step with a dense 12 x 128 K/V cache: 4680 queries over 32760 keys."""
    mla = need_gpu()
    wl = synth.WAN480P
    inp = synth.mha_inputs(wl, seed=0)
    got = _dense(mla, inp, out_dtype=torch.float32)
    rng = np.random.default_rng(5)
    i = np.concatenate([rng.integers(0, wl.n_q, 40), [0, 255, 256, wl.n_q - 1]])
    rows = np.stack([np.zeros_like(i), i, rng.integers(0, wl.n_heads, i.size)], 1)
    want = oracle.mha_attend_rows(rows, np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), wl.n_k, inp["scale"])
    assert_g2(got[rows[:, 0], rows[:, 1], rows[:, 2]], want, "480p dense")
    assert np.all(np.isfinite(got))


# ----------------------------------------------------------------- non-absorbed latent form

def _dims(mla, wl):
    return mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)


def _expanded(mla, wl, inp, out_dtype=None):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = mla.chunk_attend_expanded(_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"],
                                    inp["n_k"], inp["scale"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return np64(out)


def _latent_oracle(wl, inp):
    return oracle.chunk_attend(np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(), np64(inp["w_uk"]),
                               np64(inp["w_uv"]), np64(inp["cache"]), inp["n_k"], inp["scale"],
                               split=wl.rope_split, theta=wl.theta)


def test_expanded_tiny_bf16_and_f32_out():
    mla = need_gpu()
    wl = synth.TINY
    inp = synth.attend_inputs(wl, seed=0, capacity=wl.n_k + 9)
    want = _latent_oracle(wl, inp)
    assert_g1(_expanded(mla, wl, inp), want, "bf16 out")
    assert_g2x(_expanded(mla, wl, inp, out_dtype=torch.float32), want, "f32 out")


@pytest.mark.parametrize("d_c", [64, 128, 192, 256])
def test_expanded_dc(d_c):
    mla = need_gpu()
    wl = replace(synth.TINY, batch=2).with_dc(d_c)
    inp = synth.attend_inputs(wl, seed=1)
    assert_g2x(_expanded(mla, wl, inp, out_dtype=torch.float32), _latent_oracle(wl, inp), f"dc{d_c}")


def test_expanded_samples_not_aligned_to_wavefronts():
    """K_h and V_h are head-major: the rows of one wavefront's 32 tokens are
    contiguous only within one sample.  With 35-token frames (n_k = 280) and
    three samples, wavefronts of the expansion straddle sample boundaries."""
    mla = need_gpu()
    wl = replace(synth.TINY, name="ragged_samples", batch=3, grid_hw=(5, 7))
    inp = synth.attend_inputs(wl, seed=4, capacity=wl.n_k + 3)
    assert wl.n_k % 32 != 0
    assert_g2x(_expanded(mla, wl, inp, out_dtype=torch.float32), _latent_oracle(wl, inp), "straddling samples")


def test_expanded_agrees_with_absorbed():
    """Both forms of the same chunk step, side by side, each within the gate of the oracle."""
    mla = need_gpu()
    wl = replace(synth.TINY, name="mid", grid_hw=(12, 16))
    inp = synth.attend_inputs(wl, seed=2)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"], wl.n_k, wl.scale)
    a = np64(mla.chunk_attend(*args, out_dtype=torch.float32))
    e = np64(mla.chunk_attend_expanded(*args, out_dtype=torch.float32))
    rng = np.random.default_rng(3)
    rows = np.stack([np.zeros(60, np.int64), rng.integers(0, wl.n_q, 60), rng.integers(0, wl.n_heads, 60)], 1)
    want = oracle.chunk_attend_rows(rows, np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(), np64(inp["w_uk"]),
                                    np64(inp["w_uv"]), np64(inp["cache"]), wl.n_k, wl.scale)
    assert_g2(a[rows[:, 0], rows[:, 1], rows[:, 2]], want, "absorbed")
    assert_g2x(e[rows[:, 0], rows[:, 1], rows[:, 2]], want, "expanded")


def test_expanded_480p_sampled_rows():
    mla = need_gpu()
    wl = synth.WAN480P
    inp = synth.attend_inputs(wl, seed=0)
    got = _expanded(mla, wl, inp, out_dtype=torch.float32)
    rng = np.random.default_rng(6)
    i = np.concatenate([rng.integers(0, wl.n_q, 30), [0, wl.n_q - 1]])
    rows = np.stack([np.zeros_like(i), i, rng.integers(0, wl.n_heads, i.size)], 1)
    want = oracle.chunk_attend_rows(rows, np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(), np64(inp["w_uk"]),
                                    np64(inp["w_uv"]), np64(inp["cache"]), wl.n_k, wl.scale)
    assert_g2x(got[rows[:, 0], rows[:, 1], rows[:, 2]], want, "480p expanded")
    assert np.all(np.isfinite(got))


# ----------------------------------------------------------------- per-shape choice of the form

def test_auto_short_chunk_runs_the_absorbed_form():
    mla = need_gpu()
    wl = synth.TINY
    inp = synth.attend_inputs(wl, seed=4)
    assert mla.chunk_attend_form(_dims(mla, wl), torch.bfloat16, wl.n_q, wl.n_k) == mla.MLA_FORM_ABSORBED
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"], wl.n_k, wl.scale)
    a = mla.chunk_attend(*args, out_dtype=torch.float32)
    b = mla.chunk_attend_auto(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_auto_long_chunk_runs_the_non_absorbed_form():
    """2048 queries (16 x 32 tokens per frame, 4 frames) over 3072 keys: the expanded form."""
    mla = need_gpu()
    wl = replace(synth.TINY, name="auto_long", grid_hw=(16, 32), cache_frames=(0, 1), query_frames=(2, 3, 4, 5))
    assert (wl.n_q, wl.n_k) == (2048, 3072)
    assert mla.chunk_attend_form(_dims(mla, wl), torch.bfloat16, wl.n_q, wl.n_k) == mla.MLA_FORM_EXPANDED
    inp = synth.attend_inputs(wl, seed=5)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"], wl.n_k, wl.scale)
    a = mla.chunk_attend_expanded(*args, out_dtype=torch.float32)
    b = mla.chunk_attend_auto(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    rng = np.random.default_rng(8)
    rows = np.stack([np.zeros(40, np.int64), rng.integers(0, wl.n_q, 40), rng.integers(0, wl.n_heads, 40)], 1)
    want = oracle.chunk_attend_rows(rows, np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(), np64(inp["w_uk"]),
                                    np64(inp["w_uv"]), np64(inp["cache"]), wl.n_k, wl.scale)
    assert_g2x(np64(b)[rows[:, 0], rows[:, 1], rows[:, 2]], want, "auto long")
