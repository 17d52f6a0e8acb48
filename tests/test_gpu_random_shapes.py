"""Seeded sweep of random small shapes through every attention entry point.

Each case draws d_c, batch, head count, frame grid, the number of cached and
current frames, a ragged query prefix (one GPU's share of a query-sharded
chunk), spare cache capacity, and, for a third of the cases, a block-causal
call whose chunk length is drawn too.  The absorbed form runs with bf16 and
fp32 outputs and with fp32 inputs; the non-absorbed form and the per-shape
choice run on the same bf16 inputs.  Every output is compared with the fp64
oracle on the same inputs, under the gates of the fixed-shape tests:
G1 for bf16 outputs, G2 for fp32 outputs (the short-key and causal bound
where a row sees fewer than 148 keys or the call is block-causal; the
non-absorbed bound for that form), F32 for fp32 inputs.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import G2_CAUSAL_MAX, G2_MAX, assert_f32, assert_g1, assert_g2, assert_g2x, need_gpu, np64

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(seed: int):
    r = np.random.default_rng(90210 + seed)
    hw = (int(r.integers(1, 12)), int(r.integers(1, 16)))
    n_cache_frames = int(r.choice([int(r.integers(0, 4)), int(r.integers(4, 25))]))
    n_query_frames = int(r.integers(1, 4))
    frame = hw[0] * hw[1]
    chunk = n_query_frames * frame
    wl = replace(synth.TINY, name=f"random{seed}", batch=int(r.choice([1, 2, 3])),
                 n_heads=int(r.choice([1, 2, 5, 12])), d_c=int(r.choice([64, 128, 192, 256])), grid_hw=hw,
                 cache_frames=tuple(range(n_cache_frames)),
                 query_frames=tuple(range(n_cache_frames, n_cache_frames + n_query_frames)),
                 query_tokens=int(r.integers(1, chunk + 1)) if r.random() < 0.3 else 0)
    capacity = wl.n_k + int(r.integers(0, 41))
    causal = (wl.n_cached, int(r.integers(1, wl.n_q + 1))) if r.random() < 1 / 3 else None
    return wl, capacity, causal


def _dims(mla, wl):
    return mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)


def _oracle(wl, inp, causal):
    kw = {}
    if causal is not None:
        q_start, c = causal
        kw = dict(q_chunk=(q_start + np.arange(wl.n_q)) // c, k_chunk=np.arange(inp["n_k"]) // c)
    return oracle.chunk_attend(np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(), np64(inp["w_uk"]),
                               np64(inp["w_uv"]), np64(inp["cache"]), inp["n_k"], inp["scale"],
                               split=wl.rope_split, theta=wl.theta, **kw)


def _fewest_keys(wl, causal):
    """Keys seen by the row that sees the fewest."""
    if causal is None:
        return wl.n_k
    q_start, c = causal
    return min(wl.n_k, (q_start // c + 1) * c)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    mla = need_gpu()
    wl, capacity, causal = _case(seed)
    label = (f"seed {seed}: B={wl.batch} H={wl.n_heads} d_c={wl.d_c} n_q={wl.n_q} n_k={wl.n_k} "
             f"cap={capacity} causal={causal}")
    print(label, flush=True)
    d = _dims(mla, wl)
    gate = G2_MAX if causal is None and _fewest_keys(wl, causal) >= 148 else G2_CAUSAL_MAX

    inp = synth.attend_inputs(wl, seed=seed, capacity=capacity)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (d, dev["q"], dev["q_r"], dev["q_pos"], dev["w_uk"], dev["w_uv"], dev["cache"], wl.n_k, wl.scale)
    want = _oracle(wl, inp, causal)
    out16 = mla.chunk_attend(*args, causal=causal)
    out32 = mla.chunk_attend(*args, out_dtype=torch.float32, causal=causal)
    torch.cuda.synchronize()
    assert_g1(np64(out16), want, label + " absorbed bf16 out")
    assert_g2(np64(out32), want, label + " absorbed f32 out", max_norm=gate)
    if causal is None:
        exp32 = mla.chunk_attend_expanded(*args, out_dtype=torch.float32)
        auto32 = mla.chunk_attend_auto(*args, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_g2x(np64(exp32), want, label + " non-absorbed f32 out")
        if mla.chunk_attend_form(d, torch.bfloat16, wl.n_q, wl.n_k) == mla.MLA_FORM_EXPANDED:
            assert_g2x(np64(auto32), want, label + " per-shape choice f32 out")
        else:
            assert_g2(np64(auto32), want, label + " per-shape choice f32 out", max_norm=gate)

    inp32 = synth.attend_inputs(wl, seed=seed, dtype=torch.float32, capacity=capacity)
    dev32 = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp32.items()}
    got = mla.chunk_attend(d, dev32["q"], dev32["q_r"], dev32["q_pos"], dev32["w_uk"], dev32["w_uv"],
                           dev32["cache"], wl.n_k, wl.scale, causal=causal)
    torch.cuda.synchronize()
    assert_f32(np64(got), _oracle(wl, inp32, causal), label + " fp32 in")


# ------------------------------------------------------------ cache append
def _append_case(seed: int):
    r = np.random.default_rng(4242 + seed)
    hw = (int(r.integers(1, 12)), int(r.integers(1, 16)))
    wl = replace(synth.TINY, name=f"append{seed}", batch=int(r.choice([1, 2, 3])),
                 d_c=int(r.choice([64, 128, 192, 256])), d_model=64 * int(r.integers(1, 41)), grid_hw=hw,
                 cache_frames=(), query_frames=tuple(range(int(r.integers(1, 20)), 0, -1))[:int(r.integers(1, 4))])
    off = int(r.integers(0, 300))
    return wl, off, off + wl.n_q + int(r.integers(0, 41))


@pytest.mark.parametrize("seed", range(12))
def test_random_append(seed):
    """Append rows match the oracle's bits outside the tie zone of the fp32
    error bound; every slot outside [off, off + n) keeps its sentinel."""
    from tests.test_gpu_append import _error_bound, _run_append, _tie_zone_check
    mla = need_gpu()
    wl, off, cap = _append_case(seed)
    print(f"seed {seed}: B={wl.batch} d_c={wl.d_c} D={wl.d_model} n_new={wl.n_q} off={off} cap={cap}", flush=True)
    inp = synth.append_inputs(wl, seed=seed)
    got = _run_append(mla, wl, inp, cap, off)
    x, pos = np64(inp["x"]), inp["pos"].numpy()
    exact = oracle.latent_rows(x, np64(inp["w_dkv"]), np64(inp["w_kr"]), pos, wl.rope_split, wl.theta)
    bound = _error_bound(x, np.concatenate([np64(inp["w_dkv"]), np64(inp["w_kr"])], 0), pos, wl)
    gb = got.view(torch.int16).numpy().view(np.uint16)
    n_diff = _tie_zone_check(gb[:, off:off + wl.n_q], exact, bound)
    assert n_diff <= max(2, 1e-3 * exact.size)
    assert np.all(gb[:, :off] == 0x7F7F) and np.all(gb[:, off + wl.n_q:] == 0x7F7F)


# ------------------------------------------------- dense per-head attention
def _dense_case(seed: int):
    r = np.random.default_rng(777 + seed)
    hw = (int(r.integers(1, 12)), int(r.integers(1, 16)))
    n_cache_frames = int(r.integers(0, 12))
    wl = replace(synth.TINY, name=f"dense{seed}", batch=int(r.choice([1, 2, 3])),
                 n_heads=int(r.choice([1, 2, 5, 12])), grid_hw=hw, cache_frames=tuple(range(n_cache_frames)),
                 query_frames=tuple(range(n_cache_frames, n_cache_frames + int(r.integers(1, 4)))))
    return wl, wl.n_k + int(r.integers(0, 41))


@pytest.mark.parametrize("seed", range(12))
def test_random_dense(seed):
    mla = need_gpu()
    wl, cap = _dense_case(seed)
    print(f"seed {seed}: B={wl.batch} H={wl.n_heads} n_q={wl.n_q} n_k={wl.n_k} cap={cap}", flush=True)
    inp = synth.mha_inputs(wl, seed=seed, capacity=cap)
    out = mla.mha_attend(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["n_k"], inp["scale"],
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = oracle.mha_attend(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), inp["n_k"], inp["scale"])
    assert_g2(np64(out), want, f"dense seed {seed}", max_norm=G2_MAX if wl.n_k >= 148 else G2_CAUSAL_MAX)
