"""GPU parity of the cache-append kernel against the fp64 oracle.

Exact tier: inputs on which every fp32 partial sum is exact and the rotation
is the identity, so the bf16 bytes are fixed by the rounding rule alone; all
bytes of the cache must match the oracle (layout, offsets, token order and
round-to-nearest-even are pinned at once).

Gaussian tier: every element must be bit-identical to the oracle's direct
fp64 -> bf16 rounding, except elements whose exact value lies within the
rigorous error bound of an fp32 evaluation of a rounding midpoint; those may
differ by exactly one bf16 ulp.
"""

import numpy as np
import pytest
import torch

import oracle
from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import need_gpu, np64

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _dims(mla, wl):
    return mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)


def _run_append(mla, wl, inp, cap, off, sentinel_bits=0x7F7F):
    cache = torch.full((wl.batch, cap, wl.d_c + wl.d_r), 0, dtype=torch.int16)
    cache.fill_(np.int16(np.uint16(sentinel_bits).view(np.int16)))
    cache = cache.view(torch.bfloat16).cuda()
    mla.cache_append(_dims(mla, wl), inp["x"].cuda(), inp["w_dkv"].cuda(), inp["w_kr"].cuda(),
                     inp["pos"].cuda(), cache, off)
    torch.cuda.synchronize()
    return cache.cpu()


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("d_c", [192, 64, 128, 256])
def test_append_exact_tier_bytes(d_c):
    mla = need_gpu()
    from dataclasses import replace
    wl = replace(synth.TINY, d_c=d_c, batch=2)
    inp = synth.append_inputs_exact(wl, seed=1)
    cap, off = wl.n_q + 21, 13
    got = _run_append(mla, wl, inp, cap, off)
    sentinel = np.full((wl.batch, cap, wl.d_c + wl.d_r), 0x7F7F, np.uint16)
    ref = oracle.cache_append(np.zeros(sentinel.shape), np64(inp["x"]), np64(inp["w_dkv"]),
                              np64(inp["w_kr"]), inp["pos"].numpy(), off, split=wl.rope_split, theta=wl.theta)
    want = sentinel.copy()
    want[:, off:off + wl.n_q] = oracle.bf16_bits(ref[:, off:off + wl.n_q])
    gb = _bits(got)
    assert np.array_equal(gb, want), f"{np.count_nonzero(gb != want)} of {gb.size} bf16 values differ"


@pytest.mark.parametrize("d_model", [64, 320, 576, 2048])
def test_append_exact_tier_other_widths(d_model):
    """d_model is dealt to the four wavefronts in 64-wide chunks round robin:
    64 leaves three of them without a chunk, 320 and 576 give them unequal
    counts (one of them a single chunk), 2048 runs the steady-state loop."""
    mla = need_gpu()
    from dataclasses import replace
    wl = replace(synth.TINY, d_model=d_model, batch=2)
    inp = synth.append_inputs_exact(wl, seed=3)
    cap, off = wl.n_q + 5, 3
    got = _run_append(mla, wl, inp, cap, off)
    ref = oracle.cache_append(np.zeros((wl.batch, cap, wl.d_c + wl.d_r)), np64(inp["x"]), np64(inp["w_dkv"]),
                              np64(inp["w_kr"]), inp["pos"].numpy(), off, split=wl.rope_split, theta=wl.theta)
    want = np.full((wl.batch, cap, wl.d_c + wl.d_r), 0x7F7F, np.uint16)
    want[:, off:off + wl.n_q] = oracle.bf16_bits(ref[:, off:off + wl.n_q])
    gb = _bits(got)
    assert np.array_equal(gb, want), f"{np.count_nonzero(gb != want)} of {gb.size} bf16 values differ"


def _error_bound(x, w_all, pos, wl):
    """Rigorous bound on |fp32 GPU value - exact value| per output element."""
    D = x.shape[-1]
    gamma = D * U32 / (1 - D * U32)
    absdot = np.abs(x) @ np.abs(w_all).T                   # sum_k |x_k w_k|
    delta = 2.0 * gamma * absdot                            # any fp32 summation order, 2x margin
    raw = x @ w_all.T                                       # unrotated exact values
    dc = wl.d_c
    ang = oracle.rope3d_angles(pos, wl.rope_split, wl.theta)[None]   # [1, n, 16]
    c, s = np.abs(np.cos(ang)), np.abs(np.sin(ang))
    d0, d1 = delta[..., dc::2], delta[..., dc + 1::2]
    x0, x1 = np.abs(raw[..., dc::2]), np.abs(raw[..., dc + 1::2])
    rot = 8 * U32 * (x0 + x1)
    out = delta.copy()
    out[..., dc::2] = c * d0 + s * d1 + rot
    out[..., dc + 1::2] = s * d0 + c * d1 + rot
    return out


def _tie_zone_check(got_bits, exact, bound):
    """Bit-exact except where the fp32 error bound reaches a bf16 rounding boundary.

    An fp32 evaluation returns some value within `bound` of the exact one and
    rounds it to nearest-even, and rounding is monotonic; so a correct result
    lies in [rne(exact - bound), rne(exact + bound)].  Where that interval
    holds one bf16 value the result must equal the oracle's bits exactly.
    """
    want = oracle.bf16_rne(exact)
    want_bits = oracle.bf16_bits(want)
    diff = got_bits != want_bits
    n_diff = int(diff.sum())
    if n_diff:
        g = torch.from_numpy(got_bits[diff].view(np.int16)).view(torch.bfloat16).double().numpy()
        lo = oracle.bf16_rne(exact[diff] - bound[diff])
        hi = oracle.bf16_rne(exact[diff] + bound[diff])
        bad = (g < lo) | (g > hi)
        assert not np.any(bad), f"{int(bad.sum())} values outside the rounding interval of the fp32 bound"
    return n_diff


@pytest.mark.parametrize("wl_name,batch", [("tiny", 1), ("tiny", 3), ("wan480p", 1)])
def test_append_gaussian_tie_zone(wl_name, batch):
    mla = need_gpu()
    from dataclasses import replace
    wl = replace(synth.WORKLOADS[wl_name], batch=batch)
    inp = synth.append_inputs(wl, seed=2)
    cap, off = wl.n_q + 70, 64
    got = _run_append(mla, wl, inp, cap, off)
    x = np64(inp["x"])
    w_all = np.concatenate([np64(inp["w_dkv"]), np64(inp["w_kr"])], 0)
    pos = inp["pos"].numpy()
    exact = oracle.latent_rows(x, np64(inp["w_dkv"]), np64(inp["w_kr"]), pos, wl.rope_split, wl.theta)
    bound = _error_bound(x, w_all, pos, wl)
    gb = _bits(got)
    n_diff = _tie_zone_check(gb[:, off:off + wl.n_q], exact, bound)
    assert n_diff <= 1e-3 * exact.size
    assert np.all(gb[:, :off] == 0x7F7F) and np.all(gb[:, off + wl.n_q:] == 0x7F7F)


def test_append_ragged_token_count_and_offsets():
    mla = need_gpu()
    from dataclasses import replace
    wl = replace(synth.TINY, batch=2, grid_hw=(37, 1), query_frames=(3,))   # 37 tokens: ragged tail
    inp = synth.append_inputs(wl, seed=3)
    cap = 100
    cache = torch.zeros((2, cap, 224), dtype=torch.bfloat16).cuda()
    d = _dims(mla, wl)
    mla.cache_append(d, inp["x"].cuda(), inp["w_dkv"].cuda(), inp["w_kr"].cuda(), inp["pos"].cuda(), cache, 0)
    mla.cache_append(d, inp["x"].cuda(), inp["w_dkv"].cuda(), inp["w_kr"].cuda(), inp["pos"].cuda(), cache, cap - 37)
    torch.cuda.synchronize()
    gb = _bits(cache.cpu())
    assert np.array_equal(gb[:, :37], gb[:, cap - 37:])
    assert np.all(gb[:, 37:cap - 37] == 0)
    exact = oracle.latent_rows(np64(inp["x"]), np64(inp["w_dkv"]), np64(inp["w_kr"]), inp["pos"].numpy())
    w_all = np.concatenate([np64(inp["w_dkv"]), np64(inp["w_kr"])], 0)
    _tie_zone_check(gb[:, :37], exact, _error_bound(np64(inp["x"]), w_all, inp["pos"].numpy(), wl))


def test_append_fp32():
    mla = need_gpu()
    from dataclasses import replace
    wl = replace(synth.TINY, batch=2)
    inp = synth.append_inputs(wl, seed=4, dtype=torch.float32)
    cache = torch.zeros((2, wl.n_q + 5, 224), dtype=torch.float32).cuda()
    mla.cache_append(_dims(mla, wl), inp["x"].cuda(), inp["w_dkv"].cuda(), inp["w_kr"].cuda(),
                     inp["pos"].cuda(), cache, 5)
    torch.cuda.synchronize()
    got = np64(cache.cpu())[:, 5:]
    exact = oracle.latent_rows(np64(inp["x"]), np64(inp["w_dkv"]), np64(inp["w_kr"]), inp["pos"].numpy())
    w_all = np.concatenate([np64(inp["w_dkv"]), np64(inp["w_kr"])], 0)
    bound = _error_bound(np64(inp["x"]), w_all, inp["pos"].numpy(), wl) + 2 * U32 * np.abs(exact)
    assert np.all(np.abs(got - exact) <= bound)
