"""mla_chunk_attend_noalloc (the chunk step on the library's own static
scratch, for callers that cannot allocate) against mla_chunk_attend with a
caller workspace: same kernels, so the outputs must agree bit for bit.  Two
calls in a row, the second smaller, so the second runs over the first one's
leftover scratch contents; then a size whose workspace exceeds the scratch is
refused before anything is enqueued."""

from dataclasses import replace

import pytest
import torch

from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _dims(mla, wl):
    return mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)


def _both(mla, wl, seed, out_dtype):
    inp = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in synth.attend_inputs(wl, seed=seed).items()}
    d = _dims(mla, wl)
    args = (d, inp["q"], inp["q_r"], inp["q_pos"], inp["w_uk"], inp["w_uv"], inp["cache"], wl.n_k, wl.scale)
    want = mla.chunk_attend(*args, out_dtype=out_dtype)
    got = torch.full_like(want, float("nan"))
    mla.chunk_attend_noalloc(*args, out=got)
    torch.cuda.synchronize()
    return got, want


def test_noalloc_matches_workspace_entry_point_twice():
    mla = need_gpu()
    big = synth.WAN480P                                                          # 115 MiB of workspace
    small = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))
    d_big = _dims(mla, big)
    assert mla.workspace_bytes(d_big, torch.bfloat16, big.n_q, big.n_k) <= mla.NOALLOC_SCRATCH_BYTES
    for wl, seed, odt in ((big, 0, torch.bfloat16), (small, 1, torch.float32), (small, 2, torch.bfloat16)):
        got, want = _both(mla, wl, seed, odt)
        view = torch.int32 if odt == torch.float32 else torch.int16
        assert torch.equal(got.view(view), want.view(view)), (wl.name, seed)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    mla = need_gpu()
    wl = synth.WAN480P_B8                                                        # 860 MiB of workspace
    d = _dims(mla, wl)
    assert mla.workspace_bytes(d, torch.bfloat16, wl.n_q, wl.n_k) > mla.NOALLOC_SCRATCH_BYTES
    small = replace(wl, grid_hw=(1, 1), query_frames=(0,), cache_frames=())
    inp = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in synth.attend_inputs(small, seed=0).items()}
    # shapes are checked against the arguments first: give tensors of the large call's shapes
    q = torch.zeros((wl.batch, wl.n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    q_r = torch.zeros((wl.batch, wl.n_q, wl.n_heads, wl.d_r), dtype=torch.bfloat16, device="cuda")
    q_pos = torch.zeros((wl.n_q, 3), dtype=torch.int32, device="cuda")
    cache = torch.zeros((wl.batch, wl.n_k, wl.d_c + wl.d_r), dtype=torch.bfloat16, device="cuda")
    out = torch.full((wl.batch, wl.n_q, wl.n_heads, wl.head_dim), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MLAError, match="no-allocation entry point"):
        mla.chunk_attend_noalloc(d, q, q_r, q_pos, inp["w_uk"], inp["w_uv"], cache, wl.n_k, wl.scale, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())                                              # nothing was enqueued
