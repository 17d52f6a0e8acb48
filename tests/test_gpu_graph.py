"""A whole chunk step -- append, absorb, attention (with the chunk-causal
units kernel at the tiny shape), merge + up-projection -- captured in one
HIP graph.  The library's launches allocate nothing, record no memset nodes
and synchronize nothing, so a caller can capture them; launch-bound small
steps then pay one graph launch instead of six kernel launches.

Every replay must equal the eager step on the same inputs bit for bit (the
kernels are deterministic: fixed partition, fixed reduction orders).  The
program runs its own eager work and synchronizes between replays, and after
the inputs are rewritten in place the replays must follow the new inputs.
"""

import pytest
import torch

from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "wan480p"])
def test_chunk_step_graph_replays(name):
    mla = need_gpu()
    wl = synth.WORKLOADS[name]
    dims = mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)
    t = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in synth.attend_inputs(wl, seed=5).items()}
    a = {k: v.cuda() for k, v in synth.append_inputs(wl, seed=5).items()}
    cache = t["cache"]
    ws = mla.alloc_workspace(dims, torch.bfloat16, wl.n_q, wl.n_k)
    out = torch.empty((wl.batch, wl.n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")

    def step():
        mla.cache_append(dims, a["x"], a["w_dkv"], a["w_kr"], a["pos"], cache, wl.n_cached)
        mla.query_absorb(dims, t["q"], t["q_r"], t["q_pos"], t["w_uk"], wl.scale, wl.n_k, ws)
        mla.latent_attend(dims, cache, wl.n_q, wl.n_k, ws, causal=wl.causal)
        mla.value_upproj(dims, t["w_uv"], out, wl.n_q, wl.n_k, ws)

    def eager():
        step()
        torch.cuda.synchronize()
        return out.clone(), cache.clone()

    want, want_cache = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.fill_(0)                                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"
        assert torch.equal(cache, want_cache), f"replay {r}: cache"

    gen = torch.Generator().manual_seed(9)
    t["q"].copy_(torch.randn(t["q"].shape, generator=gen).to(torch.bfloat16))
    a["x"].copy_(torch.randn(a["x"].shape, generator=gen).to(torch.bfloat16))
    want2, want2_cache = eager()
    assert not torch.equal(want2, want)
    for r in range(2):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want2), f"replay {r} after new inputs"
        assert torch.equal(cache, want2_cache), f"replay {r} after new inputs: cache"
