"""The two-pass fallback of the single-pass softmax runs when it must and only
then, in every bf16 attention kernel (the role-split latent kernel with one or
two score wavefronts per group, the d_c = 256 single-role kernel, and the
per-head kernel of the dense and non-absorbed forms).

Rule (mla.h, MLA_ATTEND_HEADROOM): a key segment is redone exactly when some
lane's running sum of p = 2^(s - m), m the segment's first-block maximum,
exceeds 2^headroom, or an accumulator is not finite.  The single pass and the
exact pass round differently, so the output's bits show which one ran:
  * Gaussian inputs: no segment's sum comes near 2^32, so the default and the
    largest headroom (64) give the same bits, while headroom 0 (every segment
    redone) gives different bits;
  * logits with a standard deviation of about 100 log2 units: a single pass
    would overflow (2^s beyond fp32), so every segment must be redone at any
    headroom, and the default gives the bits of headroom 0, all finite.
"""

from dataclasses import replace

import pytest
import torch

from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

SHAPE = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))   # 300 q, 2100 k
FORMS = ["absorbed_dc64", "absorbed_dc128", "absorbed_dc192", "absorbed_dc256", "expanded", "dense"]


def _run(mla, form, monkeypatch, headroom, q_gain):
    if headroom is None:
        monkeypatch.delenv("MLA_ATTEND_HEADROOM", raising=False)
    else:
        monkeypatch.setenv("MLA_ATTEND_HEADROOM", str(headroom))
    if form == "dense":
        inp = synth.mha_inputs(SHAPE, seed=31)
        q = (inp["q"].float() * q_gain).to(torch.bfloat16).cuda()
        out = mla.mha_attend(q, inp["k"].cuda(), inp["v"].cuda(), inp["n_k"], inp["scale"], out_dtype=torch.float32)
    else:
        d_c = int(form.split("dc")[1]) if form.startswith("absorbed") else 192
        wl = SHAPE.with_dc(d_c)
        inp = synth.attend_inputs(wl, seed=31)
        d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        q = (d["q"].float() * q_gain).to(torch.bfloat16)
        q_r = (d["q_r"].float() * q_gain).to(torch.bfloat16)
        dims = mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                        rope=wl.rope_split, rope_theta=wl.theta)
        fn = mla.chunk_attend_expanded if form == "expanded" else mla.chunk_attend
        out = fn(dims, q, q_r, d["q_pos"], d["w_uk"], d["w_uv"], d["cache"], wl.n_k, wl.scale,
                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out.view(torch.int32).cpu()


@pytest.mark.parametrize("form", FORMS)
def test_no_fallback_on_ordinary_inputs(form, monkeypatch):
    mla = need_gpu()
    default = _run(mla, form, monkeypatch, None, 1.0)
    assert torch.equal(default, _run(mla, form, monkeypatch, 64, 1.0))
    assert not torch.equal(default, _run(mla, form, monkeypatch, 0, 1.0))


@pytest.mark.parametrize("form", FORMS)
def test_fallback_where_a_single_pass_would_overflow(form, monkeypatch):
    mla = need_gpu()
    gain = 70.0      # unit-variance logits x 70: a standard deviation of about 100 log2 units
    default = _run(mla, form, monkeypatch, None, gain)
    assert torch.isfinite(default.view(torch.float32)).all()
    assert torch.equal(default, _run(mla, form, monkeypatch, 0, gain))
