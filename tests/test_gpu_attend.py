"""GPU parity of chunk attention (absorb -> fused attend -> up-projection)
against the fp64 non-absorbed oracle, called through the C ABI.

Gates (unit-scale outputs: the values W_UV c have unit variance under the
input recipe):
  G1  bf16 output:  raw max |err| <= 2e-2, raw mean |err| <= 2e-3.
  G2  bf16 inputs, fp32 output: errors divided by RMS(oracle), max <= 2.5e-2
      and mean <= 2e-3 (the output of attention is a weighted mean, so its
      RMS is well below 1 and raw errors alone would be a weak test).  The
      bounds are derived from a model of the path's bf16 roundings in
      tests/test_tolerances.py.
  F32 fp32 inputs and output: RMS-normalised max <= 1e-4, mean <= 1e-5.
Small shapes and the whole 480P step are compared element by element; the
other full workload shapes on rows that hit every 256-row block of every
sample, which the oracle computes one by one.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import assert_f32, assert_g1, assert_g2, errors, need_gpu, np64

pytestmark = pytest.mark.gpu


def _dims(mla, wl):
    return mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)


def _dev(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _gpu(mla, wl, inp, out_dtype=None, workspace=None):
    d = _dev(inp)
    out = mla.chunk_attend(_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"],
                           inp["n_k"], inp["scale"], out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return np64(out)


def _oracle(wl, inp):
    return oracle.chunk_attend(np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(), np64(inp["w_uk"]),
                               np64(inp["w_uv"]), np64(inp["cache"]), inp["n_k"], inp["scale"],
                               split=wl.rope_split, theta=wl.theta)


def _oracle_rows(wl, inp, rows):
    return oracle.chunk_attend_rows(rows, np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(),
                                    np64(inp["w_uk"]), np64(inp["w_uv"]), np64(inp["cache"]), inp["n_k"],
                                    inp["scale"], split=wl.rope_split, theta=wl.theta)


def _sample_rows(wl, n, seed=0, heads=None):
    rng = np.random.default_rng(seed)
    hs = np.arange(wl.n_heads) if heads is None else np.asarray(heads)
    b = rng.integers(0, wl.batch, n)
    i = rng.integers(0, wl.n_q, n)
    h = rng.choice(hs, n)
    rows = np.stack([b, i, h], 1)
    edge = np.array([[0, 0, hs[0]], [wl.batch - 1, wl.n_q - 1, hs[-1]], [0, wl.n_q - 1, hs[0]]])
    return np.concatenate([edge, rows], 0)


# ----------------------------------------------------------------------- tiny
def test_tiny_bf16_g1():
    mla = need_gpu()
    wl = synth.TINY
    inp = synth.attend_inputs(wl, seed=0)
    assert_g1(_gpu(mla, wl, inp), _oracle(wl, inp), "tiny bf16")


def test_tiny_bf16_fp32_out_g2():
    mla = need_gpu()
    wl = synth.TINY
    inp = synth.attend_inputs(wl, seed=0)
    assert_g2(_gpu(mla, wl, inp, out_dtype=torch.float32), _oracle(wl, inp), "tiny bf16->f32")


def test_tiny_fp32():
    mla = need_gpu()
    wl = synth.TINY
    inp = synth.attend_inputs(wl, seed=0, dtype=torch.float32)
    assert_f32(_gpu(mla, wl, inp), _oracle(wl, inp), "tiny fp32")


# -------------------------------------------------- ragged shapes, every d_c
@pytest.mark.parametrize("d_c", [64, 128, 192, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_shapes(d_c, dtype):
    mla = need_gpu()
    # 37 queries x 3 heads (ragged row block), 150 keys (ragged key tile), 2 samples
    wl = replace(synth.TINY, batch=2, n_heads=3, d_c=d_c, grid_hw=(37, 1), query_frames=(9,),
                 cache_frames=(0, 1, 2))                  # 3*37 cached + 37 current = 148 keys
    inp = synth.attend_inputs(wl, seed=5, dtype=dtype, capacity=wl.n_k + 9)
    got = _gpu(mla, wl, inp, out_dtype=torch.float32)
    want = _oracle(wl, inp)
    if dtype == torch.float32:
        assert_f32(got, want, f"ragged f32 dc{d_c}")
    else:
        assert_g2(got, want, f"ragged bf16 dc{d_c}")


def test_stream_k_partial_segments():
    """15 row-blocks over 256 workgroups: every row-block is split across many segments."""
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))  # 300 q, 2100 k
    inp = synth.attend_inputs(wl, seed=6)
    want = _oracle(wl, inp)
    assert_g1(_gpu(mla, wl, inp), want, "stream-k bf16")
    assert_g2(_gpu(mla, wl, inp, out_dtype=torch.float32), want, "stream-k bf16->f32")


def test_unsplit_partition():
    """235 row-blocks: one workgroup per row-block, no key partition."""
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(50, 100), query_frames=(1,), cache_frames=())     # 5000 q, 5000 k
    inp = synth.attend_inputs(wl, seed=7)
    rows = _sample_rows(wl, 200, seed=1)
    got = _gpu(mla, wl, inp, out_dtype=torch.float32)
    want = _oracle_rows(wl, inp, rows)
    assert_g2(got[rows[:, 0], rows[:, 1], rows[:, 2]], want, "unsplit")


def test_peaky_logits():
    """q and q_r scaled x8: logits with std 8 exercise the running-max rescale.

    The absorbed query is rounded once to bf16 (relative error 2^-9), so the
    logit error grows in proportion to the logit magnitude; the gate is the
    unit-scale G1 gate scaled by that factor (8), halved for margin: a
    rescale bug gives errors of order 1.
    """
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(12, 10), query_frames=(4,), cache_frames=tuple(range(4)))
    inp = synth.attend_inputs(wl, seed=8)
    inp["q"] = (inp["q"].float() * 8).to(torch.bfloat16)
    inp["q_r"] = (inp["q_r"].float() * 8).to(torch.bfloat16)
    want = _oracle(wl, inp)
    for out_dtype in (None, torch.float32):
        e = errors(_gpu(mla, wl, inp, out_dtype=out_dtype), want)
        assert e["max_abs"] <= 4 * 2e-2 and e["mean_abs"] <= 4 * 2e-3, e


def test_max_key_at_tile_edges():
    """One key far above the rest, placed first, last, and at a tile boundary."""
    mla = need_gpu()
    wl = replace(synth.TINY, n_heads=2)
    for j in (0, wl.n_k - 1, 64, 63):
        inp = synth.attend_inputs(wl, seed=9)
        c = inp["cache"].float()
        q0 = inp["q"][0, 0, 0].float()
        # make key j align with query (0,0,0) through W_UK of head 0
        k_dir = inp["w_uk"][0].float().T @ q0                     # latent direction seen by that query
        c[0, j, :wl.d_c] = 6.0 * k_dir / k_dir.norm()
        inp["cache"] = c.to(torch.bfloat16)
        want = _oracle(wl, inp)
        assert_g1(_gpu(mla, wl, inp), want, f"max key at {j}")


# ---------------------------------------------------- full workload shapes
def _rows_every_block(wl, seed, per_block=1):
    """Rows (b, i, h) that hit every 256-row block of every sample (rows
    r = h * n_q + i of a sample are packed 256 to a block, and each block's
    partial states are merged from the slots of the workgroups that split it),
    plus the first and last row of every sample."""
    rng = np.random.default_rng(seed)
    rows_b = wl.n_heads * wl.n_q
    out = []
    for b in range(wl.batch):
        for r0 in range(0, rows_b, 256):
            r = rng.integers(r0, min(rows_b, r0 + 256), per_block)
            out += [[b, int(x) % wl.n_q, int(x) // wl.n_q] for x in r]
        out += [[b, 0, 0], [b, wl.n_q - 1, wl.n_heads - 1]]
    return np.array(out, np.int64)


def test_480p_every_row():
    """The headline step (4680 queries x 12 heads over 32760 keys): every one of
    the 56160 output rows against the oracle, bf16 output under G1 and fp32
    output under G2."""
    mla = need_gpu()
    wl = synth.WAN480P
    inp = synth.attend_inputs(wl, seed=0)
    got16 = _gpu(mla, wl, inp)
    got32 = _gpu(mla, wl, inp, out_dtype=torch.float32)
    want = _oracle(wl, inp)
    assert_g1(got16, want, "480p bf16 out, all rows")
    assert_g2(got32, want, "480p f32 out, all rows")


@pytest.mark.parametrize("name", ["wan720p_long", "wan480p_shard8"])
def test_full_shape_every_row_block(name):
    mla = need_gpu()
    wl = synth.WORKLOADS[name]
    inp = synth.attend_inputs(wl, seed=0)
    rows = _rows_every_block(wl, seed=2)
    got = _gpu(mla, wl, inp)
    want = _oracle_rows(wl, inp, rows)
    assert_g1(got[rows[:, 0], rows[:, 1], rows[:, 2]], want, name)
    got32 = _gpu(mla, wl, inp, out_dtype=torch.float32)
    assert_g2(got32[rows[:, 0], rows[:, 1], rows[:, 2]], want, name + " f32 out")
    assert np.all(np.isfinite(got))


def test_batched_480p_every_row_block():
    """Batch 8: 1760 row blocks (220 per sample), each checked on one row."""
    mla = need_gpu()
    wl = synth.WAN480P_B8
    inp = synth.attend_inputs(wl, seed=0)
    rows = _rows_every_block(wl, seed=3)
    got = _gpu(mla, wl, inp, out_dtype=torch.float32)
    want = _oracle_rows(wl, inp, rows)
    assert_g2(got[rows[:, 0], rows[:, 1], rows[:, 2]], want, "480p b8")


@pytest.mark.parametrize("d_c", [64, 128, 256])
def test_dc_sweep_480p_every_row_block(d_c):
    mla = need_gpu()
    wl = synth.WAN480P.with_dc(d_c)
    inp = synth.attend_inputs(wl, seed=0)
    rows = _rows_every_block(wl, seed=4)
    got = _gpu(mla, wl, inp, out_dtype=torch.float32)
    want = _oracle_rows(wl, inp, rows)
    assert_g2(got[rows[:, 0], rows[:, 1], rows[:, 2]], want, f"480p dc{d_c}")


# ------------------------------------------------------- closed forms
def _mean_of_values(inp, n_k):
    """q = q_r = 0: every score is 0, so each head's output is the plain mean of
    its values, O_h = W_UV[h] (mean_j c_j) (closed form; no softmax involved)."""
    d_c = inp["w_uk"].shape[-1]
    c_mean = np64(inp["cache"])[:, :n_k, :d_c].mean(axis=1)              # [B, d_c]
    return np.einsum("bc,hdc->bhd", c_mean, np64(inp["w_uv"]))             # [B, H, d_h]


@pytest.mark.parametrize("name", ["stream_k", "wan480p"])
def test_zero_query_gives_mean_of_values(name):
    mla = need_gpu()
    wl = (replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))
          if name == "stream_k" else synth.WAN480P)
    inp = synth.attend_inputs(wl, seed=14)
    inp["q"] = torch.zeros_like(inp["q"])
    inp["q_r"] = torch.zeros_like(inp["q_r"])
    want = np.broadcast_to(_mean_of_values(inp, wl.n_k)[:, None], (wl.batch, wl.n_q, wl.n_heads, wl.head_dim))
    got = _gpu(mla, wl, inp, out_dtype=torch.float32)
    # every p is exactly 1 and L the fp32 mean: only the bf16 hi/lo split of L
    # and the fp32 sums remain, far inside G2
    assert_g2(got, want, name + " q = 0", max_norm=1e-3, mean_norm=1e-4)


@pytest.mark.parametrize("form", ["absorbed", "expanded", "auto"])
@pytest.mark.parametrize("d_c", [64, 192, 256])
def test_single_key_gives_that_keys_value(form, d_c):
    """A one-token chunk with nothing cached (n_q = n_k = 1, the smallest
    call the ABI takes): the softmax weight is exactly 1, so every head's
    output is W_UV[h] c_0 whatever the query (a closed form)."""
    mla = need_gpu()
    wl = replace(synth.TINY, d_c=d_c, grid_hw=(1, 1), query_frames=(1,), cache_frames=())
    inp = synth.attend_inputs(wl, seed=21)
    c0 = np64(inp["cache"])[:, 0, :d_c]                                      # [B, d_c]
    want = np.einsum("bc,hdc->bhd", c0, np64(inp["w_uv"]))                    # [B, H, d_h]
    want = np.broadcast_to(want[:, None], (wl.batch, wl.n_q, wl.n_heads, wl.head_dim))
    d = _dev(inp)
    fn = {"absorbed": mla.chunk_attend, "expanded": mla.chunk_attend_expanded, "auto": mla.chunk_attend_auto}[form]
    out = fn(_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"], 1, inp["scale"],
             out_dtype=torch.float32 if form != "expanded" else None)
    torch.cuda.synchronize()
    got = np64(out)
    if form == "expanded":
        # bf16 output; V_h = W_UV[h] c_0 is itself rounded to bf16 once
        assert_g1(got, want, f"single key {form} dc{d_c}")
    else:
        # p = 1 exactly, L = c_0 exactly (bf16 hi/lo split exact); only fp32 sums remain
        assert_g2(got, want, f"single key {form} dc{d_c}", max_norm=1e-4, mean_norm=1e-5)


# ------------------------------------------------ composition and hygiene
def test_steps_compose_to_chunk_attend():
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))
    inp = _dev(synth.attend_inputs(wl, seed=10))
    d = _dims(mla, wl)
    ws = mla.alloc_workspace(d, torch.bfloat16, wl.n_q, wl.n_k)
    full = mla.chunk_attend(d, inp["q"], inp["q_r"], inp["q_pos"], inp["w_uk"], inp["w_uv"], inp["cache"],
                            wl.n_k, wl.scale, workspace=ws)
    out = torch.empty_like(full)
    mla.query_absorb(d, inp["q"], inp["q_r"], inp["q_pos"], inp["w_uk"], wl.scale, wl.n_k, ws)
    mla.latent_attend(d, inp["cache"], wl.n_q, wl.n_k, ws)
    mla.value_upproj(d, inp["w_uv"], out, wl.n_q, wl.n_k, ws)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("causal", [None, (1500, 300), (1200, 150)])
def test_attend_twice_after_one_absorb(causal):
    """Attention and up-projection read nothing of the workspace but the absorbed
    queries and what the attention call itself writes (partial states, the
    partition header, the per-row-block units): repeating them on the same
    absorbed queries, over a workspace that started as garbage, must give the
    fused call's bits every time."""
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))
    inp = _dev(synth.attend_inputs(wl, seed=13))
    d = _dims(mla, wl)
    ws = mla.alloc_workspace(d, torch.bfloat16, wl.n_q, wl.n_k)
    ws.fill_(0x55)
    outs = [torch.empty((1, wl.n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    mla.query_absorb(d, inp["q"], inp["q_r"], inp["q_pos"], inp["w_uk"], wl.scale, wl.n_k, ws)
    for o in outs:
        mla.latent_attend(d, inp["cache"], wl.n_q, wl.n_k, ws, causal=causal)
        mla.value_upproj(d, inp["w_uv"], o, wl.n_q, wl.n_k, ws)
    full = mla.chunk_attend(d, inp["q"], inp["q_r"], inp["q_pos"], inp["w_uk"], inp["w_uv"], inp["cache"],
                            wl.n_k, wl.scale, causal=causal)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), full.view(torch.int16))
    assert torch.isfinite(full.float()).all()


def test_deterministic_and_poisoned_workspace():
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))
    inp = synth.attend_inputs(wl, seed=11)
    d = _dims(mla, wl)
    ws = mla.alloc_workspace(d, torch.bfloat16, wl.n_q, wl.n_k)
    ws.fill_(0xFF)                          # NaN in every fp32 / bf16 slot
    a = _gpu(mla, wl, inp, workspace=ws)
    ws.fill_(0x7F)
    b = _gpu(mla, wl, inp, workspace=ws)
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


def test_append_then_attend_chunk_step():
    """One chunk step: append the current chunk's rows, then attend over all keys."""
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(8, 12), query_frames=(6, 7), cache_frames=tuple(range(6)))
    att = synth.attend_inputs(wl, seed=12, capacity=wl.n_k + 32)
    app = synth.append_inputs(wl, seed=12)
    d = _dims(mla, wl)
    cache = att["cache"].cuda()
    mla.cache_append(d, app["x"].cuda(), app["w_dkv"].cuda(), app["w_kr"].cuda(), app["pos"].cuda(), cache,
                     wl.n_cached)
    att_dev = _dev(att)
    out = mla.chunk_attend(d, att_dev["q"], att_dev["q_r"], att_dev["q_pos"], att_dev["w_uk"], att_dev["w_uv"],
                           cache, wl.n_k, wl.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_cache = oracle.cache_append(np64(att["cache"]), np64(app["x"]), np64(app["w_dkv"]), np64(app["w_kr"]),
                                    app["pos"].numpy(), wl.n_cached)
    inp = dict(att)
    inp["cache"] = torch.from_numpy(ref_cache).to(torch.bfloat16)
    assert_g2(np64(out), _oracle(wl, inp), "append+attend")


@pytest.mark.parametrize("headroom", ["0", "1.5"])
def test_two_pass_fallback(monkeypatch, headroom):
    """Headroom forced small from the host: segments whose max grows past it
    are redone as an exact max pass + accumulation pass."""
    mla = need_gpu()
    monkeypatch.setenv("MLA_ATTEND_HEADROOM", headroom)
    wl = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))
    inp = synth.attend_inputs(wl, seed=13)
    want = _oracle(wl, inp)
    assert_g1(_gpu(mla, wl, inp), want, "two-pass bf16")
    assert_g2(_gpu(mla, wl, inp, out_dtype=torch.float32), want, "two-pass f32 out")


def test_workspace_of_any_dtype_and_host_workspace_rejected():
    """The binding passes the workspace's size in bytes, whatever its dtype, and
    rejects a host tensor before anything is launched."""
    mla = need_gpu()
    wl = replace(synth.TINY, grid_hw=(30, 10), query_frames=(6,), cache_frames=tuple(range(6)))
    inp = synth.attend_inputs(wl, seed=13)
    d = _dims(mla, wl)
    n = mla.workspace_bytes(d, torch.bfloat16, wl.n_q, wl.n_k)
    a = _gpu(mla, wl, inp, workspace=mla.alloc_workspace(d, torch.bfloat16, wl.n_q, wl.n_k))
    b = _gpu(mla, wl, inp, workspace=torch.empty((n + 3) // 4, dtype=torch.float32, device="cuda"))
    assert np.array_equal(a, b)
    with pytest.raises(ValueError, match="workspace"):
        _gpu(mla, wl, inp, workspace=torch.empty(n, dtype=torch.uint8))
    with pytest.raises(mla.MLAError):
        _gpu(mla, wl, inp, workspace=torch.empty(n // 2, dtype=torch.uint8, device="cuda"))
