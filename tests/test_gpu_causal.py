"""GPU parity of the block-causal multi-chunk mode (mla_chunk_attend_causal)
against the fp64 oracle with the same chunk masks.

Queries span several chunks: query i is token q_start + i of the key
sequence and sees every key of its own chunk and of all earlier chunks
(chunk-causal: VideoMLA atlas.scime.ai summary, first paragraph).  The
oracle gets the same visibility as chunk indices (q_chunk, k_chunk).  Gates
as in test_gpu_attend.py, except the RMS-normalised max of the fp32-output
check (G2_CAUSAL_MAX in gpu_util.py: rows that see a single chunk do not
average the bf16 roundings of q~ and P).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import G2_CAUSAL_MAX, assert_f32, assert_g1, assert_g2, need_gpu, np64

pytestmark = pytest.mark.gpu


def _dims(mla, wl):
    return mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)


def _gpu(mla, wl, inp, causal, out_dtype=None):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = mla.chunk_attend(_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"],
                           inp["n_k"], inp["scale"], out_dtype=out_dtype, causal=causal)
    torch.cuda.synchronize()
    return np64(out)


def _chunks(n_q, n_k, causal):
    q_start, c = causal
    return (q_start + np.arange(n_q)) // c, np.arange(n_k) // c


def _oracle(wl, inp, causal):
    qc, kc = _chunks(wl.n_q, inp["n_k"], causal)
    return oracle.chunk_attend(np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(), np64(inp["w_uk"]),
                               np64(inp["w_uv"]), np64(inp["cache"]), inp["n_k"], inp["scale"],
                               split=wl.rope_split, theta=wl.theta, q_chunk=qc, k_chunk=kc)


def _oracle_rows(wl, inp, causal, rows):
    qc, kc = _chunks(wl.n_q, inp["n_k"], causal)
    return oracle.chunk_attend_rows(rows, np64(inp["q"]), np64(inp["q_r"]), inp["q_pos"].numpy(),
                                    np64(inp["w_uk"]), np64(inp["w_uv"]), np64(inp["cache"]), inp["n_k"],
                                    inp["scale"], split=wl.rope_split, theta=wl.theta, q_chunk=qc, k_chunk=kc)


# Every frame of the tiny sequence is a query: 4 chunks of 48 tokens, n_q = n_k = 192.
TINY_ALL = replace(synth.TINY, name="tiny_all", cache_frames=(), query_frames=tuple(range(8)))


def test_tiny_all_chunks_bf16():
    mla = need_gpu()
    inp = synth.attend_inputs(TINY_ALL, seed=0)
    causal = (0, 48)
    want = _oracle(TINY_ALL, inp, causal)
    assert_g1(_gpu(mla, TINY_ALL, inp, causal), want, "bf16")
    assert_g2(_gpu(mla, TINY_ALL, inp, causal, out_dtype=torch.float32), want, "bf16 f32-out",
              max_norm=G2_CAUSAL_MAX)


def test_tiny_all_chunks_fp32():
    mla = need_gpu()
    inp = synth.attend_inputs(TINY_ALL, seed=1, dtype=torch.float32)
    causal = (0, 48)
    assert_f32(_gpu(mla, TINY_ALL, inp, causal), _oracle(TINY_ALL, inp, causal), "fp32")


@pytest.mark.parametrize("d_c", [64, 128, 256])
def test_tiny_all_chunks_dc(d_c):
    mla = need_gpu()
    wl = TINY_ALL.with_dc(d_c)
    inp = synth.attend_inputs(wl, seed=2)
    causal = (0, 48)
    assert_g2(_gpu(mla, wl, inp, causal, out_dtype=torch.float32), _oracle(wl, inp, causal), f"dc{d_c}",
              max_norm=G2_CAUSAL_MAX)


@pytest.mark.parametrize("q_start,chunk_len", [(48, 50), (48, 37), (10, 64), (0, 1), (0, 192)])
def test_ragged_chunks(q_start, chunk_len):
    """Chunk boundaries off the 32-key blocks and 64-key tiles; q_start inside a chunk;
    chunk_len 1 (plain causal) and one chunk covering everything."""
    mla = need_gpu()
    n_k = 192
    wl = replace(synth.TINY, name="tiny_ragged", cache_frames=(), query_frames=tuple(range(8)))
    inp = synth.attend_inputs(wl, seed=3)
    n_q = n_k - q_start
    sub = dict(inp)
    sub["q"], sub["q_r"], sub["q_pos"] = inp["q"][:, :n_q], inp["q_r"][:, :n_q], inp["q_pos"][:n_q]
    causal = (q_start, chunk_len)
    qc, kc = (q_start + np.arange(n_q)) // chunk_len, np.arange(n_k) // chunk_len
    want = oracle.chunk_attend(np64(sub["q"]), np64(sub["q_r"]), sub["q_pos"].numpy(), np64(sub["w_uk"]),
                               np64(sub["w_uv"]), np64(sub["cache"]), n_k, sub["scale"], split=wl.rope_split,
                               theta=wl.theta, q_chunk=qc, k_chunk=kc)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in sub.items()}
    out = mla.chunk_attend(_dims(mla, wl), d["q"].contiguous(), d["q_r"].contiguous(), d["q_pos"].contiguous(),
                           d["w_uk"], d["w_uv"], d["cache"], n_k, sub["scale"], out_dtype=torch.float32,
                           causal=causal)
    torch.cuda.synchronize()
    assert_g2(np64(out), want, f"q_start={q_start} C={chunk_len}", max_norm=G2_CAUSAL_MAX)


def test_one_chunk_equals_unmasked_call():
    """q_start = n_k - n_q, chunk_len = n_q with n_k a multiple of n_q: every key is
    visible, so the causal entry point must give the unmasked result bit for bit."""
    mla = need_gpu()
    wl = synth.TINY
    inp = synth.attend_inputs(wl, seed=4)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (_dims(mla, wl), d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"], wl.n_k, wl.scale)
    a = mla.chunk_attend(*args, out_dtype=torch.float32)
    b = mla.chunk_attend(*args, out_dtype=torch.float32, causal=(wl.n_k - wl.n_q, wl.n_q))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_multi_block_stream_k():
    """108 row blocks of 256 rows over 36 key tiles: workgroups own partial ranges
    that cross row blocks, and tiles past a row block's last visible key are skipped."""
    mla = need_gpu()
    wl = replace(synth.TINY, name="mid_all", grid_hw=(12, 16), cache_frames=(), query_frames=tuple(range(12)))
    inp = synth.attend_inputs(wl, seed=5)
    causal = (0, 2 * 192)
    rows = np.array([[0, i, h] for h in (0, 11) for i in range(0, wl.n_q, 7)] + [[0, wl.n_q - 1, 5]])
    got = _gpu(mla, wl, inp, causal, out_dtype=torch.float32)
    assert_g2(got[rows[:, 0], rows[:, 1], rows[:, 2]], _oracle_rows(wl, inp, causal, rows), "mid f32-out",
              max_norm=G2_CAUSAL_MAX)
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("d_c", [64, 128, 256])
def test_multi_block_uneven_partition_dc(d_c):
    """The uneven (start-up unit) partition at every other latent width: row blocks
    see different numbers of key tiles, workgroups skip the start-up-only parts
    of row blocks, and the merge starts at each row block's first key-tile owner.
    d_c = 256 runs the single-role kernel with its 128-key tiles."""
    mla = need_gpu()
    wl = replace(synth.TINY, name="mid_all", grid_hw=(12, 16), cache_frames=(), query_frames=tuple(range(12)),
                 d_c=d_c)
    inp = synth.attend_inputs(wl, seed=14)
    causal = (0, 2 * 192)
    rows = np.array([[0, i, h] for h in (0, 7, 11) for i in range(0, wl.n_q, 23)] + [[0, wl.n_q - 1, 4]])
    got = _gpu(mla, wl, inp, causal, out_dtype=torch.float32)
    assert_g2(got[rows[:, 0], rows[:, 1], rows[:, 2]], _oracle_rows(wl, inp, causal, rows), f"mid dc{d_c}",
              max_norm=G2_CAUSAL_MAX)
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("headroom", ["0"])
def test_two_pass_fallback_causal(monkeypatch, headroom):
    mla = need_gpu()
    monkeypatch.setenv("MLA_ATTEND_HEADROOM", headroom)
    inp = synth.attend_inputs(TINY_ALL, seed=6)
    causal = (0, 48)
    assert_g2(_gpu(mla, TINY_ALL, inp, causal, out_dtype=torch.float32), _oracle(TINY_ALL, inp, causal),
              "two-pass", max_norm=G2_CAUSAL_MAX)


def test_480p_teacher_forcing_sampled_rows():
    """All 21 latent frames of the 480P sequence as queries in 7 chunks of 4680 tokens
    (n_q = n_k = 32760); rows sampled from every chunk."""
    mla = need_gpu()
    wl = replace(synth.WAN480P, name="wan480p_tf", cache_frames=(), query_frames=tuple(range(21)))
    inp = synth.attend_inputs(wl, seed=0)
    causal = (0, 4680)
    rng = np.random.default_rng(7)
    i = np.concatenate([rng.integers(c * 4680, (c + 1) * 4680, 6) for c in range(7)] + [[0, 4679, 4680, 32759]])
    rows = np.stack([np.zeros_like(i), i, rng.choice([0, 6, 11], i.size)], 1)
    got = _gpu(mla, wl, inp, causal, out_dtype=torch.float32)
    assert_g2(got[rows[:, 0], rows[:, 1], rows[:, 2]], _oracle_rows(wl, inp, causal, rows), "480p tf",
              max_norm=G2_CAUSAL_MAX)


@pytest.mark.parametrize("name,causal,uneven_rbs", [
    ("tiny_all", (0, 48), False),          # every row block holds a row of the last chunk
    ("mid_all", (0, 2 * 192), True),
    ("wan480p_tf", (0, 4680), True),
    ("wan480p", None, False),              # 220 row blocks: stream-K over 256 workgroups
    ("wan480p_shard8", None, False),       # 28 row blocks: up to 16 workgroups each
    ("wan480p_b8", None, False),           # 1760 row blocks fill 7 rounds: one workgroup each
])
def test_partition_header_matches_model(name, causal, uneven_rbs):
    """The attention kernel leaves its partition (U units, G workgroups) in the
    last 256 bytes of the workspace for the merge; the rounding model in
    tests/rounding_model.py splits row blocks the same way, so its U and G
    must be the kernel's: key tiles plus start-up units per row block when the
    row blocks see different numbers of tiles, else the plain partition."""
    import tests.rounding_model as rm
    mla = need_gpu()
    wl = {"tiny_all": TINY_ALL,
          "mid_all": replace(synth.TINY, name="mid_all", grid_hw=(12, 16), cache_frames=(),
                             query_frames=tuple(range(12))),
          "wan480p_tf": replace(synth.WAN480P, name="wan480p_tf", cache_frames=(),
                                query_frames=tuple(range(21)))}.get(name) or synth.WORKLOADS[name]
    inp = synth.attend_inputs(wl, seed=0)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    dims = _dims(mla, wl)
    ws = mla.alloc_workspace(dims, torch.bfloat16, wl.n_q, inp["n_k"], "cuda")
    ws.fill_(0xFF)
    mla.chunk_attend(dims, d["q"], d["q_r"], d["q_pos"], d["w_uk"], d["w_uv"], d["cache"], inp["n_k"],
                     inp["scale"], workspace=ws, causal=causal)
    torch.cuda.synchronize()
    tail = ws.view(torch.uint8)[-256:-240].cpu().numpy()
    U, = tail[:8].view(np.int64)
    G, per_block = tail[8:16].view(np.int32)

    kv = rm.kv_of_rows(wl.n_q, wl.n_heads, inp["n_k"], causal)
    rb_per_b = -(-kv.size // rm.ROWS_PER_BLOCK)
    bn = rm.latent_tile(wl.d_c)
    tiles = [-(-int(kv[r * rm.ROWS_PER_BLOCK:(r + 1) * rm.ROWS_PER_BLOCK].max()) // bn) for r in range(rb_per_b)]
    uneven = any(t != -(-inp["n_k"] // bn) for t in tiles)
    assert uneven == uneven_rbs
    want_U, want_G = rm.partition_size(tiles * wl.batch, spread=uneven)
    assert (int(U), int(G), int(per_block)) == (want_U, want_G, int(uneven))
    segs = rm.split_units(tiles * wl.batch, spread=uneven)
    assert all(sorted(t for a, b in sg for t in range(a, b)) == list(range(n)) for sg, n in zip(segs, tiles))
