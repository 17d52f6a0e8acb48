"""A rolling rollout through the ring cache on the GPU: every chunk is
appended into the slots mla_ring_current hands out (twice, as two denoising
steps), attended over [0, n_k), and committed.

The oracle never sees the ring: it rebuilds the visible key set in chunk
order -- the sink chunk, the most recent window chunks, the current chunk --
from its own append of those chunks' hidden states, and runs plain attention
over it.  A wrong slot, a stale chunk or a wrong n_k changes the keys and
fails the comparison; key order does not matter to softmax (pinned in
tests/test_oracle.py), which is why the ring may keep them in slot order.
"""

import numpy as np
import pytest
import torch

import oracle
from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import G2_CAUSAL_MAX, G2_MAX, assert_g2, need_gpu, np64

pytestmark = pytest.mark.gpu

GRID = (4, 6)
FRAMES_PER_CHUNK = 2
C = GRID[0] * GRID[1] * FRAMES_PER_CHUNK          # 48 tokens per chunk
SINK, WINDOW, CHUNKS = 1, 2, 7


def _max_gate(n_k):
    """The fp32-output max gate for a step over n_k keys: G2_MAX was derived
    at 148-key shapes; the first steps of a rollout see one or two 48-key
    chunks, the short-key case of G2_CAUSAL_MAX (bf16 roundings of q~ and P
    averaged over few keys; derivation in tests/gpu_util.py)."""
    return G2_MAX if n_k >= 148 else G2_CAUSAL_MAX


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


def test_rolling_rollout_matches_oracle():
    mla = need_gpu()
    dims = mla.Dims(batch=1)
    ring = mla.Ring(C, SINK, WINDOW)
    cap = ring.capacity
    rng = np.random.default_rng(11)
    D, H, dh, dc, dr = 1536, 12, 128, 192, 32
    w_dkv = _bf16(rng.standard_normal((dc, D), np.float32) / np.sqrt(D))
    w_kr = _bf16(rng.standard_normal((dr, D), np.float32) / np.sqrt(D))
    w_uk = _bf16(rng.standard_normal((H, dh, dc), np.float32) / np.sqrt(dc))
    w_uv = _bf16(rng.standard_normal((H, dh, dc), np.float32) / np.sqrt(dc))
    scale = 1.0 / np.sqrt(dh + dr)
    cache = torch.zeros((1, cap, dc + dr), dtype=torch.bfloat16, device="cuda")
    dev = lambda t: t.cuda()
    rows_of = {}                                   # chunk -> oracle cache rows (fp64 of the bf16 rounding)
    for j in range(CHUNKS):
        off, n_k = ring.current()
        pos = torch.from_numpy(synth.chunk_positions(range(FRAMES_PER_CHUNK * j, FRAMES_PER_CHUNK * (j + 1)), GRID))
        q = _bf16(rng.standard_normal((1, C, H, dh), np.float32))
        q_r = _bf16(rng.standard_normal((1, C, H, dr), np.float32))
        for step in range(2):                      # two denoising steps overwrite the same slots
            x = _bf16(rng.standard_normal((1, C, D), np.float32))
            mla.cache_append(dims, dev(x), dev(w_dkv), dev(w_kr), dev(pos), cache, off)
            out = mla.chunk_attend(dims, dev(q), dev(q_r), dev(pos), dev(w_uk), dev(w_uv), cache, n_k, scale,
                                   out_dtype=torch.float32)
            torch.cuda.synchronize()
            rows_of[j] = oracle.bf16_rne(oracle.latent_rows(np64(x), np64(w_dkv), np64(w_kr), pos.numpy()))[0]
            # the visible set in chunk order: sinks, the last WINDOW committed chunks, the current chunk
            visible = sorted(set(range(min(SINK, j + 1))) | set(range(max(SINK, j - WINDOW), j + 1)))
            keys = np.concatenate([rows_of[c] for c in visible], 0)[None]
            assert n_k == keys.shape[1], (j, n_k, visible)
            want = oracle.chunk_attend(np64(q), np64(q_r), pos.numpy(), np64(w_uk), np64(w_uv), keys, n_k, scale)
            assert_g2(np64(out), want, f"chunk {j} step {step}", max_norm=_max_gate(n_k))
        # the ring's slot map says where each chunk is; its rows must be there
        slots = ring.slot_chunks()
        got_cache = np64(cache)[0]
        for s, c in enumerate(slots):
            if c >= 0:
                np.testing.assert_allclose(got_cache[s * C:(s + 1) * C], rows_of[c], rtol=1e-2, atol=1e-2,
                                           err_msg=f"slot {s} should hold chunk {c}")
        ring.commit()
    assert ring.current()[1] == cap                 # the window is full: every slot is live


def test_samples_at_different_rollout_positions():
    """Per-sample lengths: each sample keeps its own ring over its slice of
    one [B, capacity, d_c + d_r] cache and is attended by its own call with
    its own n_k (samples are independent, so a batch of rollouts at
    different chunk indices needs no batched call).  Sample 0 rolls six
    chunks while sample 1 rolls three, interleaved step by step."""
    mla = need_gpu()
    dims = mla.Dims(batch=1)
    rings = [mla.Ring(C, SINK, WINDOW), mla.Ring(C, SINK, WINDOW)]
    cap = rings[0].capacity
    rng = np.random.default_rng(12)
    D, H, dh, dc, dr = 1536, 12, 128, 192, 32
    w_dkv = _bf16(rng.standard_normal((dc, D), np.float32) / np.sqrt(D)).cuda()
    w_kr = _bf16(rng.standard_normal((dr, D), np.float32) / np.sqrt(D)).cuda()
    w_uk = _bf16(rng.standard_normal((H, dh, dc), np.float32) / np.sqrt(dc))
    w_uv = _bf16(rng.standard_normal((H, dh, dc), np.float32) / np.sqrt(dc))
    scale = 1.0 / np.sqrt(dh + dr)
    cache = torch.zeros((2, cap, dc + dr), dtype=torch.bfloat16, device="cuda")
    rows_of = [{}, {}]
    n_chunks = [6, 3]
    for j in range(max(n_chunks)):
        for b in range(2):
            if j >= n_chunks[b]:
                continue
            ring = rings[b]
            off, n_k = ring.current()
            pos = torch.from_numpy(synth.chunk_positions(range(FRAMES_PER_CHUNK * j, FRAMES_PER_CHUNK * (j + 1)), GRID))
            x = _bf16(rng.standard_normal((1, C, D), np.float32))
            q = _bf16(rng.standard_normal((1, C, H, dh), np.float32))
            q_r = _bf16(rng.standard_normal((1, C, H, dr), np.float32))
            mine = cache[b:b + 1]                   # this sample's slots, contiguous
            mla.cache_append(dims, x.cuda(), w_dkv, w_kr, pos.cuda(), mine, off)
            out = mla.chunk_attend(dims, q.cuda(), q_r.cuda(), pos.cuda(), w_uk.cuda(), w_uv.cuda(), mine, n_k, scale,
                                   out_dtype=torch.float32)
            torch.cuda.synchronize()
            rows_of[b][j] = oracle.bf16_rne(oracle.latent_rows(np64(x), np64(w_dkv.cpu()), np64(w_kr.cpu()),
                                                               pos.numpy()))[0]
            visible = sorted(set(range(min(SINK, j + 1))) | set(range(max(SINK, j - WINDOW), j + 1)))
            keys = np.concatenate([rows_of[b][c] for c in visible], 0)[None]
            assert n_k == keys.shape[1], (b, j, n_k, visible)
            want = oracle.chunk_attend(np64(q), np64(q_r), pos.numpy(), np64(w_uk), np64(w_uv), keys, n_k, scale)
            assert_g2(np64(out), want, f"sample {b} chunk {j}", max_norm=_max_gate(n_k))
            ring.commit()
    assert rings[0].committed == 6 and rings[1].committed == 3


def test_checkpoint_and_resume_is_exact():
    """Seven chunk steps straight against three steps, a checkpoint of the ring
    state and the cache bytes, a fresh ring and cache restored from it, and four
    more steps: every output and the final cache agree bit for bit (the
    long-rollout cache of the VideoMLA arXiv abstract, resumed mid-rollout)."""
    mla = need_gpu()
    dims = mla.Dims(batch=1)
    rng = np.random.default_rng(21)
    D, H, dh, dc, dr = 1536, 12, 128, 192, 32
    w_dkv = _bf16(rng.standard_normal((dc, D), np.float32) / np.sqrt(D)).cuda()
    w_kr = _bf16(rng.standard_normal((dr, D), np.float32) / np.sqrt(D)).cuda()
    w_uk = _bf16(rng.standard_normal((H, dh, dc), np.float32) / np.sqrt(dc)).cuda()
    w_uv = _bf16(rng.standard_normal((H, dh, dc), np.float32) / np.sqrt(dc)).cuda()
    scale = 1.0 / np.sqrt(dh + dr)
    steps = []
    for j in range(CHUNKS):
        pos = torch.from_numpy(synth.chunk_positions(range(FRAMES_PER_CHUNK * j, FRAMES_PER_CHUNK * (j + 1)), GRID))
        steps.append(tuple(t.cuda() for t in (_bf16(rng.standard_normal((1, C, D), np.float32)),
                                              _bf16(rng.standard_normal((1, C, H, dh), np.float32)),
                                              _bf16(rng.standard_normal((1, C, H, dr), np.float32)), pos)))

    def run(ring, cache, chunks):
        outs = []
        for j in chunks:
            x, q, q_r, pos = steps[j]
            off, n_k = ring.current()
            mla.cache_append(dims, x, w_dkv, w_kr, pos, cache, off)
            outs.append(mla.chunk_attend(dims, q, q_r, pos, w_uk, w_uv, cache, n_k, scale))
            ring.commit()
        torch.cuda.synchronize()
        return outs

    ring = mla.Ring(C, SINK, WINDOW)
    cache = torch.zeros((1, ring.capacity, dc + dr), dtype=torch.bfloat16, device="cuda")
    straight = run(ring, cache, range(CHUNKS))

    ring_a = mla.Ring(C, SINK, WINDOW)
    cache_a = torch.zeros_like(cache)
    first = run(ring_a, cache_a, range(3))
    saved_state, saved_bytes = ring_a.state(), cache_a.cpu().view(torch.int16).clone()
    del ring_a, cache_a
    ring_b = mla.Ring.from_state(saved_state)
    cache_b = saved_bytes.view(torch.bfloat16).cuda()
    rest = run(ring_b, cache_b, range(3, CHUNKS))
    for j, (a, b) in enumerate(zip(straight, first + rest)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"chunk {j}"
    assert torch.equal(cache.view(torch.int16), cache_b.view(torch.int16))
    assert ring_b.state() == ring.state()
