"""Pins for the fp64 oracle: it is checked against things other than itself.

Each test names what fixes the expected value: a fixture of numbers the pages
print, a hand-derived closed form, an invariant of the mathematics, a library
routine for a textbook special case, or brute force on tiny inputs.  The last
group plants plausible mistakes into copies of oracle functions (on the CPU)
and checks that some pin catches each one.
"""

import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_oracle
from latent_kv_cache_chunk_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Cache footprint: the one set of numbers the pages print.
# --------------------------------------------------------------------------

def test_cache_row_footprint_matches_pages():
    g = _golden("cache_footprint.json")
    rng = np.random.default_rng(0)
    d_model = 16
    x = rng.standard_normal((1, 3, d_model))
    rows = oracle.latent_rows(x, rng.standard_normal((g["d_c"], d_model)),
                              rng.standard_normal((g["d_r"], d_model)),
                              np.zeros((3, 3), np.int32))
    assert rows.shape[-1] == g["latent_scalars_per_token"]
    assert 2 * g["n_heads"] * g["head_dim"] == g["dense_scalars_per_token"]
    reduction = 100.0 * (1 - rows.shape[-1] / g["dense_scalars_per_token"])
    assert round(reduction, 1) == g["reduction_percent_printed"]


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def test_bf16_hand_cases():
    for case in _golden("hand_cases.json")["bf16_rne"]:
        v = float.fromhex(case["in_hex"])
        want = float.fromhex(case["out_hex"])
        got = float(oracle.bf16_rne(np.array([v]))[0])
        assert got == want, case["why"]


def test_bf16_matches_torch_on_fp32_exact_values():
    # For values already exact in fp32 there is no double rounding, so torch's
    # fp32 -> bf16 conversion (round to nearest even) is an independent check.
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-36).astype(np.float32),   # near / below min normal
        np.float32([0.0, -0.0, 1.0, -2.0, 3.3895314e38]),
    ])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_rne(v.astype(np.float64))
    assert np.array_equal(got, want)


def _int_rne_bf16_scaled(n: int, frac_bits: int) -> float:
    """bf16 value of n * 2**-frac_bits by integer arithmetic (independent of frexp)."""
    if n == 0:
        return 0.0
    sign = -1 if n < 0 else 1
    a = abs(n)
    shift = a.bit_length() - 8
    if shift <= 0:
        return sign * a / 2.0 ** frac_bits
    q, r = divmod(a, 1 << shift)
    half = 1 << (shift - 1)
    if r > half or (r == half and q & 1):
        q += 1
    return sign * (q << shift) / 2.0 ** frac_bits


def test_bf16_bits_roundtrip():
    v = oracle.bf16_rne(np.random.default_rng(2).standard_normal(1000))
    bits = oracle.bf16_bits(v)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, v)
    with pytest.raises(ValueError):
        oracle.bf16_bits(np.array([1.0 + 2.0 ** -20]))


# --------------------------------------------------------------------------
# 3D RoPE
# --------------------------------------------------------------------------

def test_rope_angles_at_unit_positions():
    g = _golden("hand_cases.json")["rope_unit_position_angles"]
    a = oracle.rope3d_angles(np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1]]), g["split"], g["theta"])
    np.testing.assert_allclose(a[0, :4], g["t_axis_pos1"], rtol=1e-14)
    assert np.all(a[0, 4:] == 0)
    np.testing.assert_allclose(a[1, 4:10], g["h_axis_pos1"], rtol=1e-14)
    assert np.all(a[1, :4] == 0) and np.all(a[1, 10:] == 0)
    np.testing.assert_allclose(a[2, 10:16], g["w_axis_pos1"], rtol=1e-14)


def test_rope_identity_at_origin_and_norm():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((50, 32))
    assert np.array_equal(oracle.rope3d(v, np.zeros((50, 3), np.int32)), v)
    pos = rng.integers(0, 300, size=(50, 3))
    r = oracle.rope3d(v, pos)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-14)


def test_rope_equals_complex_rotation():
    # Each pair (x0, x1) read as x0 + i x1 is multiplied by e^{i a}.
    rng = np.random.default_rng(4)
    split = (8, 12, 12)
    v = rng.standard_normal(32)
    pos = (5, 17, 29)
    got = oracle.rope3d(v, np.array(pos))
    want = []
    for axis, width in enumerate(split):
        for i in range(width // 2):
            ang = pos[axis] * 10 ** (-8.0 * i / width)   # 1e4^(-2i/width)
            k = sum(split[:axis]) + 2 * i
            z = complex(v[k], v[k + 1]) * cmath.exp(1j * ang)
            want += [z.real, z.imag]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_rope_scores_depend_on_position_difference_only():
    rng = np.random.default_rng(5)
    a, b = rng.standard_normal((2, 40, 32))
    p = rng.integers(0, 100, size=(40, 3))
    p2 = rng.integers(0, 100, size=(40, 3))
    shift = np.array([7, 3, 11])
    s1 = np.sum(oracle.rope3d(a, p) * oracle.rope3d(b, p2), -1)
    s2 = np.sum(oracle.rope3d(a, p + shift) * oracle.rope3d(b, p2 + shift), -1)
    np.testing.assert_allclose(s1, s2, rtol=1e-10, atol=1e-10)


# --------------------------------------------------------------------------
# Cache append
# --------------------------------------------------------------------------

def test_append_exact_tier_integer_closed_form():
    wl = synth.TINY                                  # D = 1536: ~10% of values exceed 4
    inp = synth.append_inputs_exact(wl, seed=0)
    x = inp["x"].double().numpy()
    w_dkv = inp["w_dkv"].double().numpy()
    w_kr = inp["w_kr"].double().numpy()
    xi = np.rint(x).astype(np.int64)
    w_all = np.concatenate([w_dkv, w_kr], 0)
    wi = np.rint(w_all * 64).astype(np.int64)
    n_int = xi @ wi.T                                # exact integer sums, units of 2**-6
    want = np.vectorize(lambda n: _int_rne_bf16_scaled(int(n), 6))(n_int)
    cap = wl.n_q + 10
    cache0 = np.full((1, cap, 224), 7.0)
    got = oracle.cache_append(cache0, x, w_dkv, w_kr, inp["pos"].numpy(), offset=5)
    assert np.array_equal(got[:, 5:5 + wl.n_q], want)
    assert np.all(got[:, :5] == 7.0) and np.all(got[:, 5 + wl.n_q:] == 7.0)
    assert np.any(np.abs(want) > 4)                # rounding actually happens
    assert np.any(want != n_int / 64.0)


def test_append_rotates_only_positional_part():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 4, 24))
    w_dkv = rng.standard_normal((12, 24))
    w_kr = rng.standard_normal((6, 24))
    pos = rng.integers(0, 9, size=(4, 3))
    rows = oracle.latent_rows(x, w_dkv, w_kr, pos, split=(2, 2, 2))
    np.testing.assert_allclose(rows[..., :12], np.einsum("bnd,cd->bnc", x, w_dkv), rtol=1e-12)
    kr = np.einsum("bnd,rd->bnr", x, w_kr)
    for n in range(4):
        for k, (axis, i) in enumerate([(0, 0), (1, 0), (2, 0)]):
            z = complex(kr[0, n, 2 * k], kr[0, n, 2 * k + 1]) * cmath.exp(1j * pos[n, axis])
            assert abs(rows[0, n, 12 + 2 * k] - z.real) < 1e-12
            assert abs(rows[0, n, 12 + 2 * k + 1] - z.imag) < 1e-12


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _tiny_problem(seed=7, H=2, d_h=4, d_c=3, split=(2, 2, 2), n_q=3, n_k=5, B=1, scale=0.37):
    rng = np.random.default_rng(seed)
    d_r = sum(split)
    return dict(
        q=rng.standard_normal((B, n_q, H, d_h)),
        q_r=rng.standard_normal((B, n_q, H, d_r)),
        q_pos=rng.integers(0, 6, size=(n_q, 3)),
        w_uk=rng.standard_normal((H, d_h, d_c)),
        w_uv=rng.standard_normal((H, d_h, d_c)),
        cache=rng.standard_normal((B, n_k + 2, d_c + d_r)),
        n_k=n_k, scale=scale, split=split,
    )


def _brute_force(p, q_chunk=None, k_chunk=None, theta=1e4):
    """Scalar loops over Python floats; RoPE via complex multiplication."""
    q, q_r, w_uk, w_uv, cache = (p[k].tolist() for k in ("q", "q_r", "w_uk", "w_uv", "cache"))
    split, scale, n_k = p["split"], p["scale"], p["n_k"]
    B, n_q, H, d_h = p["q"].shape
    d_c = p["w_uk"].shape[-1]
    out = np.zeros((B, n_q, H, d_h))
    for b in range(B):
        for i in range(n_q):
            for h in range(H):
                qr = q_r[b][i][h]
                rot = []
                off = 0
                for axis, width in enumerate(split):
                    for k in range(width // 2):
                        ang = float(p["q_pos"][i][axis]) * theta ** (-2.0 * k / width)
                        z = complex(qr[off + 2 * k], qr[off + 2 * k + 1]) * cmath.exp(1j * ang)
                        rot += [z.real, z.imag]
                    off += width
                scores, vals = [], []
                for j in range(n_k):
                    if q_chunk is not None and k_chunk[j] > q_chunk[i]:
                        continue
                    c = cache[b][j][:d_c]
                    kr = cache[b][j][d_c:]
                    kc = [sum(w_uk[h][d][cc] * c[cc] for cc in range(d_c)) for d in range(d_h)]
                    s = sum(q[b][i][h][d] * kc[d] for d in range(d_h))
                    s += sum(rot[r] * kr[r] for r in range(len(kr)))
                    scores.append(scale * s)
                    vals.append([sum(w_uv[h][d][cc] * c[cc] for cc in range(d_c)) for d in range(d_h)])
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                tot = sum(e)
                for d in range(d_h):
                    out[b, i, h, d] = sum(e[j] * vals[j][d] for j in range(len(e))) / tot
    return out


def _oracle(p, **kw):
    return oracle.chunk_attend(p["q"], p["q_r"], p["q_pos"], p["w_uk"], p["w_uv"], p["cache"],
                               p["n_k"], p["scale"], split=p["split"], **kw)


def test_attend_matches_brute_force():
    for seed in range(3):
        p = _tiny_problem(seed=seed, B=2)
        np.testing.assert_allclose(_oracle(p), _brute_force(p), rtol=1e-12, atol=1e-13)


def test_attend_block_causal_matches_brute_force():
    p = _tiny_problem(seed=11, n_q=4, n_k=6)
    qc = [0, 0, 1, 1]
    kc = [0, 0, 0, 1, 1, 2]          # key of chunk 2 is never visible
    np.testing.assert_allclose(_oracle(p, q_chunk=qc, k_chunk=kc),
                               _brute_force(p, q_chunk=qc, k_chunk=kc), rtol=1e-12, atol=1e-13)


def _absorbed(p):
    """Absorbed form: fold w_uk into the query, attend over the latent, up-project after."""
    d_c = p["w_uk"].shape[-1]
    n_k = p["n_k"]
    c = p["cache"][:, :n_k, :d_c]
    kr = p["cache"][:, :n_k, d_c:]
    qrr = oracle.rope3d(p["q_r"], p["q_pos"][None, :, None, :], p["split"])
    qt = np.einsum("bihd,hdc->bihc", p["q"], p["w_uk"])
    s = p["scale"] * (np.einsum("bihc,bjc->bhij", qt, c) + np.einsum("bihr,bjr->bhij", qrr, kr))
    s -= s.max(-1, keepdims=True)
    e = np.exp(s)
    e /= e.sum(-1, keepdims=True)
    lat = np.einsum("bhij,bjc->bihc", e, c)
    return np.einsum("bihc,hdc->bihd", lat, p["w_uv"])


def test_absorbed_equals_non_absorbed():
    p = _tiny_problem(seed=12, H=3, d_h=16, d_c=8, split=(8, 12, 12), n_q=9, n_k=40, B=2)
    np.testing.assert_allclose(_oracle(p), _absorbed(p), rtol=1e-11, atol=1e-12)


def test_rows_are_probability_distributions():
    rng = np.random.default_rng(13)
    s = rng.standard_normal((20, 50)) * 10
    vis = rng.random((20, 50)) < 0.7
    vis[:, 0] = True
    pr = oracle.attention_probs(s, vis)
    assert np.all(pr >= 0)
    assert np.all(pr[~vis] == 0)
    np.testing.assert_allclose(pr.sum(-1), 1.0, rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_values():
    p = _tiny_problem(seed=14, H=2, d_h=8, d_c=6, n_q=4, n_k=9)
    p["q"][:] = 0
    p["q_r"][:] = 0
    c_mean = p["cache"][0, :p["n_k"], :6].mean(0)
    want = np.einsum("hdc,c->hd", p["w_uv"], c_mean)
    got = _oracle(p)[0]
    for i in range(4):
        np.testing.assert_allclose(got[i], want, rtol=1e-12, atol=1e-13)


def test_two_keys_logit_gap_ln3():
    g = _golden("hand_cases.json")["two_key_softmax"]
    scale = 0.5
    p = dict(q=np.array([[[[math.log(3.0) / scale]]]]),     # d_h = 1
             q_r=np.zeros((1, 1, 1, 2)), q_pos=np.zeros((1, 3), np.int64),
             w_uk=np.ones((1, 1, 1)), w_uv=np.ones((1, 1, 1)),
             cache=np.array([[[1.0, 0.3, -0.2], [0.0, 0.5, 0.1]]]),
             n_k=2, scale=scale, split=(2, 0, 0))
    got = _oracle(p)[0, 0, 0, 0]
    assert abs(got - g["weights"][0] * 1.0 - g["weights"][1] * 0.0) < 1e-14


def test_dominant_key_takes_all_weight():
    p = _tiny_problem(seed=15, n_q=2, n_k=7)
    p["q_r"][:] = 0
    # make key 4's content align strongly with every query of head 0
    d_c = p["w_uk"].shape[-1]
    p["cache"][0, 4, :d_c] *= 10.0
    for i in range(2):
        kvec = p["w_uk"][0] @ p["cache"][0, 4, :d_c]
        p["q"][0, i, 0] = 200.0 * kvec / (p["scale"] * kvec @ kvec)
    got = _oracle(p)[0, :, 0]
    want = p["w_uv"][0] @ p["cache"][0, 4, :d_c]
    np.testing.assert_allclose(got, np.stack([want, want]), rtol=1e-9, atol=1e-9)


def test_key_order_does_not_matter():
    p = _tiny_problem(seed=16, n_q=4, n_k=12, B=2)
    perm = np.random.default_rng(0).permutation(12)
    p2 = dict(p)
    p2["cache"] = p["cache"].copy()
    p2["cache"][:, :12] = p["cache"][:, perm]
    np.testing.assert_allclose(_oracle(p), _oracle(p2), rtol=1e-12, atol=1e-13)


def test_matches_torch_sdpa_on_reconstructed_kv():
    p = _tiny_problem(seed=17, H=3, d_h=16, d_c=12, split=(8, 12, 12), n_q=10, n_k=33, B=2)
    t = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in p.items()
         if k in ("q", "q_r", "w_uk", "w_uv", "cache")}
    d_c, n_k = 12, p["n_k"]
    c = t["cache"][:, :n_k, :d_c]
    kr = t["cache"][:, :n_k, d_c:]
    k_content = torch.einsum("bjc,hdc->bhjd", c, t["w_uk"])
    v = torch.einsum("bjc,hdc->bhjd", c, t["w_uv"])
    k = torch.cat([k_content, kr[:, None].expand(-1, 3, -1, -1)], -1)
    qrr = torch.from_numpy(oracle.rope3d(p["q_r"], p["q_pos"][None, :, None, :]))
    qq = torch.cat([t["q"], qrr], -1).permute(0, 2, 1, 3)
    want = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=p["scale"])
    np.testing.assert_allclose(_oracle(p), want.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


def test_block_causal_equals_sequential_chunk_steps():
    rng = np.random.default_rng(18)
    H, d_h, d_c, n = 2, 8, 6, 5
    p = dict(q=rng.standard_normal((1, 3 * n, H, d_h)), q_r=rng.standard_normal((1, 3 * n, H, 32)),
             q_pos=rng.integers(0, 20, size=(3 * n, 3)), w_uk=rng.standard_normal((H, d_h, d_c)),
             w_uv=rng.standard_normal((H, d_h, d_c)), cache=rng.standard_normal((1, 3 * n, d_c + 32)),
             n_k=3 * n, scale=0.3, split=(8, 12, 12))
    chunk = np.repeat(np.arange(3), n)
    multi = _oracle(p, q_chunk=chunk, k_chunk=chunk)
    for c in range(3):
        step = oracle.chunk_attend(p["q"][:, c * n:(c + 1) * n], p["q_r"][:, c * n:(c + 1) * n],
                                   p["q_pos"][c * n:(c + 1) * n], p["w_uk"], p["w_uv"], p["cache"],
                                   (c + 1) * n, p["scale"])
        np.testing.assert_allclose(multi[:, c * n:(c + 1) * n], step, rtol=1e-12, atol=1e-13)


def test_selected_rows_match_full_output():
    p = _tiny_problem(seed=19, H=3, d_h=8, d_c=6, split=(8, 12, 12), n_q=7, n_k=20, B=2)
    full = _oracle(p)
    rows = np.array([[0, 0, 0], [1, 6, 2], [0, 3, 1], [1, 3, 1]])
    got = oracle.chunk_attend_rows(rows, p["q"], p["q_r"], p["q_pos"], p["w_uk"], p["w_uv"],
                                   p["cache"], p["n_k"], p["scale"])
    np.testing.assert_allclose(got, full[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-13)


def test_selected_rows_match_full_output_block_causal():
    # row sampling must apply the same chunk-causal mask as the full output
    p = _tiny_problem(seed=21, H=2, d_h=8, d_c=6, split=(8, 12, 12), n_q=9, n_k=12, B=1)
    q_chunk = (3 + np.arange(9)) // 4          # queries are tokens 3..11 in chunks of 4
    k_chunk = np.arange(12) // 4
    full = oracle.chunk_attend(p["q"], p["q_r"], p["q_pos"], p["w_uk"], p["w_uv"], p["cache"], p["n_k"],
                               p["scale"], q_chunk=q_chunk, k_chunk=k_chunk)
    rows = np.array([[0, 0, 0], [0, 8, 1], [0, 4, 1], [0, 5, 0]])
    got = oracle.chunk_attend_rows(rows, p["q"], p["q_r"], p["q_pos"], p["w_uk"], p["w_uv"], p["cache"],
                                   p["n_k"], p["scale"], q_chunk=q_chunk, k_chunk=k_chunk)
    np.testing.assert_allclose(got, full[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-13)
    # and the mask is live: the unmasked rows differ
    open_rows = oracle.chunk_attend_rows(rows, p["q"], p["q_r"], p["q_pos"], p["w_uk"], p["w_uv"], p["cache"],
                                         p["n_k"], p["scale"])
    assert np.abs(open_rows - got).max() > 1e-3


def test_exponential_tilting_of_gaussian_latent():
    # With c ~ N(0, I) and scores a.c, the softmax-weighted mean of c tends
    # to a (mean of the exponentially tilted Gaussian).  So O -> w_uv (alpha w_uk^T q).
    rng = np.random.default_rng(20)
    d_c, d_h, n_k = 4, 4, 400000
    w_uk = rng.standard_normal((1, d_h, d_c)) / 2
    w_uv = rng.standard_normal((1, d_h, d_c))
    q = rng.standard_normal((1, 1, 1, d_h))
    scale = 0.4
    cache = np.concatenate([rng.standard_normal((1, n_k, d_c)), np.zeros((1, n_k, 2))], -1)
    got = oracle.chunk_attend(q, np.zeros((1, 1, 1, 2)), np.zeros((1, 3), np.int64), w_uk, w_uv,
                              cache, n_k, scale, split=(2, 0, 0))[0, 0, 0]
    a = scale * (w_uk[0].T @ q[0, 0, 0])
    want = w_uv[0] @ a
    np.testing.assert_allclose(got, want, atol=0.03 * np.linalg.norm(want) + 0.01)


# --------------------------------------------------------------------------
# Dense per-head attention (the K/V cache the latent replaces)
# --------------------------------------------------------------------------

def _mha_problem(seed, B=2, n_q=3, n_k=5, H=2, d=4, dv=3, cap_extra=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, n_q, H, d)), rng.standard_normal((B, n_k + cap_extra, H, d)),
            rng.standard_normal((B, n_k + cap_extra, H, dv)), n_k)


def _mha_brute(q, k, v, n_k, scale, q_chunk=None, k_chunk=None):
    """Scalar loops over Python floats."""
    B, n_q, H, d = q.shape
    out = np.zeros((B, n_q, H, v.shape[-1]))
    for b in range(B):
        for i in range(n_q):
            for h in range(H):
                js = [j for j in range(n_k) if q_chunk is None or k_chunk[j] <= q_chunk[i]]
                sc = [scale * sum(float(q[b, i, h, e]) * float(k[b, j, h, e]) for e in range(d)) for j in js]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                for e in range(v.shape[-1]):
                    out[b, i, h, e] = sum(w[t] * float(v[b, js[t], h, e]) for t in range(len(js))) / sum(w)
    return out


def test_mha_matches_brute_force():
    for seed in range(3):
        q, k, v, n_k = _mha_problem(30 + seed)
        np.testing.assert_allclose(oracle.mha_attend(q, k, v, n_k, 0.41), _mha_brute(q, k, v, n_k, 0.41),
                                   rtol=1e-12, atol=1e-13)
    q, k, v, n_k = _mha_problem(33, n_q=4, n_k=6)
    qc, kc = [0, 0, 1, 1], [0, 0, 0, 1, 1, 2]
    np.testing.assert_allclose(oracle.mha_attend(q, k, v, n_k, 0.41, q_chunk=qc, k_chunk=kc),
                               _mha_brute(q, k, v, n_k, 0.41, q_chunk=qc, k_chunk=kc), rtol=1e-12, atol=1e-13)


def test_mha_matches_torch_sdpa():
    q, k, v, n_k = _mha_problem(34, B=2, n_q=9, n_k=31, H=3, d=16, dv=16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a[:, :n_k] if a is not q else a)).permute(0, 2, 1, 3)
    want = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.2)
    np.testing.assert_allclose(oracle.mha_attend(q, k, v, n_k, 0.2), want.permute(0, 2, 1, 3).numpy(),
                               rtol=1e-11, atol=1e-12)


def test_mha_zero_query_gives_mean_of_values():
    q, k, v, n_k = _mha_problem(35, n_k=11)
    got = oracle.mha_attend(np.zeros_like(q), k, v, n_k, 0.5)
    for i in range(q.shape[1]):
        np.testing.assert_allclose(got[:, i], v[:, :n_k].mean(1), rtol=1e-12, atol=1e-13)


def test_mha_on_reconstructed_kv_equals_latent_attention():
    """The non-absorbed MLA definition is dense attention over
    K_h = [C W_UK[h]^T || RoPE'd k_R] and V_h = C W_UV[h]^T."""
    p = _tiny_problem(seed=36, H=3, d_h=8, d_c=6, split=(8, 12, 12), n_q=5, n_k=17, B=2)
    d_c, n_k = 6, p["n_k"]
    c, kr = p["cache"][:, :, :d_c], p["cache"][:, :, d_c:]
    k = np.concatenate([np.einsum("bjc,hdc->bjhd", c, p["w_uk"]),
                        np.broadcast_to(kr[:, :, None], kr.shape[:2] + (3, kr.shape[-1]))], -1)
    v = np.einsum("bjc,hdc->bjhd", c, p["w_uv"])
    qq = np.concatenate([p["q"], oracle.rope3d(p["q_r"], p["q_pos"][None, :, None, :])], -1)
    np.testing.assert_allclose(oracle.mha_attend(qq, k, v, n_k, p["scale"]), _oracle(p), rtol=1e-11, atol=1e-12)


def test_mha_selected_rows_match_full_output():
    q, k, v, n_k = _mha_problem(37, B=2, n_q=6, n_k=13, H=3, d=8, dv=5)
    full = oracle.mha_attend(q, k, v, n_k, 0.3)
    rows = np.array([[0, 0, 0], [1, 5, 2], [0, 3, 1], [1, 2, 0]])
    np.testing.assert_allclose(oracle.mha_attend_rows(rows, q, k, v, n_k, 0.3),
                               full[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-13)


@pytest.mark.parametrize("mutation", ["kv_swapped", "keys_past_n_k", "head_mixed"])
def test_mha_planted_mistakes_are_caught(mutation):
    q, k, v, n_k = _mha_problem(38, B=1, n_q=3, n_k=5, H=2, d=4, dv=4)
    want = _mha_brute(q, k, v, n_k, 0.41)
    if mutation == "kv_swapped":
        got = oracle.mha_attend(q, v, k, n_k, 0.41)
    elif mutation == "keys_past_n_k":
        got = oracle.mha_attend(q, k, v, n_k + 2, 0.41)
    else:
        got = oracle.mha_attend(q, k[:, :, ::-1], v, n_k, 0.41)
    assert not np.allclose(got, want, rtol=1e-6, atol=1e-6), mutation


# --------------------------------------------------------------------------
# Planted mistakes: each one must be caught by a pin above.
# --------------------------------------------------------------------------

def _rope_sign_flipped(v, pos, split=(8, 12, 12), theta=1e4):
    a = oracle.rope3d_angles(pos, split, theta)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(np.broadcast_shapes(v.shape, a.shape[:-1] + (v.shape[-1],)))
    out[..., 0::2] = v[..., 0::2] * np.cos(a) + v[..., 1::2] * np.sin(a)
    out[..., 1::2] = -v[..., 0::2] * np.sin(a) + v[..., 1::2] * np.cos(a)
    return out


def _rope_half_freq(pos, split=(8, 12, 12), theta=1e4):
    parts = []
    for axis, width in enumerate(split):
        i = np.arange(width // 2, dtype=np.float64)
        parts.append(np.asarray(pos)[..., axis:axis + 1] * theta ** (-i / width))
    return np.concatenate(parts, -1)


@pytest.mark.parametrize("mutation", ["rope_sign", "rope_freq", "drop_positional", "uv_for_uk",
                                      "wrong_scale", "mask_ignored"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    p = _tiny_problem(seed=21, B=2, n_q=4, n_k=6, split=(8, 12, 12))
    p["q_pos"] = np.array([[3, 1, 2], [5, 4, 0], [1, 2, 3], [2, 3, 5]])
    qc, kc = [0, 0, 1, 1], [0, 0, 1, 1, 1, 2]
    want = _brute_force(p, q_chunk=qc, k_chunk=kc)
    if mutation == "rope_sign":
        monkeypatch.setattr(mla_oracle, "rope3d", _rope_sign_flipped)
    elif mutation == "rope_freq":
        monkeypatch.setattr(mla_oracle, "rope3d_angles", _rope_half_freq)
    elif mutation == "drop_positional":
        orig = mla_oracle._head_qkv
        monkeypatch.setattr(mla_oracle, "_head_qkv", lambda q, qr, wuk, wuv, c, kr, b, h:
                            orig(q, qr * 0, wuk, wuv, c, kr, b, h))
    elif mutation == "uv_for_uk":
        orig = mla_oracle._head_qkv
        monkeypatch.setattr(mla_oracle, "_head_qkv", lambda q, qr, wuk, wuv, c, kr, b, h:
                            orig(q, qr, wuv, wuv, c, kr, b, h))
    elif mutation == "wrong_scale":
        monkeypatch.setattr(mla_oracle, "attention_probs",
                            lambda s, visible=None: oracle.attention_probs(s / 0.37 * 0.5, visible))
    elif mutation == "mask_ignored":
        monkeypatch.setattr(mla_oracle, "_chunk_visibility", lambda qch, kch, nq, nk: None)
    got = mla_oracle.chunk_attend(p["q"], p["q_r"], p["q_pos"], p["w_uk"], p["w_uv"], p["cache"],
                                  p["n_k"], p["scale"], split=p["split"], q_chunk=qc, k_chunk=kc)
    assert not np.allclose(got, want, rtol=1e-6, atol=1e-6), mutation


def test_planted_bf16_truncation_is_caught():
    # Truncation instead of round-to-nearest-even must fail the hand cases.
    def trunc(v):
        v = np.asarray(v, np.float64)
        m, e = np.frexp(v)
        return np.ldexp(np.trunc(m * 256.0), e - 8)
    cases = _golden("hand_cases.json")["bf16_rne"]
    assert any(float(trunc(np.array([float.fromhex(c["in_hex"])]))[0]) != float.fromhex(c["out_hex"])
               for c in cases)
