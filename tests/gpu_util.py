"""Helpers shared by the GPU parity tests (comparison metrics only)."""

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    from latent_kv_cache_chunk_amd import mla  # noqa: F401  (fails loudly if the library is missing)
    return mla


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def errors(got: np.ndarray, want: np.ndarray) -> dict:
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    rms = float(np.sqrt(np.mean(np.square(want))))
    return dict(max_abs=float(d.max()), mean_abs=float(d.mean()), rms_ref=rms,
                max_norm=float(d.max() / rms), mean_norm=float(d.mean() / rms))


# Gates on chunk attention output (see the test docstrings for the reasoning):
#   G1 raw absolute error of the bf16 output on unit-scale values
G1_MAX, G1_MEAN = 2e-2, 2e-3
#   G2 error of the fp32-output path divided by the RMS of the reference output.
#   Mean 2e-3.  Max 3e-2: emulating in fp64 only the roundings any bf16 MFMA
#   path must make (absorbed query and P rounded once to bf16, L in fp32)
#   gives normalised max errors of 0.010-0.016 against the oracle with the
#   exact running max and 0.015-0.021 with the first-block reference max the
#   kernel uses (rows dominated by one key no longer get p = 1 exactly), at
#   148-key shapes for d_c 64 and 192 over three seeds; mean errors 1.5-1.7e-3
#   either way.
G2_MAX, G2_MEAN = 3e-2, 2e-3
#   Chunk-causal calls include rows that see only one chunk (down to a single
#   key), where the bf16 roundings of q~ and P are not averaged over many keys.
#   The same fp64 emulation on the tiny causal shapes (chunk 1, 48, 50; three
#   seeds) gives normalised max errors of 0.019-0.041 and means of
#   1.25-1.65e-3, so the max gate for these calls is 5e-2 (mean unchanged).
G2_CAUSAL_MAX = 5e-2
#   fp32 inputs, fp32 output, divided by the RMS of the reference output
F32_MAX, F32_MEAN = 1e-4, 1e-5


def assert_g1(got, want, label=""):
    e = errors(got, want)
    assert np.all(np.isfinite(got)), label
    assert e["max_abs"] <= G1_MAX and e["mean_abs"] <= G1_MEAN, (label, e)
    return e


def assert_g2(got, want, label="", max_norm=G2_MAX):
    e = errors(got, want)
    assert np.all(np.isfinite(got)), label
    assert e["max_norm"] <= max_norm and e["mean_norm"] <= G2_MEAN, (label, e)
    return e


def assert_f32(got, want, label=""):
    e = errors(got, want)
    assert np.all(np.isfinite(got)), label
    assert e["max_norm"] <= F32_MAX and e["mean_norm"] <= F32_MEAN, (label, e)
    return e
