"""Host-side tests of the C ABI: symbols, status codes, validation, planning.

None of these enqueue GPU work: every call here either is pure host logic or
fails validation before anything is launched, so they run without a GPU.
"""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

mla = pytest.importorskip("latent_kv_cache_chunk_amd.mla",
                          reason="libmla_hip.so not built (python -m latent_kv_cache_chunk_amd.build)")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = mla.raw()
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/mla.h but not exported"
    assert set(names) == set(mla.EXPORTED)


def test_exported_symbols_are_c_linkage():
    # nm on our own build output: the ABI symbols must be unmangled.
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in _declared_functions():
        assert n in syms


def test_status_strings_and_version():
    lib = mla.raw()
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(-1) == b"MLA_ERR_INVALID_ARG"
    assert lib.mla_status_string(-2) == b"MLA_ERR_UNSUPPORTED"
    assert lib.mla_status_string(-3) == b"MLA_ERR_WORKSPACE"
    assert lib.mla_status_string(-4) == b"MLA_ERR_HIP"
    assert lib.mla_status_string(17) == b"MLA_ERR_UNKNOWN"
    assert b"gfx950" in lib.mla_version()


def _dims(**kw):
    base = dict(batch=1, n_heads=12, head_dim=128, d_c=192, d_r=32, rope=(8, 12, 12), rope_theta=1e4)
    base.update(kw)
    return mla.Dims(**base).c()


def _ws(d, dt=0, n_q=48, n_k=192):
    return mla.raw().mla_chunk_attend_workspace_bytes(ctypes.byref(d), dt, n_q, n_k)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), -2), (dict(d_c=100), -2), (dict(d_c=320), -2), (dict(d_r=64, rope=(16, 24, 24)), -2),
    (dict(rope=(8, 12, 10)), -2), (dict(rope=(7, 13, 12)), -2), (dict(batch=0), -1), (dict(n_heads=0), -1),
    (dict(rope_theta=0.0), -1),
])
def test_invalid_dims_are_rejected(kw, code):
    assert _ws(_dims(**kw)) == code


def test_invalid_sizes_and_dtypes():
    d = _dims()
    assert _ws(d, n_q=0, n_k=10) == -1
    assert _ws(d, n_q=50, n_k=49) == -1          # the chunk's own keys are part of n_k
    assert _ws(d, dt=7) == -2
    assert mla.raw().mla_chunk_attend_workspace_bytes(None, 0, 48, 192) == -1


def test_workspace_plan_sizes():
    # 480P: 56160 rows -> 220 row-blocks of 256; 512 key tiles of 64; stream-K over 256 workgroups, whose
    # partial states take one slot per (workgroup, row block) pair: fewer than 256 + 220.
    d = _dims()
    n480 = _ws(d, 0, 4680, 32760)
    rows_pad = 220 * 256
    qt = rows_pad * 224 * 2
    slots = 256 + 220
    states = slots * 256 * (192 + 2) * 4
    units = (220 + 1) * 8
    assert n480 >= qt + states + units
    assert n480 < qt + states + units + 4096
    # fp32 variant: one slot per row-block
    n32 = _ws(d, 1, 48, 192)
    assert n32 >= 3 * 256 * 224 * 4 + 3 * 256 * 194 * 4


def test_calls_fail_validation_without_launching():
    lib = mla.raw()
    d = _dims()
    fake = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: validation fails first
    # null query pointer
    rc = lib.mla_chunk_attend(ctypes.byref(d), 0, 0, None, fake, fake, 48, fake, fake, fake, 192, 192,
                              ctypes.c_float(0.08), fake, fake, 1 << 40, None)
    assert rc == -1 and b"q is null" in lib.mla_last_error()
    # misaligned cache
    rc = lib.mla_chunk_attend(ctypes.byref(d), 0, 0, fake, fake, fake, 48, fake, fake, ctypes.c_void_p(0x10002),
                              192, 192, ctypes.c_float(0.08), fake, fake, 1 << 40, None)
    assert rc == -1 and b"aligned" in lib.mla_last_error()
    # n_k beyond capacity
    rc = lib.mla_chunk_attend(ctypes.byref(d), 0, 0, fake, fake, fake, 48, fake, fake, fake, 100, 192,
                              ctypes.c_float(0.08), fake, fake, 1 << 40, None)
    assert rc == -1 and b"capacity" in lib.mla_last_error()
    # workspace too small
    rc = lib.mla_chunk_attend(ctypes.byref(d), 0, 0, fake, fake, fake, 48, fake, fake, fake, 192, 192,
                              ctypes.c_float(0.08), fake, fake, 1024, None)
    assert rc == -3
    # bad scale
    rc = lib.mla_chunk_attend(ctypes.byref(d), 0, 0, fake, fake, fake, 48, fake, fake, fake, 192, 192,
                              ctypes.c_float(-1.0), fake, fake, 1 << 40, None)
    assert rc == -1
    # append: offset + n_new beyond capacity, bad d_model
    rc = lib.mla_cache_append(ctypes.byref(d), 0, fake, 1536, 48, fake, fake, fake, fake, 100, 60, None)
    assert rc == -1
    rc = lib.mla_cache_append(ctypes.byref(d), 0, fake, 1568, 48, fake, fake, fake, fake, 100, 0, None)
    assert rc == -2
    rc = lib.mla_cache_append(ctypes.byref(d), 0, fake, 1536, -1, fake, fake, fake, fake, 100, 0, None)
    assert rc == -1
    # append of zero tokens is a valid no-op (nothing enqueued)
    rc = lib.mla_cache_append(ctypes.byref(d), 0, fake, 1536, 0, fake, fake, fake, fake, 100, 100, None)
    assert rc == 0
    # steps share the size checks
    assert lib.mla_latent_attend(ctypes.byref(d), 0, fake, 100, 48, 192, fake, 1 << 40, None) == -1
    assert lib.mla_value_upproj(ctypes.byref(d), 0, 5, 48, 192, fake, fake, fake, 1 << 40, None) == -2
    assert lib.mla_query_absorb(ctypes.byref(d), 0, fake, fake, fake, 48, fake, ctypes.c_float(0.1), 192,
                                None, 1 << 40, None) == -3


def test_causal_validation():
    lib = mla.raw()
    d = _dims()
    fake = ctypes.c_void_p(0x10000)

    def call(cz, n_q=48, n_k=192):
        return lib.mla_chunk_attend_causal(ctypes.byref(d), 0, 0, fake, fake, fake, n_q, fake, fake, fake, 192, n_k,
                                           cz, ctypes.c_float(0.08), fake, fake, 1 << 40, None)

    assert call(None) == -1 and b"causal is null" in lib.mla_last_error()
    assert call(ctypes.byref(mla.MlaCausal(0, 0))) == -1 and b"chunk_len" in lib.mla_last_error()
    assert call(ctypes.byref(mla.MlaCausal(-1, 48))) == -1
    assert call(ctypes.byref(mla.MlaCausal(150, 48))) == -1 and b"q_start" in lib.mla_last_error()
    assert lib.mla_latent_attend_causal(ctypes.byref(d), 0, fake, 192, 48, 192, None, fake, 1 << 40, None) == -1
    assert lib.mla_latent_attend_causal(ctypes.byref(d), 0, fake, 192, 48, 192,
                                        ctypes.byref(mla.MlaCausal(144, 0)), fake, 1 << 40, None) == -1


def test_key_count_limit_of_32_bit_offsets():
    lib = mla.raw()
    d = _dims()                                          # d_c + d_r = 224: 448 bytes per key
    limit = (1 << 32) // 448
    assert lib.mla_chunk_attend_workspace_bytes(ctypes.byref(d), 0, 48, limit) > 0
    assert lib.mla_chunk_attend_workspace_bytes(ctypes.byref(d), 0, 48, limit + 1) == -2
    assert b"4 GiB" in lib.mla_last_error()
    assert lib.mla_chunk_attend_workspace_bytes(ctypes.byref(d), 1, 48, limit + 1) > 0   # fp32 kernels use 64-bit offsets


def test_mha_validation_and_workspace():
    lib = mla.raw()
    fake = ctypes.c_void_p(0x10000)
    ws_dense = lib.mla_mha_attend_workspace_bytes(1, 12, 128, 4680, 32760)
    assert ws_dense > 0 and ws_dense % 256 == 0
    assert lib.mla_mha_attend_workspace_bytes(1, 12, 64, 4680, 32760) == -2
    assert lib.mla_mha_attend_workspace_bytes(1, 12, 128, 0, 32760) == -1
    assert lib.mla_mha_attend_workspace_bytes(1, 12, 128, 100, 99) == -1

    def dense(head_dim=128, q=fake, n_q=48, cap=192, n_k=192, scale=0.08, ws_bytes=1 << 40):
        return lib.mla_mha_attend(1, 12, head_dim, 0, q, n_q, fake, fake, cap, n_k, ctypes.c_float(scale), fake,
                                  fake, ws_bytes, None)

    assert dense(head_dim=96) == -2
    assert dense(q=None) == -1 and b"q is null" in lib.mla_last_error()
    assert dense(cap=100) == -1 and b"cache_capacity" in lib.mla_last_error()
    assert dense(scale=0.0) == -1
    assert dense(ws_bytes=1024) == -3
    assert dense(cap=(1 << 21)) == -2        # one sample's K would pass 4 GiB

    d = _dims()
    ws_exp = lib.mla_chunk_attend_expanded_workspace_bytes(ctypes.byref(d), 4680, 32760)
    # the materialised per-head K (160 wide) and V (128 wide) dominate
    assert ws_exp > 32760 * 12 * (160 + 128) * 2
    bad = _dims(head_dim=64)
    assert lib.mla_chunk_attend_expanded_workspace_bytes(ctypes.byref(bad), 48, 192) == -2

    def expanded(q_pos=fake, n_k=192, cap=192, ws_bytes=1 << 40):
        return lib.mla_chunk_attend_expanded(ctypes.byref(d), 0, fake, fake, q_pos, 48, fake, fake, fake, cap, n_k,
                                             ctypes.c_float(0.08), fake, fake, ws_bytes, None)

    assert expanded(q_pos=None) == -1 and b"q_pos" in lib.mla_last_error()
    assert expanded(n_k=200) == -1
    assert expanded(ws_bytes=4096) == -3


def test_chunk_attend_form_rule():
    lib = mla.raw()
    form = lambda d, dt, n_q, n_k=32760: lib.mla_chunk_attend_form(ctypes.byref(d), dt, n_q, n_k)
    d192 = _dims()
    assert form(d192, 0, 4680) == 1                     # 480P chunk: non-absorbed (4864 rows per head)
    assert form(d192, 0, 1560) == 1
    assert form(d192, 0, 1279) == 0                     # below 1280 queries at d_c = 192
    assert form(d192, 0, 1280) == 1
    assert form(d192, 1, 4680) == 0                     # fp32 inputs: absorbed only
    assert form(_dims(d_c=128), 0, 4680) == 0           # d_c <= 128: absorbed at every size
    assert form(_dims(d_c=256), 0, 4680) == 1
    assert form(_dims(d_c=256), 0, 447) == 0            # below 448 queries at d_c = 256
    assert form(_dims(d_c=256), 0, 448) == 1
    assert form(d192, 0, 0) == -1                       # arguments mla_chunk_attend rejects
    ws_auto = lib.mla_chunk_attend_auto_workspace_bytes(ctypes.byref(d192), 0, 4680, 32760)
    assert ws_auto == lib.mla_chunk_attend_expanded_workspace_bytes(ctypes.byref(d192), 4680, 32760)
    assert lib.mla_chunk_attend_auto_workspace_bytes(ctypes.byref(d192), 0, 48, 192) == \
        lib.mla_chunk_attend_workspace_bytes(ctypes.byref(d192), 0, 48, 192)


def test_binding_checks_tensors_on_host():
    d = mla.Dims(batch=1)
    with pytest.raises(ValueError):
        mla.cache_append(d, torch.zeros(1, 4, 64, dtype=torch.bfloat16), torch.zeros(192, 64, dtype=torch.bfloat16),
                         torch.zeros(32, 64, dtype=torch.bfloat16), torch.zeros(4, 3, dtype=torch.int32),
                         torch.zeros(1, 8, 224, dtype=torch.bfloat16), 0)


def test_last_error_is_per_thread():
    """Validation messages are kept per thread: two threads failing different
    checks at the same time each read back their own message."""
    import threading
    lib = mla.raw()
    fake = ctypes.c_void_p(0x10000)
    seen = {"null": [], "capacity": []}

    def worker(kind, n):
        d = _dims()
        for _ in range(n):
            if kind == "null":
                rc = lib.mla_chunk_attend(ctypes.byref(d), 0, 0, None, fake, fake, 48, fake, fake, fake, 192, 192,
                                          ctypes.c_float(0.08), fake, fake, 1 << 40, None)
            else:
                rc = lib.mla_chunk_attend(ctypes.byref(d), 0, 0, fake, fake, fake, 48, fake, fake, fake, 100, 192,
                                          ctypes.c_float(0.08), fake, fake, 1 << 40, None)
            seen[kind].append((rc, lib.mla_last_error()))

    threads = [threading.Thread(target=worker, args=(k, 2000)) for k in ("null", "capacity")]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(rc == -1 and b"q is null" in m for rc, m in seen["null"])
    assert all(rc == -1 and b"capacity" in m for rc, m in seen["capacity"])
