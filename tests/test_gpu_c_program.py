"""One chunk step driven from plain C through the ABI: hipMalloc'd buffers,
mla_cache_append, the workspace query and mla_chunk_attend on the null
stream -- no Python, no torch on the path.  The program is compiled with the
system C compiler against include/mla.h and HIP's C runtime header.

The appended rows (Gaussian inputs at the chunk's real positions) must match
the oracle's bits except where the fp32 error bound reaches a bf16 rounding
boundary, the rule the append tests apply; the rows before the write offset
must be untouched; the fp32 output must match the oracle run on the cache the
GPU wrote, within the fp32-output gate.
"""

import os
import shutil
import subprocess
from dataclasses import replace

import numpy as np
import pytest

import oracle
from latent_kv_cache_chunk_amd import synth
from tests.gpu_util import assert_g2, need_gpu, np64
from tests.test_gpu_append import _error_bound, _tie_zone_check

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "latent_kv_cache_chunk_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "mla.h"
#include "sizes.h"

static void* upload(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  void* host = malloc(bytes);
  void* dev = NULL;
  FILE* f;
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "rb");
  if (!f || fread(host, 1, bytes, f) != bytes) { fprintf(stderr, "read %s\n", path); exit(2); }
  fclose(f);
  if (hipMalloc(&dev, bytes) != hipSuccess || hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "upload %s\n", name);
    exit(3);
  }
  free(host);
  return dev;
}

static void download(const char* dir, const char* name, const void* dev, size_t bytes) {
  char path[4096];
  void* host = malloc(bytes);
  FILE* f;
  if (hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) { fprintf(stderr, "download\n"); exit(4); }
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "wb");
  fwrite(host, 1, bytes, f);
  fclose(f);
  free(host);
}

int main(int argc, char** argv) {
  const char* dir = argc > 1 ? argv[1] : ".";
  mla_dims d = {B, H, DH, DC, DR, RT, RH, RW, 10000.0};
  const size_t w = DC + DR;
  void* x = upload(dir, "x.bin", (size_t)B * NQ * D * 2);
  void* w_dkv = upload(dir, "w_dkv.bin", (size_t)DC * D * 2);
  void* w_kr = upload(dir, "w_kr.bin", (size_t)DR * D * 2);
  int32_t* pos = (int32_t*)upload(dir, "pos.bin", (size_t)NQ * 3 * 4);
  void* q = upload(dir, "q.bin", (size_t)B * NQ * H * DH * 2);
  void* q_r = upload(dir, "q_r.bin", (size_t)B * NQ * H * DR * 2);
  void* w_uk = upload(dir, "w_uk.bin", (size_t)H * DH * DC * 2);
  void* w_uv = upload(dir, "w_uv.bin", (size_t)H * DH * DC * 2);
  void* cache = upload(dir, "cache.bin", (size_t)B * CAP * w * 2);
  void* out = NULL;
  void* ws = NULL;
  int64_t ws_bytes;
  int32_t st;
  if (hipMalloc(&out, (size_t)B * NQ * H * DH * 4) != hipSuccess) return 5;
  st = mla_cache_append(&d, MLA_BF16, x, D, NQ, w_dkv, w_kr, pos, cache, CAP, OFF, NULL);
  printf("append %d\n", (int)st);
  ws_bytes = mla_chunk_attend_workspace_bytes(&d, MLA_BF16, NQ, NK);
  if (ws_bytes <= 0 || hipMalloc(&ws, (size_t)ws_bytes) != hipSuccess) return 6;
  st = mla_chunk_attend(&d, MLA_BF16, MLA_F32, q, q_r, pos, NQ, w_uk, w_uv, cache, CAP, NK, SCALE, out, ws, ws_bytes,
                        NULL);
  printf("attend %d\n", (int)st);
  printf("sync %d\n", (int)hipDeviceSynchronize());
  download(dir, "out.bin", out, (size_t)B * NQ * H * DH * 4);
  download(dir, "cache_out.bin", cache, (size_t)B * CAP * w * 2);
  return 0;
}
"""


def test_chunk_step_from_c(tmp_path):
    need_gpu()
    import torch
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    wl = replace(synth.TINY, batch=2)
    att = synth.attend_inputs(wl, seed=6, capacity=wl.n_k + 5)
    app = synth.append_inputs(wl, seed=6)
    cap, off = wl.n_k + 5, wl.n_cached
    files = {"x.bin": app["x"], "w_dkv.bin": app["w_dkv"], "w_kr.bin": app["w_kr"], "q.bin": att["q"],
             "q_r.bin": att["q_r"], "w_uk.bin": att["w_uk"], "w_uv.bin": att["w_uv"], "cache.bin": att["cache"]}
    for name, t in files.items():
        (tmp_path / name).write_bytes(t.contiguous().view(torch.int16).numpy().tobytes())
    pos = app["pos"].numpy().astype(np.int32)
    (tmp_path / "pos.bin").write_bytes(np.ascontiguousarray(pos).tobytes())
    (tmp_path / "sizes.h").write_text(
        f"#define B {wl.batch}\n#define NQ {wl.n_q}\n#define NK {wl.n_k}\n#define CAP {cap}\n#define OFF {off}\n"
        f"#define D {wl.d_model}\n#define H {wl.n_heads}\n#define DH {wl.head_dim}\n#define DC {wl.d_c}\n"
        f"#define DR {wl.d_r}\n#define RT {wl.rope_split[0]}\n#define RH {wl.rope_split[1]}\n"
        f"#define RW {wl.rope_split[2]}\n#define SCALE {wl.scale!r}f\n")
    (tmp_path / "prog.c").write_text(PROGRAM)
    exe = tmp_path / "prog"
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", str(tmp_path), str(tmp_path / "prog.c"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-L", LIB_DIR, "-lmla_hip",
           "-Wl,-rpath," + LIB_DIR, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("running the C program", flush=True)
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split() == ["append", "0", "attend", "0", "sync", "0"], r.stdout

    width = wl.d_c + wl.d_r
    got_cache = np.frombuffer((tmp_path / "cache_out.bin").read_bytes(), np.uint16).reshape(wl.batch, cap, width)
    # appended rows: the oracle's bits outside the tie zone of the fp32 bound
    x = np64(app["x"])
    exact = oracle.latent_rows(x, np64(app["w_dkv"]), np64(app["w_kr"]), pos, wl.rope_split, wl.theta)
    bound = _error_bound(x, np.concatenate([np64(app["w_dkv"]), np64(app["w_kr"])], 0), pos, wl)
    n_diff = _tie_zone_check(got_cache[:, off:off + wl.n_q], exact, bound)
    assert n_diff <= 1e-3 * exact.size
    # the rows before the offset are untouched
    before = att["cache"].contiguous().view(torch.int16).numpy().view(np.uint16)[:, :off]
    assert np.array_equal(got_cache[:, :off], before)
    # the output against the oracle on the cache the GPU wrote
    cache64 = (got_cache.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = np.frombuffer((tmp_path / "out.bin").read_bytes(), np.float32).reshape(wl.batch, wl.n_q, wl.n_heads,
                                                                                wl.head_dim)
    want = oracle.chunk_attend(np64(att["q"]), np64(att["q_r"]), pos, np64(att["w_uk"]), np64(att["w_uv"]), cache64,
                               wl.n_k, wl.scale, split=wl.rope_split, theta=wl.theta)
    assert_g2(out.astype(np.float64), want, "C program")
