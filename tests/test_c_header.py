"""include/mla.h is a C header: a C99 program (no C++, no HIP headers)
compiles against it with -pedantic -Werror, links against the built library
and runs its host-only entry points -- version and status strings, cache
byte counts, the ring bookkeeping and the workspace query -- with no GPU.
The values it prints are checked against what the header documents."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "latent_kv_cache_chunk_amd")

PROGRAM = r"""
#include <stdio.h>
#include "mla.h"

int main(void) {
  mla_dims d = {1, 12, 128, 192, 32, 8, 12, 12, 10000.0};
  mla_ring r;
  int32_t off = -1, n_k = -1;
  int64_t ws;
  printf("version %s\n", mla_version());
  printf("status %s %s\n", mla_status_string(MLA_OK), mla_status_string(MLA_ERR_WORKSPACE));
  printf("latent %lld dense %lld\n", (long long)mla_cache_bytes(&d, MLA_BF16, 32760),
         (long long)mla_dense_kv_bytes(&d, MLA_BF16, 32760));
  if (mla_ring_init(&r, 48, 1, 2) != MLA_OK) return 1;
  printf("capacity %d\n", (int)r.capacity);
  mla_ring_current(&r, &off, &n_k);
  printf("chunk0 %d %d\n", (int)off, (int)n_k);
  mla_ring_commit(&r);
  mla_ring_commit(&r);
  mla_ring_current(&r, &off, &n_k);
  printf("chunk2 %d %d\n", (int)off, (int)n_k);
  ws = mla_chunk_attend_workspace_bytes(&d, MLA_BF16, 4680, 32760);
  printf("workspace %d\n", ws > 0);
  printf("bad_dims %d\n", (int)(mla_chunk_attend_workspace_bytes(NULL, MLA_BF16, 4680, 32760) < 0));
  return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    lib = os.path.join(LIB_DIR, "libmla_hip.so")
    if not os.path.exists(lib):
        pytest.skip("libmla_hip.so is not built")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    cmd = [cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-L", LIB_DIR, "-lmla_hip", "-Wl,-rpath," + LIB_DIR, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert out["version"].endswith("gfx950")
    assert out["status"] == "MLA_OK MLA_ERR_WORKSPACE"
    # 224 bf16 per token against 2 x 12 x 128 (atlas.scime.ai summary, "Key results")
    assert out["latent"] == f"{32760 * 224 * 2} dense {32760 * 3072 * 2}"
    # one sink chunk, a window of two, one slot for the current chunk
    assert out["capacity"] == str((1 + 2 + 1) * 48)
    assert out["chunk0"] == "0 48"
    assert out["chunk2"] == f"{2 * 48} {3 * 48}"
    assert out["workspace"] == "1"
    assert out["bad_dims"] == "1"
