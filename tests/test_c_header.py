"""The C ABI from plain C: include/hk.h compiles as strict C99 (no C++ in the header),
a C program links against libhk.so and calls the host-side parts (status strings,
workspace sizes, argument checks) -- nothing that needs a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "hash_top_kv_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "hk.h"

int main(void) {
  int bad = 0;
  /* status strings */
  if (strcmp(hk_strerror(HK_OK), "success") != 0) bad |= 1;
  if (hk_strerror((hk_status)99) == NULL) bad |= 2;
  /* workspace sizes grow with the context */
  if (!(hk_retrieve_topk_workspace(128, 1, 8, 524288, 0, 0, 1024) >
        hk_retrieve_topk_workspace(128, 1, 8, 65536, 0, 0, 1024))) bad |= 4;
  if (hk_evict_workspace(64, 4, 4, 262144, 4, 64) != 16 * 128 * 8) bad |= 8;
  /* host-side argument checks enqueue nothing and need no device */
  if (hk_retrieve_topk(NULL, NULL, 96, 1, 1, 10, 10, 0, 0, 3, NULL, NULL, NULL, 0, NULL) !=
      HK_ERR_UNSUPPORTED) bad |= 16;
  if (hk_lse_merge(NULL, NULL, 0, 4, 128, NULL, NULL, NULL) != HK_ERR_INVALID_ARGUMENT) bad |= 32;
  {
    hk_hash h;
    memset(&h, 0, sizeof h);
    h.kind = HK_HASH_LSH; h.dtype = HK_BF16; h.d = 64; h.bits = 128;
    if (hk_encode_keys(&h, NULL, 1, 1, 10, 0, 10, NULL, NULL) != HK_ERR_UNSUPPORTED) bad |= 64;
  }
  printf("%d\n", bad);
  return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c99_and_links(tmp_path):
    lib = os.path.join(LIBDIR, "libhk.so")
    if not os.path.exists(lib):
        pytest.skip("libhk.so is not built")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-L", LIBDIR, "-lhk",
           "-Wl,-rpath," + LIBDIR, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.stdout, r.stderr)
