"""The boundary from plain C: include/dit_attn.h compiles as strict C99 (no C++
in the declarations) and a C program links libditattn.so and calls it.  Only
host-side paths run (argument validation, error text, the balanced plan with
an explicit slot count), so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

import diffusion_transformer_attention_amd as dta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = r"""
#include <stdio.h>
#include <stddef.h>
#include "dit_attn.h"
int main(void) {
  size_t ws = 7;
  int rc = dit_attn_fwd_balanced_workspace(1, 10, 32768, 32768, 128, 256, &ws);
  if (rc != DIT_OK || ws != 0) return 1;               /* five whole waves: no split */
  rc = dit_attn_fwd_balanced_workspace(1, 10, 75600, 75600, 128, 256, &ws);
  if (rc != DIT_OK || ws == 0) return 2;
  if (dit_attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 96, 0.1f, DIT_BF16, NULL)
      != DIT_EUNSUPPORTED) return 3;                   /* D = 96: rejected before any launch */
  if (dit_attn_merge(NULL, NULL, 0, NULL, NULL, 1, 1, 1, 128, DIT_BF16, NULL) != DIT_EINVAL)
    return 4;
  if (ulysses_seq2head(NULL, NULL, 4, 1, 6, 64, 128, 2, NULL) != DIT_EINVAL) return 5;
  printf("abi %d: %s\n", dit_abi_version(), dit_strerror(DIT_EALIGN));
  return dit_abi_version() == DIT_ABI_VERSION ? 0 : 6;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c99_and_links(tmp_path):
    if not os.path.exists(dta.LIB_PATH):
        pytest.fail("libditattn.so not built: run __graft_entry__.build()")
    src = tmp_path / "use_abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_abi"
    libdir = os.path.dirname(dta.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I" + os.path.join(ROOT, "include"), str(src), "-L" + libdir, "-lditattn",
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("abi 1: ")
