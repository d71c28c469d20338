"""The C ABI from a C program: include/qha.h compiles as strict C99, every function it declares links
against libqha.so, and the host-only helpers give the documented results when called from C (no GPU
call is made)."""
import os
import re
import shutil
import subprocess

import pytest

from quantized_halo_aggregation_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "qha.h")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "qha.h"

typedef void (*fn)(void);
static const fn every_entry_point[] = { %(table)s };

int main(void) {
  /* every declared function links (its address is taken) */
  for (size_t i = 0; i < sizeof every_entry_point / sizeof every_entry_point[0]; ++i)
    if (!every_entry_point[i]) return 10;
  if (qha_abi_version() != QHA_ABI_VERSION) return 11;
  if (!qha_status_string(QHA_OK) || !qha_status_string(QHA_ERR_INVALID_ARG)) return 12;

  /* d = 128: 4, 8, 16, 32 words for 1, 2, 4, 8 bits, 128 raw words for 32 bits */
  const uint8_t bits[5] = {1, 2, 4, 8, 32};
  uint32_t off[6];
  uint64_t total = 0;
  if (qha_pack_layout(bits, 5, 128, off, &total) != QHA_OK) return 13;
  const uint32_t want[6] = {0, 4, 12, 28, 60, 188};
  if (memcmp(off, want, sizeof want) != 0 || total != 188) return 14;
  const uint8_t bad[1] = {3};
  if (qha_pack_layout(bad, 1, 128, off, &total) != QHA_ERR_INVALID_ARG) return 15;
  if (!qha_last_error() || !qha_last_error()[0]) return 16;

  /* [[0 1 0], [1 0 1]] as a 2 x 3 CSR, transposed to 3 x 2 */
  const int32_t rowptr[3] = {0, 1, 3}, colidx[3] = {1, 0, 2};
  int32_t colptr[4], rowidx[3];
  if (qha_validate_csr(2, 3, rowptr, colidx, 1) != QHA_OK) return 17;
  if (qha_csr_transpose(2, 3, rowptr, colidx, colptr, rowidx) != QHA_OK) return 18;
  const int32_t wp[4] = {0, 1, 2, 3}, wi[3] = {1, 0, 1};
  if (memcmp(colptr, wp, sizeof wp) != 0 || memcmp(rowidx, wi, sizeof wi) != 0) return 19;

  /* a device call with a bad argument is rejected before it touches the GPU */
  if (qha_quantize_pack(0, 128, 0, 1, 128, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != QHA_ERR_INVALID_ARG) return 20;
  printf("ok %%d\n", (int)(sizeof every_entry_point / sizeof every_entry_point[0]));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_header_is_c99_and_links_from_c(tmp_path):
    names = sorted(set(re.findall(r"\b(qha_[a-z0-9_]+)\s*\(", open(HDR).read())))
    assert names
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM % {"table": ", ".join(f"(fn){n}" for n in names)})
    exe = tmp_path / "consumer"
    lib_dir = os.path.dirname(B.LIB_PATH)
    build = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                            f"-I{os.path.dirname(HDR)}", str(src),
                            f"-L{lib_dir}", "-l:" + os.path.basename(B.LIB_PATH), f"-Wl,-rpath,{lib_dir}",
                            "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.strip() == f"ok {len(names)}"
