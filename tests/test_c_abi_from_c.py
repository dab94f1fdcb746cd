"""The boundary is a C ABI: the header compiles as strict C99 and a plain C
program links against the library and calls its host-side entry points
(argument checks and queries only; no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
INCLUDE = os.path.join(REPO, "include")
LIBDIR = os.path.join(REPO, "selective_state_space_scan_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "ssm_scan.h"

int main(void) {
  ssm_scan_dims dims;
  memset(&dims, 0, sizeof dims);
  dims.batch = 2; dims.seqlen = 100; dims.dim = 32; dims.dstate = 16; dims.io_dtype = SSM_IO_BF16;
  dims.delta_softplus = 1;
  int fails = 0;
  /* every pointer valid-looking, NULL handle: rejected on the host with INVALID_ARG */
  char* base = (char*)0x100000;
  int rc = ssm_selective_scan_fwd(NULL, base, base + 0x10000, (const float*)(base + 0x20000), base + 0x30000,
                                  base + 0x40000, NULL, NULL, base + 0x50000, (float*)(base + 0x60000), &dims, NULL);
  if (rc != SSM_ERR_INVALID_ARG) { printf("fwd rc %d\n", rc); ++fails; }
  dims.dstate = 8;
  rc = ssm_selective_scan_fwd(NULL, base, base, NULL, base, base, NULL, NULL, base, NULL, &dims, NULL);
  if (rc != SSM_ERR_UNSUPPORTED) { printf("dstate rc %d\n", rc); ++fails; }
  dims.dstate = 16;
  if (ssm_scan_chunk_len(16) != 128 || ssm_scan_bwd_chunk_len(16) != 32) { printf("chunk lens\n"); ++fails; }
  if (ssm_scan_workspace_bytes(&dims, 1) != 0) { printf("workspace\n"); ++fails; }
  if (ssm_scan_bwd_workspace_bytes(&dims) <= 0) { printf("bwd workspace\n"); ++fails; }
  if (ssm_scan_auto_time_parts(NULL, &dims) != 1) { printf("auto parts\n"); ++fails; }
  if (strcmp(ssm_scan_error_string(SSM_OK), "ok") != 0) { printf("error string\n"); ++fails; }
  if (ssm_scan_destroy(NULL) != SSM_OK) { printf("destroy\n"); ++fails; }
  ssm_scan_t h = (ssm_scan_t)1;
  if (ssm_scan_create(NULL, 0) != SSM_ERR_INVALID_ARG) { printf("create\n"); ++fails; }
  (void)h;
  printf("%s\n", fails ? "FAIL" : "OK");
  return fails;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_c99(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "ssm_scan.h"\nint main(void) { return 0; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, "-c", str(src),
                    "-o", str(tmp_path / "h.o")], check=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_links_and_calls_host_entry_points(tmp_path):
    import selective_state_space_scan_amd as ssm
    if not os.path.exists(ssm.library_path()):
        pytest.skip("HIP library not built")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", INCLUDE, str(src), "-o", str(exe), f"-L{LIBDIR}",
                    "-lssmscan", f"-Wl,-rpath,{LIBDIR}"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout + res.stderr
