"""The C ABI from plain C: include/skipattn.h compiles as C99 with every
warning an error, and a C program linked against libskipattn.so calls the
validation entry points, the workspace-size query and the SAS entry points
with a rejected degree (no GPU needed)."""
import os
import shutil
import subprocess
import textwrap

import pytest

import long_context_tiled_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = textwrap.dedent(r"""
    #include <math.h>
    #include <stdint.h>
    #include <stdio.h>
    #include <string.h>
    #include "skipattn.h"

    #define P ((void*)(uintptr_t)0x10000)   /* fake aligned device address */

    int main(void) {
      int bad = 0;
      /* decode workspace: B * Hq * ceil(L / 4096) * (d + 1) * 4 bytes */
      size_t ws = attn_decode_workspace_bytes(16, 64, 131072, 128);
      if (ws != (size_t)16 * 64 * 32 * 129 * 4) { printf("ws %zu\n", ws); bad = 1; }
      if (attn_decode_workspace_bytes(0, 64, 131072, 128) != 0) bad = 1;
      /* valid prefill arguments pass; a NaN tau and an odd head ratio fail */
      if (attn_prefill_check(P, P, P, (float*)P, (float*)P, 1, 8, 1, 131072, 128, 1,
                             INFINITY, NULL) != SKIPATTN_OK) bad = 1;
      if (attn_prefill_check(P, P, P, (float*)P, (float*)P, 1, 8, 1, 1024, 128, 1,
                             NAN, NULL) != SKIPATTN_EINVAL) bad = 1;
      if (strlen(attn_last_error()) == 0) bad = 1;
      if (attn_prefill_check(P, P, P, (float*)P, (float*)P, 1, 7, 2, 1024, 128, 1,
                             4.0f, NULL) != SKIPATTN_EINVAL) bad = 1;
      /* a causal chunk must start on a tile boundary */
      if (attn_prefill_chunk_check(P, P, P, (float*)P, (float*)P, 1, 8, 1, 64, 1000, 128,
                                   1, 4.0f, NULL) != SKIPATTN_EUNSUPPORTED) bad = 1;
      /* decode: too small a workspace is its own error */
      if (attn_decode_check(P, P, P, (float*)P, (float*)P, 16, 64, 8, 131072, 128,
                            INFINITY, NULL, P, 16) != SKIPATTN_EWORKSPACE) bad = 1;
      if (attn_decode_check(P, P, P, (float*)P, (float*)P, 16, 64, 8, 131072, 128,
                            INFINITY, NULL, P, ws) != SKIPATTN_OK) bad = 1;
      /* SAS degrees other than 0, 2, 3 are rejected before any launch */
      if (attn_decode_sas(P, P, P, (float*)P, (float*)P, 16, 64, 8, 131072, 128,
                          INFINITY, 5, NULL, P, ws, NULL) != SKIPATTN_EINVAL) bad = 1;
      if (attn_decode_q4_sas(P, (const uint8_t*)P, (const uint32_t*)P, (const uint8_t*)P,
                             (const uint32_t*)P, (float*)P, (float*)P, 16, 64, 8, 131072,
                             128, INFINITY, 1, NULL, P, ws, NULL) != SKIPATTN_EINVAL) bad = 1;
      if (attn_decode_q2_sas(P, (const uint8_t*)P, (const uint32_t*)P, (const uint8_t*)P,
                             (const uint32_t*)P, (float*)P, (float*)P, 16, 64, 8, 131072,
                             128, INFINITY, -2, NULL, P, ws, NULL) != SKIPATTN_EINVAL) bad = 1;
      printf(bad ? "FAIL\n" : "OK\n");
      return bad;
    }
""")


@pytest.fixture(scope="module")
def built_program(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib.load()  # the library must exist (built in-tree)
    d = tmp_path_factory.mktemp("cabi")
    src = d / "use_skipattn.c"
    src.write_text(PROGRAM)
    exe = d / "use_skipattn"
    libdir = os.path.dirname(lib.LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-lskipattn", "-lm", "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_header_is_c99_and_links(built_program):
    r = subprocess.run([str(built_program)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr
