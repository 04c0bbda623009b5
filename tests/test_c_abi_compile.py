"""The header is plain C: a C99 program that includes include/lightning_attn.h
compiles with -Wall -Wextra -Werror, links against the library and calls the
entry points that return before any HIP call (status strings, ABI version,
empty launches and host-side argument errors).  CPU only."""
import os
import shutil
import subprocess

import pytest

from long_context_layers_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "lightning_attn.h"

int main(void) {
    if (la_abi_version() != LA_ABI_VERSION) return 10;
    if (strncmp(la_status_string(LA_OK), "LA_OK", 5) != 0) return 11;
    if (strcmp(la_status_string(1234), "unknown status") != 0) return 12;
    float slopes[2] = {0.5f, 0.25f};
    static float state[2 * 64 * 64] __attribute__((aligned(16)));
    /* empty prefill: no-op, null activations allowed, no HIP call */
    if (la_prefill(NULL, NULL, NULL, slopes, NULL, state, 1, 2, 0, 64, NULL) != LA_OK) return 13;
    /* host-side argument errors, reported before any HIP call */
    if (la_prefill(NULL, NULL, NULL, slopes, NULL, state, 1, 2, 0, 96, NULL) != LA_ERR_UNSUPPORTED) return 14;
    if (la_prefill(NULL, NULL, NULL, NULL, NULL, state, 1, 2, 0, 64, NULL) != LA_ERR_INVALID_ARG) return 15;
    if (la_decode_multi(NULL, NULL, NULL, slopes, NULL, state, NULL, 1, 2, 4, 64, NULL)
        != LA_ERR_INVALID_ARG) return 16;
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_c99_and_the_library_links(tmp_path):
    lib = binding.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(lib)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-llightning_attn", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
