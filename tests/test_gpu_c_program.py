"""The C ABI from a plain C99 program on the GPU: tests/c/la_c_program.c
(built with gcc by the package build, HIP runtime C API for memory and
streams, no Python or torch in the process) checks prefill + decode
continuation against one longer prefill, packed prefill against per-sequence
calls (bitwise), the host-side argument errors, the workspace split call
against the plain one, and the outputs-only packed call from zero against
zero states (bitwise)."""
import os
import subprocess

import pytest

from long_context_layers_amd import build
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def test_c_program_runs_clean():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    assert os.path.exists(build.C_PROGRAM), "tests/c/la_c_program is built by the package build"
    log("plain C program: prefill + decode continuation, packed prefill, errors, split, outputs only")
    r = subprocess.run([build.C_PROGRAM], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
