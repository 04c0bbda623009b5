"""The allocation-free prefill (la_prefill_noalloc) through the C ABI against
la_prefill_ws with a workspace from torch: two calls in a row on the library's
scratch, the second smaller, each equal to the workspace call (same kernels,
same split: bitwise), and the oracle bar as a second check."""
import pytest
import torch

from long_context_layers_amd import binding, inputs
from tests.gpu_util import BF16_TOL, log, oracle_prefill, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _call(fn, inp, out, st, *extra):
    B, H, N, d = inp.q.shape
    return fn(inp.q.data_ptr(), inp.k.data_ptr(), inp.v.data_ptr(), inp.slopes.data_ptr(),
              out.data_ptr(), st.data_ptr(), B, H, N, d, *extra,
              torch.cuda.current_stream().cuda_stream)


def test_noalloc_equals_the_workspace_call_twice_in_a_row():
    lib = binding.load_library()
    shapes = [(32, 40000, 801), (16, 12000, 802)]          # second call smaller (8 and 2 MiB)
    planned = [binding.prefill_workspace_bytes(1, H, N, 128, DEV) for H, N, _ in shapes]
    if not all(planned):
        pytest.skip(f"no sequence split planned on this device ({planned})")
    assert planned[1] < planned[0]
    for (H, N, seed), ws in zip(shapes, planned):
        log(f"noalloc prefill B1 H{H} N{N} d128 (split workspace {ws} B)")
        inp = inputs.make_prefill(1, H, N, 128, torch.bfloat16, seed, init_state=True, device=DEV)
        out_n, st_n = torch.empty_like(inp.q), inp.state.clone()
        assert _call(lib.la_prefill_noalloc, inp, out_n, st_n) == 0
        work = torch.empty(ws, dtype=torch.uint8, device=DEV)
        out_w, st_w = torch.empty_like(inp.q), inp.state.clone()
        assert _call(lib.la_prefill_ws, inp, out_w, st_w, work.data_ptr(), ws) == 0
        torch.cuda.synchronize()
        assert torch.equal(out_n, out_w) and torch.equal(st_n, st_w)
        o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state)
        eo, es = rel_l2(out_n, o_ref), rel_l2(st_n, s_ref)
        log(f"  bitwise equal to la_prefill_ws; oracle out {eo:.3e} state {es:.3e}")
        assert eo <= BF16_TOL and es <= BF16_TOL
