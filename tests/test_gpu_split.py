"""GPU checks of the dense prefill's sequence split (la_prefill_ws): a B = 1
launch whose column-slice workgroups fill at most half the device runs S
segments of each head's sequence at once, chains their states and corrects
the later segments (the report's §4.1.1 / Fig. 10 decomposition on one
device).  Checked against the fp64 oracle (outputs and final states, bf16 bar
2e-2 and the 4e-3 guard) with slow, unit and infinite-slope decays, ragged
lengths and a random initial state; against the unsplit launch; and the
workspace rules (too small, null, misaligned) are refused before any launch."""
import ctypes
import math

import pytest
import torch

from long_context_layers_amd import binding, inputs
from tests.gpu_util import BF16_GUARD, BF16_TOL, F32_TOL, log, oracle_prefill, rel_l2
from tests.test_gpu_strided import heads_view, pack_token_major

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def need_split(B, H, N, d=128):
    ws = binding.prefill_workspace_bytes(B, H, N, d, DEV)
    if ws == 0:
        pytest.skip(f"no split for B{B} H{H} N{N} on this device "
                    f"({torch.cuda.get_device_properties(0).multi_processor_count} compute units)")
    return ws


def unsplit(inp, state):
    out = torch.empty_like(inp.q)
    B, H, N, d = inp.q.shape
    rc = binding.load_library().la_prefill(inp.q.data_ptr(), inp.k.data_ptr(), inp.v.data_ptr(),
                                           inp.slopes.data_ptr(), out.data_ptr(), state.data_ptr(),
                                           B, H, N, d, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return out


@pytest.mark.parametrize("H,N,slopes", [
    (64, 40000, None),                                   # 2 segments, ragged, the model's decays
    (32, 40000, None),                                   # 4 segments
    (8, 65536 + 77, [0.0, 1e-4, 1e-3, 0.01, 0.1, 1.0, 5.0, math.inf]),   # 16 segments; lambda = 1 .. 0
    (64, 262144, None),                                  # the 256K workload's shape: 2 segments
    (1, 70000, [1e-4]),                                  # 17 segments, slow decay: full corrections
    (64, 16384 + 100, None),                             # 2 segments of ~8K (full device unsplit)
    (32, 8192 + 5, None),                                # 2 segments of ~4K (half the device unsplit)
    (8, 16384 + 33, [0.0, 1e-4, 1e-3, 0.01, 0.1, 1.0, 5.0, 2.0 ** -8]),   # 4 segments of ~4K
    (1, 33000, [2.0 ** -8]),                             # 8 segments, the slowest model decay
])
def test_split_matches_oracle(H, N, slopes):
    ws = need_split(1, H, N)
    inp = inputs.make_prefill(1, H, N, 128, torch.bfloat16, 700 + H, init_state=True, device=DEV)
    if slopes is not None:
        inp = inputs.PrefillInputs(inp.q, inp.k, inp.v,
                                   torch.tensor(slopes, dtype=torch.float32, device=DEV), inp.state)
    log(f"split prefill B1 H{H} N{N} d128 (workspace {ws} B), slopes {slopes or 'model'}")
    st = inp.state.clone()
    out = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state)
    eo, es = rel_l2(out, o_ref), rel_l2(st, s_ref)
    # and the unsplit launch on the same inputs
    st1 = inp.state.clone()
    out1 = unsplit(inp, st1)
    torch.cuda.synchronize()
    eo1, es1 = rel_l2(out1, o_ref), rel_l2(st1, s_ref)
    log(f"  split: out {eo:.3e} state {es:.3e}; unsplit: out {eo1:.3e} state {es1:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
    assert eo <= BF16_GUARD and es <= BF16_GUARD, "precision regression"


def test_split_is_deterministic():
    H, N = 32, 40000
    need_split(1, H, N)
    inp = inputs.make_prefill(1, H, N, 128, torch.bfloat16, 711, init_state=True, device=DEV)
    st1, st2 = inp.state.clone(), inp.state.clone()
    o1 = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st1)
    o2 = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)


def test_workspace_rules_are_checked_before_any_launch():
    H, N, d = 32, 40000, 128
    ws = need_split(1, H, N)
    inp = inputs.make_prefill(1, H, N, d, torch.bfloat16, 712, init_state=True, device=DEV)
    out = torch.full_like(inp.q, 3.0)
    st = inp.state.clone()
    work = torch.empty(ws + 512, dtype=torch.uint8, device=DEV)
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream

    def call(wp, nb):
        return lib.la_prefill_ws(inp.q.data_ptr(), inp.k.data_ptr(), inp.v.data_ptr(),
                                 inp.slopes.data_ptr(), out.data_ptr(), st.data_ptr(), 1, H, N, d,
                                 wp, nb, s)
    assert call(None, ws) == 1                          # null workspace
    assert call(work.data_ptr(), ws - 1) == 1           # too small
    assert call(work.data_ptr() + 128, ws) == 1         # not 256-byte aligned
    assert call(out.data_ptr(), ws) == 1                # overlaps out
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and torch.equal(st, inp.state)   # nothing ran
    assert call(work.data_ptr(), ws) == 0
    torch.cuda.synchronize()
    assert not bool((out == 3.0).all())


def test_split_plan():
    # segments of 64-column workgroups (d = 128) or 32-column ones (d = 64):
    # 64 heads of 128 split in two on 256 compute units, 128 heads of 64 fill
    # the device unsplit, B > 1 never splits; segments of at least 8192 tokens
    # where la_prefill's grid fills the device, of at least 4096 where it
    # leaves compute units idle
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip("the expected plans are those of a 256-CU device")
    d128 = 64 * 128 * 128 * 4
    assert binding.prefill_workspace_bytes(1, 64, 262144, 128, DEV) == 2 * d128 + 256
    assert binding.prefill_workspace_bytes(1, 32, 262144, 128, DEV) == 4 * d128 // 2 + 256
    assert binding.prefill_workspace_bytes(1, 128, 262144, 64, DEV) == 0
    assert binding.prefill_workspace_bytes(2, 32, 262144, 128, DEV) == 0
    assert binding.prefill_workspace_bytes(1, 64, 16384, 128, DEV) == 2 * d128 + 256
    assert binding.prefill_workspace_bytes(1, 64, 16383, 128, DEV) == 0     # too short to split
    assert binding.prefill_workspace_bytes(1, 64, 8192, 128, DEV) == 0
    assert binding.prefill_workspace_bytes(1, 32, 8192, 128, DEV) == d128 + 256
    assert binding.prefill_workspace_bytes(1, 32, 8191, 128, DEV) == 0
    assert binding.prefill_workspace_bytes(1, 8, 16384, 128, DEV) == 4 * d128 // 8 + 256
    # one head: 64 segments of 4096 (at most 64), 65 offsets in the tail
    assert binding.prefill_workspace_bytes(1, 1, 262144, 128, DEV) == 64 * d128 // 64 + 768


@pytest.mark.parametrize("H,N,d", [(32, 40000, 128), (64, 65536 + 300, 64)])
def test_strided_split_bitwise_equals_contiguous_split(H, N, d):
    # q, k, v from one token-major projection buffer, out token-major
    # (la_prefill_strided_ws), against la_prefill_ws on the same values, and
    # the oracle
    ws = need_split(1, H, N, d)
    log(f"strided split prefill B1 H{H} N{N} d{d} (workspace {ws} B)")
    x = inputs.make_prefill(1, H, N, d, torch.bfloat16, 730 + H, init_state=True, device=DEV)
    st_ref = x.state.clone()
    out_ref = binding.prefill(x.q, x.k, x.v, x.slopes, st_ref)
    _, (qv, kv, vv) = pack_token_major([x.q, x.k, x.v], pad=8)
    obuf = torch.empty((1, N, H * d), dtype=torch.bfloat16, device=DEV)
    st = x.state.clone()
    binding.prefill(qv, kv, vv, x.slopes, st, out=heads_view(obuf, 0, H, d))
    torch.cuda.synchronize()
    assert torch.equal(heads_view(obuf, 0, H, d), out_ref) and torch.equal(st, st_ref)
    o_ref, s_ref = oracle_prefill(x.q, x.k, x.v, x.slopes, x.state)
    eo, es = rel_l2(out_ref, o_ref), rel_l2(st_ref, s_ref)
    log(f"  bitwise equal; oracle out {eo:.3e} state {es:.3e}")
    assert eo <= BF16_GUARD and es <= BF16_GUARD


# ---- the fp32 split (la_prefill_f32_ws): the fp32 kernel's segments, the same
# fold, an fp32 correction ----

def need_f32_split(H, N, d=128):
    ws = binding.prefill_f32_workspace_bytes(1, H, N, d, DEV)
    if ws == 0:
        pytest.skip(f"no fp32 split for B1 H{H} N{N} d{d} on this device")
    return ws


@pytest.mark.parametrize("H,N,d,slopes", [
    (64, 32768 + 21, 128, None),                         # the fp32 benchmark's shape: 2 segments
    (32, 32768 + 300, 128, None),                        # 4 segments
    (8, 65536 + 77, 128, [0.0, 1e-4, 1e-3, 0.01, 0.1, 1.0, 5.0, math.inf]),   # 8; lambda = 1 .. 0
    (1, 40000, 128, [1e-4]),                             # 4 segments, slow decay: full corrections
    (1, 70000, 128, [2.0 ** -8]),                        # 8 segments, the slowest model decay
    (64, 65536 + 5, 64, None),                           # d = 64: 4 segments
])
def test_f32_split_matches_oracle(H, N, d, slopes):
    ws = need_f32_split(H, N, d)
    inp = inputs.make_prefill(1, H, N, d, torch.float32, 740 + H, init_state=True, device=DEV)
    if slopes is not None:
        inp = inputs.PrefillInputs(inp.q, inp.k, inp.v,
                                   torch.tensor(slopes, dtype=torch.float32, device=DEV), inp.state)
    log(f"fp32 split prefill B1 H{H} N{N} d{d} (workspace {ws} B), slopes {slopes or 'model'}")
    st = inp.state.clone()
    out = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st)
    st1 = inp.state.clone()
    out1 = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st1, split=False)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state)
    eo, es = rel_l2(out, o_ref), rel_l2(st, s_ref)
    eo1, es1 = rel_l2(out1, o_ref), rel_l2(st1, s_ref)
    log(f"  split: out {eo:.3e} state {es:.3e}; unsplit: out {eo1:.3e} state {es1:.3e}")
    assert eo <= F32_TOL and es <= F32_TOL
    assert eo1 <= F32_TOL and es1 <= F32_TOL
    # fp32 throughout: both sit near single-precision rounding
    assert max(eo, es, eo1, es1) <= 1e-5, "precision regression"


def test_f32_split_is_deterministic():
    H, N = 32, 40000
    need_f32_split(H, N)
    inp = inputs.make_prefill(1, H, N, 128, torch.float32, 751, init_state=True, device=DEV)
    st1, st2 = inp.state.clone(), inp.state.clone()
    o1 = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st1)
    o2 = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)


def test_f32_workspace_rules_are_checked_before_any_launch():
    H, N, d = 64, 32768, 128
    ws = need_f32_split(H, N, d)
    inp = inputs.make_prefill(1, H, N, d, torch.float32, 752, init_state=True, device=DEV)
    out = torch.full_like(inp.q, 3.0)
    st = inp.state.clone()
    work = torch.empty(ws + 512, dtype=torch.uint8, device=DEV)
    lib = binding.load_library()
    s = torch.cuda.current_stream().cuda_stream

    def call(wp, nb):
        return lib.la_prefill_f32_ws(inp.q.data_ptr(), inp.k.data_ptr(), inp.v.data_ptr(),
                                     inp.slopes.data_ptr(), out.data_ptr(), st.data_ptr(), 1, H, N,
                                     d, wp, nb, s)
    assert call(None, ws) == 1                          # null workspace
    assert call(work.data_ptr(), ws - 1) == 1           # too small
    assert call(work.data_ptr() + 128, ws) == 1         # not 256-byte aligned
    assert call(out.data_ptr(), ws) == 1                # overlaps out
    assert call(st.data_ptr(), ws) == 1                 # overlaps the state
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and torch.equal(st, inp.state)   # nothing ran
    assert call(work.data_ptr(), ws) == 0
    torch.cuda.synchronize()
    assert not bool((out == 3.0).all())


def test_f32_split_plan():
    # fp32 workgroups of 32 columns, two per compute unit: a B = 1 launch splits
    # into S = min(2 x CUs / workgroups, N / 8192, 64) segments when S >= 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip("the expected plans are those of a 256-CU device")
    slot = lambda H, d: H * d * d * 4
    assert binding.prefill_f32_workspace_bytes(1, 64, 32768, 128, DEV) == 2 * slot(64, 128) + 256
    assert binding.prefill_f32_workspace_bytes(1, 64, 16384, 128, DEV) == 2 * slot(64, 128) + 256
    assert binding.prefill_f32_workspace_bytes(1, 64, 16383, 128, DEV) == 0
    assert binding.prefill_f32_workspace_bytes(1, 32, 32768, 128, DEV) == 4 * slot(32, 128) + 256
    assert binding.prefill_f32_workspace_bytes(1, 128, 65536, 128, DEV) == 0   # fills the device
    assert binding.prefill_f32_workspace_bytes(2, 64, 65536, 128, DEV) == 0
    assert binding.prefill_f32_workspace_bytes(1, 64, 65536, 64, DEV) == 4 * slot(64, 64) + 256
    assert binding.prefill_f32_workspace_bytes(1, 1, 1 << 20, 128, DEV) == 64 * slot(1, 128) + 768
