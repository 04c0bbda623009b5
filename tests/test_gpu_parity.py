"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on
the same seeded bytes.  Bar: max over (b, h) of the relative L2 error of the
outputs and of the final states <= 2e-2 for bf16 activations and <= 1e-3 for
fp32 activations."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_layers_amd import binding, inputs
from tests.gpu_util import (BF16_GUARD, BF16_TOL, DECODE_STATE_GUARD, F32_TOL, log, np64,
                            oracle_prefill, rel_l2)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def gpu_prefill(inp, state=None):
    st = (inp.state if state is None else state).clone()
    out = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st)
    torch.cuda.synchronize()
    return out, st


def check_prefill(inp, tol, heads=None, what="", guard=None):
    out, st = gpu_prefill(inp)
    o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state, heads)
    if heads is not None:
        idx = torch.tensor(heads, device=out.device)
        out, st = out.index_select(1, idx), st.index_select(1, idx)
    eo, es = rel_l2(out, o_ref), rel_l2(st, s_ref)
    log(f"  {what}: out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}  (tol {tol:g})")
    assert eo <= tol and es <= tol
    if guard is not None:
        assert eo <= guard and es <= guard, f"precision regression: {eo:.3e} / {es:.3e} > {guard:g}"
    return eo, es


# ---- the named workloads ---------------------------------------------------

def test_tiny_f32_workload():
    log("tiny_f32: B1 H2 N256 d64 fp32")
    inp = inputs.make_workload("tiny_f32", device=DEV)
    check_prefill(inp, F32_TOL, what="tiny_f32")


def test_prefill_4k_workload():
    log("prefill_4k: B1 H64 N4096 d128 bf16")
    inp = inputs.make_workload("prefill_4k", device=DEV)
    check_prefill(inp, BF16_TOL, what="prefill_4k", guard=BF16_GUARD)


def test_prefill_32k_with_initial_state():
    log("prefill_32k_state: B1 H64 N32768 d128 bf16 + fp32 initial state")
    inp = inputs.make_workload("prefill_32k_state", device=DEV)
    check_prefill(inp, BF16_TOL, what="prefill_32k_state", guard=BF16_GUARD)


def test_prefill_256k_all_heads():
    # the full 256K launch as timed by the benchmark, every one of the 64 heads
    # against the oracle (16 heads at a time to bound host memory)
    log("prefill_256k: B1 H64 N262144 d128 bf16, oracle on all 64 heads in groups of 16")
    inp = inputs.make_workload("prefill_256k", device=DEV)
    st = inp.state.clone()
    out = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st)
    torch.cuda.synchronize()
    worst_o = worst_s = 0.0
    for h0 in range(0, 64, 16):
        heads = list(range(h0, h0 + 16))
        o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state, heads=heads)
        idx = torch.tensor(heads, device=DEV)
        eo = rel_l2(out.index_select(1, idx), o_ref)
        es = rel_l2(st.index_select(1, idx), s_ref)
        log(f"  heads {h0}..{h0 + 15}: out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        del o_ref, s_ref
    assert worst_o <= BF16_TOL and worst_s <= BF16_TOL
    assert worst_o <= BF16_GUARD and worst_s <= BF16_GUARD, "precision regression"


def test_prefill_beyond_4gib_per_tensor():
    # maximum size: two 256K sequences (8 GiB per tensor, 2^32 elements), so
    # the second sequence's slices lie past 4 GiB from each tensor's base.
    # That sequence alone, launched from a view at its own base (offsets
    # below 4 GiB, no split), must give the same bits; heads 0 and 63 of it
    # against the oracle, from a random initial state.
    B, H, N, d = 2, 64, 262144, 128
    log(f"prefill B{B} H{H} N{N} d{d} bf16 (8 GiB per tensor) + fp32 initial state")
    inp = inputs.make_prefill(B, H, N, d, torch.bfloat16, 1013, init_state=True, device=DEV)
    st = inp.state.clone()
    out = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st)
    torch.cuda.synchronize()
    st1 = inp.state[1:2].clone()
    out1 = binding.prefill(inp.q[1:2], inp.k[1:2], inp.v[1:2], inp.slopes, st1, split=False)
    torch.cuda.synchronize()
    assert torch.equal(out[1:2], out1), "second sequence: outputs differ from its own launch"
    assert torch.equal(st[1:2], st1), "second sequence: final states differ from its own launch"
    del out1, st1
    heads = [0, 63]
    idx = torch.tensor(heads, device=DEV)
    o_ref, s_ref = oracle_prefill(inp.q[1:2], inp.k[1:2], inp.v[1:2], inp.slopes, inp.state[1:2],
                                  heads=heads)
    eo = rel_l2(out[1:2].index_select(1, idx), o_ref)
    es = rel_l2(st[1:2].index_select(1, idx), s_ref)
    log(f"  bitwise equal to its own launch; heads 0, 63 of the second sequence: "
        f"out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
    assert eo <= BF16_GUARD and es <= BF16_GUARD, "precision regression"


def test_prefill_flash_heads_32k():
    # the flash models' 32 heads of 128 (report §2.1.1, Table 1): 128 column-slice
    # workgroups on a 256-CU device, a long sequence from a random initial state
    log("prefill flash heads: B1 H32 N32768 d128 bf16 + fp32 initial state")
    inp = inputs.make_prefill(1, 32, 32768, 128, torch.bfloat16, 1012, init_state=True, device=DEV)
    check_prefill(inp, BF16_TOL, what="flash heads 32K", guard=BF16_GUARD)


def test_decode_b256_64_steps():
    log("decode_b256: B256 H64 d128, 64 steps")
    inp = inputs.make_workload("decode_b256", device=DEV)
    st = inp.state.clone()
    ref_st = np64(inp.state)
    s64 = np64(inp.slopes)
    worst = 0.0
    for t in range(inp.q.shape[0]):
        o = binding.decode_step(inp.q[t], inp.k[t], inp.v[t], inp.slopes, st)
        o_ref, ref_st = oracle.decode_step(np64(inp.q[t]), np64(inp.k[t]), np64(inp.v[t]),
                                           s64, ref_st, inplace=True)
        e = rel_l2(o, o_ref)
        worst = max(worst, e)
        assert e <= BF16_TOL, (t, e)
    es = rel_l2(st, ref_st)
    log(f"  decode_b256: worst step out rel-L2 {worst:.3e}  final state {es:.3e}")
    assert es <= BF16_TOL
    assert worst <= BF16_GUARD and es <= DECODE_STATE_GUARD, "precision regression"


def test_prefill_f32_beyond_4gib_per_tensor():
    # fp32 activations at the 256K shape: 8 GiB per tensor, the later heads'
    # rows past 4 GiB (the split call: two segments, fold, fp32 correction);
    # heads 0 and 63 against the oracle from a random initial state
    B, H, N, d = 1, 64, 262144, 128
    log(f"prefill fp32 B{B} H{H} N{N} d{d} (8 GiB per tensor) + fp32 initial state")
    inp = inputs.make_prefill(B, H, N, d, torch.float32, 1016, init_state=True, device=DEV)
    out, st = gpu_prefill(inp)
    heads = [0, 63]
    idx = torch.tensor(heads, device=DEV)
    o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state, heads=heads)
    eo = rel_l2(out.index_select(1, idx), o_ref)
    es = rel_l2(st.index_select(1, idx), s_ref)
    log(f"  heads 0, 63: out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
    assert eo <= F32_TOL and es <= F32_TOL


def test_decode_states_beyond_4gib():
    # maximum size: 1100 sequences of 64 heads hold 4.3 GiB of fp32 states, so
    # the last 76 sequences' states lie past 4 GiB; two steps, the last 8
    # sequences (every head) against the oracle, and the first sequence too
    B, H, d = 1100, 64, 128
    log(f"decode B{B} H{H} d{d} bf16 (4.3 GiB of states), 2 steps")
    dec = inputs.make_decode(B, H, d, 2, torch.bfloat16, seed=1014, device=DEV)
    st = dec.state.clone()
    rows = list(range(B - 8, B)) + [0]
    idx = torch.tensor(rows, device=DEV)
    ref = np64(dec.state.index_select(0, idx))
    s64 = np64(dec.slopes)
    for t in range(2):
        o = binding.decode_step(dec.q[t], dec.k[t], dec.v[t], dec.slopes, st)
        o_ref, ref = oracle.decode_step(np64(dec.q[t].index_select(0, idx)),
                                        np64(dec.k[t].index_select(0, idx)),
                                        np64(dec.v[t].index_select(0, idx)), s64, ref)
        e = rel_l2(o.index_select(0, idx), o_ref)
        log(f"  step {t}: out rel-L2 {e:.3e} (sequences {B - 8}..{B - 1} and 0)")
        assert e <= BF16_TOL and e <= BF16_GUARD, (t, e)
    es = rel_l2(st.index_select(0, idx), ref)
    log(f"  final states rel-L2 {es:.3e}")
    assert es <= DECODE_STATE_GUARD


# ---- edge cases ------------------------------------------------------------

EDGE_SLOPES = [0.0, 0.5, 30.0]       # lambda = 1, 0.61, ~1e-13


def small_inputs(B, H, N, d, dtype, seed, slopes=None, state=True):
    inp = inputs.make_prefill(B, H, N, d, dtype, seed, init_state=state, device="cpu")
    s = inp.slopes if slopes is None else torch.tensor(slopes, dtype=torch.float32)
    return inputs.PrefillInputs(inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV), s.to(DEV),
                                inp.state.to(DEV))


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 5, 63, 64, 65, 200, 1000])
def test_ragged_lengths_and_decay_extremes(dtype, tol, d, N):
    inp = small_inputs(2, 3, N, d, dtype, seed=N * 7 + d, slopes=EDGE_SLOPES)
    check_prefill(inp, tol, what=f"{dtype} d{d} N{N}")


@pytest.mark.parametrize("dtype,tol,N", [(torch.float32, F32_TOL, 8192),
                                         (torch.bfloat16, BF16_TOL, 32768)])
def test_long_sequence_with_slow_decay(dtype, tol, N):
    # decays close to 1 (lambda = 0.9999 .. 0.999) let the state accumulate over
    # the whole sequence, so the inter term (the state's bf16 copy in the bf16
    # kernel, the fp32 state registers on the fp32 matrix cores in the fp32
    # one) dominates the outputs
    inp = small_inputs(1, 2, N, 128, dtype, seed=N + 17, slopes=[1e-4, 1e-3])
    check_prefill(inp, tol, what=f"{dtype} N{N} slow decay")


def test_fp32_at_the_benchmarked_shape():
    # the fp32 path at the shape its benchmark line times (64 heads, 32K tokens
    # and a ragged tail, 128 channels, a random fp32 initial state): all 256
    # workgroups, every head against the oracle at the fp32 bar
    x = inputs.make_prefill(1, 64, 32768 + 21, 128, torch.float32, seed=1012, init_state=True,
                            device=DEV)
    log("fp32 prefill B1 H64 N32789 d128, random initial state")
    st = x.state.clone()
    out = binding.prefill(x.q, x.k, x.v, x.slopes, st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(x.q, x.k, x.v, x.slopes, x.state)
    eo, es = rel_l2(out, o_ref), rel_l2(st, s_ref)
    log(f"  out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
    assert eo <= F32_TOL and es <= F32_TOL


@pytest.mark.parametrize("H", [1, 2, 5, 8])
def test_head_counts_and_grid_mapping(H):
    # grids that are and are not multiples of the 8 XCDs
    inp = small_inputs(1, H, 300, 128, torch.bfloat16, seed=H)
    check_prefill(inp, BF16_TOL, what=f"H{H}")


def test_infinite_slope_means_no_memory():
    inp = small_inputs(1, 2, 130, 128, torch.bfloat16, seed=3, slopes=[math.inf, 1.0])
    check_prefill(inp, BF16_TOL, what="slope inf")


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
@pytest.mark.parametrize("m", [64, 100, 1])
def test_split_with_carried_state(dtype, tol, m):
    N = 333
    inp = small_inputs(1, 4, N, 128, dtype, seed=m)
    o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state)
    st = inp.state.clone()
    o1 = binding.prefill(inp.q[:, :, :m].contiguous(), inp.k[:, :, :m].contiguous(),
                         inp.v[:, :, :m].contiguous(), inp.slopes, st)
    o2 = binding.prefill(inp.q[:, :, m:].contiguous(), inp.k[:, :, m:].contiguous(),
                         inp.v[:, :, m:].contiguous(), inp.slopes, st)
    torch.cuda.synchronize()
    out = torch.cat([o1, o2], dim=2)
    assert rel_l2(out, o_ref) <= tol and rel_l2(st, s_ref) <= tol


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
def test_decode_after_prefill_equals_longer_prefill(dtype, tol):
    N, T = 150, 6
    inp = small_inputs(2, 3, N + T, 128, dtype, seed=11)
    o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state)
    st = inp.state.clone()
    binding.prefill(inp.q[:, :, :N].contiguous(), inp.k[:, :, :N].contiguous(),
                    inp.v[:, :, :N].contiguous(), inp.slopes, st)
    outs = []
    for t in range(N, N + T):
        outs.append(binding.decode_step(inp.q[:, :, t].contiguous(), inp.k[:, :, t].contiguous(),
                                        inp.v[:, :, t].contiguous(), inp.slopes, st))
    torch.cuda.synchronize()
    dec = torch.stack(outs, dim=2)
    assert rel_l2(dec, o_ref[:, :, N:]) <= tol
    assert rel_l2(st, s_ref) <= tol


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_step_matches_oracle(dtype, tol, d):
    dec = inputs.make_decode(3, 5, d, 4, dtype, seed=d, device="cpu")
    st = dec.state.to(DEV)
    s = torch.tensor([0.0, 0.2, 1.0, 7.0, math.inf], dtype=torch.float32)
    ref = np64(dec.state)
    for t in range(4):
        o = binding.decode_step(dec.q[t].to(DEV), dec.k[t].to(DEV), dec.v[t].to(DEV), s.to(DEV), st)
        o_ref, ref = oracle.decode_step(np64(dec.q[t]), np64(dec.k[t]), np64(dec.v[t]), np64(s), ref)
        assert rel_l2(o, o_ref) <= tol
    assert rel_l2(st, ref) <= tol


def test_empty_sequence_leaves_state_untouched():
    inp = small_inputs(1, 2, 0, 128, torch.bfloat16, seed=1)
    st = inp.state.clone()
    out = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st)
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 128) and torch.equal(st, inp.state)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bitwise_deterministic(dtype):
    inp = small_inputs(1, 8, 777, 128, dtype, seed=5)
    o1, s1 = gpu_prefill(inp)
    o2, s2 = gpu_prefill(inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_aliasing_output_is_rejected():
    inp = small_inputs(1, 2, 64, 128, torch.bfloat16, seed=2)
    st = inp.state.clone()
    with pytest.raises(binding.LightningAttnError):
        binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st, out=inp.q)
    q1 = inp.q[:, :, 0].contiguous()
    with pytest.raises(binding.LightningAttnError):
        binding.decode_step(q1, q1, q1, inp.slopes, st, out=q1)


def test_runs_on_a_non_default_stream():
    inp = small_inputs(1, 4, 500, 128, torch.bfloat16, seed=9)
    o_ref, s_ref = oracle_prefill(inp.q, inp.k, inp.v, inp.slopes, inp.state)
    s = torch.cuda.Stream()
    st = inp.state.clone()
    torch.cuda.current_stream().synchronize()
    with torch.cuda.stream(s):
        out = binding.prefill(inp.q, inp.k, inp.v, inp.slopes, st)
    s.synchronize()
    assert rel_l2(out, o_ref) <= BF16_TOL and rel_l2(st, s_ref) <= BF16_TOL


def test_large_values_stay_finite():
    # |q.k| up to ~1e2 per token and lambda = 1 over 2000 tokens: state grows
    # to O(1e3); fp32 accumulation must keep the same relative accuracy
    inp = small_inputs(1, 2, 2000, 128, torch.bfloat16, seed=4, slopes=[0.0, 0.001])
    scale = 10.0
    inp = inputs.PrefillInputs((inp.q.float() * scale).bfloat16(), (inp.k.float() * scale).bfloat16(),
                               inp.v, inp.slopes, inp.state)
    check_prefill(inp, BF16_TOL, what="large values")
