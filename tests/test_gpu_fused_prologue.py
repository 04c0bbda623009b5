"""GPU parity of the prefill with QK Norm + RoPE fused into its loads
(la_prefill_qk_norm_rope_ws) through the C ABI: the raw q and k of a packed
token-major projection buffer go in, and the output and final state are held
to the fp64 oracle chain (oracle/layer_ops.py's qk_norm_rope, then the
prefill oracle) on the same seeded bytes: bf16 bar 2e-2 and the 4e-3 guard.
Cases: every supported rotary dim, positions far from 0, a batch, a ragged
tail, a random initial state, the sequence split (with decays slow enough
that the correction spans whole segments), the 256K layer shape on sampled
heads, and agreement with the two-call path (la_qk_norm_rope in place, then
la_prefill_strided_ws) on every head."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_layers_amd import binding, inputs
from oracle import layer_ops as lo
from tests.gpu_util import BF16_GUARD, BF16_TOL, log, np64, rel_l2
from tests.test_gpu_strided import heads_view

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 128
THETA, EPS = 6.0e6, 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def projection(B, N, H, seed, pad=8):
    """one [B,N,3*H*d + pad] bf16 buffer (a fused QKV projection's output) and
    the [B,H,N,d] views of q, k and v inside it"""
    g = torch.Generator(device=DEV).manual_seed(seed)
    buf = torch.randn((B, N, 3 * H * D + pad), generator=g, device=DEV).to(torch.bfloat16)
    return buf, [heads_view(buf, i * H * D, H, D) for i in range(3)]


def weights(seed):
    # q's weight also carries 1/sqrt(d), so the synthetic scores stay in a
    # typical range (RoPE is linear, so the scale passes through it)
    g = torch.Generator(device=DEV).manual_seed(seed)
    wq = ((1 + 0.1 * torch.randn(D, generator=g, device=DEV)) / math.sqrt(D)).float()
    wk = (1 + 0.1 * torch.randn(D, generator=g, device=DEV)).float()
    return wq, wk


def oracle_chain(q, k, v, wq, wk, slopes, state0, rot, pos0, heads=None):
    """fp64: QK Norm + RoPE on the raw rows, then the prefill (optionally a
    subset of heads)"""
    if heads is not None:
        idx = torch.tensor(heads, device=DEV)
        q, k, v = (t.index_select(1, idx) for t in (q, k, v))
        slopes, state0 = slopes.index_select(0, idx), state0.index_select(1, idx)
    tm = [np64(t).transpose(0, 2, 1, 3) for t in (q, k, v)]       # [B,N,H,d]
    rq, rk, rv = lo.qk_norm_rope(*tm, np64(wq), np64(wk), THETA, rot, pos0, EPS)
    return oracle.prefill(rq, rk, rv, np64(slopes), np64(state0))


def check(out, st, ref, what, heads=None):
    o, s = out, st
    if heads is not None:
        idx = torch.tensor(heads, device=DEV)
        o, s = out.index_select(1, idx), st.index_select(1, idx)
    eo, es = rel_l2(o, ref[0]), rel_l2(s, ref[1])
    log(f"  {what}: out rel-L2 {eo:.3e}  state {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
    assert eo <= BF16_GUARD and es <= BF16_GUARD, "precision regression"


@pytest.mark.parametrize("B,H,N,rot,pos0", [
    (2, 4, 300, 64, 0),          # the layer's rotary dim, a ragged tail, a batch
    (1, 4, 300, 64, 1000),
    (1, 3, 129, 0, 0),           # no rotation
    (1, 4, 200, 16, 7),
    (1, 4, 200, 32, 0),
    (2, 2, 190, 128, 12345),     # every channel rotates
    (1, 2, 64, 64, 0),           # exactly one block
    (1, 2, 1, 64, 5),            # one token
    (2, 64, 300, 64, 3),         # a batch at 64 heads: 64-column workgroups without the split
])
def test_fused_prologue_matches_oracle(B, H, N, rot, pos0):
    log(f"fused prologue B{B} H{H} N{N} d{D} rot{rot} pos0 {pos0}")
    _, (q, k, v) = projection(B, N, H, 900 + N + rot)
    wq, wk = weights(901 + rot)
    slopes = inputs.slopes(H, DEV)
    st0 = inputs.make_prefill(B, H, 1, D, torch.bfloat16, 902, init_state=True, device=DEV).state
    st = st0.clone()
    out = binding.prefill_qk_norm_rope(q, k, v, slopes, st, wq, wk, THETA, rot, pos0, EPS)
    torch.cuda.synchronize()
    check(out, st, oracle_chain(q, k, v, wq, wk, slopes, st0, rot, pos0), "fused")


def test_fused_prologue_far_positions_token_major_out():
    # positions near 2^20: the fastest pair turns by ~10^6 rad, so the angle
    # reduction must be exact; the output goes to a token-major buffer
    B, H, N, rot, pos0 = 1, 4, 333, 64, (1 << 20) - 100
    log(f"fused prologue at positions {pos0}.., token-major out")
    _, (q, k, v) = projection(B, N, H, 910)
    wq, wk = weights(911)
    slopes = inputs.slopes(H, DEV)
    st0 = torch.zeros((B, H, D, D), device=DEV)
    obuf = torch.full((B, N, H * D + 8), -7.0, dtype=torch.bfloat16, device=DEV)
    out = heads_view(obuf, 0, H, D)
    st = st0.clone()
    binding.prefill_qk_norm_rope(q, k, v, slopes, st, wq, wk, THETA, rot, pos0, EPS, out=out)
    torch.cuda.synchronize()
    check(out, st, oracle_chain(q, k, v, wq, wk, slopes, st0, rot, pos0), "fused, token-major")
    assert bool((obuf[..., H * D:] == -7.0).all()), "padding columns written"


def need_split(H, N):
    ws = binding.prefill_workspace_bytes(1, H, N, D, DEV)
    if ws == 0:
        pytest.skip(f"no split for H{H} N{N} on this device")
    return ws


@pytest.mark.parametrize("H,N,slopes,pos0", [
    (8, 40000 + 77, [0.0, 1e-4, 1e-3, 0.01, 0.1, 1.0, 5.0, math.inf], 0),
    (64, 40000, None, 3000),
])
def test_fused_prologue_split_matches_oracle(H, N, slopes, pos0):
    ws = need_split(H, N)
    log(f"fused prologue, split: B1 H{H} N{N} pos0 {pos0} (workspace {ws} B), slopes {slopes or 'model'}")
    _, (q, k, v) = projection(1, N, H, 920 + H)
    wq, wk = weights(921)
    sl = (torch.tensor(slopes, dtype=torch.float32, device=DEV) if slopes is not None
          else inputs.slopes(H, DEV))
    st0 = inputs.make_prefill(1, H, 1, D, torch.bfloat16, 922, init_state=True, device=DEV).state
    st = st0.clone()
    out = binding.prefill_qk_norm_rope(q, k, v, sl, st, wq, wk, THETA, 64, pos0, EPS)
    torch.cuda.synchronize()
    heads = list(range(H)) if H <= 8 else [0, 1, H // 2, H - 1]
    check(out, st, oracle_chain(q, k, v, wq, wk, sl, st0, 64, pos0, heads=heads),
          f"fused split, heads {heads}", heads=heads)


def test_fused_prologue_layer_256k():
    # the layer's shape: B1 H64 N262144 from one packed projection buffer, as
    # the benchmark times it; the oracle on 4 heads (slowest and fastest decay
    # among them), the two-call GPU path on all 64
    B, H, N = 1, 64, 262144
    log(f"fused prologue, layer shape B{B} H{H} N{N}")
    buf, (q, k, v) = projection(B, N, H, 930)
    wq, wk = weights(931)
    slopes = inputs.slopes(H, DEV)
    st0 = torch.zeros((B, H, D, D), device=DEV)
    st = st0.clone()
    out = binding.prefill_qk_norm_rope(q, k, v, slopes, st, wq, wk, THETA, 64, 0, EPS)
    torch.cuda.synchronize()
    heads = [0, 21, 42, 63]
    check(out, st, oracle_chain(q, k, v, wq, wk, slopes, st0, 64, 0, heads=heads),
          f"fused 256K, heads {heads}", heads=heads)
    # the two-call path: QK Norm + RoPE in place over the projection, then the
    # strided prefill (differs only in where q and k are rounded to bf16)
    qk = buf[..., :2 * H * D]
    binding.qk_norm_rope(qk[..., :H * D], qk[..., H * D:], None, wq, wk, H, THETA, 64, 0, EPS,
                         inplace=True)
    st2 = st0.clone()
    out2 = binding.prefill(q, k, v, slopes, st2)
    torch.cuda.synchronize()
    e_o, e_s = rel_l2(out, out2), rel_l2(st, st2)
    log(f"  fused vs two-call, all heads: out {e_o:.3e}  state {e_s:.3e}")
    assert e_o <= BF16_GUARD and e_s <= BF16_GUARD


def test_fused_prologue_deterministic():
    B, H, N = 1, 8, 40000
    _, (q, k, v) = projection(B, N, H, 940)
    wq, wk = weights(941)
    slopes = inputs.slopes(H, DEV)
    outs = []
    for _ in range(2):
        st = torch.zeros((B, H, D, D), device=DEV)
        outs.append((binding.prefill_qk_norm_rope(q, k, v, slopes, st, wq, wk), st))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_fused_prologue_batch_without_split_contiguous_inputs():
    # B > 1 never splits: one workgroup per (b, head, 32 columns) through 129
    # blocks; q, k, v contiguous [B,H,N,d] (token stride d) rather than views
    B, H, N, rot, pos0 = 2, 4, 8192 + 33, 64, 17
    log(f"fused prologue B{B} H{H} N{N} contiguous, no split")
    _, (q, k, v) = projection(B, N, H, 950)
    q, k, v = (t.contiguous() for t in (q, k, v))
    assert binding.prefill_workspace_bytes(B, H, N, D, DEV) == 0
    wq, wk = weights(951)
    slopes = inputs.slopes(H, DEV)
    st0 = inputs.make_prefill(B, H, 1, D, torch.bfloat16, 952, init_state=True, device=DEV).state
    st = st0.clone()
    out = binding.prefill_qk_norm_rope(q, k, v, slopes, st, wq, wk, THETA, rot, pos0, EPS)
    torch.cuda.synchronize()
    check(out, st, oracle_chain(q, k, v, wq, wk, slopes, st0, rot, pos0), "fused, B2 contiguous")


def test_fused_prologue_positions_near_2_40():
    # the exact fp64 reduction of the angles at positions about 10^12 (the
    # fastest pair turns by about 10^12 rad) and the block-to-block turns from there
    B, H, N, rot, pos0 = 1, 2, 2000, 64, (1 << 40) + 12345
    log(f"fused prologue at positions {pos0}..")
    _, (q, k, v) = projection(B, N, H, 960)
    wq, wk = weights(961)
    slopes = inputs.slopes(H, DEV)
    st0 = torch.zeros((B, H, D, D), device=DEV)
    st = st0.clone()
    out = binding.prefill_qk_norm_rope(q, k, v, slopes, st, wq, wk, THETA, rot, pos0, EPS)
    torch.cuda.synchronize()
    check(out, st, oracle_chain(q, k, v, wq, wk, slopes, st0, rot, pos0), "fused, positions ~2^40")


def test_fused_prologue_empty_sequence_is_a_noop():
    B, H = 1, 2
    _, (q, k, v) = projection(B, 1, H, 970)
    q, k, v = (t[:, :, :0] for t in (q, k, v))
    wq, wk = weights(971)
    st = torch.randn((B, H, D, D), device=DEV)
    ref = st.clone()
    out = binding.prefill_qk_norm_rope(q, k, v, inputs.slopes(H, DEV), st, wq, wk)
    torch.cuda.synchronize()
    assert out.shape == (B, H, 0, D) and torch.equal(st, ref)


def test_fused_prologue_replayed_from_a_graph():
    # the call with a caller-held workspace captured once and replayed: each
    # replay bitwise against the eager call on the same inputs
    B, H, N = 1, 32, 40000
    ws = binding.prefill_workspace_bytes(B, H, N, D, DEV)
    log(f"graph: la_prefill_qk_norm_rope_ws B{B} H{H} N{N} (workspace {ws} B), 3 replays")
    lib = binding.load_library()
    buf, (q, k, v) = projection(B, N, H, 980)
    wq, wk = weights(981)
    slopes = inputs.slopes(H, DEV)
    st0 = inputs.make_prefill(B, H, 1, D, torch.bfloat16, 982, init_state=True, device=DEV).state
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=DEV)
    state = st0.clone()
    si = q.stride()[:-1]

    def call(o, stt):
        rc = lib.la_prefill_qk_norm_rope_ws(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), wq.data_ptr(), wk.data_ptr(),
            THETA, 64, 0, EPS, o.data_ptr(), stt.data_ptr(), B, H, N, D, *si, *o.stride()[:-1],
            work.data_ptr() if ws else None, ws, torch.cuda.current_stream().cuda_stream)
        assert rc == 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(torch.empty_like(out), st0.clone())
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, state)
    for r in range(3):
        state.copy_(st0)
        g.replay()
        ref_state = st0.clone()
        ref = torch.empty_like(out)
        call(ref, ref_state)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert torch.equal(state, ref_state), r
