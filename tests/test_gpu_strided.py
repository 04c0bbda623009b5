"""GPU checks of the strided calls (la_prefill_strided, la_prefill_varlen_strided,
in-place la_qk_norm_rope, la_group_norm_gate on a token-major o) through the
C ABI.  A strided call does the same arithmetic in the same order as the
contiguous call on the same values, so the bar is bitwise equality with the
contiguous results (themselves held to the fp64 oracle by the other GPU
tests), plus one direct oracle comparison and checks that padding between
strided output rows is never written."""
import numpy as np
import pytest
import torch

import oracle
from long_context_layers_amd import binding, inputs
from oracle import layer_ops as lo
from tests.gpu_util import BF16_TOL, log, np64, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = -7.0          # exactly representable in bf16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def heads_view(buf, col0, H, d):
    """[B,N,X] token-major buffer -> [B,H,N,d] view of columns col0 .. col0+H*d"""
    return buf[..., col0:col0 + H * d].unflatten(-1, (H, d)).transpose(-3, -2)


def pack_token_major(tensors, pad):
    """[B,H,N,d] tensors -> one [B,N,len*H*d + pad] buffer (pad columns hold the
    sentinel) and the [B,H,N,d] views of each tensor inside it"""
    B, H, N, d = tensors[0].shape
    buf = torch.full((B, N, len(tensors) * H * d + pad), SENTINEL, dtype=tensors[0].dtype,
                     device=DEV)
    views = []
    for i, t in enumerate(tensors):
        v = heads_view(buf, i * H * d, H, d)
        v.copy_(t)
        views.append(v)
    return buf, views


@pytest.mark.parametrize("d", [64, 128])
def test_strided_prefill_bitwise_equals_contiguous(d):
    B, H, N = 2, 4, 300                               # 4 full blocks and a ragged tail
    log(f"strided prefill B{B} H{H} N{N} d{d}")
    x = inputs.make_prefill(B, H, N, d, torch.bfloat16, seed=90 + d, init_state=True, device=DEV)
    st_ref = x.state.clone()
    out_ref = binding.prefill(x.q, x.k, x.v, x.slopes, st_ref)
    _, (qv, kv, vv) = pack_token_major([x.q, x.k, x.v], pad=24)
    obuf = torch.full((B, N, H * d + 40), SENTINEL, dtype=torch.bfloat16, device=DEV)
    ov = heads_view(obuf, 0, H, d)
    st = x.state.clone()
    binding.prefill(qv, kv, vv, x.slopes, st, out=ov)
    torch.cuda.synchronize()
    assert qv.stride() == (N * (3 * H * d + 24), d, 3 * H * d + 24, 1)
    assert torch.equal(ov, out_ref), "strided output differs from the contiguous call"
    assert torch.equal(st, st_ref), "strided final state differs from the contiguous call"
    assert bool((obuf[..., H * d:] == SENTINEL).all()), "padding between output rows was written"


def test_strided_prefill_matches_oracle():
    B, H, N, d = 1, 2, 200, 128
    log(f"strided prefill vs oracle B{B} H{H} N{N} d{d}")
    x = inputs.make_prefill(B, H, N, d, torch.bfloat16, seed=95, init_state=True, device=DEV)
    _, (qv, kv, vv) = pack_token_major([x.q, x.k, x.v], pad=0)
    st = x.state.clone()
    o = binding.prefill(qv, kv, vv, x.slopes, st)       # contiguous out, strided inputs
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.prefill(np64(x.q), np64(x.k), np64(x.v), np64(x.slopes), np64(x.state))
    eo, es = rel_l2(o, o_ref), rel_l2(st, s_ref)
    log(f"  out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_strided_prefill_contiguous_inputs_strided_output():
    B, H, N, d = 1, 3, 129, 64
    log(f"strided output only B{B} H{H} N{N} d{d}")
    x = inputs.make_prefill(B, H, N, d, torch.bfloat16, seed=96, device=DEV)
    st_ref = x.state.clone()
    out_ref = binding.prefill(x.q, x.k, x.v, x.slopes, st_ref)
    obuf = torch.full((B, N, H * d), SENTINEL, dtype=torch.bfloat16, device=DEV)
    st = x.state.clone()
    binding.prefill(x.q, x.k, x.v, x.slopes, st, out=heads_view(obuf, 0, H, d))
    torch.cuda.synchronize()
    assert torch.equal(heads_view(obuf, 0, H, d), out_ref) and torch.equal(st, st_ref)


MIXED = [0, 1, 63, 64, 65, 130, 0, 1000, 7, 257]


@pytest.mark.parametrize("d", [64, 128])
def test_strided_varlen_bitwise_equals_contiguous(d):
    H = 4
    log(f"strided varlen {MIXED} H{H} d{d}")
    x = inputs.make_varlen(H, MIXED, d, torch.bfloat16, seed=97 + d, init_state=True, device=DEV)
    st_ref = x.states.clone()
    out_ref = binding.prefill_varlen(x.q, x.k, x.v, x.slopes, x.cu_seqlens, st_ref)
    # packed token-major buffer [T, q|k|v|pad]; [H,T,d] views
    _, (qv, kv, vv) = pack_token_major([t[None] for t in (x.q, x.k, x.v)], pad=16)
    qv, kv, vv = qv[0], kv[0], vv[0]
    T = sum(MIXED)
    obuf = torch.full((T, H * d + 8), SENTINEL, dtype=torch.bfloat16, device=DEV)
    ov = obuf[:, :H * d].unflatten(-1, (H, d)).transpose(0, 1)
    st = x.states.clone()
    binding.prefill_varlen(qv, kv, vv, x.slopes, x.cu_seqlens, st, out=ov)
    torch.cuda.synchronize()
    assert torch.equal(ov, out_ref) and torch.equal(st, st_ref)
    assert bool((obuf[:, H * d:] == SENTINEL).all())


def test_strided_prefill_full_256k_bitwise():
    # the 256K-token, 64-head, d = 128 workload in the launch the layer uses:
    # q, k, v read from one token-major projection buffer, out written
    # token-major, against the contiguous launch on the same values (both
    # with the sequence split: la_prefill_strided_ws against la_prefill_ws)
    w = inputs.WORKLOADS["prefill_256k"]
    log(f"strided prefill 256K: B{w.B} H{w.H} N{w.N} d{w.d}")
    x = inputs.make_workload("prefill_256k", device=DEV)
    st_ref = x.state.clone()
    out_ref = binding.prefill(x.q, x.k, x.v, x.slopes, st_ref)    # la_prefill_ws (the split)
    _, (qv, kv, vv) = pack_token_major([x.q, x.k, x.v], pad=0)
    obuf = torch.empty((w.B, w.N, w.H * w.d), dtype=torch.bfloat16, device=DEV)
    st = torch.zeros_like(st_ref)
    binding.prefill(qv, kv, vv, x.slopes, st, out=heads_view(obuf, 0, w.H, w.d))
    torch.cuda.synchronize()
    assert torch.equal(heads_view(obuf, 0, w.H, w.d), out_ref)
    assert torch.equal(st, st_ref)


def test_strided_fp32_is_refused():
    # the strided calls take bf16 only: fp32 views raise in the binding
    buf = torch.zeros((1, 64, 3 * 2 * 64), dtype=torch.float32, device=DEV)
    q, k, v = (heads_view(buf, i * 128, 2, 64) for i in range(3))
    with pytest.raises(ValueError):
        binding.prefill(q, k, v, inputs.slopes(2, DEV), torch.zeros((1, 2, 64, 64), device=DEV))


def projection(B, N, H, d, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    buf = torch.randn((B, N, 4 * H * d), generator=g, device=DEV).to(torch.bfloat16)
    return buf, [buf[..., i * H * d:(i + 1) * H * d] for i in range(4)]


@pytest.mark.parametrize("d,rot", [(128, 64), (64, 32)])
def test_qk_norm_rope_in_place_bitwise(d, rot):
    B, N, H = 2, 37, 4
    log(f"qk_norm_rope in place B{B} N{N} H{H} d{d} rot{rot}")
    buf, (q, k, v, _) = projection(B, N, H, d, 700 + d)
    wq = torch.linspace(0.5, 1.5, d, device=DEV)
    wk = torch.linspace(1.5, 0.5, d, device=DEV)
    qo, ko, vo = binding.qk_norm_rope(q, k, v, wq, wk, H, rot_dim=rot, pos0=17)
    v_before = v.clone()
    rest_before = buf[..., 2 * H * d:].clone()
    qi, ki, none = binding.qk_norm_rope(q, k, None, wq, wk, H, rot_dim=rot, pos0=17, inplace=True)
    torch.cuda.synchronize()
    assert none is None
    assert qi.data_ptr() == q.data_ptr() and ki.data_ptr() == k.data_ptr()
    assert torch.equal(qi, qo) and torch.equal(ki, ko)
    assert torch.equal(buf[..., 2 * H * d:], rest_before), "v or gate columns were written"
    assert torch.equal(vo, v_before.unflatten(-1, (H, d)).transpose(1, 2))


def test_qk_norm_rope_in_place_with_v_copied_out():
    # q, k normed and rotated in place while v is still moved to [B,H,N,d]
    B, N, H, d = 1, 40, 4, 128
    log(f"qk_norm_rope in place with v out B{B} N{N} H{H} d{d}")
    buf, (q, k, v, _) = projection(B, N, H, d, 750)
    w = torch.linspace(0.7, 1.3, d, device=DEV)
    qo, ko, vo = binding.qk_norm_rope(q, k, v, w, w, H, rot_dim=64)
    v_ref = v.clone()
    qi, ki, vi = binding.qk_norm_rope(q, k, v, w, w, H, rot_dim=64, inplace=True)
    torch.cuda.synchronize()
    assert torch.equal(qi, qo) and torch.equal(ki, ko)
    assert torch.equal(vi, vo) and torch.equal(v, v_ref)          # v copied out, not changed


def test_group_norm_gate_token_major_o_bitwise():
    B, N, H, d = 2, 37, 4, 128
    log(f"group_norm_gate token-major o B{B} N{N} H{H} d{d}")
    g = torch.Generator(device=DEV).manual_seed(800)
    o = torch.randn((B, H, N, d), generator=g, device=DEV).to(torch.bfloat16)
    _, (_, _, _, gate) = projection(B, N, H, d, 801)
    w = (1 + 0.1 * torch.randn(H * d, generator=g, device=DEV)).float()
    y_ref = binding.group_norm_gate(o, gate, w, group=64)
    o_tm = torch.empty((B, N, H * d), dtype=torch.bfloat16, device=DEV)
    heads_view(o_tm, 0, H, d).copy_(o)
    y = binding.group_norm_gate(heads_view(o_tm, 0, H, d), gate, w, group=64)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)


def test_layer_chain_without_layout_copies():
    # projection buffer -> QK norm + RoPE in place -> strided prefill straight
    # from the buffer, token-major output -> grouped norm x gate: bitwise the
    # chain through the kernel layout, and within the bf16 bar of the fp64 chain
    B, N, H, d = 1, 300, 4, 128
    log(f"layer chain, strided: B{B} N{N} H{H} d{d}")
    buf, (q, k, v, gate) = projection(B, N, H, d, 900)
    raw = buf.clone()
    wq, wk = torch.linspace(0.8, 1.2, d, device=DEV), torch.linspace(1.2, 0.8, d, device=DEV)
    wo = torch.linspace(0.9, 1.1, H * d, device=DEV)
    slopes = inputs.slopes(H, DEV)
    # through the kernel layout
    qo, ko, vo = binding.qk_norm_rope(q, k, v, wq, wk, H)
    qo.mul_(1.0 / np.sqrt(d))
    st1 = torch.zeros((B, H, d, d), device=DEV)
    y_ref = binding.group_norm_gate(binding.prefill(qo, ko, vo, slopes, st1), gate, wo)
    # no layout copies
    qi, ki, _ = binding.qk_norm_rope(q, k, None, wq, wk, H, inplace=True)
    qi.mul_(1.0 / np.sqrt(d))
    st2 = torch.zeros((B, H, d, d), device=DEV)
    o_tm = torch.empty((B, N, H * d), dtype=torch.bfloat16, device=DEV)
    binding.prefill(qi, ki, heads_view(buf, 2 * H * d, H, d), slopes, st2,
                    out=heads_view(o_tm, 0, H, d))
    y = binding.group_norm_gate(heads_view(o_tm, 0, H, d), gate, wo)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(st2, st1)
    rq, rk, rv = lo.qk_norm_rope(*(np64(t).reshape(B, N, H, d)
                                   for t in (raw[..., :H * d], raw[..., H * d:2 * H * d],
                                             raw[..., 2 * H * d:3 * H * d])),
                                 np64(wq), np64(wk), 6e6, 64, 0, 1e-6)
    ro, _ = oracle.prefill(rq / np.sqrt(d), rk, rv, np64(slopes))
    ry = lo.group_norm_gate(ro, np64(raw[..., 3 * H * d:]), np64(wo), d, 1e-6)
    e = float(np.max(np.linalg.norm(np64(y).reshape(-1, H * d) - ry.reshape(-1, H * d), axis=1)
                     / np.linalg.norm(ry.reshape(-1, H * d), axis=1)))
    log(f"  y rel-L2 {e:.3e} (bar 2e-2)")
    assert e <= 2e-2


@pytest.mark.parametrize("d", [64, 128])
def test_decode_step_strided_bitwise(d):
    # one new token per sequence, q | k | v of all heads in one row per sequence
    B, H = 5, 4
    log(f"strided decode step B{B} H{H} d{d}")
    x = inputs.make_decode(B, H, d, 1, torch.bfloat16, seed=120 + d, device=DEV)
    st_ref = x.state.clone()
    o_ref = binding.decode_step(x.q[0], x.k[0], x.v[0], x.slopes, st_ref)
    row = torch.full((B, 3 * H * d + 16), SENTINEL, dtype=torch.bfloat16, device=DEV)
    qv, kv, vv = (row[:, i * H * d:(i + 1) * H * d].unflatten(-1, (H, d)) for i in range(3))
    for dst, src in ((qv, x.q[0]), (kv, x.k[0]), (vv, x.v[0])):
        dst.copy_(src)
    st = x.state.clone()
    o = binding.decode_step(qv, kv, vv, x.slopes, st)
    torch.cuda.synchronize()
    assert qv.stride() == (3 * H * d + 16, d, 1)
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_multi_strided_bitwise(d):
    # draft tokens straight from a [B, T, 4*H*d] projection buffer
    B, H, T = 3, 4, 4
    log(f"strided multi-token decode B{B} H{H} T{T} d{d}")
    x = inputs.make_decode(B, H, d, T, torch.bfloat16, seed=130 + d, device=DEV)
    q, k, v = (t.permute(1, 2, 0, 3).contiguous() for t in (x.q, x.k, x.v))   # [B,H,T,d]
    ncommit = torch.tensor([1, 4, 0], dtype=torch.int32, device=DEV)
    st_ref = x.state.clone()
    o_ref = binding.decode_multi(q, k, v, x.slopes, st_ref, n_commit=ncommit)
    buf = torch.full((B, T, 4 * H * d), SENTINEL, dtype=torch.bfloat16, device=DEV)
    views = [heads_view(buf, i * H * d, H, d) for i in range(3)]
    for dst, src in zip(views, (q, k, v)):
        dst.copy_(src)
    st = x.state.clone()
    o = binding.decode_multi(*views, x.slopes, st, n_commit=ncommit)
    torch.cuda.synchronize()
    assert views[0].stride() == (T * 4 * H * d, d, 4 * H * d, 1)
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref)
