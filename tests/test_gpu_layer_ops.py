"""GPU parity for the layer's neighbouring ops (la_qk_norm_rope,
la_group_norm_gate) through the C ABI, against the fp64 oracle in
oracle/layer_ops.py on the same seeded bytes.  Bar: max over rows of the
relative L2 error <= 1e-2 (one bf16 rounding of the output is at most 2^-9
relative per element; the fp32 arithmetic adds ~1e-6), v bitwise."""
import numpy as np
import pytest
import torch

from long_context_layers_amd import binding
from oracle import layer_ops as lo
from tests.gpu_util import log, np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def rows_err(x, ref):
    x = np.asarray(x, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    num = np.linalg.norm(x - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))


def packed_projection(B, N, H, d, seed, extra=1):
    """one [B,N,(3+extra)*H*d] bf16 buffer, as a fused projection writes it"""
    g = torch.Generator(device=DEV).manual_seed(seed)
    buf = torch.randn((B, N, (3 + extra) * H * d), generator=g, device=DEV).to(torch.bfloat16)
    return buf, [buf[..., i * H * d:(i + 1) * H * d] for i in range(3 + extra)]


@pytest.mark.parametrize("d,rot", [(128, 64), (128, 0), (128, 16), (128, 128), (64, 64), (64, 32)])
def test_qk_norm_rope_matches_oracle(d, rot):
    B, N, H = 2, 37, 4
    pos0 = 1000
    log(f"qk_norm_rope B{B} N{N} H{H} d{d} rot{rot} pos0 {pos0}")
    _, (q, k, v, _) = packed_projection(B, N, H, d, 200 + d + rot)
    g = torch.Generator(device=DEV).manual_seed(300 + d)
    wq = (1 + 0.1 * torch.randn(d, generator=g, device=DEV)).float()
    wk = (1 + 0.1 * torch.randn(d, generator=g, device=DEV)).float()
    qo, ko, vo = binding.qk_norm_rope(q, k, v, wq, wk, H, theta=6e6, rot_dim=rot, pos0=pos0)
    torch.cuda.synchronize()
    r = lo.qk_norm_rope(*(np64(x).reshape(B, N, H, d) for x in (q, k, v)), np64(wq), np64(wk),
                        6e6, rot, pos0, 1e-6)
    eq, ek = rows_err(np64(qo), r[0]), rows_err(np64(ko), r[1])
    log(f"  q rel-L2 {eq:.3e}  k rel-L2 {ek:.3e}")
    assert eq <= TOL and ek <= TOL
    assert torch.equal(vo, v.reshape(B, N, H, d).permute(0, 2, 1, 3))


def test_qk_norm_rope_long_context_positions():
    # positions near 256K with the pages' base (6e6) and rotary dim (64): the
    # fastest pair turns by ~262,000 rad, so the angle must be reduced exactly
    B, N, H, d = 1, 40, 8, 128
    pos0 = 262144 - N
    log(f"qk_norm_rope at positions {pos0}..{pos0 + N - 1}")
    _, (q, k, v, _) = packed_projection(B, N, H, d, 210)
    w = torch.ones(d, device=DEV)
    qo, ko, _ = binding.qk_norm_rope(q, k, v, w, w, H, theta=6e6, rot_dim=64, pos0=pos0)
    torch.cuda.synchronize()
    r = lo.qk_norm_rope(*(np64(x).reshape(B, N, H, d) for x in (q, k, v)), np64(w), np64(w),
                        6e6, 64, pos0, 1e-6)
    eq, ek = rows_err(np64(qo), r[0]), rows_err(np64(ko), r[1])
    log(f"  q rel-L2 {eq:.3e}  k rel-L2 {ek:.3e}")
    assert eq <= TOL and ek <= TOL


@pytest.mark.parametrize("d,group", [(128, 128), (128, 64), (128, 8), (64, 64), (64, 16)])
def test_group_norm_gate_matches_oracle(d, group):
    B, N, H = 2, 37, 4
    log(f"group_norm_gate B{B} N{N} H{H} d{d} group {group}")
    g = torch.Generator(device=DEV).manual_seed(400 + d + group)
    o = torch.randn((B, H, N, d), generator=g, device=DEV).to(torch.bfloat16)
    _, (_, _, _, gate) = packed_projection(B, N, H, d, 500 + d)
    w = (1 + 0.1 * torch.randn(H * d, generator=g, device=DEV)).float()
    y = binding.group_norm_gate(o, gate, w, group=group)
    torch.cuda.synchronize()
    ref = lo.group_norm_gate(np64(o), np64(gate), np64(w), group, 1e-6)
    e = rows_err(np64(y), ref)
    log(f"  y rel-L2 {e:.3e}")
    assert e <= TOL


def test_layer_ops_at_256k_sampled_tokens():
    # the bench's shape (B1 N262144 H64 d128, a 16 GiB projection buffer):
    # both kernels over every token, checked against the oracle on the first,
    # middle and last 64 tokens (every head; rotary positions up to 2^18)
    B, N, H, d = 1, 262144, 64, 128
    log(f"layer ops at B{B} N{N} H{H} d{d}, sampled tokens against the oracle")
    _, (q, k, v, gate) = packed_projection(B, N, H, d, 700)
    g = torch.Generator(device=DEV).manual_seed(701)
    wq = (1 + 0.1 * torch.randn(d, generator=g, device=DEV)).float()
    wk = (1 + 0.1 * torch.randn(d, generator=g, device=DEV)).float()
    w = (1 + 0.1 * torch.randn(H * d, generator=g, device=DEV)).float()
    qo, ko, vo = binding.qk_norm_rope(q, k, v, wq, wk, H, theta=6e6, rot_dim=64, pos0=0)
    y = binding.group_norm_gate(qo, gate, w, group=d)
    torch.cuda.synchronize()
    for t0 in (0, N // 2 - 32, N - 64):
        t1 = t0 + 64
        r = lo.qk_norm_rope(*(np64(x[:, t0:t1]).reshape(B, t1 - t0, H, d) for x in (q, k, v)),
                            np64(wq), np64(wk), 6e6, 64, t0, 1e-6)
        eq, ek = rows_err(np64(qo[:, :, t0:t1]), r[0]), rows_err(np64(ko[:, :, t0:t1]), r[1])
        assert torch.equal(vo[:, :, t0:t1], v[:, t0:t1].reshape(B, t1 - t0, H, d).permute(0, 2, 1, 3))
        ref = lo.group_norm_gate(np64(qo[:, :, t0:t1]), np64(gate[:, t0:t1]), np64(w), d, 1e-6)
        ey = rows_err(np64(y[:, t0:t1]), ref)
        log(f"  tokens {t0}..{t1 - 1}: q {eq:.3e}  k {ek:.3e}  y {ey:.3e}")
        assert eq <= TOL and ek <= TOL and ey <= TOL


def test_layer_chain_matches_oracle():
    # projection outputs -> QK norm + RoPE -> prefill -> grouped norm x gate,
    # every stage on the GPU, against the same chain in fp64 (bar 2e-2: the
    # prefill's own bf16 bound)
    B, N, H, d = 1, 300, 4, 128
    log(f"layer chain B{B} N{N} H{H} d{d}")
    _, (q, k, v, gate) = packed_projection(B, N, H, d, 600)
    gw = torch.Generator(device=DEV).manual_seed(601)
    wq, wk = ((1 + 0.1 * torch.randn(d, generator=gw, device=DEV)).float() for _ in range(2))
    wo = (1 + 0.1 * torch.randn(H * d, generator=gw, device=DEV)).float()
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], device=DEV)
    qo, ko, vo = binding.qk_norm_rope(q, k, v, wq, wk, H, rot_dim=64)
    qo.mul_(1.0 / np.sqrt(d))        # keep the synthetic scores in a typical range
    st = torch.zeros((B, H, d, d), device=DEV)
    o = binding.prefill(qo, ko, vo, slopes, st)
    y = binding.group_norm_gate(o, gate, wo)
    torch.cuda.synchronize()
    import oracle
    rq, rk, rv = lo.qk_norm_rope(*(np64(x).reshape(B, N, H, d) for x in (q, k, v)), np64(wq),
                                 np64(wk), 6e6, 64, 0, 1e-6)
    ro, _ = oracle.prefill(rq / np.sqrt(d), rk, rv, np64(slopes))
    ry = lo.group_norm_gate(ro, np64(gate), np64(wo), d, 1e-6)
    e = rows_err(np64(y), ry)
    log(f"  y rel-L2 {e:.3e} (bar 2e-2)")
    assert e <= 2e-2
