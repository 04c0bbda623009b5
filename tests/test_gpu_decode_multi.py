"""GPU parity for multi-token decode (la_decode_multi[_f32]) through the C
ABI: against the fp64 oracle on the same seeded bytes (2e-2 bf16, 1e-3 fp32,
max over (b, h) and tokens of the relative L2 error; committed states
likewise), and bitwise against single-token decode steps."""
import numpy as np
import pytest
import torch

import oracle
from long_context_layers_amd import binding, inputs
from tests.gpu_util import BF16_TOL, F32_TOL, log, np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def tokens(dec, T):
    """[B,H,T,d] views of the first T decode tokens ([T,B,H,d] -> [B,H,T,d])."""
    return tuple(x[:T].permute(1, 2, 0, 3).contiguous() for x in (dec.q, dec.k, dec.v))


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
def test_decode_multi_matches_oracle(T, d, dtype, tol):
    B, H = 6, 4
    log(f"decode_multi B{B} H{H} T{T} d{d} {dtype}")
    dec = inputs.make_decode(B, H, d, T, dtype, seed=91 + T + d, device=DEV)
    q, k, v = tokens(dec, T)
    n = torch.tensor([(b * 3) % (T + 1) for b in range(B)], dtype=torch.int32, device=DEV)
    st = dec.state.clone()
    out = binding.decode_multi(q, k, v, dec.slopes, st, n_commit=n)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode_multi(np64(q), np64(k), np64(v), np64(dec.slopes),
                                       np64(dec.state), n.cpu().numpy())
    eo = oracle.rel_l2(np64(out), o_ref, axes=(-1,))
    es = oracle.rel_l2(np64(st), s_ref)
    log(f"  out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}  (tol {tol:g})")
    assert eo <= tol and es <= tol
    for b in range(B):
        if int(n[b]) == 0:
            assert torch.equal(st[b], dec.state[b])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_multi_equals_single_steps_bitwise(dtype):
    B, H, T, d = 8, 8, 4, 128
    log(f"decode_multi vs {T} decode steps, B{B} H{H} d{d} {dtype}")
    dec = inputs.make_decode(B, H, d, T, dtype, seed=95, device=DEV)
    q, k, v = tokens(dec, T)
    st_m = dec.state.clone()
    out_m = binding.decode_multi(q, k, v, dec.slopes, st_m)
    st_s = dec.state.clone()
    outs = [binding.decode_step(dec.q[t], dec.k[t], dec.v[t], dec.slopes, st_s) for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(st_m, st_s)
    for t in range(T):
        assert torch.equal(out_m[:, :, t], outs[t]), f"token {t}"


def test_decode_multi_commit_counts_are_clamped():
    B, H, T, d = 4, 2, 3, 64
    dec = inputs.make_decode(B, H, d, T, torch.bfloat16, seed=96, device=DEV)
    q, k, v = tokens(dec, T)
    n = torch.tensor([-5, 0, 3, 99], dtype=torch.int32, device=DEV)
    st = dec.state.clone()
    binding.decode_multi(q, k, v, dec.slopes, st, n_commit=n)
    st_all = dec.state.clone()
    binding.decode_multi(q, k, v, dec.slopes, st_all)
    torch.cuda.synchronize()
    assert torch.equal(st[0], dec.state[0]) and torch.equal(st[1], dec.state[1])
    assert torch.equal(st[2], st_all[2]) and torch.equal(st[3], st_all[3])


def test_decode_multi_mtp_workload():
    # the benchmark's draft-verification workload: B256 H64 d128, 4 draft
    # tokens, commit counts 1..4; the oracle checks every sequence's first head
    B, H, T, d = 256, 64, 4, 128
    log(f"decode_multi B{B} H{H} T{T} d{d} bf16, random commit counts")
    dec = inputs.make_decode(B, H, d, T, torch.bfloat16, seed=1006, device=DEV)
    q, k, v = tokens(dec, T)
    g = torch.Generator().manual_seed(1006)
    n = torch.randint(1, T + 1, (B,), generator=g, dtype=torch.int32).to(DEV)
    st = dec.state.clone()
    out = binding.decode_multi(q, k, v, dec.slopes, st, n_commit=n)
    torch.cuda.synchronize()
    h = [0, 63]
    o_ref, s_ref = oracle.decode_multi(np64(q[:, h]), np64(k[:, h]), np64(v[:, h]),
                                       np64(dec.slopes[h]), np64(dec.state[:, h]), n.cpu().numpy())
    eo = oracle.rel_l2(np64(out[:, h]), o_ref, axes=(-1,))
    es = oracle.rel_l2(np64(st[:, h]), s_ref)
    log(f"  heads 0, 63: out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
