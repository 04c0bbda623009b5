"""GPU parity for the sequence-sharded (context-parallel) prefill steps
(la_cp_fold, la_cp_correct) through the C ABI, against the fp64 oracle's
cp_fold / cp_correct on the same bytes, and end to end: every shard run by
la_prefill from a zero state, folded and corrected, against the oracle's
recurrence over the unsplit sequence.  Bars: fp32 fold 1e-5 (fp32 sums of at
most 65 terms), bf16 outputs and states 2e-2 (as for the prefill)."""
import numpy as np
import pytest
import torch

import oracle
from long_context_layers_amd import binding, inputs
from tests.gpu_util import BF16_TOL, log, np64, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FOLD_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def slopes_of(kind, H):
    # the pages' per-head decays, or decays close to 1 so that states carry
    # across many shards
    if kind == "pages":
        return inputs.slopes(H, DEV)
    return torch.linspace(1e-4, 3e-3, H, device=DEV)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["pages", "slow"])
def test_cp_fold_matches_oracle(d, kind):
    lens = [100, 0, 37, 1, 64]
    R, B, H = len(lens), 2, 4
    log(f"cp_fold R{R} {lens} B{B} H{H} d{d} slopes {kind}")
    g = torch.Generator(device=DEV).manual_seed(40 + d)
    loc = 0.1 * torch.randn((R, B, H, d, d), generator=g, device=DEV)
    init = 0.1 * torch.randn((B, H, d, d), generator=g, device=DEV)
    s = slopes_of(kind, H)
    for r in range(R + 1):
        for with_init in (True, False):
            got = binding.cp_fold(loc, lens, r, s, init if with_init else None)
            torch.cuda.synchronize()
            ref = oracle.cp_fold(np64(loc), lens, np64(s), r, np64(init) if with_init else None)
            e = rel_l2(got, ref)
            assert e <= FOLD_TOL, (r, with_init, e)
    # in place: state_in is state_init
    st = init.clone()
    binding.cp_fold(loc, lens, 3, s, st, out=st)
    torch.cuda.synchronize()
    assert rel_l2(st, oracle.cp_fold(np64(loc), lens, np64(s), 3, np64(init))) <= FOLD_TOL
    # rank 0 without an initial state is zero
    z = binding.cp_fold(loc, lens, 0, s)
    torch.cuda.synchronize()
    assert bool((z == 0).all())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 31, 33, 1000])
def test_cp_correct_matches_oracle(d, L):
    B, H = 2, 3
    log(f"cp_correct B{B} H{H} L{L} d{d}")
    g = torch.Generator(device=DEV).manual_seed(50 + L + d)
    q = (torch.randn((B, H, L, d), generator=g, device=DEV) / np.sqrt(d)).to(torch.bfloat16)
    o_loc = (0.3 * torch.randn((B, H, L, d), generator=g, device=DEV)).to(torch.bfloat16)
    S = 0.1 * torch.randn((B, H, d, d), generator=g, device=DEV)
    s = slopes_of("slow", H)
    out = o_loc.clone()
    binding.cp_correct(q, s, S, out)
    torch.cuda.synchronize()
    ref = oracle.cp_correct(np64(q), np64(s), np64(S), np64(o_loc))
    e = rel_l2(out, ref)
    log(f"  out rel-L2 {e:.3e}")
    assert e <= BF16_TOL


def run_sharded(x, lens):
    """every shard by la_prefill from zero, then fold and correct per shard"""
    B, H, N, d = x.q.shape
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    locs, outs = [], []
    for j in range(len(lens)):
        a, b = starts[j], starts[j + 1]
        st = torch.zeros((B, H, d, d), device=DEV)
        o = binding.prefill(x.q[:, :, a:b].contiguous(), x.k[:, :, a:b].contiguous(),
                            x.v[:, :, a:b].contiguous(), x.slopes, st)
        locs.append(st)
        outs.append(o)
    loc = torch.stack(locs)                            # what an all-gather would hand every rank
    for r in range(len(lens)):
        a, b = starts[r], starts[r + 1]
        s_in = binding.cp_fold(loc, lens, r, x.slopes, x.state)
        binding.cp_correct(x.q[:, :, a:b].contiguous(), x.slopes, s_in, outs[r])
    final = binding.cp_fold(loc, lens, len(lens), x.slopes, x.state)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=2), final


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["pages", "slow"])
def test_cp_end_to_end_equals_the_unsplit_sequence(d, kind):
    lens = [600, 1, 0, 333, 566]
    B, H, N = 1, 4, sum(lens)
    log(f"cp end to end {lens} B{B} H{H} d{d} slopes {kind}")
    x = inputs.make_prefill(B, H, N, d, torch.bfloat16, seed=60 + d, init_state=True, device=DEV)
    x.slopes = slopes_of(kind, H)
    out, final = run_sharded(x, lens)
    o_ref, s_ref = oracle.prefill(np64(x.q), np64(x.k), np64(x.v), np64(x.slopes), np64(x.state))
    eo, es = rel_l2(out, o_ref), rel_l2(final, s_ref)
    log(f"  out rel-L2 {eo:.3e}  final state rel-L2 {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_cp_256k_in_8_shards_sampled_heads():
    # the 256K, 64-head workload split into 8 shards of 32K tokens (the shape
    # one rank of an 8-way split runs), every head on the GPU; the oracle
    # checks heads 0 and 63 over the whole sequence
    w = inputs.WORKLOADS["prefill_256k"]
    R = 8
    lens = [w.N // R] * R
    log(f"cp 256K: B{w.B} H{w.H} N{w.N} d{w.d} in {R} shards of {lens[0]}")
    x = inputs.make_workload("prefill_256k", device=DEV)
    out, final = run_sharded(x, lens)
    heads = [0, w.H - 1]
    idx = torch.tensor(heads, device=DEV)
    o_ref, s_ref = oracle.prefill(*(np64(t.index_select(1, idx)) for t in (x.q, x.k, x.v)),
                                  np64(x.slopes.index_select(0, idx)))
    eo = rel_l2(out.index_select(1, idx), o_ref)
    es = rel_l2(final.index_select(1, idx), s_ref)
    log(f"  heads {heads}: out rel-L2 {eo:.3e}  final state rel-L2 {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("R", [1, 64])
def test_cp_fold_shard_count_limits(R):
    # one shard, and the most shards a call takes (64), with uneven lengths
    B, H, d = 1, 2, 64
    lens = [(7 * j) % 5 for j in range(R)]
    log(f"cp_fold with {R} shards {lens[:8]}...")
    g = torch.Generator(device=DEV).manual_seed(70 + R)
    loc = 0.1 * torch.randn((R, B, H, d, d), generator=g, device=DEV)
    init = 0.1 * torch.randn((B, H, d, d), generator=g, device=DEV)
    s = slopes_of("slow", H)
    for r in sorted({0, 1, R // 2, R}):
        got = binding.cp_fold(loc, lens, r, s, init)
        torch.cuda.synchronize()
        ref = oracle.cp_fold(np64(loc), lens, np64(s), r, np64(init))
        assert rel_l2(got, ref) <= FOLD_TOL, r
