"""GPU checks of the packed prefill's sequence walk: one workgroup per (head,
32 output columns) runs every sequence of the batch in order, handing each
sequence's final state out and the next one's initial state in at the
boundaries.  On a 256-CU MI355X it is taken for short sequences at H = 64
(d = 128) and H = 128 (d = 64), whose workgroups fill the device; with fewer
heads the sequences are cut into groups (by tokens) walked side by side so
that the workgroups still fill it (32 heads: 2 groups, 16: 4, 8: 8, 3: 21).
Checked against the fp64 packed oracle (bf16 bar 2e-2) and bitwise against
launches over each sequence alone (which never walk), with empty, one-token,
one-block and back-to-back one-block sequences, and through the strided call."""
import numpy as np
import pytest
import torch

import oracle
from long_context_layers_amd import binding, inputs
from tests.gpu_util import BF16_TOL, log, np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HEADS = {128: 64, 64: 128}          # heads that make the walk fill 256 compute units
# (d, H); fewer heads than fill the device walk their sequences as groups side
# by side (32 heads: 2 groups, 16: 4, 8: 8 on 256 compute units)
SHAPES = [(128, 64), (128, 32), (64, 128), (128, 16), (128, 8)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def need_walk(nseq, H, T, d):
    if not binding.prefill_varlen_walks(nseq, H, T, d):
        pytest.skip(f"this device does not walk nseq={nseq} H={H} d={d} "
                    f"({torch.cuda.get_device_properties(0).multi_processor_count} compute units)")


def per_sequence(x, lens):
    """each sequence by its own dense launch (one workgroup per head slice)"""
    cu = x.cu_seqlens.cpu().tolist()
    outs, sts = [], []
    for i in range(len(lens)):
        a, b = cu[i], cu[i + 1]
        s1 = x.states[i:i + 1].clone()
        if b > a:
            q, k, v = (t[:, a:b].unsqueeze(0).contiguous() for t in (x.q, x.k, x.v))
            outs.append(binding.prefill(q, k, v, x.slopes, s1)[0])
        sts.append(s1[0])
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1) if outs else None, torch.stack(sts)


CASES = {
    "mixed": [0, 1, 63, 64, 65, 130, 0, 1000, 7, 257],
    "one_block_runs": [64, 1, 64, 2, 64, 64, 3, 64],          # a boundary at every block
    "edges_empty": [0, 0, 100, 0, 0],
    "two": [5, 700],
    # many short prompts (the report's §4.1.2 pain point), 0..120 tokens
    "short_many": [int(n) for n in np.random.default_rng(664).integers(0, 121, size=300)],
    # one long sequence among many short ones: the groups of a walk split the
    # tokens, not the sequences, evenly (the long one fills a group alone)
    "skewed": [3000, 1, 0, 2] + [int(n) for n in np.random.default_rng(665).integers(0, 41, size=150)],
}


@pytest.mark.parametrize("d,H", SHAPES)
@pytest.mark.parametrize("case", sorted(CASES))
def test_walk_matches_oracle_and_per_sequence_launches(case, d, H):
    # (a case the plan does not walk on this device runs the same checks on
    # the per-sequence grid, which must give the same bits)
    lens = CASES[case]
    path = "walk" if binding.prefill_varlen_walks(len(lens), H, sum(lens), d) else "grid"
    log(f"{path} {case} {lens[:12]}{'...' if len(lens) > 12 else ''} ({len(lens)}) H{H} d{d} bf16")
    x = inputs.make_varlen(H, lens, d, torch.bfloat16, seed=600 + d + len(case), init_state=True,
                           device=DEV)
    st = x.states.clone()
    out = binding.prefill_varlen(x.q, x.k, x.v, x.slopes, x.cu_seqlens, st)
    torch.cuda.synchronize()
    # bitwise: the walk computes every block exactly as a launch over its sequence alone
    o1, s1 = per_sequence(x, lens)
    if o1 is not None:
        assert torch.equal(out, o1), "outputs differ from per-sequence launches"
    assert torch.equal(st, s1), "states differ from per-sequence launches"
    for i, n in enumerate(lens):
        if n == 0:
            assert torch.equal(st[i], x.states[i]), f"empty sequence {i} changed its state"
    # and the oracle
    o_ref, s_ref = oracle.prefill_varlen(np64(x.q), np64(x.k), np64(x.v), np64(x.slopes),
                                         x.cu_seqlens.cpu().numpy(), np64(x.states))
    cu = x.cu_seqlens.cpu().tolist()
    eo = es = 0.0
    o64, s64 = np64(out), np64(st)
    for i in range(len(lens)):
        a, b = cu[i], cu[i + 1]
        if b > a:
            eo = max(eo, oracle.rel_l2(o64[:, a:b], o_ref[:, a:b]))
        es = max(es, oracle.rel_l2(s64[i], s_ref[i]))
    log(f"  out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("d,H", SHAPES)
def test_walk_strided_bitwise_equals_contiguous(d, H):
    lens = CASES["mixed"] if H * d // 32 >= 256 else CASES["one_block_runs"]
    need_walk(len(lens), H, sum(lens), d)
    log(f"walk through la_prefill_varlen_strided {lens} H{H} d{d}")
    x = inputs.make_varlen(H, lens, d, torch.bfloat16, seed=661 + d, init_state=True, device=DEV)
    st_ref = x.states.clone()
    out_ref = binding.prefill_varlen(x.q, x.k, x.v, x.slopes, x.cu_seqlens, st_ref)
    T = x.q.shape[1]
    # q, k, v as [H,T,d] views of one token-major [T, 3, H, d] buffer; out token-major
    buf = torch.stack([t.transpose(0, 1) for t in (x.q, x.k, x.v)], dim=1).contiguous()
    qv, kv, vv = (buf[:, j].transpose(0, 1) for j in range(3))
    ob = torch.empty((T, H, d), dtype=torch.bfloat16, device=DEV)
    st = x.states.clone()
    binding.prefill_varlen(qv, kv, vv, x.slopes, x.cu_seqlens, st, out=ob.transpose(0, 1))
    torch.cuda.synchronize()
    assert torch.equal(ob.transpose(0, 1), out_ref) and torch.equal(st, st_ref)


@pytest.mark.parametrize("H,d", [(3, 128), (5, 64), (12, 128), (24, 128), (48, 64)])
def test_walk_groups_at_odd_head_counts(H, d):
    # group counts 21, 25, 5, 2, 2 on 256 compute units; head slots that are
    # not a multiple of 8 take the plain workgroup placement
    rng = np.random.default_rng(666 + H)
    lens = [int(n) for n in rng.integers(0, 150, size=90)] + [700, 0, 3]
    need_walk(len(lens), H, sum(lens), d)
    log(f"walk groups: H{H} d{d}, {len(lens)} sequences of 0..700 tokens")
    x = inputs.make_varlen(H, lens, d, torch.bfloat16, seed=667 + H, init_state=True, device=DEV)
    st = x.states.clone()
    out = binding.prefill_varlen(x.q, x.k, x.v, x.slopes, x.cu_seqlens, st)
    torch.cuda.synchronize()
    o1, s1 = per_sequence(x, lens)
    bad = [i for i in range(len(lens)) if not torch.equal(st[i], s1[i])]
    assert not bad, f"states differ for sequences {bad[:8]}"
    assert torch.equal(out, o1), "outputs differ from per-sequence launches"
    o_ref, s_ref = oracle.prefill_varlen(np64(x.q), np64(x.k), np64(x.v), np64(x.slopes),
                                         x.cu_seqlens.cpu().numpy(), np64(x.states))
    eo = oracle.rel_l2(np64(out), o_ref)
    es = max(oracle.rel_l2(np64(st)[i], s_ref[i]) for i in range(len(lens)))
    log(f"  out rel-L2 {eo:.3e}  state rel-L2 {es:.3e}")
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_packed_256k_workload_equals_per_sequence_launches():
    # the packed 256K workload (74 sequences, 64 heads), whichever work split
    # the plan takes for it (the grid of 64-column workgroups on a 256-CU
    # device): every sequence's output and state bitwise against its own launch
    x = inputs.make_workload("varlen_256k", device=DEV)
    lens = x.lens
    H, T, d = x.q.shape
    walks = binding.prefill_varlen_walks(len(lens), H, sum(lens), d)
    log(f"packed varlen_256k: H{H} T{T} d{d}, {len(lens)} sequences ({min(lens)}..{max(lens)}), "
        f"walk={walks}")
    st = x.states.clone()
    out = binding.prefill_varlen(x.q, x.k, x.v, x.slopes, x.cu_seqlens, st)
    o1, s1 = per_sequence(x, lens)
    bad = [i for i in range(len(lens)) if not torch.equal(st[i], s1[i])]
    assert not bad, f"states differ for sequences {bad[:8]}"
    assert torch.equal(out, o1), "outputs differ from per-sequence launches"


@pytest.mark.parametrize("H", [64, 32])
def test_walk_more_sequences_than_one_table(H):
    # 1100 short sequences (some empty): walked 1024 at a time, two launches
    # (at 32 heads each in two groups)
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(0, 40, size=1100)]
    d = 128
    need_walk(len(lens), H, sum(lens), d)
    log(f"walk over {len(lens)} sequences of 0..39 tokens, H{H} d{d}")
    x = inputs.make_varlen(H, lens, d, torch.bfloat16, seed=662, init_state=True, device=DEV)
    st = x.states.clone()
    out = binding.prefill_varlen(x.q, x.k, x.v, x.slopes, x.cu_seqlens, st)
    o1, s1 = per_sequence(x, lens)
    bad = [i for i in range(len(lens)) if not torch.equal(st[i], s1[i])]
    assert not bad, f"states differ for sequences {bad[:8]}"
    assert torch.equal(out, o1), "outputs differ from per-sequence launches"


MALFORMED = {
    # out of order, negative and past the end: sequence 2 clamps to rows 100..1099
    "past_end": ([0, 300, 100, 1200, -5, 700, 1000], None),
    # out of order and negative, nothing past row 999: rows 1000..1099 in no sequence
    "short_tail": ([0, 300, 100, 900, -5, 700, 1000], 1000),
}


@pytest.mark.parametrize("case", sorted(MALFORMED))
@pytest.mark.parametrize("H", [4, 16, 64])
def test_malformed_offsets_stay_inside_the_tensors(H, case):
    # the results are unspecified, but every access stays inside q, k, v, out
    # and the states (offsets are clamped into [0, T]), and rows outside every
    # clamped sequence are not written.  H = 4: one workgroup per sequence;
    # H = 16: the walk in groups; H = 64: the walk (on a 256-CU device).
    offsets, free_from = MALFORMED[case]
    d, T = 128, 1100
    cu = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    nseq = cu.numel() - 1
    log(f"malformed offsets {offsets} H{H} T{T} d{d}, walk={binding.prefill_varlen_walks(nseq, H, T, d)}")
    g = torch.Generator(device=DEV).manual_seed(663)
    q, k, v = ((torch.randn((H, T, d), generator=g, device=DEV) / d ** 0.5).to(torch.bfloat16)
               for _ in range(3))
    guard = 4096
    canary = torch.tensor(-7.0, dtype=torch.bfloat16)
    flat = torch.full((2 * guard + H * T * d,), float(canary), dtype=torch.bfloat16, device=DEV)
    out = flat[guard:guard + H * T * d].view(H, T, d)
    sflat = torch.full(((nseq + 2) * H * d * d,), 3.5, device=DEV)
    states = sflat[H * d * d:(nseq + 1) * H * d * d].view(nseq, H, d, d)
    states.normal_(generator=g).mul_(0.01)
    binding.prefill_varlen(q, k, v, inputs.slopes(H, DEV), cu, states, out=out)
    torch.cuda.synchronize()
    assert bool((flat[:guard] == canary).all()) and bool((flat[-guard:] == canary).all())
    assert bool((sflat[:H * d * d] == 3.5).all()) and bool((sflat[-H * d * d:] == 3.5).all())
    end = T if free_from is None else free_from
    assert bool(torch.isfinite(out[:, :end].float()).all()) and bool(torch.isfinite(states).all())
    if free_from is not None:
        assert bool((out[:, free_from:] == canary).all())
