"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test checks the recurrent C oracle against something the mathematics
fixes: the definition's double sum on tiny inputs, closed forms (lambda = 1,
lambda = 0, d = 1 geometric series, zero keys), the block decomposition, and
invariants (split with carried state, prefill == decode steps, linearity,
head/batch equivariance).  The decayed linear-attention recurrence itself is
the one the Ling and Ring 2.6 Technical Report (§4.1.1) describes as an
RNN-style recurrence over a [B,H,D,D] state.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, H, N, d, with_state=True):
    q = rng.standard_normal((B, H, N, d)) / math.sqrt(d)
    k = rng.standard_normal((B, H, N, d)) / math.sqrt(d)
    v = rng.standard_normal((B, H, N, d))
    S0 = 0.1 * rng.standard_normal((B, H, d, d)) if with_state else None
    return q, k, v, S0


def slopes_for(lams):
    return np.array([math.inf if l == 0 else -math.log(l) for l in lams])


LAMS = [0.0, 0.4, 0.94, 0.996, 1.0]


@pytest.mark.parametrize("N,d", [(1, 1), (7, 3), (37, 8), (64, 5)])
def test_recurrent_matches_quadratic_definition(N, d):
    rng = np.random.default_rng(N * 100 + d)
    B, H = 2, len(LAMS)
    q, k, v, S0 = rand_inputs(rng, B, H, N, d)
    s = slopes_for(LAMS)
    o_r, f_r = oracle.prefill(q, k, v, s, S0)
    o_q, f_q = oracle.quadratic(q, k, v, s, S0)
    assert oracle.rel_l2(o_r, o_q) <= 1e-12
    assert oracle.rel_l2(f_r, f_q) <= 1e-12


def test_non_square_roles_are_not_transposed():
    # asymmetric state and distinct q/k/v: a transposed S (S[j][i]) or swapped
    # q/k roles changes the result; the double sum fixes which is right.
    rng = np.random.default_rng(7)
    q, k, v, S0 = rand_inputs(rng, 1, 1, 9, 4)
    s = slopes_for([0.7])
    o_r, f_r = oracle.prefill(q, k, v, s, S0)
    o_q, f_q = oracle.quadratic(q, k, v, s, S0)
    assert oracle.rel_l2(o_r, o_q) <= 1e-12
    o_t, _ = oracle.quadratic(q, k, v, s, np.swapaxes(S0, -1, -2))
    assert oracle.rel_l2(o_t, o_q) > 1e-3        # the transpose is detectable
    o_s, _ = oracle.quadratic(k, q, v, s, S0)
    assert oracle.rel_l2(o_s, o_q) > 1e-3        # swapping q and k is detectable


def test_lambda_one_is_plain_causal_linear_attention():
    # lambda = 1: o_t = q_t (S_init + sum_{s<=t} k_s^T v_s), final S_init + K^T V
    rng = np.random.default_rng(11)
    B, H, N, d = 2, 2, 33, 6
    q, k, v, S0 = rand_inputs(rng, B, H, N, d)
    s = np.zeros(H)
    o, f = oracle.prefill(q, k, v, s, S0)
    kv = np.einsum("bhti,bhtj->bhtij", k, v)
    pref = S0[:, :, None] + np.cumsum(kv, axis=2)
    o_ref = np.einsum("bhti,bhtij->bhtj", q, pref)
    assert oracle.rel_l2(o, o_ref) <= 1e-12
    assert oracle.rel_l2(f, S0 + np.einsum("bhti,bhtj->bhij", k, v)) <= 1e-12


def test_lambda_zero_keeps_only_the_diagonal():
    # lambda = 0 (slope +inf): o_t = (q_t . k_t) v_t, final k_{N-1}^T v_{N-1}
    rng = np.random.default_rng(12)
    B, H, N, d = 1, 3, 10, 5
    q, k, v, S0 = rand_inputs(rng, B, H, N, d)
    s = np.full(H, math.inf)
    o, f = oracle.prefill(q, k, v, s, S0)
    o_ref = np.sum(q * k, axis=-1, keepdims=True) * v
    assert oracle.rel_l2(o, o_ref) <= 1e-15
    f_ref = np.einsum("bhi,bhj->bhij", k[:, :, -1], v[:, :, -1])
    assert oracle.rel_l2(f, f_ref) <= 1e-15


def test_geometric_series_worked_values():
    with open(os.path.join(GOLDEN, "geometric_d1.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        N = c["N"]
        one = np.ones((1, 1, N, 1))
        s = slopes_for([c["lambda"]])
        S0 = np.full((1, 1, 1, 1), c["S_init"])
        o, f = oracle.prefill(one, one, one, s, S0)
        np.testing.assert_allclose(o[0, 0, :, 0], c["out"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(f[0, 0, 0, 0], c["final"], rtol=1e-14, atol=1e-15)


def test_geometric_closed_form_long():
    # d = 1, q = k = v = 1: o_t = (1 - lam^(t+1)) / (1 - lam) + lam^(t+1) S0
    N = 300
    lams = [0.3, 0.9, 0.999]
    one = np.ones((1, 3, N, 1))
    S0 = np.array([0.5, -1.0, 3.0]).reshape(1, 3, 1, 1)
    o, f = oracle.prefill(one, one, one, slopes_for(lams), S0)
    t = np.arange(N)
    for h, lam in enumerate(lams):
        lam = math.exp(-slopes_for([lam])[0])
        ref = (1 - lam ** (t + 1)) / (1 - lam) + lam ** (t + 1) * S0[0, h, 0, 0]
        np.testing.assert_allclose(o[0, h, :, 0], ref, rtol=1e-12)


def test_initial_state_decays_at_the_first_token():
    # zero keys: o_t = lam^(t+1) q_t S_init and final = lam^N S_init
    rng = np.random.default_rng(3)
    B, H, N, d = 1, 2, 12, 4
    q, _, v, S0 = rand_inputs(rng, B, H, N, d)
    k = np.zeros_like(q)
    lams = [0.8, 0.5]
    o, f = oracle.prefill(q, k, v, slopes_for(lams), S0)
    for h, lam in enumerate(lams):
        lam = math.exp(-slopes_for([lam])[0])
        for t in range(N):
            ref = lam ** (t + 1) * (q[0, h, t] @ S0[0, h])
            np.testing.assert_allclose(o[0, h, t], ref, rtol=1e-13)
        np.testing.assert_allclose(f[0, h], lam ** N * S0[0, h], rtol=1e-13)


@pytest.mark.parametrize("C", [1, 3, 32, 64, 70])
def test_blockwise_decomposition_reaches_the_definition(C):
    rng = np.random.default_rng(C)
    B, H, N, d = 1, 3, 70, 8
    q, k, v, S0 = rand_inputs(rng, B, H, N, d)
    s = slopes_for([0.4, 0.94, 0.996])
    o_r, f_r = oracle.prefill(q, k, v, s, S0)
    o_b, f_b = oracle.blockwise(q, k, v, s, S0, C=C)
    assert oracle.rel_l2(o_b, o_r) <= 1e-12
    assert oracle.rel_l2(f_b, f_r) <= 1e-12


@pytest.mark.parametrize("m", [1, 32, 33, 63])
def test_split_with_carried_state_is_bitwise_identical(m):
    rng = np.random.default_rng(m)
    B, H, N, d = 2, 2, 64, 8
    q, k, v, S0 = rand_inputs(rng, B, H, N, d)
    s = slopes_for([0.5, 0.99])
    o, f = oracle.prefill(q, k, v, s, S0)
    o1, f1 = oracle.prefill(q[:, :, :m], k[:, :, :m], v[:, :, :m], s, S0)
    o2, f2 = oracle.prefill(q[:, :, m:], k[:, :, m:], v[:, :, m:], s, f1)
    assert np.array_equal(np.concatenate([o1, o2], axis=2), o)
    assert np.array_equal(f2, f)


def test_prefill_equals_decode_steps():
    rng = np.random.default_rng(5)
    B, H, N, d = 2, 3, 9, 6
    q, k, v, S0 = rand_inputs(rng, B, H, N, d)
    s = slopes_for([0.3, 0.9, 1.0])
    o, f = oracle.prefill(q, k, v, s, S0)
    st = S0
    for t in range(N):
        ot, st = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], s, st)
        assert np.array_equal(ot, o[:, :, t])
    assert np.array_equal(st, f)


def test_linear_in_v_and_q_bilinear_in_k_v():
    rng = np.random.default_rng(9)
    B, H, N, d = 1, 2, 20, 5
    q, k, v1, _ = rand_inputs(rng, B, H, N, d, with_state=False)
    v2 = rng.standard_normal(v1.shape)
    q2 = rng.standard_normal(q.shape)
    s = slopes_for([0.6, 0.97])
    a, b = 1.75, -0.5
    o1, f1 = oracle.prefill(q, k, v1, s)
    o2, f2 = oracle.prefill(q, k, v2, s)
    o12, f12 = oracle.prefill(q, k, a * v1 + b * v2, s)
    assert oracle.rel_l2(o12, a * o1 + b * o2) <= 1e-13
    assert oracle.rel_l2(f12, a * f1 + b * f2) <= 1e-13
    oq, _ = oracle.prefill(q2, k, v1, s)
    oqq, _ = oracle.prefill(a * q + b * q2, k, v1, s)
    assert oracle.rel_l2(oqq, a * o1 + b * oq) <= 1e-13
    ok, fk = oracle.prefill(q, 2.0 * k, v1, s)
    assert oracle.rel_l2(ok, 2.0 * o1) <= 1e-14 and oracle.rel_l2(fk, 2.0 * f1) <= 1e-14


def test_heads_and_batch_are_independent():
    rng = np.random.default_rng(21)
    B, H, N, d = 3, 4, 15, 4
    q, k, v, S0 = rand_inputs(rng, B, H, N, d)
    s = slopes_for([0.2, 0.5, 0.9, 0.99])
    o, f = oracle.prefill(q, k, v, s, S0)
    pb = [2, 0, 1]
    ph = [3, 1, 0, 2]
    qp, kp, vp, Sp = (x[pb][:, ph] for x in (q, k, v, S0))
    op, fp = oracle.prefill(qp, kp, vp, s[ph], Sp)
    assert np.array_equal(op, o[pb][:, ph]) and np.array_equal(fp, f[pb][:, ph])


def test_empty_sequence_leaves_state():
    rng = np.random.default_rng(1)
    q, k, v, S0 = rand_inputs(rng, 1, 2, 0, 4)
    o, f = oracle.prefill(q, k, v, slopes_for([0.5, 0.9]), S0)
    assert o.shape == (1, 2, 0, 4) and np.array_equal(f, S0)


# --- the pins catch plausible mistakes: planted in a Python copy of the
# recurrence (CPU only), each mistake must fail the double-sum comparison.

def _mutant_recurrence(q, k, v, lam, S0, mutation):
    N, d = q.shape
    S = S0.copy()
    o = np.zeros((N, d))
    for t in range(N):
        if mutation == "read_before_update":
            o[t] = q[t] @ S
            S = lam * S + np.outer(k[t], v[t])
            continue
        if mutation == "no_decay_on_state":
            S = S + np.outer(k[t], v[t])
        elif mutation == "decay_on_new_term":
            S = lam * (S + np.outer(k[t], v[t]))
        elif mutation == "transposed_update":
            S = lam * S + np.outer(v[t], k[t])
        else:
            S = lam * S + np.outer(k[t], v[t])
        o[t] = (S @ q[t]) if mutation == "transposed_read" else (q[t] @ S)
    return o


@pytest.mark.parametrize("mutation", ["read_before_update", "no_decay_on_state",
                                      "decay_on_new_term", "transposed_update",
                                      "transposed_read"])
def test_pins_detect_planted_mistakes(mutation):
    rng = np.random.default_rng(99)
    N, d = 11, 4
    q, k, v, S0 = rand_inputs(rng, 1, 1, N, d)
    v = rng.standard_normal(v.shape)
    lam = 0.8
    o_q, _ = oracle.quadratic(q, k, v, slopes_for([lam]), S0)
    good = _mutant_recurrence(q[0, 0], k[0, 0], v[0, 0], lam, S0[0, 0], None)
    assert oracle.rel_l2(good, o_q[0, 0]) <= 1e-12
    bad = _mutant_recurrence(q[0, 0], k[0, 0], v[0, 0], lam, S0[0, 0], mutation)
    assert oracle.rel_l2(bad, o_q[0, 0]) > 1e-3


# --- packed variable-length batches (the report's §4.1.2: packed
# sub-sequences each attend only within themselves) -------------------------

def _packed(rng, H, lens, d):
    T = sum(lens)
    q = rng.standard_normal((H, T, d)) / math.sqrt(d)
    k = rng.standard_normal((H, T, d)) / math.sqrt(d)
    v = rng.standard_normal((H, T, d))
    S0 = 0.1 * rng.standard_normal((len(lens), H, d, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, S0, cu


def test_varlen_matches_quadratic_per_sequence():
    # each sequence against the double sum on its own rows from its own state
    rng = np.random.default_rng(31)
    lens = [0, 1, 5, 17, 0, 9]
    q, k, v, S0, cu = _packed(rng, len(LAMS), lens, 4)
    s = slopes_for(LAMS)
    o, f = oracle.prefill_varlen(q, k, v, s, cu, S0)
    for i in range(len(lens)):
        a, b = cu[i], cu[i + 1]
        oq, fq = oracle.quadratic(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], s, S0[i:i + 1])
        if b > a:
            assert oracle.rel_l2(o[:, a:b], oq[0]) <= 1e-12
        assert oracle.rel_l2(f[i], fq[0]) <= 1e-12


def test_varlen_with_chained_states_is_one_dense_run():
    # start sequence i from the dense state after cu[i] tokens (double sum on
    # the prefix): the packed run must then reproduce the dense definition
    rng = np.random.default_rng(32)
    lens = [3, 0, 11, 6, 1]
    q, k, v, S0, cu = _packed(rng, 3, lens, 5)
    s = slopes_for([0.3, 0.9, 1.0])
    chained = np.zeros_like(S0)
    for i in range(len(lens)):
        _, fp = oracle.quadratic(q[None, :, :cu[i]], k[None, :, :cu[i]], v[None, :, :cu[i]], s, S0[:1])
        chained[i] = fp[0]
    o, f = oracle.prefill_varlen(q, k, v, s, cu, chained)
    od, fd = oracle.quadratic(q[None], k[None], v[None], s, S0[:1])
    assert oracle.rel_l2(o, od[0]) <= 1e-12
    assert oracle.rel_l2(f[-1], fd[0]) <= 1e-12


def test_varlen_empty_sequences_keep_their_state():
    rng = np.random.default_rng(33)
    q, k, v, S0, cu = _packed(rng, 2, [0, 4, 0], 3)
    _, f = oracle.prefill_varlen(q, k, v, slopes_for([0.5, 0.9]), cu, S0)
    assert np.array_equal(f[0], S0[0]) and np.array_equal(f[2], S0[2])
    assert not np.array_equal(f[1], S0[1])


def test_varlen_pin_detects_a_missing_reset():
    # planted mistake: one dense run over the packed tokens (state carried
    # across sequence boundaries) must fail the per-sequence double sum
    rng = np.random.default_rng(34)
    lens = [6, 7]
    q, k, v, S0, cu = _packed(rng, 1, lens, 4)
    s = slopes_for([0.9])
    leaky, _ = oracle.prefill(q[None], k[None], v[None], s, S0[:1])
    a, b = cu[1], cu[2]
    oq, _ = oracle.quadratic(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], s, S0[1:2])
    assert oracle.rel_l2(leaky[0][:, a:b], oq[0]) > 1e-3
    good, _ = oracle.prefill_varlen(q, k, v, s, cu, S0)
    assert oracle.rel_l2(good[:, a:b], oq[0]) <= 1e-12


def test_varlen_rejects_bad_offsets():
    rng = np.random.default_rng(35)
    q, k, v, S0, _ = _packed(rng, 1, [4, 4], 2)
    for cu in ([0, 9, 8], [1, 4, 8], [0, 4, 7], [0, 8, 4]):
        with pytest.raises(ValueError):
            oracle.prefill_varlen(q, k, v, slopes_for([0.5]), np.array(cu), None)


# --- several tokens per sequence with a committed prefix (draft
# verification in serving with multi-token prediction) ----------------------

def test_decode_multi_matches_quadratic():
    rng = np.random.default_rng(41)
    B, H, T, d = 5, len(LAMS), 4, 6
    q, k, v, S0 = rand_inputs(rng, B, H, T, d)
    s = slopes_for(LAMS)
    n = np.array([0, 1, 2, 3, 4])
    o, st = oracle.decode_multi(q, k, v, s, S0, n)
    oq, _ = oracle.quadratic(q, k, v, s, S0)
    assert oracle.rel_l2(o, oq) <= 1e-12                       # every token's output
    for b in range(B):
        _, fq = oracle.quadratic(q[b:b + 1, :, :n[b]], k[b:b + 1, :, :n[b]], v[b:b + 1, :, :n[b]],
                                 s, S0[b:b + 1])
        assert oracle.rel_l2(st[b], fq[0]) <= 1e-12             # state after n[b] tokens
    assert np.array_equal(st[0], S0[0])                         # nothing committed


def test_decode_multi_outputs_ignore_the_commit_count():
    rng = np.random.default_rng(42)
    q, k, v, S0 = rand_inputs(rng, 3, 2, 3, 4)
    s = slopes_for([0.5, 0.97])
    o1, s1 = oracle.decode_multi(q, k, v, s, S0, [3, 3, 3])
    o2, _ = oracle.decode_multi(q, k, v, s, S0, [0, 1, 2])
    o3, s3 = oracle.decode_multi(q, k, v, s, S0, None)
    assert np.array_equal(o1, o2) and np.array_equal(o1, o3) and np.array_equal(s1, s3)
    # clamping: counts beyond [0, T]
    _, s4 = oracle.decode_multi(q, k, v, s, S0, [-2, 7, 3])
    assert np.array_equal(s4[0], S0[0]) and np.array_equal(s4[1], s1[1])


def test_decode_multi_pin_detects_committing_every_token():
    # planted mistake: storing the state after all T tokens whatever the
    # commit count must fail the double sum over the committed prefix
    rng = np.random.default_rng(43)
    q, k, v, S0 = rand_inputs(rng, 1, 1, 4, 5)
    s = slopes_for([0.9])
    _, full = oracle.decode_multi(q, k, v, s, S0, [4])
    _, fq = oracle.quadratic(q[:, :, :2], k[:, :, :2], v[:, :, :2], s, S0)
    assert oracle.rel_l2(full, fq) > 1e-3
    _, good = oracle.decode_multi(q, k, v, s, S0, [2])
    assert oracle.rel_l2(good, fq) <= 1e-12


# ---- sequence-sharded (context-parallel) prefill: fold and correct ----------
# Ling and Ring 2.6 Technical Report, §4.1.1 and Fig. 10: each rank runs its
# shard from a zero state (local output, local state), the local states are
# all-gathered, and each rank folds the states before it into its incoming
# state and corrects its local output.  Pinned against the recurrence over the
# unsplit sequence (the state after a prefix; the output rows of a shard).

CP_LENS = [5, 0, 17, 1, 9]           # uneven, with an empty and a one-token shard


def cp_setup(seed, lens=CP_LENS, d=4):
    rng = np.random.default_rng(seed)
    H = len(LAMS)
    q, k, v, S0 = rand_inputs(rng, 2, H, sum(lens), d)
    s = slopes_for(LAMS)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    loc_out, loc_st = [], []
    for j in range(len(lens)):
        a, b = starts[j], starts[j + 1]
        o, st = oracle.prefill(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], s)   # zero state
        loc_out.append(o)
        loc_st.append(st)
    return q, k, v, S0, s, starts, loc_out, np.stack(loc_st)


def test_cp_fold_is_the_state_after_the_prefix():
    q, k, v, S0, s, starts, _, loc = cp_setup(11)
    for r in range(len(CP_LENS) + 1):
        m = starts[r]
        _, ref = oracle.prefill(q[:, :, :m], k[:, :, :m], v[:, :, :m], s, S0)
        got = oracle.cp_fold(loc, CP_LENS, s, r, S0)
        assert oracle.rel_l2(got, ref) <= 1e-12, r
        # no initial state: the prefix from zero
        _, ref0 = oracle.prefill(q[:, :, :m], k[:, :, :m], v[:, :, :m], s)
        assert oracle.rel_l2(oracle.cp_fold(loc, CP_LENS, s, r), ref0) <= 1e-12, r


def test_cp_correct_gives_the_unsplit_output():
    q, k, v, S0, s, starts, loc_out, loc = cp_setup(12)
    full, _ = oracle.prefill(q, k, v, s, S0)
    for r in range(len(CP_LENS)):
        a, b = starts[r], starts[r + 1]
        S_in = oracle.cp_fold(loc, CP_LENS, s, r, S0)
        got = oracle.cp_correct(q[:, :, a:b], s, S_in, loc_out[r])
        assert oracle.rel_l2(got, full[:, :, a:b]) <= 1e-12, r


def test_cp_single_shard_is_the_carried_state_run():
    # one shard: the fold at rank 1 is the final state, the correction of the
    # zero-state output is the output from S_init (a closed check by hand)
    rng = np.random.default_rng(13)
    q, k, v, S0 = rand_inputs(rng, 1, 2, 9, 3)
    s = slopes_for([0.5, 0.9])
    o0, st0 = oracle.prefill(q, k, v, s)
    full, fin = oracle.prefill(q, k, v, s, S0)
    lam = np.exp(-s)[None, :, None, None]
    assert oracle.rel_l2(oracle.cp_fold(st0[None], [9], s, 1, S0), lam ** 9 * S0 + st0) <= 1e-14
    assert oracle.rel_l2(oracle.cp_fold(st0[None], [9], s, 1, S0), fin) <= 1e-12
    assert oracle.rel_l2(oracle.cp_correct(q, s, S0, o0), full) <= 1e-12


def _fold_mutant(kind):
    def fold(loc, lens, slopes, rank, S0):
        lam = np.exp(-np.asarray(slopes, np.float64))[None, :, None, None]
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.float64)
        out = np.zeros(loc.shape[1:])
        if kind != "no_init_decay":
            out += lam ** starts[rank] * S0
        else:
            out += S0
        for j in range(rank):
            if kind == "decay_own_shard":
                e = starts[rank] - starts[j]
            elif kind == "reversed_order":
                e = starts[j + 1]
            else:
                e = starts[rank] - starts[j + 1]
            out += lam ** e * loc[j]
        return out
    return fold


@pytest.mark.parametrize("kind", ["no_init_decay", "decay_own_shard", "reversed_order"])
def test_cp_fold_pin_detects_planted_mistakes(kind):
    q, k, v, S0, s, starts, _, loc = cp_setup(14)
    bad = _fold_mutant(kind)
    worst = 0.0
    for r in range(len(CP_LENS) + 1):
        m = starts[r]
        _, ref = oracle.prefill(q[:, :, :m], k[:, :, :m], v[:, :, :m], s, S0)
        worst = max(worst, oracle.rel_l2(bad(loc, CP_LENS, s, r, S0), ref))
    assert worst > 1e-3


@pytest.mark.parametrize("kind", ["power_a", "transposed_state"])
def test_cp_correct_pin_detects_planted_mistakes(kind):
    q, k, v, S0, s, starts, loc_out, loc = cp_setup(15)
    full, _ = oracle.prefill(q, k, v, s, S0)
    worst = 0.0
    for r in range(len(CP_LENS)):
        a, b = starts[r], starts[r + 1]
        S_in = oracle.cp_fold(loc, CP_LENS, s, r, S0)
        L = b - a
        idx = np.arange(L, dtype=np.float64)
        lam = np.exp(-s)[:, None] ** (idx[None, :] + (0.0 if kind == "power_a" else 1.0))
        S_use = np.swapaxes(S_in, -1, -2) if kind == "transposed_state" else S_in
        bad = loc_out[r] + lam[None, :, :, None] * (q[:, :, a:b] @ S_use)
        worst = max(worst, oracle.rel_l2(bad, full[:, :, a:b]))
    assert worst > 1e-3


def test_cp_fold_rejects_bad_arguments():
    _, _, _, S0, s, _, _, loc = cp_setup(16)
    with pytest.raises(ValueError):
        oracle.cp_fold(loc, CP_LENS[:-1], s, 1, S0)
    with pytest.raises(ValueError):
        oracle.cp_fold(loc, CP_LENS, s, len(CP_LENS) + 1, S0)


# --- the parity checker itself: max over (b, h) slices of the relative L2
# error, ||x - ref||_2 / ||ref||_2, absolute where ||ref||_2 = 0.  Every value
# below is worked by hand; a checker that took one global ratio over all
# slices, an absolute norm, a mean over slices, or the wrong axes gives a
# different number.

def _slice_3_4(scale=1.0):
    """A [4, 5] slice with ||ref||_2 = 5 * scale: entries 3 and 4, rest 0."""
    r = np.zeros((4, 5))
    r[1, 2], r[3, 0] = 3.0, 4.0
    return r * scale


def test_rel_l2_is_the_worst_slice_not_a_global_ratio():
    # [2, 3] slices of [4, 5]; every reference slice has norm 5.  Slice
    # (1, 2) is off by (0, 0, ..., 2.5 at one entry): 2.5 / 5 = 0.5.  All
    # other slices are exact.  A global ratio would give
    # 2.5 / sqrt(6 * 25) = 0.2041, a mean over slices 0.5 / 6 = 0.0833.
    ref = np.stack([np.stack([_slice_3_4() for _ in range(3)]) for _ in range(2)])
    x = ref.copy()
    x[1, 2, 0, 4] += 2.5
    assert oracle.rel_l2(x, ref) == pytest.approx(0.5, abs=1e-15)
    # one bad slice of 64 (the shape of a 64-head launch): still its own error
    ref64 = np.ones((1, 64, 8, 16))                   # each slice norm sqrt(128)
    x64 = ref64.copy()
    x64[0, 37] *= 1.05                                # that slice: exactly 0.05
    assert oracle.rel_l2(x64, ref64) == pytest.approx(0.05, rel=1e-12)


@pytest.mark.parametrize("scale", [1e-150, 1e-3, 1.0, 1e3, 1e150])
def test_rel_l2_is_relative_at_any_magnitude(scale):
    # x = 7 ref: ||6 ref|| / ||ref|| = 6 whatever the magnitude
    ref = np.stack([_slice_3_4(scale), 2.0 * _slice_3_4(scale)])[None]   # [1, 2, 4, 5]
    assert oracle.rel_l2(7.0 * ref, ref) == pytest.approx(6.0, rel=1e-14)
    # and a relative error of 1e-3 in every element stays 1e-3
    assert oracle.rel_l2(ref * (1 + 1e-3), ref) == pytest.approx(1e-3, rel=1e-9)


def test_rel_l2_zero_reference_slice_uses_the_absolute_norm():
    ref = np.stack([np.zeros((4, 5)), _slice_3_4()])[None]      # [1, 2, 4, 5]
    x = ref.copy()
    x[0, 0, 2, 1], x[0, 0, 0, 3] = 3.0, 4.0     # ||x - 0|| = 5, absolute
    assert oracle.rel_l2(x, ref) == pytest.approx(5.0, abs=1e-15)
    x2 = ref.copy()
    x2[0, 0, 0, 0] = 1e-4                       # small absolute error stays small
    assert oracle.rel_l2(x2, ref) == pytest.approx(1e-4, rel=1e-12)
    assert oracle.rel_l2(np.zeros((2, 3, 4)), np.zeros((2, 3, 4))) == 0.0


def test_rel_l2_nan_or_inf_fails_any_tolerance():
    ref = np.ones((1, 2, 4, 5))
    for bad in (np.nan, np.inf, -np.inf):
        x = ref.copy()
        x[0, 1, 2, 3] = bad
        r = oracle.rel_l2(x, ref)
        assert not (r <= 1.0)          # a NaN or inf result never passes a bar


def test_rel_l2_per_row_axes_for_decode_outputs():
    # decode outputs [B, H, d] are compared per (b, h) row: axes=(-1,).
    ref = np.zeros((2, 3, 5))
    ref[..., 0], ref[..., 1] = 3.0, 4.0          # every row norm 5
    x = ref.copy()
    x[1, 0, 4] = 1.25                            # that row: 1.25 / 5 = 0.25
    assert oracle.rel_l2(x, ref, axes=(-1,)) == pytest.approx(0.25, abs=1e-15)
    # the same arrays sliced per b over (h, d) dilute it: 1.25 / sqrt(75)
    assert oracle.rel_l2(x, ref, axes=(-2, -1)) == pytest.approx(1.25 / math.sqrt(75.0), rel=1e-14)


def test_gpu_parity_helper_picks_the_slice_axes():
    # tests/gpu_util.rel_l2 (what every GPU parity test calls) slices [B,H,N,d]
    # and [B,H,d,d] tensors per (b, h) over the last two axes, [B,H,d] per row
    gpu_util = pytest.importorskip("gpu_util")
    ref4 = np.ones((1, 4, 6, 8))
    x4 = ref4.copy()
    x4[0, 2] *= 1.1                              # one head: 0.1
    assert gpu_util.rel_l2(x4, ref4) == pytest.approx(0.1, rel=1e-12)
    ref3 = np.ones((2, 4, 8))
    x3 = ref3.copy()
    x3[1, 3, :] *= 0.7                           # one row: 0.3
    assert gpu_util.rel_l2(x3, ref3) == pytest.approx(0.3, rel=1e-12)
    with pytest.raises(AssertionError):
        gpu_util.rel_l2(np.ones((1, 2, 3, 4)), np.ones((1, 2, 4, 3)))


def _mutant_rel_l2(x, ref, kind, axes=(-2, -1)):
    """Plausible wrong checkers, each planted in a copy (CPU only)."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if kind == "global_ratio":
        return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    if kind == "absolute":
        return float(np.max(num))
    if kind == "mean_over_slices":
        return float(np.mean(num / den))
    if kind == "squared":
        return float(np.max(num ** 2 / den ** 2))
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["global_ratio", "absolute", "mean_over_slices", "squared"])
def test_rel_l2_pins_detect_planted_checker_mistakes(kind):
    ref = np.stack([np.stack([_slice_3_4() for _ in range(3)]) for _ in range(2)])
    x = ref.copy()
    x[1, 2, 0, 4] += 2.5
    assert oracle.rel_l2(x, ref) == pytest.approx(0.5, abs=1e-15)
    assert _mutant_rel_l2(x, ref, kind) != pytest.approx(0.5, rel=1e-3)
