"""fp64 CPU oracle for decayed causal linear attention (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library and
never imports it.

Definition followed (Ling and Ring 2.6 Technical Report, §4.1.1: linear
attention as an RNN-style recurrence over a per-(batch, head) D x D state):

    o_t = sum_{s <= t} lambda_h^(t-s) (q_t . k_s) v_s  +  lambda_h^(t+1) q_t S_init
    S_t = lambda_h S_{t-1} + k_t^T v_t,   o_t = q_t S_t,   S_{-1} = S_init
    lambda_h = exp(-s_h)

Several statements of it live here:

* ``prefill`` / ``decode_step``: the recurrence, in plain C (``la_oracle.c``),
  fp64, OpenMP over the B*H slices.  This is the oracle the GPU is compared to.
* ``prefill_varlen``: a packed batch of independent sequences (the report's
  §4.1.2: packed sub-sequences, each attending only within itself), i.e. the
  same recurrence restarted from each sequence's own state.
* ``decode_multi``: several tokens per sequence from the carried state with
  only a leading prefix committed to the stored state (draft verification in
  serving with multi-token prediction, the report's §4.3 and Appendix B),
  i.e. ``decode_step`` applied token after token.
* ``quadratic``: the definition's double sum written out as a masked
  decay-weighted score matrix (NumPy, fp64, tiny sizes only).
* ``blockwise``: the block decomposition the GPU kernels follow (intra-block
  masked scores times V, plus the inter-block term from the carried state,
  plus the decayed state scan), NumPy fp64.  It exists to show that the
  decomposition reaches the definition at any block length.
* ``cp_fold`` / ``cp_correct``: the two steps of the sequence-sharded
  (context-parallel) prefill of the report's §4.1.1 and Fig. 10 that follow
  each rank's local pass from a zero state: the incoming state of rank r from
  the all-gathered local states, and the correction of the rank's local
  output with it.  NumPy fp64.

Inputs are NumPy arrays (or anything ``np.asarray`` takes) that are widened
exactly to fp64; bf16/fp32 tensors are widened by the caller (exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblaoracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile la_oracle.c with gcc (host code only, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = build(force=False)
            lib = ctypes.CDLL(path)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.la_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64]
            lib.la_oracle_prefill.restype = ctypes.c_int
            lib.la_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64]
            lib.la_oracle_decode_step.restype = ctypes.c_int
            lib.la_oracle_set_threads.argtypes = [ctypes.c_int]
            lib.la_oracle_set_threads.restype = None
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


last_threads = 0


def set_threads(n: int) -> None:
    """Thread count of the C oracle's OpenMP loops from now on (timing aid;
    results are independent of it)."""
    _load().la_oracle_set_threads(int(n))


def prefill(q, k, v, slopes, state_init=None, want_out: bool = True):
    """Recurrent fp64 prefill.

    q, k, v: [B,H,N,d]; slopes: [H]; state_init: [B,H,d,d] or None (zeros).
    Returns (out [B,H,N,d] fp64 or None, final_state [B,H,d,d] fp64).
    """
    global last_threads
    q, k, v, s = _f64(q), _f64(k), _f64(v), _f64(slopes)
    B, H, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and s.shape == (H,)
    st = np.zeros((B, H, d, d)) if state_init is None else _f64(state_init).copy()
    assert st.shape == (B, H, d, d)
    out = np.zeros((B, H, N, d)) if want_out else None
    r = _load().la_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(st),
                                  _ptr(out) if want_out else None, B, H, N, d)
    if r < 0:
        raise ValueError("la_oracle_prefill rejected its arguments")
    last_threads = min(r, B * H)
    return out, st


def prefill_varlen(q, k, v, slopes, cu_seqlens, states_init=None, want_out: bool = True):
    """Packed prefill over independent sequences, fp64.

    q, k, v: [H,T,d]; cu_seqlens: nseq+1 non-decreasing offsets, cu[0] = 0,
    cu[nseq] = T; states_init: [nseq,H,d,d] or None (zeros).  Sequence i is
    rows cu[i]:cu[i+1] of every head; it runs the recurrence of ``prefill``
    from its own initial state and never sees another sequence's tokens.
    Returns (out [H,T,d] or None, final states [nseq,H,d,d]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, T, d = q.shape
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    nseq = len(cu) - 1
    if nseq < 1 or cu[0] != 0 or cu[-1] != T or any(a > b for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to T")
    st = np.zeros((nseq, H, d, d)) if states_init is None else _f64(states_init).copy()
    assert st.shape == (nseq, H, d, d)
    out = np.zeros((H, T, d)) if want_out else None
    for i in range(nseq):
        a, b = cu[i], cu[i + 1]
        if a == b:
            continue                                   # an empty sequence keeps its state
        o, fin = prefill(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], slopes,
                         st[i:i + 1], want_out)
        st[i] = fin[0]
        if want_out:
            out[:, a:b] = o[0]
    return out, st


def decode_step(q, k, v, slopes, state, inplace: bool = False):
    """One decode step: q, k, v [B,H,d]; state [B,H,d,d].

    Returns (out [B,H,d], new_state).  The state is copied unless ``inplace``
    is set and it is already a contiguous fp64 array (then it is updated)."""
    q, k, v, s = _f64(q), _f64(k), _f64(v), _f64(slopes)
    B, H, d = q.shape
    if inplace and isinstance(state, np.ndarray) and state.dtype == np.float64 \
            and state.flags.c_contiguous:
        st = state
    else:
        st = _f64(state).copy()
    out = np.zeros((B, H, d))
    r = _load().la_oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(st),
                                      _ptr(out), B, H, d)
    if r < 0:
        raise ValueError("la_oracle_decode_step rejected its arguments")
    return out, st


def decode_multi(q, k, v, slopes, state, n_commit=None):
    """T tokens per sequence from the carried state, fp64.

    q, k, v: [B,H,T,d]; state: [B,H,d,d]; n_commit: B integers or None (= T).
    Token t: S_t = lambda S_{t-1} + k_t^T v_t, o_t = q_t S_t, S_{-1} = state.
    Returns (out [B,H,T,d] for every token, committed state [B,H,d,d] =
    S_{n-1} with n = n_commit[b] clamped to [0, T]; the entry state for n = 0).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, d = q.shape
    S = _f64(state).copy()
    n = [T] * B if n_commit is None else [min(max(int(x), 0), T) for x in np.asarray(n_commit)]
    committed = S.copy()
    out = np.zeros((B, H, T, d))
    for t in range(T):
        o, S = decode_step(q[:, :, t], k[:, :, t], v[:, :, t], slopes, S)
        out[:, :, t] = o
        for b in range(B):
            if n[b] == t + 1:
                committed[b] = S[b]
    return out, committed


def quadratic(q, k, v, slopes, state_init=None):
    """The definition's double sum, O(N^2) per slice (tiny inputs only).

    o_t = sum_{s<=t} lambda^(t-s) (q_t.k_s) v_s + lambda^(t+1) q_t S_init,
    final = lambda^N S_init + sum_s lambda^(N-1-s) k_s^T v_s.
    """
    q, k, v, s = _f64(q), _f64(k), _f64(v), _f64(slopes)
    B, H, N, d = q.shape
    S0 = np.zeros((B, H, d, d)) if state_init is None else _f64(state_init)
    out = np.zeros((B, H, N, d))
    fin = np.zeros((B, H, d, d))
    t = np.arange(N)
    for h in range(H):
        lam = np.exp(-s[h])
        # decay matrix lambda^(t-s) on s <= t, zero above the diagonal (0**0 == 1)
        expo = (t[:, None] - t[None, :]).astype(np.float64)
        dec = np.where(expo >= 0, lam ** np.maximum(expo, 0.0), 0.0)
        for b in range(B):
            scores = q[b, h] @ k[b, h].T                     # [N, N], (q_t . k_s)
            out[b, h] = (scores * dec) @ v[b, h]
            out[b, h] += (lam ** (t + 1.0))[:, None] * (q[b, h] @ S0[b, h])
            w = lam ** (N - 1.0 - t)                         # weight of token s in the final state
            fin[b, h] = (lam ** float(N)) * S0[b, h] + (k[b, h] * w[:, None]).T @ v[b, h]
    return out, fin


def blockwise(q, k, v, slopes, state_init=None, C: int = 64):
    """Block decomposition with block length C (any C >= 1), fp64.

    For the block of c tokens starting at t0, with local indices a, b < c:
      P      = (Q K^T) * D,  D[a,b] = lambda^(a-b) for b <= a, else 0
      O      = P V + diag(lambda^(a+1)) Q S_prev
      S_next = lambda^c S_prev + (diag(lambda^(c-1-b)) K)^T V
    """
    q, k, v, s = _f64(q), _f64(k), _f64(v), _f64(slopes)
    B, H, N, d = q.shape
    S0 = np.zeros((B, H, d, d)) if state_init is None else _f64(state_init)
    out = np.zeros((B, H, N, d))
    fin = np.zeros((B, H, d, d))
    for h in range(H):
        lam = np.exp(-s[h])
        for b in range(B):
            S = S0[b, h].copy()
            for t0 in range(0, N, C):
                c = min(C, N - t0)
                Q, K, V = q[b, h, t0:t0 + c], k[b, h, t0:t0 + c], v[b, h, t0:t0 + c]
                ai = np.arange(c)
                expo = (ai[:, None] - ai[None, :]).astype(np.float64)
                D = np.where(expo >= 0, lam ** np.maximum(expo, 0.0), 0.0)
                P = (Q @ K.T) * D
                out[b, h, t0:t0 + c] = P @ V + (lam ** (ai + 1.0))[:, None] * (Q @ S)
                S = (lam ** float(c)) * S + (K * (lam ** (c - 1.0 - ai))[:, None]).T @ V
            fin[b, h] = S
    return out, fin


def cp_fold(local_states, shard_lens, slopes, rank, state_init=None):
    """Incoming state of shard ``rank`` of a sequence split into consecutive
    shards (the report's §4.1.1, Fig. 10: each rank's local state is the
    decayed sum of k^T v over its own tokens from a zero state; the local
    states are all-gathered and every rank folds in those of the shards before
    it).

    local_states: [R,B,H,d,d], shard j's state after its L_j tokens from zero;
    shard_lens: R lengths L_j; rank in 0..R (R gives the state after the
    whole sequence).  With start_r = L_0 + ... + L_{r-1}:

        S_in(r) = lambda^start_r S_init + sum_{j<r} lambda^(start_r - start_{j+1}) S_loc(j)

    (shard j's state is decayed by the tokens that follow it up to start_r).
    Returns [B,H,d,d] fp64.
    """
    loc = _f64(local_states)
    s = _f64(slopes)
    lens = [int(x) for x in np.asarray(shard_lens).reshape(-1)]
    R, B, H, d, _ = loc.shape
    if len(lens) != R or not 0 <= rank <= R or any(n < 0 for n in lens):
        raise ValueError("bad shard lengths or rank")
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.float64)
    lam = np.exp(-s)[None, :, None, None]                       # [1,H,1,1]
    out = np.zeros((B, H, d, d))
    if state_init is not None:
        out += lam ** starts[rank] * _f64(state_init)
    for j in range(rank):
        out += lam ** (starts[rank] - starts[j + 1]) * loc[j]
    return out


def cp_correct(q, slopes, state_in, out_local):
    """Shard output from its local output (computed from a zero state) and its
    incoming state: o_a = o_local_a + lambda^(a+1) q_a S_in for local token
    index a (the report's §4.1.1, Fig. 10: the rank corrects its local O once
    the preceding states are known).

    q, out_local: [B,H,L,d]; state_in: [B,H,d,d].  Returns [B,H,L,d] fp64.
    """
    q, s, S = _f64(q), _f64(slopes), _f64(state_in)
    B, H, L, d = q.shape
    a = np.arange(L, dtype=np.float64)
    lam = np.exp(-s)[:, None] ** (a[None, :] + 1.0)              # [H, L]
    return _f64(out_local) + lam[None, :, :, None] * (q @ S)


def rel_l2(x, ref, axes=(-2, -1)):
    """max over leading slices of ||x - ref||_2 / ||ref||_2 (absolute if ||ref|| == 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(np.max(r)) if r.size else 0.0
