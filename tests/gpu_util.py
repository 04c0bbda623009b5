"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

import oracle

BF16_TOL = 2e-2      # max over (b, h) of relative L2 error, bf16 activations
F32_TOL = 1e-3       # same, fp32 activations

# Regression guards on the named bf16 workloads, below the pass bars: the
# kernels measure 2.4e-3 .. 2.8e-3 (outputs: the bf16 scores, the bf16 copy of
# the state and the bf16 output each round at ~2^-9 relative) and 1.7e-3 for
# prefill states, 1.7e-6 for decode states (fp32, never rounded).  A change
# that loses precision (an extra bf16 rounding, a state kept in bf16) moves
# these well before it reaches the 2e-2 bar.
BF16_GUARD = 4e-3     # outputs and prefill final states
DECODE_STATE_GUARD = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (bf16 / fp32) tensor to fp64 on the host."""
    return t.detach().to("cpu", torch.float32).double().numpy()


def rel_l2(x, ref):
    """max over (b, h) slices of ||x - ref|| / ||ref|| (fp64).

    [B,H,N,d] / [B,H,d,d] tensors are sliced per (b, h) over the last two
    axes, [B,H,d] decode outputs per (b, h) over the last axis."""
    x = x if isinstance(x, np.ndarray) else np64(x)
    ref = ref if isinstance(ref, np.ndarray) else np64(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    return oracle.rel_l2(x, ref, axes=(-1,) if x.ndim == 3 else (-2, -1))


def oracle_prefill(q, k, v, slopes, state0, heads=None):
    """Run the fp64 oracle on device tensors (optionally on a subset of heads)."""
    if heads is not None:
        idx = torch.tensor(heads, device=q.device)
        q, k, v = (t.index_select(1, idx) for t in (q, k, v))
        slopes = slopes.index_select(0, idx)
        state0 = state0.index_select(1, idx)
    return oracle.prefill(np64(q), np64(k), np64(v), np64(slopes), np64(state0))
