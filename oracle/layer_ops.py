"""fp64 CPU oracle for the linear-attention layer's neighbouring ops
(TEST INFRASTRUCTURE: only tests/, the smoke entry and the benchmark's CPU
leg may import it; it shares no code with the GPU library).

Ling and Ring 2.6 Technical Report, Fig. 2 (the layer: QKV projection ->
QK Norm -> RoPE -> linear attention -> grouped RMSNorm, times sigmoid of the
gate projection -> output projection) and §2.1.1 (RMSNorm epsilon 1e-6, RoPE
base 6e6, rotary dimension 64 out of the head dimension 128).

Readings where the pages are silent: QK Norm is an RMSNorm over each head's d
channels with one [d] weight per tensor; RoPE is the rotate-half form on the
first rot_dim channels (pairs j, j + rot_dim/2, frequency theta^(-2j/rot_dim))
at position pos0 + t; the grouped RMSNorm normalises groups of `group`
consecutive channels of the [H*d] output row with one [H*d] weight.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, weight, eps, axis=-1):
    """x / sqrt(mean(x^2) + eps) * weight along `axis` (fp64)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=axis, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(weight)


def rope_angles(n_pos, rot_dim, theta, pos0=0):
    """[n_pos, rot_dim/2] angles (pos0 + t) * theta^(-2j/rot_dim), fp64."""
    j = np.arange(rot_dim // 2, dtype=np.float64)
    freq = float(theta) ** (-2.0 * j / rot_dim)
    pos = pos0 + np.arange(n_pos, dtype=np.float64)
    return pos[:, None] * freq[None, :]


def rope(x, rot_dim, theta, pos0=0):
    """Rotate-half RoPE on the first rot_dim channels of x [..., N, H, d]
    (positions along axis -3)."""
    x = _f64(x).copy()
    if rot_dim == 0:
        return x
    h = rot_dim // 2
    ang = rope_angles(x.shape[-3], rot_dim, theta, pos0)[:, None, :]      # [N, 1, h]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h].copy(), x[..., h:rot_dim].copy()
    x[..., :h] = a * c - b * s
    x[..., h:rot_dim] = b * c + a * s
    return x


def qk_norm_rope(q, k, v, q_weight, k_weight, theta, rot_dim, pos0, eps):
    """q, k, v: [B,N,H,d] -> (q', k', v') [B,H,N,d]: RMSNorm over d, then RoPE
    for q and k; v only changes layout."""
    qn = rope(rms_norm(q, q_weight, eps), rot_dim, theta, pos0)
    kn = rope(rms_norm(k, k_weight, eps), rot_dim, theta, pos0)
    return tuple(np.ascontiguousarray(np.transpose(_f64(x), (0, 2, 1, 3))) for x in (qn, kn, v))


def group_norm_gate(o, gate, weight, group, eps):
    """o: [B,H,N,d], gate: [B,N,H*d], weight: [H*d] -> y [B,N,H*d]:
    RMSNorm over groups of `group` consecutive channels, times sigmoid(gate)."""
    o = _f64(o)
    B, H, N, d = o.shape
    x = np.transpose(o, (0, 2, 1, 3)).reshape(B, N, H * d // group, group)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    xn = (x / np.sqrt(ms + eps)).reshape(B, N, H * d) * _f64(weight)
    return xn / (1.0 + np.exp(-_f64(gate)))
