"""Pins for the fp64 oracle of the layer's neighbouring ops (QK RMSNorm +
partial RoPE, grouped RMSNorm x sigmoid gate): hand-worked values, rotation
and normalisation invariants, and planted mistakes (CPU only)."""
import math

import numpy as np
import pytest

from oracle import layer_ops as lo


def test_rope_hand_worked_values():
    # d = rot = 16, theta = 10^4, position 1: pair j couples channels j and
    # j + 8 and turns by theta^(-2j/16) radians
    x = np.zeros((1, 2, 1, 16))              # [B, N, H, d], positions 0 and 1
    x[0, :, 0, 0] = 1.0                      # unit vector on channel 0
    y = lo.rope(x, 16, 1e4)
    assert np.allclose(y[0, 0, 0], x[0, 0, 0], atol=0)            # position 0: identity
    assert abs(y[0, 1, 0, 0] - 0.5403023058681398) < 1e-15         # cos 1
    assert abs(y[0, 1, 0, 8] - 0.8414709848078965) < 1e-15         # sin 1
    assert np.count_nonzero(y[0, 1, 0]) == 2
    x = np.zeros((1, 2, 1, 16))
    x[0, :, 0, 9] = 1.0                      # channel 9 = second half of pair 1
    y = lo.rope(x, 16, 1e4)
    a = 1e4 ** (-2.0 / 16)                   # 0.31622776601683794 rad
    assert abs(y[0, 1, 0, 1] + math.sin(a)) < 1e-15 and abs(y[0, 1, 0, 9] - math.cos(a)) < 1e-15


def test_rope_partial_keeps_the_rest_and_preserves_norms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 9, 3, 128))
    y = lo.rope(x, 64, 6e6, pos0=1000)
    assert np.array_equal(y[..., 64:], x[..., 64:])
    h = 32
    assert np.allclose(y[..., :h] ** 2 + y[..., h:64] ** 2, x[..., :h] ** 2 + x[..., h:64] ** 2)
    assert np.array_equal(lo.rope(x, 0, 6e6, 5), x)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 1, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    def score(m, n):
        return float(np.sum(lo.rope(q, 64, 6e6, m) * lo.rope(k, 64, 6e6, n)))
    s = score(10, 3)
    for shift in (1, 57, 262000):
        assert abs(score(10 + shift, 3 + shift) - s) < 1e-9 * (1 + abs(s))
    assert abs(score(11, 3) - s) > 1e-6


def test_rms_norm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 5, 6, 128)) * 3
    y = lo.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0)
    assert np.allclose(lo.rms_norm(7.5 * x, np.ones(128), 0.0), y)
    w = rng.standard_normal(128)
    assert np.allclose(lo.rms_norm(x, w, 0.0), y * w)


def test_qk_norm_rope_layouts_and_order():
    rng = np.random.default_rng(4)
    B, N, H, d = 2, 5, 3, 16
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    wq, wk = rng.standard_normal(d), rng.standard_normal(d)
    qo, ko, vo = lo.qk_norm_rope(q, k, v, wq, wk, 1e4, 16, 7, 1e-6)
    assert qo.shape == (B, H, N, d)
    assert np.array_equal(vo, np.transpose(v, (0, 2, 1, 3)))
    b, t, h = 1, 3, 2                        # one row by hand: norm, then rotate
    r = q[b, t, h] / math.sqrt(np.mean(q[b, t, h] ** 2) + 1e-6) * wq
    ang = (7 + t) * 1e4 ** (-2.0 * np.arange(8) / 16)
    want = np.concatenate([r[:8] * np.cos(ang) - r[8:] * np.sin(ang),
                           r[8:] * np.cos(ang) + r[:8] * np.sin(ang)])
    assert np.allclose(qo[b, h, t], want, rtol=1e-14, atol=1e-14)


def test_group_norm_gate_against_a_loop_over_groups():
    rng = np.random.default_rng(5)
    B, H, N, d = 2, 3, 4, 32
    o = rng.standard_normal((B, H, N, d))
    g = rng.standard_normal((B, N, H * d))
    w = rng.standard_normal(H * d)
    for group in (8, 16, 32):
        y = lo.group_norm_gate(o, g, w, group, 1e-6)
        for b in range(B):
            for t in range(N):
                row = np.concatenate([o[b, h, t] for h in range(H)])
                for s in range(0, H * d, group):
                    seg = row[s:s + group]
                    want = seg / math.sqrt(np.mean(seg ** 2) + 1e-6) * w[s:s + group] \
                        / (1 + np.exp(-g[b, t, s:s + group]))
                    assert np.allclose(y[b, t, s:s + group], want, rtol=1e-13, atol=1e-13)


def test_group_norm_gate_special_cases():
    rng = np.random.default_rng(6)
    o = rng.standard_normal((1, 2, 3, 16))
    ones = np.ones(32)
    y0 = lo.group_norm_gate(o, np.zeros((1, 3, 32)), ones, 16, 0.0)       # sigmoid(0) = 1/2
    y1 = lo.group_norm_gate(o, np.full((1, 3, 32), 60.0), ones, 16, 0.0)  # sigmoid -> 1
    assert np.allclose(2 * y0, y1)
    assert np.allclose(np.mean(y1.reshape(1, 3, 2, 16) ** 2, axis=-1), 1.0)


@pytest.mark.parametrize("mutation", ["interleaved_pairs", "reverse_rotation", "rope_before_norm"])
def test_layer_pins_detect_planted_mistakes(mutation):
    # planted mistakes in a copy of the prologue must fail the hand-worked row
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 4, 1, 16)) + 0.5
    w = rng.standard_normal(16)
    good = lo.rope(lo.rms_norm(x, w, 1e-6), 16, 1e4, 3)
    if mutation == "interleaved_pairs":
        xn = lo.rms_norm(x, w, 1e-6)
        bad = xn.copy()
        ang = lo.rope_angles(4, 16, 1e4, 3)[:, None, :]
        a, b = xn[..., 0::2], xn[..., 1::2]
        bad[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
        bad[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
    elif mutation == "reverse_rotation":
        xn = lo.rms_norm(x, w, 1e-6)
        bad = lo.rope(xn, 16, 1e4, 3)
        ang = lo.rope_angles(4, 16, 1e4, 3)[:, None, :]
        bad[..., :8] = xn[..., :8] * np.cos(ang) + xn[..., 8:] * np.sin(ang)
        bad[..., 8:] = xn[..., 8:] * np.cos(ang) - xn[..., :8] * np.sin(ang)
    else:
        bad = lo.rms_norm(lo.rope(x, 16, 1e4, 3), w, 1e-6)
    assert np.max(np.abs(bad - good)) > 1e-3
