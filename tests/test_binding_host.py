"""Host logic of the binding, on the CPU: which tensor views go to the strided
entry points and with which element strides, and which are refused before
any library call."""
import pytest
import torch

from long_context_layers_amd import binding

CPU = torch.device("cpu")


def heads(buf, col0, H, d):
    return buf[..., col0:col0 + H * d].unflatten(-1, (H, d)).transpose(-3, -2)


def test_view_strides_of_a_projection_slice():
    B, N, H, d = 2, 5, 3, 8
    buf = torch.zeros((B, N, 4 * H * d), dtype=torch.bfloat16)
    q = heads(buf, 0, H, d)
    assert tuple(q.shape) == (B, H, N, d)
    assert binding._view(q, "q", torch.bfloat16, CPU, (B, H, N, d)) == (N * 4 * H * d, d, 4 * H * d)


def test_contiguous_tensors_take_the_dense_call():
    x = torch.zeros((1, 2, 4, 8), dtype=torch.bfloat16)
    assert binding._strided(x, x, x, None, torch.bfloat16, CPU, (1, 2, 4, 8)) is False
    assert binding._strided(x, x, x, x.clone(), torch.bfloat16, CPU, (1, 2, 4, 8)) is False


def test_views_take_the_strided_call():
    B, N, H, d = 1, 4, 2, 8
    buf = torch.zeros((B, N, 3 * H * d), dtype=torch.bfloat16)
    q, k, v = (heads(buf, i * H * d, H, d) for i in range(3))
    assert binding._strided(q, k, v, None, torch.bfloat16, CPU, (B, H, N, d)) is True
    # contiguous inputs with a strided output also take it
    c = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    out = heads(torch.zeros((B, N, H * d), dtype=torch.bfloat16), 0, H, d)
    assert binding._strided(c, c, c, out, torch.bfloat16, CPU, (B, H, N, d)) is True


def test_inputs_with_different_strides_are_refused():
    B, N, H, d = 1, 4, 2, 8
    buf = torch.zeros((B, N, 3 * H * d), dtype=torch.bfloat16)
    q, k = heads(buf, 0, H, d), heads(buf, H * d, H, d)
    v = torch.zeros((B, H, N, d), dtype=torch.bfloat16)          # contiguous: other strides
    with pytest.raises(ValueError):
        binding._strided(q, k, v, None, torch.bfloat16, CPU, (B, H, N, d))


def test_fp32_views_are_refused():
    buf = torch.zeros((1, 4, 3 * 16), dtype=torch.float32)
    q, k, v = (heads(buf, i * 16, 2, 8) for i in range(3))
    with pytest.raises(ValueError):
        binding._strided(q, k, v, None, torch.float32, CPU, (1, 2, 4, 8))


def test_non_unit_channel_stride_is_refused():
    x = torch.zeros((1, 2, 8, 4), dtype=torch.bfloat16).transpose(2, 3)   # channels strided
    with pytest.raises(ValueError):
        binding._view(x, "q", torch.bfloat16, CPU, (1, 2, 4, 8))


def test_wrong_dtype_device_or_shape_is_refused():
    x = torch.zeros((1, 2, 4, 8), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        binding._view(x.float(), "q", torch.bfloat16, CPU, (1, 2, 4, 8))
    with pytest.raises(ValueError):
        binding._view(x, "q", torch.bfloat16, CPU, (1, 2, 4, 9))
    with pytest.raises(TypeError):
        binding._view(x, "q", torch.bfloat16, torch.device("meta"), (1, 2, 4, 8))


def test_rows_helper_reads_the_token_stride():
    buf = torch.zeros((2, 5, 4 * 16), dtype=torch.bfloat16)
    assert binding._rows(buf[..., 16:32], "k", CPU, (2, 5, 16)) == 64
    with pytest.raises(ValueError):
        binding._rows(buf.transpose(0, 1)[..., :16], "k", CPU, (5, 2, 16))   # batch stride != N * token stride


def test_gpu_only_calls_refuse_cpu_tensors():
    x = torch.zeros((1, 2, 4, 8), dtype=torch.bfloat16)
    s = torch.zeros(2)
    with pytest.raises(ValueError):
        binding.cp_correct(x, s, torch.zeros(1, 2, 8, 8), x.clone())
    with pytest.raises(ValueError):
        binding.cp_fold(torch.zeros(2, 1, 2, 8, 8), [1, 1], 1, s)
    with pytest.raises(ValueError):
        binding.prefill_varlen(x[0], x[0], x[0], s, torch.zeros(2, dtype=torch.int64),
                               torch.zeros(1, 2, 8, 8))
