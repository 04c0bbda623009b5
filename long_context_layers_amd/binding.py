"""ctypes binding of liblightning_attn.so (argument marshalling only).

Every function here checks dtypes, devices, shapes and strides, then passes
raw device pointers, sizes and element strides and the current HIP stream to
the C ABI declared in ``include/lightning_attn.h``.  PyTorch only provides
device memory and streams; all of the layer's arithmetic runs in the
library's HIP kernels.
There is no fallback: if the library is missing or a call fails, an error is
raised.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "liblightning_attn.so")

# names and signatures of the C ABI (include/lightning_attn.h)
_P, _I64, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "la_prefill": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "la_prefill_f32": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "la_prefill_workspace_bytes": ([_I64, _I64, _I64, _I64, ctypes.POINTER(_I64)], _INT),
    "la_prefill_ws": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P], _INT),
    "la_prefill_f32_workspace_bytes": ([_I64, _I64, _I64, _I64, ctypes.POINTER(_I64)], _INT),
    "la_prefill_f32_ws": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P], _INT),
    "la_prefill_noalloc": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "la_prefill_varlen": ([_P, _P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I64, _P], _INT),
    "la_prefill_varlen_f32": ([_P, _P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I64, _P], _INT),
    "la_prefill_strided": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                            _I64, _I64, _I64, _I64, _I64, _I64, _P], _INT),
    "la_prefill_strided_ws": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                               _I64, _I64, _I64, _I64, _I64, _I64, _P, _I64, _P], _INT),
    "la_prefill_qk_norm_rope_ws": ([_P, _P, _P, _P, _P, _P, ctypes.c_double, _I64, _I64,
                                    ctypes.c_float, _P, _P, _I64, _I64, _I64, _I64,
                                    _I64, _I64, _I64, _I64, _I64, _I64, _P, _I64, _P], _INT),
    "la_prefill_varlen_from_zero": ([_P, _P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I64,
                                     _I64, _I64, _I64, _I64, _P], _INT),
    "la_prefill_varlen_strided": ([_P, _P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I64,
                                   _I64, _I64, _I64, _I64, _P], _INT),
    "la_decode_step": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], _INT),
    "la_decode_multi": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "la_decode_multi_f32": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "la_decode_step_f32": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], _INT),
    "la_decode_step_strided": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P], _INT),
    "la_decode_multi_strided": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64,
                                 _I64, _P], _INT),
    "la_qk_norm_rope": ([_P, _P, _P, _I64, _P, _P, ctypes.c_double, _I64, _I64, ctypes.c_float,
                         _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "la_group_norm_gate": ([_P, _I64, _I64, _I64, _P, _I64, _P, _I64, ctypes.c_float, _P,
                            _I64, _I64, _I64, _I64, _P], _INT),
    "la_cp_fold": ([_P, _P, _I64, _I64, _P, _P, _P, _I64, _I64, _I64, _P], _INT),
    "la_cp_correct": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "la_status_string": ([_INT], ctypes.c_char_p),
    "la_prefill_varlen_plan": ([_I64, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_int)], _INT),
    "la_abi_version": ([], _INT),
}
ABI_VERSION = 8

_lock = threading.Lock()
_lib = None


class LightningAttnError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise LightningAttnError(
                    f"{path} is missing: build it with `python -m long_context_layers_amd.build` "
                    "(there is no CPU fallback)")
            lib = ctypes.CDLL(path)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            if lib.la_abi_version() != ABI_VERSION:
                raise LightningAttnError("liblightning_attn.so ABI version mismatch")
            _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load_library().la_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise LightningAttnError(f"{what}: {status_string(code)} (status {code})")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, dev, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _view(t: torch.Tensor, name: str, dtype, dev, shape):
    """A bf16 view of `shape` with unit channel stride: its other strides."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev or t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} on {dev}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name} must have a unit channel stride")
    return tuple(t.stride()[:-1])


def _strided(q, k, v, out, dt, dev, shape) -> bool:
    """True if q, k, v or out is a non-contiguous view that the strided
    bf16 prefill takes (q, k, v sharing one set of strides)."""
    ts = (q, k, v) if out is None else (q, k, v, out)
    if all(isinstance(t, torch.Tensor) and t.is_contiguous() for t in ts):
        return False
    if dt != torch.bfloat16:
        raise ValueError("strided q/k/v/out are taken for bfloat16 only; pass contiguous fp32 tensors")
    st = _view(q, "q", dt, dev, shape)
    for t, n in ((k, "k"), (v, "v")):
        if _view(t, n, dt, dev, shape) != st:
            raise ValueError("q, k and v must share one set of strides")
    return True


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, slopes: torch.Tensor,
            state: torch.Tensor, out: Optional[torch.Tensor] = None,
            split: bool = True) -> torch.Tensor:
    """Blockwise decayed causal linear attention over N tokens.

    q, k, v: [B,H,N,d] bf16 or fp32 on one GPU; slopes: [H] fp32;
    state: [B,H,d,d] fp32, IN = initial state, OUT = final state (in place).
    Returns out [B,H,N,d] (same dtype as q).  Enqueued on the current stream.
    bf16 q, k, v (sharing one set of strides) and out may be strided views
    with a unit channel stride, e.g. head-split slices of a token-major
    projection buffer; such calls go to ``la_prefill_strided``.  bf16 calls
    go to ``la_prefill_ws`` / ``la_prefill_strided_ws`` (the sequence split,
    with a workspace from torch's allocator) when a split is planned, fp32
    calls to ``la_prefill_f32_ws``, unless ``split`` is False (then
    ``la_prefill`` / ``la_prefill_strided`` / ``la_prefill_f32``).
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B,H,N,d] tensor")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("prefill runs on a GPU tensor only (no CPU path)")
    B, H, N, d = q.shape
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _view(t, n, dt, dev, (B, H, N, d))
    _need(slopes, "slopes", torch.float32, dev, (H,))
    _need(state, "state", torch.float32, dev, (B, H, d, d))
    if _strided(q, k, v, out, dt, dev, (B, H, N, d)):
        if out is None:
            out = torch.empty((B, H, N, d), dtype=dt, device=dev)
        so = _view(out, "out", dt, dev, (B, H, N, d))
        si = q.stride()[:-1]
        ws = prefill_workspace_bytes(B, H, N, d, dev) if split else 0
        with torch.cuda.device(dev):
            if ws > 0:
                work = torch.empty(ws, dtype=torch.uint8, device=dev)
                rc = load_library().la_prefill_strided_ws(
                    q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), out.data_ptr(),
                    state.data_ptr(), B, H, N, d, *si, *so, work.data_ptr(), ws, _stream(dev))
                _check(rc, "la_prefill_strided_ws")
                return out
            rc = load_library().la_prefill_strided(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), out.data_ptr(),
                state.data_ptr(), B, H, N, d, *si, *so, _stream(dev))
        _check(rc, "la_prefill_strided")
        return out
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", dt, dev, (B, H, N, d))
    lib = load_library()
    if dt == torch.bfloat16 and split:
        ws = prefill_workspace_bytes(B, H, N, d, dev)
        if ws > 0:
            # the sequence split over the whole device (la_prefill_ws); the
            # workspace comes from torch's caching allocator
            work = torch.empty(ws, dtype=torch.uint8, device=dev)
            with torch.cuda.device(dev):
                rc = lib.la_prefill_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(),
                                       out.data_ptr(), state.data_ptr(), B, H, N, d,
                                       work.data_ptr(), ws, _stream(dev))
            _check(rc, "la_prefill_ws")
            return out
    if dt == torch.float32 and split:
        ws = prefill_f32_workspace_bytes(B, H, N, d, dev)
        if ws > 0:
            work = torch.empty(ws, dtype=torch.uint8, device=dev)
            with torch.cuda.device(dev):
                rc = lib.la_prefill_f32_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(),
                                           out.data_ptr(), state.data_ptr(), B, H, N, d,
                                           work.data_ptr(), ws, _stream(dev))
            _check(rc, "la_prefill_f32_ws")
            return out
    fn = lib.la_prefill if dt == torch.bfloat16 else lib.la_prefill_f32
    with torch.cuda.device(dev):
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), out.data_ptr(),
                state.data_ptr(), B, H, N, d, _stream(dev))
    _check(rc, "la_prefill" if dt == torch.bfloat16 else "la_prefill_f32")
    return out


def prefill_qk_norm_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, slopes: torch.Tensor,
                         state: torch.Tensor, q_norm_weight: torch.Tensor,
                         k_norm_weight: torch.Tensor, theta: float = 6.0e6, rot_dim: int = 64,
                         pos0: int = 0, eps: float = 1e-6,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The prefill straight from the projection's raw q and k
    (``la_prefill_qk_norm_rope_ws``): QK RMSNorm + RoPE (as ``qk_norm_rope``
    defines them) applied inside the attention kernels, then the decayed
    linear attention.

    q, k, v: [B,H,N,128] bf16 views sharing one set of strides with a unit
    channel stride (e.g. head-split slices of a packed [B,N,4*H*d]
    projection output); weights [128] fp32; state [B,H,d,d] fp32 in/out.
    Returns out [B,H,N,d] (or writes the given bf16 view).  The sequence
    split's workspace, when planned, comes from torch's allocator.
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B,H,N,d] tensor")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("prefill_qk_norm_rope runs on GPU tensors only (no CPU path)")
    B, H, N, d = q.shape
    dt = torch.bfloat16
    si = _view(q, "q", dt, dev, (B, H, N, d))
    for t, n in ((k, "k"), (v, "v")):
        if _view(t, n, dt, dev, (B, H, N, d)) != si:
            raise ValueError("q, k and v must share one set of strides")
    _need(slopes, "slopes", torch.float32, dev, (H,))
    _need(state, "state", torch.float32, dev, (B, H, d, d))
    _need(q_norm_weight, "q_norm_weight", torch.float32, dev, (d,))
    _need(k_norm_weight, "k_norm_weight", torch.float32, dev, (d,))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=dt, device=dev)
    so = _view(out, "out", dt, dev, (B, H, N, d))
    ws = prefill_workspace_bytes(B, H, N, d, dev)
    with torch.cuda.device(dev):
        work = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
        rc = load_library().la_prefill_qk_norm_rope_ws(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), q_norm_weight.data_ptr(),
            k_norm_weight.data_ptr(), float(theta), rot_dim, pos0, float(eps), out.data_ptr(),
            state.data_ptr(), B, H, N, d, *si, *so, None if work is None else work.data_ptr(), ws,
            _stream(dev))
    _check(rc, "la_prefill_qk_norm_rope_ws")
    return out


def prefill_workspace_bytes(B: int, H: int, N: int, d: int, device=None) -> int:
    """Workspace bytes la_prefill_ws needs for a dense bf16 prefill of these
    sizes on `device` (0: no sequence split, la_prefill is used)."""
    n = ctypes.c_int64(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        rc = load_library().la_prefill_workspace_bytes(B, H, N, d, ctypes.byref(n))
    _check(rc, "la_prefill_workspace_bytes")
    return int(n.value)


def prefill_f32_workspace_bytes(B: int, H: int, N: int, d: int, device=None) -> int:
    """Workspace bytes la_prefill_f32_ws needs for a dense fp32 prefill of
    these sizes on `device` (0: no sequence split, la_prefill_f32 is used)."""
    n = ctypes.c_int64(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        rc = load_library().la_prefill_f32_workspace_bytes(B, H, N, d, ctypes.byref(n))
    _check(rc, "la_prefill_f32_workspace_bytes")
    return int(n.value)


def prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, slopes: torch.Tensor,
                   cu_seqlens: torch.Tensor, states: Optional[torch.Tensor],
                   out: Optional[torch.Tensor] = None, from_zero: bool = False) -> torch.Tensor:
    """Packed variable-length prefill: independent sequences in one launch.

    q, k, v: [H,T,d] bf16 or fp32 (sequence i is rows cu_seqlens[i]:cu_seqlens[i+1]
    of every head); cu_seqlens: [nseq+1] int64 on the same GPU (0 = cu[0] <= ... <=
    cu[nseq] = T); slopes: [H] fp32; states: [nseq,H,d,d] fp32, IN = initial states,
    OUT = final states (in place).  Returns out [H,T,d].  Enqueued on the current
    stream; the offsets are not read on the host.  bf16 q, k, v (sharing one
    set of strides) and out may be strided [H,T,d] views with a unit channel
    stride (``la_prefill_varlen_strided``).  from_zero (bf16): every sequence
    starts from a zero state and ``states`` is only written, never read
    (``la_prefill_varlen_from_zero``; empty sequences get zero states);
    ``states=None`` with from_zero: outputs only, no state is written.
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [H,T,d] tensor")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("prefill_varlen runs on GPU tensors only (no CPU path)")
    H, T, d = q.shape
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _view(t, n, dt, dev, (H, T, d))
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a [nseq+1] tensor with nseq >= 1")
    nseq = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", torch.int64, dev, (nseq + 1,))
    _need(slopes, "slopes", torch.float32, dev, (H,))
    if states is not None or not from_zero:
        _need(states, "states", torch.float32, dev, (nseq, H, d, d))
    if from_zero:
        if dt != torch.bfloat16:
            raise ValueError("from_zero is taken for bfloat16 only")
        if out is None:
            out = torch.empty((H, T, d), dtype=dt, device=dev)
        so = _view(out, "out", dt, dev, (H, T, d))
        si = q.stride()[:-1]
        with torch.cuda.device(dev):
            rc = load_library().la_prefill_varlen_from_zero(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(),
                cu_seqlens.data_ptr(), nseq, out.data_ptr(),
                None if states is None else states.data_ptr(), H, T, d, *si, *so, _stream(dev))
        _check(rc, "la_prefill_varlen_from_zero")
        return out
    if _strided(q, k, v, out, dt, dev, (H, T, d)):
        if out is None:
            out = torch.empty((H, T, d), dtype=dt, device=dev)
        so = _view(out, "out", dt, dev, (H, T, d))
        si = q.stride()[:-1]
        with torch.cuda.device(dev):
            rc = load_library().la_prefill_varlen_strided(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(),
                cu_seqlens.data_ptr(), nseq, out.data_ptr(), states.data_ptr(), H, T, d,
                *si, *so, _stream(dev))
        _check(rc, "la_prefill_varlen_strided")
        return out
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", dt, dev, (H, T, d))
    lib = load_library()
    fn = lib.la_prefill_varlen if dt == torch.bfloat16 else lib.la_prefill_varlen_f32
    with torch.cuda.device(dev):
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), cu_seqlens.data_ptr(),
                nseq, out.data_ptr(), states.data_ptr(), H, T, d, _stream(dev))
    _check(rc, "la_prefill_varlen" if dt == torch.bfloat16 else "la_prefill_varlen_f32")
    return out


def prefill_varlen_walks(nseq: int, H: int, T: int, d: int, device=None) -> bool:
    """Whether a packed bf16 prefill of nseq sequences, H heads and T tokens
    walks the sequences in one workgroup per (head, 32 output columns) on
    ``device`` (``la_prefill_varlen_plan``); otherwise each (sequence, head,
    column slice) has a workgroup of its own.  Both give the same results,
    bitwise."""
    walks = ctypes.c_int(0)
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        _check(load_library().la_prefill_varlen_plan(nseq, H, T, d, ctypes.byref(walks)),
               "la_prefill_varlen_plan")
    return bool(walks.value)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, slopes: torch.Tensor,
                state: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One recurrent step: state = lambda*state + k^T v (in place); returns q . state.

    q, k, v: [B,H,d] bf16 or fp32; slopes [H] fp32; state [B,H,d,d] fp32.
    bf16 q, k, v may be strided views sharing one set of strides (unit
    channel stride), e.g. head-split slices of a projection buffer
    (``la_decode_step_strided``); out is [B,H,d] contiguous.
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B,H,d] tensor")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_step runs on a GPU tensor only (no CPU path)")
    B, H, d = q.shape
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _view(t, n, dt, dev, (B, H, d))
    _need(slopes, "slopes", torch.float32, dev, (H,))
    _need(state, "state", torch.float32, dev, (B, H, d, d))
    if out is None:
        out = torch.empty((B, H, d), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, dev, (B, H, d))
    if _strided(q, k, v, None, dt, dev, (B, H, d)):
        with torch.cuda.device(dev):
            rc = load_library().la_decode_step_strided(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), state.data_ptr(),
                out.data_ptr(), B, H, d, *q.stride()[:-1], _stream(dev))
        _check(rc, "la_decode_step_strided")
        return out
    lib = load_library()
    fn = lib.la_decode_step if dt == torch.bfloat16 else lib.la_decode_step_f32
    with torch.cuda.device(dev):
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(), state.data_ptr(),
                out.data_ptr(), B, H, d, _stream(dev))
    _check(rc, "la_decode_step" if dt == torch.bfloat16 else "la_decode_step_f32")
    return out


def decode_multi(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, slopes: torch.Tensor,
                 state: torch.Tensor, n_commit: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """T draft tokens per sequence (1 <= T <= 8) from the carried state.

    q, k, v: [B,H,T,d] bf16 or fp32; slopes [H] fp32; state [B,H,d,d] fp32,
    updated in place to the state after n_commit[b] tokens (all T if n_commit
    is None); n_commit: [B] int32 on the same GPU.  Returns out [B,H,T,d] with
    o_t = q_t S_t for every token.  bf16 q, k, v may be strided views sharing
    one set of strides, e.g. [B,T,H*d] projection slices viewed as [B,H,T,d]
    (``la_decode_multi_strided``).
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B,H,T,d] tensor")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_multi runs on GPU tensors only (no CPU path)")
    B, H, T, d = q.shape
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _view(t, n, dt, dev, (B, H, T, d))
    _need(slopes, "slopes", torch.float32, dev, (H,))
    _need(state, "state", torch.float32, dev, (B, H, d, d))
    if n_commit is not None:
        _need(n_commit, "n_commit", torch.int32, dev, (B,))
    if out is None:
        out = torch.empty((B, H, T, d), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, dev, (B, H, T, d))
    if _strided(q, k, v, None, dt, dev, (B, H, T, d)):
        with torch.cuda.device(dev):
            rc = load_library().la_decode_multi_strided(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(),
                None if n_commit is None else n_commit.data_ptr(), state.data_ptr(),
                out.data_ptr(), B, H, T, d, *q.stride()[:-1], _stream(dev))
        _check(rc, "la_decode_multi_strided")
        return out
    lib = load_library()
    fn = lib.la_decode_multi if dt == torch.bfloat16 else lib.la_decode_multi_f32
    with torch.cuda.device(dev):
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), slopes.data_ptr(),
                None if n_commit is None else n_commit.data_ptr(), state.data_ptr(),
                out.data_ptr(), B, H, T, d, _stream(dev))
    _check(rc, "la_decode_multi" if dt == torch.bfloat16 else "la_decode_multi_f32")
    return out


def _rows(t: torch.Tensor, name: str, dev, shape):
    """[B,N,X] bf16 rows with a contiguous last dim (any token stride)."""
    if not isinstance(t, torch.Tensor) or t.device != dev or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bfloat16 tensor on {dev}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.stride(2) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
        raise ValueError(f"{name} must be [B,N,X] rows with unit channel stride and equal token strides")
    return t.stride(1)


def qk_norm_rope(q_in: torch.Tensor, k_in: torch.Tensor, v_in: Optional[torch.Tensor],
                 q_norm_weight: torch.Tensor, k_norm_weight: torch.Tensor, H: int,
                 theta: float = 6.0e6, rot_dim: int = 64, pos0: int = 0, eps: float = 1e-6,
                 outs=None, inplace: bool = False):
    """QK RMSNorm + partial RoPE, and the move of q, k, v to the kernel layout.

    q_in, k_in, v_in: [B,N,H*d] bf16 views (a shared token stride is allowed,
    e.g. slices of one packed projection output); weights [d] fp32.
    Returns (q, k, v) as [B,H,N,d] bf16 (written into ``outs`` if given).
    v_in None: v is not touched and the third result is None.
    inplace: q and k are written back over q_in and k_in, and the results are
    [B,H,N,d] views of them (v, if given, is still copied out), ready for the
    strided prefill.
    """
    dev = q_in.device
    if dev.type != "cuda":
        raise ValueError("qk_norm_rope runs on GPU tensors only (no CPU path)")
    B, N, HD = q_in.shape
    d = HD // H
    if d * H != HD:
        raise ValueError("last dimension must be H*d")
    st = _rows(q_in, "q_in", dev, (B, N, HD))
    ins = (k_in, "k_in"), (v_in, "v_in")
    for t, n in ins if v_in is not None else ins[:1]:
        if _rows(t, n, dev, (B, N, HD)) != st:
            raise ValueError("q_in, k_in, v_in must share one token stride")
    _need(q_norm_weight, "q_norm_weight", torch.float32, dev, (d,))
    _need(k_norm_weight, "k_norm_weight", torch.float32, dev, (d,))
    if outs is None:
        def new():
            return torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
        outs = (None if inplace else new(), None if inplace else new(),
                None if v_in is None else new())
    if inplace:
        if outs[0] is not None or outs[1] is not None:
            raise ValueError("inplace: q and k are written over q_in and k_in (outs[0:2] must be None)")
        outs = (q_in.unflatten(2, (H, d)).transpose(1, 2), k_in.unflatten(2, (H, d)).transpose(1, 2),
                outs[2])
    else:
        for t, n in zip(outs[:2], ("q_out", "k_out")):
            _need(t, n, torch.bfloat16, dev, (B, H, N, d))
    if (v_in is None) != (outs[2] is None):
        raise ValueError("v_in and v_out must both be given or both be None")
    if outs[2] is not None:
        _need(outs[2], "v_out", torch.bfloat16, dev, (B, H, N, d))
    lib = load_library()
    qo = q_in.data_ptr() if inplace else outs[0].data_ptr()
    ko = k_in.data_ptr() if inplace else outs[1].data_ptr()
    with torch.cuda.device(dev):
        rc = lib.la_qk_norm_rope(q_in.data_ptr(), k_in.data_ptr(),
                                 None if v_in is None else v_in.data_ptr(), st,
                                 q_norm_weight.data_ptr(), k_norm_weight.data_ptr(), float(theta),
                                 rot_dim, pos0, float(eps), qo, ko,
                                 None if outs[2] is None else outs[2].data_ptr(), B, N, H, d,
                                 _stream(dev))
    _check(rc, "la_qk_norm_rope")
    return tuple(outs)


def group_norm_gate(o: torch.Tensor, gate: torch.Tensor, norm_weight: torch.Tensor,
                    group: Optional[int] = None, eps: float = 1e-6,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Grouped RMSNorm of the kernel output times sigmoid(gate), back to [B,N,H*d].

    o: [B,H,N,d] bf16, any strides with a unit channel stride (la_prefill's
    contiguous output, or a token-major one from the strided prefill);
    gate: [B,N,H*d] bf16 view (any token stride); norm_weight: [H*d] fp32;
    group: channels per group (default d, one head).
    """
    if not isinstance(o, torch.Tensor) or o.dim() != 4:
        raise ValueError("o must be a [B,H,N,d] tensor")
    dev = o.device
    if dev.type != "cuda":
        raise ValueError("group_norm_gate runs on GPU tensors only (no CPU path)")
    B, H, N, d = o.shape
    os_ = _view(o, "o", torch.bfloat16, dev, (B, H, N, d))
    gst = _rows(gate, "gate", dev, (B, N, H * d))
    _need(norm_weight, "norm_weight", torch.float32, dev, (H * d,))
    if out is None:
        out = torch.empty((B, N, H * d), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, dev, (B, N, H * d))
    lib = load_library()
    with torch.cuda.device(dev):
        rc = lib.la_group_norm_gate(o.data_ptr(), *os_, gate.data_ptr(), gst,
                                    norm_weight.data_ptr(), d if group is None else group,
                                    float(eps), out.data_ptr(), B, N, H, d, _stream(dev))
    _check(rc, "la_group_norm_gate")
    return out


def cp_fold(local_states: torch.Tensor, shard_lens, rank: int, slopes: torch.Tensor,
            state_init: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """State entering shard ``rank`` of a sequence-sharded prefill.

    local_states: [R,B,H,d,d] fp32 (each shard's la_prefill final state from a
    zero state, e.g. the result of an all-gather); shard_lens: R token counts
    (host ints); rank in 0..R; state_init: [B,H,d,d] fp32 or None (zero).
    Returns [B,H,d,d] fp32 (``out`` may be ``state_init`` itself).
    """
    if not isinstance(local_states, torch.Tensor) or local_states.dim() != 5:
        raise ValueError("local_states must be a [R,B,H,d,d] tensor")
    dev = local_states.device
    if dev.type != "cuda":
        raise ValueError("cp_fold runs on GPU tensors only (no CPU path)")
    R, B, H, d, _ = local_states.shape
    _need(local_states, "local_states", torch.float32, dev, (R, B, H, d, d))
    lens = [int(x) for x in shard_lens]
    if len(lens) != R:
        raise ValueError("shard_lens must have one entry per shard")
    _need(slopes, "slopes", torch.float32, dev, (H,))
    if state_init is not None:
        _need(state_init, "state_init", torch.float32, dev, (B, H, d, d))
    if out is None:
        out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, dev, (B, H, d, d))
    arr = (ctypes.c_int64 * max(R, 1))(*lens)
    with torch.cuda.device(dev):
        rc = load_library().la_cp_fold(local_states.data_ptr(), ctypes.cast(arr, ctypes.c_void_p),
                                       R, int(rank), slopes.data_ptr(),
                                       None if state_init is None else state_init.data_ptr(),
                                       out.data_ptr(), B, H, d, _stream(dev))
    _check(rc, "la_cp_fold")
    return out


def cp_correct(q: torch.Tensor, slopes: torch.Tensor, state_in: torch.Tensor,
               out: torch.Tensor) -> torch.Tensor:
    """Correct a shard's local output in place: out_a += lambda^(a+1) q_a S_in.

    q, out: [B,H,L,d] bf16 (out = la_prefill's output over the shard from a
    zero state); state_in: [B,H,d,d] fp32 (``cp_fold`` for this shard).
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B,H,L,d] tensor")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("cp_correct runs on GPU tensors only (no CPU path)")
    B, H, L, d = q.shape
    _need(q, "q", torch.bfloat16, dev, (B, H, L, d))
    _need(out, "out", torch.bfloat16, dev, (B, H, L, d))
    _need(slopes, "slopes", torch.float32, dev, (H,))
    _need(state_in, "state_in", torch.float32, dev, (B, H, d, d))
    with torch.cuda.device(dev):
        rc = load_library().la_cp_correct(q.data_ptr(), slopes.data_ptr(), state_in.data_ptr(),
                                          out.data_ptr(), B, H, L, d, _stream(dev))
    _check(rc, "la_cp_correct")
    return out
