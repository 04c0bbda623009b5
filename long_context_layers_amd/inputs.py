"""Seeded synthetic inputs for the decayed linear-attention layer.

This module only draws random tensors and the per-head slope values; it holds
none of the layer's arithmetic (no decay powers, no products, no scan).  The
GPU path and the CPU oracle both consume the exact tensors produced here.

Workload shapes follow the model the pages describe: 64 heads of head
dimension 128 (Ling and Ring 2.6 Technical Report, §2.1.1 "inherited
design"), contexts at the training stages 4K / 32K / 256K (§2.3), and a
decode batch large enough that the per-sequence states do not fit in
on-chip caches.

Recipe (every workload):
  * ``g = torch.Generator(device).manual_seed(seed)``;
  * draw order: q, k, v (per head, shape ``[B, N, d]`` each, fp32
    ``randn / sqrt(d)``), then the initial state (per head ``[B, d, d]``,
    fp32 ``randn * 0.1``, i.e. variance 0.01), then for decode the per-step
    tokens (step-major: q, k, v of shape ``[B, H, d]``);
  * every tensor is drawn in fp32 and rounded once (round-to-nearest-even) to
    its storage dtype; both sides read those stored bytes;
  * slopes ``s_h = 2**(-8 (h+1) / H)`` for h = 0..H-1, computed in fp64 and
    stored fp32 (so lambda_h = exp(-s_h); h = 0 decays fastest).

Packed variable-length batches (``make_varlen``): sub-sequence lengths come
from ``varlen_lengths`` (log-uniform between ``lo`` and ``hi`` from a CPU
generator, the last piece cut to fit the total), then q, k, v are drawn as
the dense recipe with B = 1 over all T packed rows (shape ``[H, T, d]``),
then the per-sequence initial states ``[nseq, H, d, d]``.  This stands in for
packed training samples made of many short sub-sequences (the report's
§4.1.2); no dataset is involved.

Drawing on the GPU uses torch's device generator (fast for the 256K
workload); drawing on the CPU uses torch's CPU generator.  The two give
different numbers for the same seed; each parity check draws once and hands
the same bytes to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload (sizes, dtype, seed)."""
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    seed: int
    init_state: bool = False
    decode_steps: int = 0          # > 0: a decode workload (N unused)
    block: int = 64                # block length named for the workload (FLOP count)
    note: str = ""


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 256, 64, torch.float32, 1000, block=32,
                         note="fp32 correctness case, zero initial state"),
    "prefill_4k": Workload("prefill_4k", 1, 64, 4096, 128, torch.bfloat16, 1001,
                           note="one layer prefill, zero initial state"),
    "prefill_32k_state": Workload("prefill_32k_state", 1, 64, 32768, 128, torch.bfloat16, 1002,
                                  init_state=True,
                                  note="32K crossover, chunked continuation from a random fp32 state"),
    "prefill_256k": Workload("prefill_256k", 1, 64, 262144, 128, torch.bfloat16, 1003,
                             note="full 256K context on one device, zero initial state"),
    "decode_b256": Workload("decode_b256", 256, 64, 0, 128, torch.bfloat16, 1004,
                            init_state=True, decode_steps=64,
                            note="batched decode, 64 steps of fresh tokens"),
    "varlen_256k": Workload("varlen_256k", 1, 64, 262144, 128, torch.bfloat16, 1005,
                            init_state=True,
                            note="256K packed tokens in sub-sequences of 256..16384 tokens "
                                 "(log-uniform), each with its own random fp32 state"),
}

VARLEN_RANGE = (256, 16384)        # sub-sequence lengths of the varlen_256k workload


def slopes(H: int, device="cpu") -> torch.Tensor:
    """Per-head slopes s_h = 2^(-8(h+1)/H), fp64 -> fp32, shape [H]."""
    s = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]
    return torch.tensor(s, dtype=torch.float64).to(torch.float32).to(device)


def _gen(device, seed: int) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g


def _draw_heads(g, B, H, rows, cols, scale, dtype, device) -> torch.Tensor:
    """[B, H, rows, cols] drawn head by head (bounded fp32 temporaries)."""
    out = torch.empty((B, H, rows, cols), dtype=dtype, device=device)
    for h in range(H):
        x = torch.randn((B, rows, cols), generator=g, dtype=torch.float32, device=device)
        x.mul_(scale)
        out[:, h].copy_(x)          # one rounding to the storage dtype (RNE)
        del x
    return out


@dataclass
class PrefillInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    slopes: torch.Tensor
    state: torch.Tensor            # [B,H,d,d] fp32: the initial state (zeros if none)


def make_prefill(B: int, H: int, N: int, d: int, dtype=torch.bfloat16, seed: int = 0,
                 init_state: bool = False, device="cpu") -> PrefillInputs:
    g = _gen(device, seed)
    sc = 1.0 / math.sqrt(d)
    q = _draw_heads(g, B, H, N, d, sc, dtype, device)
    k = _draw_heads(g, B, H, N, d, sc, dtype, device)
    v = _draw_heads(g, B, H, N, d, sc, dtype, device)
    if init_state:
        st = _draw_heads(g, B, H, d, d, 0.1, torch.float32, device)
    else:
        st = torch.zeros((B, H, d, d), dtype=torch.float32, device=device)
    return PrefillInputs(q, k, v, slopes(H, device), st)


@dataclass
class DecodeInputs:
    q: torch.Tensor                # [T,B,H,d] (T decode steps)
    k: torch.Tensor
    v: torch.Tensor
    slopes: torch.Tensor
    state: torch.Tensor            # [B,H,d,d] fp32 initial state


def make_decode(B: int, H: int, d: int, steps: int, dtype=torch.bfloat16, seed: int = 0,
                device="cpu") -> DecodeInputs:
    g = _gen(device, seed)
    sc = 1.0 / math.sqrt(d)
    st = _draw_heads(g, B, H, d, d, 0.1, torch.float32, device)
    qs, ks, vs = [], [], []
    for _ in range(steps):
        for lst in (qs, ks, vs):
            x = torch.randn((B, H, d), generator=g, dtype=torch.float32, device=device)
            lst.append((x * sc).to(dtype))
    if steps:
        q, k, v = torch.stack(qs), torch.stack(ks), torch.stack(vs)
    else:
        q = k = v = torch.empty((0, B, H, d), dtype=dtype, device=device)
    return DecodeInputs(q, k, v, slopes(H, device), st)


def varlen_lengths(total: int, seed: int, lo: int = VARLEN_RANGE[0],
                   hi: int = VARLEN_RANGE[1]) -> list:
    """Seeded sub-sequence lengths summing to ``total``: log-uniform in
    [lo, hi], the last one cut to fit."""
    g = torch.Generator().manual_seed(seed)
    lens, rem = [], total
    while rem > 0:
        u = float(torch.rand((), generator=g, dtype=torch.float64))
        n = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
        n = max(1, min(n, rem))
        lens.append(n)
        rem -= n
    return lens


@dataclass
class VarlenInputs:
    q: torch.Tensor                # [H,T,d]: sequence i is rows cu[i]:cu[i+1] of every head
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens: torch.Tensor       # [nseq+1] int64
    slopes: torch.Tensor
    states: torch.Tensor           # [nseq,H,d,d] fp32 initial states (zeros if none)
    lens: list = field(default_factory=list)


def make_varlen(H: int, lens, d: int, dtype=torch.bfloat16, seed: int = 0,
                init_state: bool = False, device="cpu") -> VarlenInputs:
    lens = [int(n) for n in lens]
    T = sum(lens)
    g = _gen(device, seed)
    sc = 1.0 / math.sqrt(d)
    q = _draw_heads(g, 1, H, T, d, sc, dtype, device)[0]
    k = _draw_heads(g, 1, H, T, d, sc, dtype, device)[0]
    v = _draw_heads(g, 1, H, T, d, sc, dtype, device)[0]
    if init_state:
        st = _draw_heads(g, len(lens), H, d, d, 0.1, torch.float32, device)
    else:
        st = torch.zeros((len(lens), H, d, d), dtype=torch.float32, device=device)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    return VarlenInputs(q, k, v, torch.tensor(cu, dtype=torch.int64, device=device),
                        slopes(H, device), st, lens)


def make_workload(name: str, device="cpu", N: Optional[int] = None):
    """Inputs of a named workload; ``N`` overrides the sequence length (the
    total packed length for a varlen workload)."""
    w = WORKLOADS[name]
    if name.startswith("varlen"):
        lens = varlen_lengths(N if N is not None else w.N, w.seed)
        return make_varlen(w.H, lens, w.d, w.dtype, w.seed, w.init_state, device)
    if w.decode_steps:
        return make_decode(w.B, w.H, w.d, w.decode_steps, w.dtype, w.seed, device)
    return make_prefill(w.B, w.H, N if N is not None else w.N, w.d, w.dtype, w.seed,
                        w.init_state, device)
