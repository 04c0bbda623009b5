"""Benchmark: decayed causal linear attention (Lightning Attention) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the whole hot path over resident synthetic inputs:
  * prefill of B=1, H=64, N=262,144, d=128 bf16 tokens from a zero state
    (la_prefill: blockwise intra scores, inter term from the carried state,
    decayed state scan), and
  * one batched decode step of B=256 sequences, H=64, d=128 with fp32 states
    (la_decode_step), cycling through 64 pre-staged bf16 tokens.
The JSON line's ``value`` is the prefill throughput in algorithmic TFLOP/s
(B*H*N*(4 d^2 + 2 (C+1) d) with C = 64, i.e. 82,176 flop per token-head,
whatever block length the kernel uses), from HIP events around each prefill
launch on its stream.  Decode is reported in GB/s of state traffic, from the
64 pre-staged steps chained as one timed region after the step loop (the one
decode step inside each timed step, right after a 4 GB prefill, is kept as
``decode.in_step_ms``).
``roofline`` is the prefill kernel's HBM roofline (algorithmic bytes per
launch / launch time against 8 TB/s); ``cpu_baseline`` times the fp64 CPU
oracle on a bounded sample of the same workload; ``ceilings`` holds what the
same GPU sustains in probe kernels (lib/liblapeak.so: an MFMA loop and read,
write and copy streams) and the prefill and decode against them.

Outside the timed step, two more launches are measured the same way (HIP
events on the launch stream, median of ``--extra-reps`` after 3 warm-ups):
  * ``varlen``: packed prefill of 262,144 tokens split into 74 sub-sequences
    of 256..16,384 tokens (seeded log-uniform lengths), H=64, d=128 bf16, each
    sequence with its own fp32 state (la_prefill_varlen, one launch);
  * ``decode_multi``: draft verification, B=256 sequences x H=64, 4 draft
    tokens each, seeded commit counts 1..4 (la_decode_multi), next to the
    same tokens as 4 single decode steps;
  * ``layer_ops``: the layer's neighbouring fused ops at the 256K shape
    (B=1, N=262,144, H=64, d=128 bf16), in two arrangements: through the
    kernel layout (la_qk_norm_rope moves q, k, v from one packed projection
    buffer to [B,H,N,d]; la_prefill; la_group_norm_gate back to the
    token-major layout), and with no layout copies (QK norm + RoPE in place
    in the projection buffer, la_prefill_strided reading q, k, v from it and
    writing [B,H,N,d], la_group_norm_gate on that output); the strided
    prefill writing its output token-major is timed beside it;
  * ``sizes``: the prefill at the other context lengths of the metric's range:
    4K (B=1, H=64, d=128, zero state; a 512 MB buffer is read between
    launches so the 256 MB MALL does not serve the ~200 MB of inputs - a read,
    because a written buffer would leave its write-back to the timed launch) and
    the 32K crossover continuing from a random fp32 state (3 warm-ups, median
    of 20 launches each);
  * ``decode_latency``: one sequence (B=1, H=64, d=128) decoded for 64
    steps, launched one call at a time and replayed from one captured HIP
    graph (torch.cuda.CUDAGraph): per-step latency of each;
  * ``cp``: one rank's share of the 256K sequence split 8 ways (32,768 tokens,
    H=64, d=128 bf16, the last rank): its prefill from a zero state
    (la_prefill), the fold of the 8 gathered local states into its incoming
    state (la_cp_fold) and the correction of its output (la_cp_correct).
With ``--power``, ``power`` holds the package power and graphics clock
(`amd-smi metric -p -c`, run as a child process) sampled while the dense 256K
prefill (and its strided launch on a packed projection buffer), the B=256
decode step and the probe kernels (MFMA loops on constant
and on changing random operands, HBM copy, L2 hits, LDS reads, integer adds)
each run back to back for 8 s, with the
package power limit (`rocm-smi --showmaxpower`), the energy per launch and the
probes' energy per byte above the integer-work probe.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Lightning-attn prefill TFLOP/s (H=64,d=128,N=32K-256K); decode state GB/s"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA
C_COUNT = 64                     # block length the flop count is fixed at

PREFILL = dict(B=1, H=64, N=262144, d=128, seed=1003)
DECODE = dict(B=256, H=64, d=128, steps=64, seed=1004)
MTP = dict(B=256, H=64, T=4, d=128, seed=1006)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_256k_traffic.txt")
FUSED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_qk_norm_rope_256k_traffic.txt")

# the kernels of one timed call, in launch order: the headline la_prefill_ws
# call, and the layer's la_prefill_qk_norm_rope_ws (64 rotary dims)
TRAFFIC_CALLS = {
    "split": dict(
        kernels=["split_prep_kernel", "prefill_bf16_kernel<128, false, false, 2, -1>",
                 "split_fold_kernel", "cp_correct_kernel<128, -1>"],
        what=["HBM traffic of the prefill call bench.py times (la_prefill_ws: split_prep_kernel,",
              "prefill_bf16_kernel<128, false, false, 2, -1> over two segments per head,",
              "split_fold_kernel, cp_correct_kernel<128, -1>) on the 256K prefill workload",
              "(B={B}, H={H}, N={N}, d={d}, bf16, zero initial state)"],
        out=TRAFFIC_FILE),
    "fused": dict(
        kernels=["split_prep_kernel", "prefill_bf16_kernel<128, true, false, 2, 64>",
                 "split_fold_kernel", "cp_correct_kernel<128, 64>"],
        what=["HBM traffic of the layer's fused call bench.py times (la_prefill_qk_norm_rope_ws:",
              "split_prep_kernel, prefill_bf16_kernel<128, true, false, 2, 64> over two segments",
              "per head with QK Norm + RoPE in its loads, split_fold_kernel, cp_correct_kernel<128, 64>)",
              "on the 256K layer workload (B={B}, H={H}, N={N}, d={d}, bf16; raw q, k, v in one",
              "[B, N, 4*H*d] projection buffer, [B,H,N,d] output, zero initial state)"],
        out=FUSED_TRAFFIC_FILE)}
# the sources of the timed prefill calls' kernels, the headers they include
# among them (the traffic profiles are keyed by their hash)
KERNEL_SRCS = [os.path.join(ROOT, "long_context_layers_amd", "csrc", f)
               for f in ("prefill_bf16.hip", "cp.hip", "la_internal.h", "qk_prologue.h")]


def prefill_flops(B, H, N, d):
    return B * H * N * (4 * d * d + 2 * (C_COUNT + 1) * d)


def prefill_bytes(B, H, N, d):
    # q, k, v read and out written in bf16, plus the fp32 state read and written
    return B * H * N * d * 2 * 4 + B * H * d * d * 4 * 2


def decode_bytes(B, H, d, T=1):
    # state read + written (fp32), q, k, v read and out written (bf16), T tokens
    return B * H * (2 * 4 * d * d + 4 * 2 * d * T)


def time_launches(stream, fn, reps, warmups=3):
    """median ms of `reps` launches of fn() on `stream` (HIP events on that
    stream), after `warmups` untimed launches."""
    import torch
    for _ in range(warmups):
        fn()
    stream.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    stream.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return ts[len(ts) // 2] if len(ts) % 2 else 0.5 * (ts[len(ts) // 2 - 1] + ts[len(ts) // 2])


def smi_sample(args, timeout=30):
    """stdout of one `amd-smi` / `rocm-smi` query, run as a child process (None if
    the tool is missing or fails)."""
    import shutil
    import subprocess
    exe = shutil.which(args[0]) or os.path.join("/opt/rocm/bin", args[0])
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe] + args[1:], capture_output=True, text=True, timeout=timeout)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout if r.returncode == 0 else None


def parse_power_clock(text):
    """socket power (W) and the mean graphics clock over the XCDs (MHz) from
    the text of `amd-smi metric -p -c`."""
    if not text:
        return None, None
    m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    gfx = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", text)]
    return (float(m.group(1)) if m else None), (round(sum(gfx) / len(gfx)) if gfx else None)


def measure_power(stream, workloads, seconds=8.0):
    """Package power and graphics clock while each workload's launches run back
    to back: `amd-smi metric -p -c` sampled twice from a child process, from
    2.5 s into `seconds` of launches (the first seconds let the power controller
    settle), with the launches timed by HIP events on `stream` meanwhile.
    `workloads`: (name, launch function, launches per timed batch, bytes moved
    per launch or None, wave instructions of interest per launch or None)."""
    import threading
    import torch
    cap = None
    t = smi_sample(["rocm-smi", "--showmaxpower"])
    if t:
        m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", t)
        cap = float(m.group(1)) if m else None
    stream.synchronize()
    time.sleep(2.0)
    idle_w, idle_mhz = parse_power_clock(smi_sample(["amd-smi", "metric", "-p", "-c"]))
    res = {"tool": "amd-smi metric -p -c (socket power, graphics clock of each XCD), sampled "
                   "twice while the launches run back to back; energies per byte and per "
                   "instruction are taken above the idle sample (the GPU 2 s after the last "
                   "work, clock as given); the probes' figures include their own few vector "
                   "instructions per access",
           "power_cap_w": cap, "idle_w": idle_w, "idle_gfx_mhz": idle_mhz}
    for name, fn, per, nbytes, ninsts in workloads:
        samples = []

        def sampler():
            for delay in (2.5, 1.5):
                time.sleep(delay)
                samples.append(parse_power_clock(smi_sample(["amd-smi", "metric", "-p", "-c"])))

        th = threading.Thread(target=sampler)
        ms = []
        t_end = time.time() + seconds
        th.start()
        while time.time() < t_end:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(per):
                fn()
            b.record(stream)
            stream.synchronize()
            ms.append(a.elapsed_time(b) / per)
        th.join()
        watts = [w for w, _ in samples if w is not None]
        mhz = [c for _, c in samples if c is not None]
        ms_launch = sorted(ms)[len(ms) // 2]
        w = sum(watts) / len(watts) if watts else None
        res[name] = {"ms_per_launch": round(ms_launch, 4), "socket_w": watts, "gfx_mhz": mhz,
                     "energy_j_per_launch": round(w * ms_launch * 1e-3, 3) if w else None}
        if nbytes:
            res[name]["gbs"] = round(nbytes / (ms_launch * 1e-3) / 1e9, 1)
        if w and idle_w and nbytes:
            res[name]["pj_per_byte_above_idle"] = round((w - idle_w) / (nbytes / (ms_launch * 1e-3)) * 1e12, 2)
        if w and idle_w and ninsts:
            res[name]["nj_per_wave_instruction_above_idle"] = round(
                (w - idle_w) / (ninsts / (ms_launch * 1e-3)) * 1e9, 3)
        print(f"[bench] power {name}: {ms_launch:.3f} ms per launch, {watts} W, {mhz} MHz",
              file=sys.stderr, flush=True)
    return res


def measure_power_all(dev, stream, p, pstate, out, dcd, dstate, dout):
    """measure_power over the dense 256K prefill, the B256 decode step and two
    probe kernels (the bf16 MFMA loop and the HBM copy stream of lib/liblapeak.so)."""
    import ctypes
    import torch
    from long_context_layers_amd import binding, build
    lib = ctypes.CDLL(build.PEAK_LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.la_peak_mfma_bf16.argtypes = [I64, I64, P, P]
    lib.la_peak_copy.argtypes = [P, P, I64, P]
    lib.la_peak_l2_read.argtypes = [P, I64, I64, I64, P, P]
    lib.la_peak_lds_read.argtypes = [I64, I64, P, P]
    lib.la_peak_valu.argtypes = [I64, I64, P, P]
    lib.la_peak_mfma_bf16_data.argtypes = [I64, I64, P, P]
    for f in (lib.la_peak_mfma_bf16, lib.la_peak_copy, lib.la_peak_l2_read, lib.la_peak_lds_read,
              lib.la_peak_valu, lib.la_peak_lds_bytes_per_iter, lib.la_peak_mfma_chains,
              lib.la_peak_mfma_bf16_data):
        f.restype = ctypes.c_int
    h = stream.cuda_stream
    B, H, N, d = p.q.shape
    with torch.cuda.stream(stream):
        a = torch.zeros(1 << 29, dtype=torch.float32, device=dev)       # 2 GiB
        b = torch.zeros(1 << 29, dtype=torch.float32, device=dev)
        sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
        # the strided launch of the layer: q, k, v read from one packed
        # [B,N,4*H*d] projection buffer (token stride 4*H*d)
        proj = torch.empty((B, N, 4 * H * d), dtype=torch.bfloat16, device=dev)
        proj.normal_(0.0, d ** -0.5, generator=torch.Generator(device=dev).manual_seed(11))
        sq, sk, sv = (proj[..., i * H * d:(i + 1) * H * d].unflatten(-1, (H, d)).transpose(1, 2)
                      for i in range(3))

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")

    l2_region, l2_reps, lds_iters, blocks = 2 << 20, 40, 6000, 1024
    lds_bytes = blocks * lib.la_peak_lds_bytes_per_iter() * lds_iters
    mfma_iters, valu_iters = 20000, 500000
    work = [("prefill_256k", lambda: binding.prefill(p.q, p.k, p.v, p.slopes, pstate, out=out), 100,
             None, None),
            ("prefill_256k_strided", lambda: binding.prefill(sq, sk, sv, p.slopes, pstate, out=out), 100,
             None, None),
            ("decode_b256", lambda: binding.decode_step(dcd.q[0], dcd.k[0], dcd.v[0], dcd.slopes,
                                                         dstate, out=dout), 1000, None, None),
            # wave instructions: MFMAs (4 waves x chains per iteration), integer adds (4 per iteration)
            ("mfma_probe", lambda: check(lib.la_peak_mfma_bf16(mfma_iters, blocks, sink.data_ptr(), h)),
             100, None, blocks * 4 * mfma_iters * lib.la_peak_mfma_chains()),
            ("mfma_data_probe", lambda: check(lib.la_peak_mfma_bf16_data(mfma_iters, blocks,
                                                                          sink.data_ptr(), h)),
             100, None, blocks * 4 * mfma_iters * lib.la_peak_mfma_chains()),
            ("copy_probe_2gib", lambda: check(lib.la_peak_copy(a.data_ptr(), b.data_ptr(), 2 << 30, h)),
             500, 4 << 30, None),
            ("l2_read_probe", lambda: check(lib.la_peak_l2_read(a.data_ptr(), l2_region, l2_reps, blocks,
                                                                 sink.data_ptr(), h)), 100,
             blocks * l2_region * l2_reps, None),
            ("lds_read_probe", lambda: check(lib.la_peak_lds_read(lds_iters, blocks, sink.data_ptr(), h)),
             100, lds_bytes, None),
            ("valu_probe", lambda: check(lib.la_peak_valu(valu_iters, blocks, sink.data_ptr(), h)), 100,
             None, blocks * 4 * valu_iters * 4)]
    with torch.cuda.stream(stream):
        res = measure_power(stream, work)
    del a, b, sink, proj, sq, sk, sv
    return res


def measure_varlen(dev, stream, reps, dense_tflops):
    """Packed prefill: the 256K packed workload (74 sequences, log-uniform
    lengths) and, beside it, 512 sequences of 512 tokens (short prompts)."""
    import torch
    from long_context_layers_amd import binding, inputs

    def one(make, what, from_zero=False, states_out=True):
        with torch.cuda.stream(stream):
            inp = make()
            st = inp.states.clone()
            out = torch.empty_like(inp.q)
        stream.synchronize()
        H, T, d = inp.q.shape
        nseq = len(inp.lens)

        def run():
            binding.prefill_varlen(inp.q, inp.k, inp.v, inp.slopes, inp.cu_seqlens,
                                   st if states_out else None, out=out, from_zero=from_zero)

        with torch.cuda.stream(stream):
            ms = time_launches(stream, run, reps)
        fl = H * T * (4 * d * d + 2 * (C_COUNT + 1) * d)
        # q, k, v, out, and the states written (and read unless from zero)
        by = H * T * d * 2 * 4 + (nseq * H * d * d * 4 * (1 if from_zero else 2) if states_out else 0)
        tflops = fl / (ms * 1e-3) / 1e12
        gbs = by / (ms * 1e-3) / 1e9
        lo, hi = min(inp.lens), max(inp.lens)
        walks = binding.prefill_varlen_walks(nseq, H, T, d, dev)
        # the grid's column tiles per workgroup (as the library chooses them:
        # 64 columns when those workgroups still fill the device)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        njt = 2 if d == 128 and 2 * H * nseq >= cus else 1
        del inp, st, out
        return {"workload": f"packed prefill H{H} T{T} d{d} bf16: {nseq} sequences of "
                            f"{lo}..{hi} tokens ({what}), "
                            + ("per-sequence fp32 states" if states_out else "outputs only")
                            + (" written from zero (la_prefill_varlen_from_zero)" if from_zero and states_out
                               else " from zero (la_prefill_varlen_from_zero, null states)" if from_zero
                               else ""),
                "nseq": nseq, "ms": round(ms, 4), "tflops": round(tflops, 3),
                "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": by,
                "vs_dense_256k_tflops": round(tflops / dense_tflops, 4),
                "kernel": ("prefill_bf16_kernel<128, false, true, 1, -1>: one workgroup per head and "
                           "32 columns walks every sequence of its group (groups of sequences walked side "
                           "by side fill the device)" if walks else
                           f"prefill_bf16_kernel<128, false, false, {njt}, -1>: one workgroup per "
                           f"sequence, head and {32 * njt} columns")}

    res = one(lambda: inputs.make_workload("varlen_256k", device=dev), "seeded log-uniform")
    res["short_sequences"] = one(
        lambda: inputs.make_varlen(64, [512] * 512, 128, torch.bfloat16, seed=1006,
                                   init_state=True, device=dev), "short prompts")
    # the report's pain point (many short packed sub-sequences, §4.1.2)
    res["many_short_sequences"] = one(
        lambda: inputs.make_varlen(64, [64] * 4096, 128, torch.bfloat16, seed=1007,
                                   init_state=True, device=dev), "one block each")
    # the same fresh requests from zero states: the states only written
    res["many_short_sequences_from_zero"] = one(
        lambda: inputs.make_varlen(64, [64] * 4096, 128, torch.bfloat16, seed=1007,
                                   init_state=False, device=dev), "one block each", from_zero=True)
    # and with no states at all: a forward pass whose final states are not
    # needed (training or scoring over packed sequences)
    res["many_short_sequences_outputs_only"] = one(
        lambda: inputs.make_varlen(64, [64] * 4096, 128, torch.bfloat16, seed=1007,
                                   init_state=False, device=dev), "one block each", from_zero=True,
        states_out=False)
    # the flash models' 32 heads (§2.1.1, Table 1): 128 column-slice workgroups
    # fill half of the device, so only very short sequences walk
    res["flash_heads"] = {
        "many_short_sequences": one(
            lambda: inputs.make_varlen(32, [64] * 4096, 128, torch.bfloat16, seed=1008,
                                       init_state=True, device=dev), "one block each"),
        "short_sequences": one(
            lambda: inputs.make_varlen(32, [512] * 512, 128, torch.bfloat16, seed=1009,
                                       init_state=True, device=dev), "short prompts"),
        "mixed": one(
            lambda: inputs.make_varlen(32, inputs.varlen_lengths(262144, 1005), 128,
                                       torch.bfloat16, seed=1010, init_state=True, device=dev),
            "seeded log-uniform")}
    return res


def measure_layer_ops(dev, stream, reps, pre_ms):
    import torch
    from long_context_layers_amd import binding, inputs
    B, N, H, d = 1, PREFILL["N"], PREFILL["H"], PREFILL["d"]
    g = torch.Generator(device=dev).manual_seed(1007)
    with torch.cuda.stream(stream):
        proj = torch.empty((B, N, 4 * H * d), dtype=torch.bfloat16, device=dev)
        proj.normal_(generator=g)                     # packed q | k | v | gate rows
        q, k, v, gate = (proj[..., i * H * d:(i + 1) * H * d] for i in range(4))
        outs = tuple(torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
        y = torch.empty((B, N, H * d), dtype=torch.bfloat16, device=dev)
        o_tm = torch.empty((B, N, H * d), dtype=torch.bfloat16, device=dev)
        wq = torch.ones(d, device=dev)
        wo = torch.ones(H * d, device=dev)
        slopes = inputs.slopes(H, dev)
        st = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)

    def heads(t):                                     # [B,N,H*d] -> [B,H,N,d] view
        return t.unflatten(-1, (H, d)).transpose(1, 2)

    stream.synchronize()

    def pro():
        binding.qk_norm_rope(q, k, v, wq, wq, H, theta=6e6, rot_dim=64, outs=outs)

    def epi():
        binding.group_norm_gate(outs[0], gate, wo, out=y)

    def pro_inplace():
        binding.qk_norm_rope(q, k, None, wq, wq, H, theta=6e6, rot_dim=64, inplace=True)

    def attn_strided():
        binding.prefill(heads(q), heads(k), heads(v), slopes, st, out=outs[1])

    def attn_strided_tm():
        binding.prefill(heads(q), heads(k), heads(v), slopes, st, out=heads(o_tm))

    def epi_tm():
        binding.group_norm_gate(heads(o_tm), gate, wo, out=y)

    def attn_fused():                                 # QK Norm + RoPE inside the prefill's loads
        binding.prefill_qk_norm_rope(heads(q), heads(k), heads(v), slopes, st, wq, wq,
                                     theta=6e6, rot_dim=64, out=outs[2])

    with torch.cuda.stream(stream):
        ms_pro = time_launches(stream, pro, reps)
        ms_epi = time_launches(stream, epi, reps)
        ms_pro_ip = time_launches(stream, pro_inplace, reps)
        ms_attn = time_launches(stream, attn_strided, reps)
        ms_attn_tm = time_launches(stream, attn_strided_tm, reps)
        ms_epi_tm = time_launches(stream, epi_tm, reps)
        ms_fused = time_launches(stream, attn_fused, reps)
    elems = B * N * H * d
    by_pro, by_epi, by_pro_ip = elems * 2 * 6, elems * 2 * 3, elems * 2 * 4
    del proj, q, k, v, gate, outs, y, o_tm, st

    def line(ms, by, kernel):
        gb = by / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "gbs": round(gb, 1), "frac_of_hbm_peak": round(gb / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": by, "kernel": kernel}

    fl = prefill_flops(B, H, N, d)
    return {"workload": f"B{B} N{N} H{H} d{d} bf16; q,k,v,gate in one packed [B,N,4*H*d] "
                        "projection buffer; RoPE base 6e6, rotary dim 64; norm group d",
            "qk_norm_rope": line(ms_pro, by_pro, "qk_norm_rope_kernel<128>"),
            "group_norm_gate": line(ms_epi, by_epi, "group_norm_gate_kernel<128>"),
            "layer_ms": round(ms_pro + pre_ms + ms_epi, 4),
            "no_layout_copies": {
                "qk_norm_rope_in_place": line(ms_pro_ip, by_pro_ip, "qk_norm_rope_kernel<128>"),
                "prefill_strided": {"ms": round(ms_attn, 4),
                                    "tflops": round(fl / (ms_attn * 1e-3) / 1e12, 3),
                                    "vs_contiguous": round(pre_ms / ms_attn, 4),
                                    "kernel": "prefill_bf16_kernel<128, true, false, 2, -1> (token stride "
                                              "4*H*d in, [B,H,N,d] out)"},
                "layer_ms": round(ms_pro_ip + ms_attn + ms_epi, 4),
                "token_major_out": {
                    "prefill_strided_ms": round(ms_attn_tm, 4),
                    "group_norm_gate": line(ms_epi_tm, by_epi, "group_norm_gate_kernel<128>"),
                    "layer_ms": round(ms_pro_ip + ms_attn_tm + ms_epi_tm, 4)}},
            "fused_prologue": {
                "prefill_qk_norm_rope_ms": round(ms_fused, 4),
                "tflops": round(fl / (ms_fused * 1e-3) / 1e12, 3),
                "vs_prefill_alone": round(ms_attn / ms_fused, 4),
                "kernel": "prefill_bf16_kernel<128, true, false, 2, 64> (QK Norm + RoPE with 64 rotary "
                          "dims in the producers' loads) and cp_correct_kernel<128, 64>",
                "layer_ms": round(ms_fused + ms_epi, 4)}}


def measure_decode_multi(dev, stream, reps):
    import torch
    from long_context_layers_amd import binding, inputs
    B, H, T, d = MTP["B"], MTP["H"], MTP["T"], MTP["d"]
    with torch.cuda.stream(stream):
        dec = inputs.make_decode(B, H, d, T, torch.bfloat16, MTP["seed"], dev)
        q, k, v = (x.permute(1, 2, 0, 3).contiguous() for x in (dec.q, dec.k, dec.v))
        g = torch.Generator().manual_seed(MTP["seed"])
        n = torch.randint(1, T + 1, (B,), generator=g, dtype=torch.int32).to(dev)
        st = dec.state.clone()
        out = torch.empty_like(q)
        o1 = torch.empty_like(dec.q[0])
    stream.synchronize()

    def multi():
        binding.decode_multi(q, k, v, dec.slopes, st, n_commit=n, out=out)

    def singles():
        for t in range(T):
            binding.decode_step(dec.q[t], dec.k[t], dec.v[t], dec.slopes, st, out=o1)

    with torch.cuda.stream(stream):
        ms = time_launches(stream, multi, reps)
        ms_single = time_launches(stream, singles, reps)
    by = decode_bytes(B, H, d, T)
    gbs = by / (ms * 1e-3) / 1e9
    del dec, q, k, v, st, out
    return {"workload": f"draft verification B{B} H{H} d{d} bf16, {T} draft tokens per "
                        "sequence, seeded commit counts 1..4 (fp32 states)",
            "ms_per_call": round(ms, 4), "gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "algorithmic_bytes_per_call": by,
            "four_single_steps_ms": round(ms_single, 4),
            "speedup_vs_single_steps": round(ms_single / ms, 3),
            "kernel": "decode_multi_kernel<bf16,128>"}


def measure_ceilings(dev, stream, pre_ms, pre_tflops, dec_gbs):
    """Probe kernels on this GPU: bf16 MFMA loop, HBM read / write / copy /
    in-place update streams; the prefill's time floor at the measured read and
    write rates (its reads and writes taken one after the other, as the copy
    stream shows they are), and decode against the in-place update stream."""
    import ctypes
    import torch
    from long_context_layers_amd import build
    lib = ctypes.CDLL(build.PEAK_LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.la_peak_mfma_bf16.argtypes = [I64, I64, P, P]
    lib.la_peak_read.argtypes = [P, I64, P, P]
    lib.la_peak_write.argtypes = [P, I64, P]
    lib.la_peak_copy.argtypes = [P, P, I64, P]
    lib.la_peak_update.argtypes = [P, I64, P]
    lib.la_peak_mix3.argtypes = [P, P, P, P, I64, P]
    lib.la_peak_stream_persistent.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, P, P]
    lib.la_peak_pair_pattern.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, I64, I64, P]
    for f in (lib.la_peak_mfma_bf16, lib.la_peak_read, lib.la_peak_write, lib.la_peak_copy,
              lib.la_peak_update, lib.la_peak_mix3, lib.la_peak_stream_persistent,
              lib.la_peak_pair_pattern):
        f.restype = ctypes.c_int
    h = stream.cuda_stream
    nbytes = 4 << 30
    with torch.cuda.stream(stream):
        a = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)
        b = torch.zeros(nbytes // 8, dtype=torch.float32, device=dev)
        sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
    stream.synchronize()
    blocks, iters = 256 * 4, 20000
    chains = 4

    def best(fn, n=3):
        def call():
            rc = fn()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
        return min(time_launches(stream, call, 1) for _ in range(n))

    with torch.cuda.stream(stream):
        ms_mfma = best(lambda: lib.la_peak_mfma_bf16(iters, blocks, sink.data_ptr(), h))
        ms_read = best(lambda: lib.la_peak_read(a.data_ptr(), nbytes, sink.data_ptr(), h))
        ms_write = best(lambda: lib.la_peak_write(a.data_ptr(), nbytes, h))
        ms_copy = best(lambda: lib.la_peak_copy(a.data_ptr(), b.data_ptr(), nbytes // 2, h))
        ms_upd = best(lambda: lib.la_peak_update(a.data_ptr(), nbytes // 2, h))
        q4 = nbytes // 4                        # three quarters of a read, b's first half written
        ms_mix = best(lambda: lib.la_peak_mix3(a.data_ptr(), a.data_ptr() + q4, a.data_ptr() + 2 * q4,
                                               b.data_ptr(), q4, h))
        # the persistent forms (a fixed grid, each workgroup streaming its own region)
        pers = {}
        for nb in (1024, 2048):
            pers[("read", nb)] = best(lambda: lib.la_peak_stream_persistent(
                0, a.data_ptr(), None, None, None, nbytes, nb, sink.data_ptr(), h))
            pers[("write", nb)] = best(lambda: lib.la_peak_stream_persistent(
                1, None, None, None, a.data_ptr(), nbytes, nb, None, h))
            pers[("mix3", nb)] = best(lambda: lib.la_peak_stream_persistent(
                2, a.data_ptr(), a.data_ptr() + q4, a.data_ptr() + 2 * q4, b.data_ptr(), q4, nb, None, h))
        # the prefill's pattern without arithmetic: 128 head slots of 32K tokens x 256 B
        # rows (1 GiB per buffer), q and k rows read by both workgroups of a slot or halved
        pat = {(mode, nf): best(lambda: lib.la_peak_pair_pattern(
            mode, nf, a.data_ptr(), a.data_ptr() + q4, a.data_ptr() + 2 * q4, b.data_ptr(),
            128, q4 // (128 * 256), h)) for mode in (0, 1, 2) for nf in (1, 4)}
    del a, b, sink
    p_rd = max(nbytes / (ms * 1e-3) / 1e9 for (k, _), ms in pers.items() if k == "read")
    p_wr = max(nbytes / (ms * 1e-3) / 1e9 for (k, _), ms in pers.items() if k == "write")
    p_mx = max(nbytes / (ms * 1e-3) / 1e9 for (k, _), ms in pers.items() if k == "mix3")
    tf = blocks * 4 * iters * chains * 32768 / (ms_mfma * 1e-3) / 1e12
    rd, wr, cp, up, mx = (x / (ms * 1e-3) / 1e9 for x, ms in
                          ((nbytes, ms_read), (nbytes, ms_write), (nbytes, ms_copy), (nbytes, ms_upd),
                           (nbytes, ms_mix)))
    chunk_rates = {"read": round(rd, 1), "write": round(wr, 1), "mix3": round(mx, 1)}
    rd, wr, mx = max(rd, p_rd), max(wr, p_wr), max(mx, p_mx)
    B, H, N, d = PREFILL["B"], PREFILL["H"], PREFILL["N"], PREFILL["d"]
    st = B * H * d * d * 4
    rbytes, wbytes = B * H * N * d * 2 * 3 + st, B * H * N * d * 2 + st
    floor_ms = (rbytes / (rd * 1e9) + wbytes / (wr * 1e9)) * 1e3
    return {"mfma_bf16_tflops": round(tf, 1), "hbm_read_gbs": round(rd, 1),
            "hbm_write_gbs": round(wr, 1), "hbm_copy_gbs": round(cp, 1),
            "hbm_update_gbs": round(up, 1), "hbm_mix3_gbs": round(mx, 1),
            "probes": "lib/liblapeak.so: v_mfma_f32_32x32x16_bf16 chains on registers "
                      f"({blocks} workgroups of 4 waves, {chains} chains each); streams over "
                      "4 GiB in 64 KB chunks, one per workgroup, each chunk's 16-byte "
                      "nontemporal accesses all in flight (copy and in-place update: 2 GiB "
                      "read + 2 GiB written, counted as 4 GiB; mix3: 3 GiB read + 1 GiB "
                      "written, the prefill's 3:1 mix); read, write and mix3 also from 1024 "
                      "and 2048 persistent workgroups each streaming its own region in 128 KB "
                      "bursts, the better form reported; best of 3",
            "chunked_form_gbs": chunk_rates,
            "persistent_form_gbs": {"read": round(p_rd, 1), "write": round(p_wr, 1),
                                    "mix3": round(p_mx, 1)},
            "prefill_pattern_gbs": {
                f"{name}_{nf}_in_flight": round(nbytes / (pat[(mode, nf)] * 1e-3) / 1e9, 1)
                for mode, name in ((0, "column_split"), (1, "own_half_rows"), (2, "own_whole_rows"))
                for nf in (1, 4)} | {
                "probe": "la_peak_pair_pattern: 128 head slots x 32K tokens x 256-byte rows in "
                         "q, k, v (read) and o (written), a workgroup pair per slot on one XCD "
                         "walking 64-token blocks, 1 or 4 blocks loaded before their outputs are "
                         "written; column_split: each reads the full q and k rows (the partner's "
                         "copy an L2 hit, as the prefill's two column workgroups of a head) and "
                         "its half of every v and o row; own_half_rows: each moves only its half "
                         "of every row (the same HBM bytes); own_whole_rows: each moves the whole "
                         "rows of its own tokens (a full-width split); GB/s of HBM bytes"},
            "prefill_frac_of_mfma_loop": round(pre_tflops / tf, 4),
            "prefill_floor_ms_at_stream_rates": round(floor_ms, 4),
            "prefill_frac_of_stream_floor": round(floor_ms / pre_ms, 4),
            "prefill_frac_of_mix3_stream": round((rbytes + wbytes) / (pre_ms * 1e-3) / 1e9 / mx, 4),
            "decode_frac_of_update_stream": round(dec_gbs / up, 4)}


def measure_sizes(dev, stream, reps):
    import torch
    from long_context_layers_amd import binding, inputs
    res = {}
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)      # 512 MB
    sink = torch.empty((), dtype=torch.float32, device=dev)
    for name in ("prefill_4k", "prefill_32k_state"):
        w = inputs.WORKLOADS[name]
        with torch.cuda.stream(stream):
            x = inputs.make_workload(name, device=dev)
            st = x.state.clone()
            out = torch.empty_like(x.q)
        stream.synchronize()
        n = max(reps, 20)                                               # short launches: 20 repetitions
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        with torch.cuda.stream(stream):
            for _ in range(3):                                          # warm-ups
                binding.prefill(x.q, x.k, x.v, x.slopes, st, out=out)
            for a, b in evs:
                torch.sum(flush, dim=0, out=sink)                       # evicts the MALL
                st.copy_(x.state)
                a.record(stream)
                binding.prefill(x.q, x.k, x.v, x.slopes, st, out=out)
                b.record(stream)
        stream.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        ms = 0.5 * (ts[(n - 1) // 2] + ts[n // 2])                      # median
        fl = prefill_flops(w.B, w.H, w.N, w.d)
        by = prefill_bytes(w.B, w.H, w.N, w.d)
        res[name] = {"config": f"B{w.B} H{w.H} N{w.N} d{w.d} bf16, "
                               + ("random fp32 initial state" if w.init_state else "zero state"),
                     "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 3),
                     "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del x, st, out
    del flush, sink
    # the flash models' head count (32 heads of 128, §2.1.1 and Table 1) at
    # 256K tokens: 128 column-slice workgroups, half of the device
    B, H, N, d = 1, 32, PREFILL["N"], 128
    with torch.cuda.stream(stream):
        x = inputs.make_prefill(B, H, N, d, torch.bfloat16, 1011, False, dev)
        out = torch.empty_like(x.q)
        ms = time_launches(stream, lambda: binding.prefill(x.q, x.k, x.v, x.slopes, x.state,
                                                           out=out), max(reps, 5))
    fl, by = prefill_flops(B, H, N, d), prefill_bytes(B, H, N, d)
    res["prefill_256k_flash_heads"] = {
        "config": f"B{B} H{H} N{N} d{d} bf16, zero state (128 workgroups)",
        "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 3),
        "gbs": round(by / (ms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del x, out
    # the fp32 path (fp32 q, k, v, out and state; fp32 matrix cores) at the 32K
    # continuation shape: bound by the fp32 MFMA rate, not by memory
    B, H, N, d = 1, 64, 32768, 128
    with torch.cuda.stream(stream):
        x = inputs.make_prefill(B, H, N, d, torch.float32, 1012, True, dev)
        st = x.state.clone()
        out = torch.empty_like(x.q)
        ms = time_launches(stream, lambda: binding.prefill(x.q, x.k, x.v, x.slopes, st, out=out),
                           max(reps, 5))
        ms1 = time_launches(stream, lambda: binding.prefill(x.q, x.k, x.v, x.slopes, st, out=out,
                                                            split=False), max(reps, 5))
        nseg = binding.prefill_f32_workspace_bytes(B, H, N, d, dev) // (H * d * d * 4)
    fl = prefill_flops(B, H, N, d)
    by = B * H * N * d * 4 * 4 + 2 * B * H * d * d * 4
    res["prefill_32k_fp32"] = {
        "config": f"B{B} H{H} N{N} d{d} fp32, random fp32 initial state",
        "kernel": "prefill_f32_kernel<128> (v_mfma_f32_32x32x2_f32)"
                  + (f", {nseg} segments per head (la_prefill_f32_ws)" if nseg > 1 else ""),
        "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 3),
        "frac_of_fp32_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
        "gbs": round(by / (ms * 1e-3) / 1e9, 1),
        "unsplit_ms": round(ms1, 4)}
    del x, st, out
    return res


def measure_decode_latency(dev, stream, reps):
    import torch
    from long_context_layers_amd import binding, inputs
    B, H, d, steps = 1, DECODE["H"], DECODE["d"], 64
    x = inputs.make_decode(B, H, d, steps, torch.bfloat16, DECODE["seed"], dev)
    st = x.state.clone()
    out = torch.empty_like(x.q[0])

    def run():
        for t in range(steps):
            binding.decode_step(x.q[t], x.k[t], x.v[t], x.slopes, st, out=out)

    with torch.cuda.stream(stream):
        ms_eager = min(time_launches(stream, run, 1) for _ in range(reps)) / steps
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    with torch.cuda.stream(stream):
        ms_graph = min(time_launches(stream, g.replay, 1) for _ in range(reps)) / steps
    torch.cuda.synchronize()
    by = decode_bytes(B, H, d)
    del g, x, st, out
    return {"workload": f"B{B} H{H} d{d} bf16, {steps} decode steps of one sequence",
            "eager_us_per_step": round(ms_eager * 1e3, 2),
            "graph_us_per_step": round(ms_graph * 1e3, 2),
            "graph_speedup": round(ms_eager / ms_graph, 3),
            "graph_gbs": round(by / (ms_graph * 1e-3) / 1e9, 1),
            "algorithmic_bytes_per_step": by,
            "kernel": "decode_kernel<bf16,128,4>: 4 column slices per head, 256 workgroups "
                      "per step"}


def corrected_tokens(slopes, L):
    """token-heads of an L-token shard whose correction factor
    lambda^(a+1) = exp(-s (a+1)) is not 0 in fp32: below 2^-150 it rounds to
    zero, so head s contributes the tokens with s (a+1) < 150 ln 2."""
    lim = 150.0 * math.log(2.0)
    return sum(min(L, max(0, math.ceil(lim / s) - 1)) if s > 0 else L for s in slopes)


def measure_cp(dev, stream, reps):
    import torch
    from long_context_layers_amd import binding, inputs
    R = 8
    B, H, d = PREFILL["B"], PREFILL["H"], PREFILL["d"]
    L = PREFILL["N"] // R
    with torch.cuda.stream(stream):
        x = inputs.make_prefill(B, H, L, d, torch.bfloat16, seed=1008, init_state=False, device=dev)
        g = torch.Generator(device=dev).manual_seed(1009)
        loc = 0.1 * torch.randn((R, B, H, d, d), generator=g, device=dev)   # gathered local states
        init = 0.1 * torch.randn((B, H, d, d), generator=g, device=dev)
        st = torch.zeros((B, H, d, d), device=dev)
        s_in = torch.empty((B, H, d, d), device=dev)
        out = torch.empty_like(x.q)
    stream.synchronize()

    def local():
        binding.prefill(x.q, x.k, x.v, x.slopes, st, out=out)

    def fold():
        binding.cp_fold(loc, [L] * R, R - 1, x.slopes, init, out=s_in)

    def correct():
        binding.cp_correct(x.q, x.slopes, s_in, out)

    with torch.cuda.stream(stream):
        ms_loc = time_launches(stream, local, reps)
        ms_fold = time_launches(stream, fold, reps)
        ms_corr = time_launches(stream, correct, reps)
    state_bytes = B * H * d * d * 4
    by_fold = (R - 1 + 2) * state_bytes                 # 7 local states + S_init read, S_in written
    # q, out read, out written for the tokens whose factor lambda^(a+1) is not 0
    # in fp32 (the others add exactly nothing and are skipped); S_in read
    ntok = B * corrected_tokens(x.slopes.tolist(), L)
    by_corr = ntok * d * 2 * 3 + state_bytes
    del x, loc, init, st, s_in, out
    gf, gc = by_fold / (ms_fold * 1e-3) / 1e9, by_corr / (ms_corr * 1e-3) / 1e9
    return {"workload": f"rank {R - 1} of {R}: shard B{B} H{H} L{L} d{d} bf16 of the 256K "
                        "sequence; the all-gather of the local states is not run (one GPU)",
            "local_prefill_ms": round(ms_loc, 4),
            "local_prefill_tflops": round(prefill_flops(B, H, L, d) / (ms_loc * 1e-3) / 1e12, 3),
            "cp_fold": {"ms": round(ms_fold, 4), "gbs": round(gf, 1),
                        "frac_of_hbm_peak": round(gf / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes": by_fold, "kernel": "cp_fold_kernel"},
            "cp_correct": {"ms": round(ms_corr, 4), "gbs": round(gc, 1),
                           "frac_of_hbm_peak": round(gc / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes": by_corr, "corrected_token_heads": ntok,
                           "kernel": "cp_correct_kernel<128, -1>"},
            "overhead_vs_local_prefill": round((ms_fold + ms_corr) / ms_loc, 4)}


def kernel_hash():
    """sha256 (first 16 hex digits) of the prefill call's kernel sources with
    comments and blank space removed, so comment edits keep the recorded
    counters."""
    text = "\n".join(open(f).read() for f in KERNEL_SRCS)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per prefill launch from the committed rocprofv3 counter
    summary, or None when it is absent or was taken on another kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def _counter_rows(path):
    """(kernel name, grid size, value) per dispatch, in dispatch order, from a
    rocprofv3 --pmc csv (one counter per run), or from every
    *counter_collection.csv under a directory."""
    import csv
    import glob
    files = [path] if os.path.isfile(path) else sorted(
        glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r.get("Dispatch_Id") or 0), r["Kernel_Name"],
                             int(float(r.get("Grid_Size") or 0)), float(r["Counter_Value"])))
    rows.sort()
    return [(k, g, v) for _, k, g, v in rows]


def write_traffic_summary(fetch, write, copy_fetch, copy_write, commands, out=None, call="split"):
    """The HBM bytes per launch of a timed call (TRAFFIC_CALLS) from FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) of a restricted bench run, each scaled by
    what the same counter reads for a plain device copy of known size; written
    with the hash of the kernel source the counters belong to."""
    B, H, N, d = PREFILL["B"], PREFILL["H"], PREFILL["N"], PREFILL["d"]
    spec = TRAFFIC_CALLS[call]
    out = out or spec["out"]
    copy_kib = (1 << 30) / 1024.0
    parts = [(k, k) for k in spec["kernels"]]

    def per(rows, pick):
        return [v for k, g, v in rows if pick(k)]
    is_copy = lambda k: "copyBuffer" in k or "copy" in k.lower()
    fetch_rows, write_rows = _counter_rows(fetch), _counter_rows(write)
    f_cp, w_cp = per(_counter_rows(copy_fetch), is_copy), per(_counter_rows(copy_write), is_copy)
    if not (f_cp and w_cp):
        raise SystemExit("missing copy dispatches in the counter files")
    kf, kw = copy_kib / min(f_cp), copy_kib / min(w_cp)      # KiB counted per KiB moved, inverted
    steady = lambda xs: xs[len(xs) // 2:]                     # the first dispatches carry earlier dirt
    raw, fr, wr = [], 0.0, 0.0
    for label, key in parts:
        fv, wv = per(fetch_rows, lambda k: key in k), per(write_rows, lambda k: key in k)
        if not (fv and wv):
            raise SystemExit(f"missing dispatches of {label} in the counter files")
        fr += sum(steady(fv)) / len(steady(fv)) * kf * 1024
        wr += sum(steady(wv)) / len(steady(wv)) * kw * 1024
        raw += [f"  {label}  FETCH_SIZE {', '.join('%.0f' % x for x in fv)}",
                f"  {label}  WRITE_SIZE {', '.join('%.0f' % x for x in wv)}"]
    algo = prefill_bytes(B, H, N, d)
    lines = [
        *[w.format(B=B, H=H, N=N, d=d) for w in spec["what"]],
        f"MI355X, rocprofv3 PMC, written by `python bench.py --traffic-summary --traffic-call {call}`",
        "from the counter files (no value typed by hand).",
        "",
        f"kernel_source_sha256_16: {kernel_hash()}   (code with comments and blank space removed)",
        "",
        "Commands (one counter per run, from /tmp with TMPDIR=/tmp; the repository at $R):",
        *["  " + c for c in commands],
        "",
        "Raw counters (KiB per dispatch, in dispatch order):",
        f"  copy 1 GiB  FETCH_SIZE {', '.join('%.0f' % x for x in f_cp)} -> factor {kf:.4f}",
        f"  copy 1 GiB  WRITE_SIZE {', '.join('%.0f' % x for x in w_cp)} -> factor {kw:.4f}",
        *raw,
        "",
        "Per prefill call (each kernel's steady state: the second half of its dispatches averaged,",
        "calibrated, then summed over the call's kernels; the counters need a few launches to",
        "settle after the inputs are written):",
        f"  reads  {fr / 1e9:.3f} GB   writes {wr / 1e9:.3f} GB",
        f"hbm_bytes_per_launch: {fr + wr:.0f}",
        f"algorithmic_bytes_per_launch: {algo}   (ratio {(fr + wr) / algo:.4f})",
        ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def cpu_baseline(pre, target_s=12.0):
    """The fp64 oracle on a bounded sample of the prefill workload: groups of
    16 heads over all N tokens, group after group until about ``target_s``
    seconds of oracle time have accumulated (or every head is done)."""
    import torch
    import oracle
    H, N, d = pre["H"], pre["N"], pre["d"]
    spent, heads_done, threads = 0.0, 0, 0
    for h0 in range(0, H, 16):
        idx = torch.arange(h0, min(H, h0 + 16), device=pre["q"].device)
        q, k, v = (t.index_select(1, idx).float().cpu().double().numpy()
                   for t in (pre["q"], pre["k"], pre["v"]))
        s = pre["slopes"].index_select(0, idx).cpu().double().numpy()
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, s)
        spent += time.perf_counter() - t0
        threads = max(threads, oracle.last_threads)
        heads_done += len(idx)
        del q, k, v
        if spent >= target_s:
            break
    fl = prefill_flops(1, heads_done, N, d)
    # one thread on the 4K workload (B1 H64 N4096 d128), for a per-core figure
    one = inputs_4k = None
    try:
        from long_context_layers_amd import inputs
        inputs_4k = inputs.make_workload("prefill_4k", device="cpu")
        q4, k4, v4 = (t.float().double().numpy() for t in (inputs_4k.q, inputs_4k.k, inputs_4k.v))
        s4 = inputs_4k.slopes.double().numpy()
        oracle.set_threads(1)
        t0 = time.perf_counter()
        oracle.prefill(q4, k4, v4, s4)
        one = time.perf_counter() - t0
    finally:
        oracle.set_threads(max(1, threads))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": fl / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 recurrent oracle (OpenMP over heads) on heads 0..{heads_done - 1} "
                      f"x all {N} tokens of the prefill workload ({heads_done}/{H} heads, "
                      f"{spent:.1f} s of oracle time); flops counted as on the GPU "
                      f"(B*H*N*(4d^2+2(C+1)d), C=64)",
            "seconds": round(spent, 2),
            "host_threads_available": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model,
            "one_thread_prefill_4k_s": None if one is None else round(one, 2),
            "one_thread_prefill_4k_tflops": None if one is None else
            round(prefill_flops(1, 64, 4096, 128) / one / 1e12, 5)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timing (for profiler runs)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the probe kernels that measure this GPU's MFMA and HBM ceilings")
    ap.add_argument("--power", action="store_true",
                    help="also sample package power and graphics clock (amd-smi) while the "
                         "prefill, the decode step and the probe kernels run back to back")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the prefill's HBM-traffic profile from four rocprofv3 --pmc "
                         "outputs (files or directories: FETCH_SIZE and WRITE_SIZE of a "
                         "--no-ceilings --extra-reps 0 run, then of a --copy-only run); no GPU")
    ap.add_argument("--traffic-call", choices=sorted(TRAFFIC_CALLS), default="split",
                    help="which timed call the --traffic-summary counters cover: the headline "
                         "la_prefill_ws (split) or the layer's la_prefill_qk_norm_rope_ws (fused)")
    ap.add_argument("--traffic-commands", nargs="*", default=[],
                    help="the commands that made those outputs, recorded in the profile")
    ap.add_argument("--extras", default="",
                    help="comma-separated subset of the extra measurements to run (varlen, "
                         "decode_multi, layer_ops, sizes, decode_latency, cp; default all)")
    ap.add_argument("--extra-reps", type=int, default=5,
                    help="launches timed for the packed-prefill and draft-verification lines "
                         "(0 skips them)")
    args = ap.parse_args()
    if args.traffic_summary:
        write_traffic_summary(*args.traffic_summary, commands=args.traffic_commands,
                              call=args.traffic_call)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(heads and batch shard across GPUs with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_layers_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.load_library()

    if args.copy_only:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": max(args.steps, 1)}))
        return

    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        p = inputs.make_prefill(PREFILL["B"], PREFILL["H"], PREFILL["N"], PREFILL["d"],
                                torch.bfloat16, PREFILL["seed"], False, dev)
        dcd = inputs.make_decode(DECODE["B"], DECODE["H"], DECODE["d"], DECODE["steps"],
                                 torch.bfloat16, DECODE["seed"], dev)
        out = torch.empty_like(p.q)
        pstate = torch.zeros_like(p.state)
        dstate = dcd.state.clone()
        dout = torch.empty_like(dcd.q[0])
    stream.synchronize()
    print(f"[bench] inputs resident: prefill {tuple(p.q.shape)} bf16, decode states "
          f"{tuple(dstate.shape)} fp32", file=sys.stderr, flush=True)

    def step(i, ev=None):
        pstate.zero_()
        if ev is not None:
            ev[0].record(stream)
        binding.prefill(p.q, p.k, p.v, p.slopes, pstate, out=out)
        if ev is not None:
            ev[1].record(stream)
        t = i % DECODE["steps"]
        binding.decode_step(dcd.q[t], dcd.k[t], dcd.v[t], dcd.slopes, dstate, out=dout)
        if ev is not None:
            ev[2].record(stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        stream.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i, evs[i])
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dec_step_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    # the decode rate: all 64 pre-staged steps chained as one timed region
    # (each step reads and writes every state once)
    with torch.cuda.stream(stream):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for t in range(DECODE["steps"]):
            binding.decode_step(dcd.q[t], dcd.k[t], dcd.v[t], dcd.slopes, dstate, out=dout)
        c1.record(stream)
        stream.synchronize()
    dec_ms = c0.elapsed_time(c1) / DECODE["steps"]
    print(f"[bench] {args.steps} steps: prefill {pre_ms:.3f} ms, decode {dec_step_ms:.3f} ms "
          f"(in the step), {dec_ms:.3f} ms ({DECODE['steps']} chained steps), "
          f"wall {wall * 1e3 / args.steps:.3f} ms/step", file=sys.stderr, flush=True)

    B, H, N, d = PREFILL["B"], PREFILL["H"], PREFILL["N"], PREFILL["d"]
    fl = prefill_flops(B, H, N, d)
    by = prefill_bytes(B, H, N, d)
    tflops = fl / (pre_ms * 1e-3) / 1e12
    gbs = by / (pre_ms * 1e-3) / 1e9
    dby = decode_bytes(DECODE["B"], DECODE["H"], DECODE["d"])
    dgbs = dby / (dec_ms * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill B1 H64 N262144 d128 bf16 from a zero state (la_prefill_ws: "
                        "two segments per head on 64-column workgroups, states folded, the "
                        "second segment corrected) + one decode step B256 H64 d128 (fp32 states)",
            "prefill": {"B": B, "H": H, "N": N, "d": d, "flop_count_block": C_COUNT},
            "decode": {"B": DECODE["B"], "H": DECODE["H"], "d": DECODE["d"]},
        },
        "prefill_ms": round(pre_ms, 4),
        "prefill_tflops_frac_of_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        # the same launch at the pure recurrent count (4 d^2 per token-head: the inter
        # term and the state update, no intra-block work)
        "prefill_tflops_recurrent_count": round(B * H * N * 4 * d * d / (pre_ms * 1e-3) / 1e12, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": by,
            "kernel": "prefill_bf16_kernel<128, false, false, 2, -1> (64-column workgroups, the "
                      "sequence in two segments per head), timed with the rest of its la_prefill_ws "
                      "call: split_prep_kernel, split_fold_kernel, cp_correct_kernel<128, -1>",
            "binding_limit": "memory traffic: a copy of the kernel with its compute removed "
                             "(same loads and stores) takes as long; against the 3:1 read/write "
                             "stream this chip sustains (ceilings.hbm_mix3_gbs) the gap is the "
                             "second pass of each head's Q and K rows through L2 by its other "
                             "column workgroup (a memory-only probe of that pattern: 3.7 against "
                             "5.5 TB/s with each workgroup reading only its own bytes); not "
                             "package power (with the redundant score tiles skipped the power "
                             "drops below the limit and the clock rises 12% at the same time)",
        },
        "context": {
            "pages_kernel_numbers": "none: the Ling and Ring 2.6 Technical Report gives no "
                                    "kernel-level throughput for this path, so vs_baseline is null",
            "attention_flop_share": "in the GQA predecessor attention takes more than 60% of "
                                    "all FLOPs once contexts pass 32K tokens (report, §1 and "
                                    "§2.1.3; hardware not stated)",
            "context_parallel_speedup": "AllGather context parallelism with variable-length "
                                        "fusion sped linear-attention training at 256K up by "
                                        "about 68% end to end (report, §4.1.2; hardware not "
                                        "stated); its on-GPU arithmetic is the cp line below",
        },
        "decode": {
            "value": round(dgbs, 1),
            "timing": f"{DECODE['steps']} chained steps as one region (HIP events), per step; "
                      "in_step_ms: the one step of each timed step, right after its prefill",
            "in_step_ms": round(dec_step_ms, 4),
            "unit": "GB/s",
            "ms_per_step": round(dec_ms, 4),
            "frac_of_hbm_peak": round(dgbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": dby,
            "kernel": "decode_kernel<bf16,128>",
        },
    }
    if args.power:
        print("[bench] package power and clock", file=sys.stderr, flush=True)
        res["power"] = measure_power_all(dev, stream, p, pstate, out, dcd, dstate, dout)
        torch.cuda.empty_cache()
    if not args.no_ceilings:
        print("[bench] ceilings (MFMA loop, HBM streams)", file=sys.stderr, flush=True)
        res["ceilings"] = measure_ceilings(dev, stream, pre_ms, tflops, dgbs)
        torch.cuda.empty_cache()
    extras = [
        ("varlen", "packed variable-length prefill",
         lambda: measure_varlen(dev, stream, args.extra_reps, tflops)),
        ("decode_multi", "multi-token decode", lambda: measure_decode_multi(dev, stream, args.extra_reps)),
        ("layer_ops", "layer ops (QK norm + RoPE, grouped norm x gate, the fused prologue)",
         lambda: measure_layer_ops(dev, stream, args.extra_reps, pre_ms)),
        ("sizes", "prefill at 4K and 32K", lambda: measure_sizes(dev, stream, args.extra_reps)),
        ("decode_latency", "single-sequence decode latency (eager, HIP graph)",
         lambda: measure_decode_latency(dev, stream, args.extra_reps)),
        ("cp", "sequence-sharded prefill steps", lambda: measure_cp(dev, stream, args.extra_reps))]
    wanted = set(args.extras.split(",")) if args.extras else {k for k, _, _ in extras}
    unknown = wanted - {k for k, _, _ in extras}
    if unknown:
        raise SystemExit(f"unknown --extras {sorted(unknown)}")
    if args.extra_reps > 0:
        for key, what, fn in extras:
            if key not in wanted:
                continue
            print(f"[bench] {what}", file=sys.stderr, flush=True)
            res[key] = fn()
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(dict(q=p.q, k=p.k, v=p.v, slopes=p.slopes, N=N, d=d, H=H))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
