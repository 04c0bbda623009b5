"""Host-side pieces of bench.py: the single-GPU guard and the parsing of the
package power / clock query (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# the layout `amd-smi metric -p -c` prints (values made up)
SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1234 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 2000 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 2100 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
        VCLK_0:
            CLK: 59 MHz
"""


def test_parse_power_clock():
    w, mhz = bench.parse_power_clock(SMI_TEXT)
    assert w == 1234.0
    assert mhz == 2050          # mean of the GFX clocks only, not MEM or VCLK


@pytest.mark.parametrize("text", [None, "", "no such fields\n"])
def test_parse_power_clock_missing(text):
    assert bench.parse_power_clock(text) == (None, None)


def test_smi_sample_missing_tool():
    assert bench.smi_sample(["no-such-smi-tool-here"]) is None


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _pmc_csv(path, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w") as f:
        f.write(",".join(f'"{c}"' for c in cols) + "\n")
        for i, (name, val) in enumerate(rows):
            r = dict.fromkeys(cols, "0")
            r.update(Dispatch_Id=str(i + 1), Kernel_Name=name, Grid_Size="131072",
                     Counter_Name="X", Counter_Value=str(val))
            f.write(",".join(f'"{r[c]}"' for c in cols) + "\n")


def test_traffic_summary_is_calibrated_and_keyed_by_the_source(tmp_path, monkeypatch):
    # made-up counters: the copy reads count twice (factor 1/2), writes once;
    # the prefill's steady dispatches (3..) read 6,000,000 KiB and write 4,000,000
    pre = "void la::(anonymous namespace)::prefill_bf16_kernel<128, false, false, 2, -1>(...)"
    prep, fold = "la::split_prep_kernel(...)", "la::split_fold_kernel(...)"
    corr = "void la::(anonymous namespace)::cp_correct_kernel<128, -1>(...)"
    cp = "__amd_rocclr_copyBuffer"
    gib = 1 << 20
    call = lambda a, b, c, e: [(prep, a), (pre, b), (fold, c), (corr, e)]
    _pmc_csv(tmp_path / "f.csv", call(9, 7e6, 9, 90) + call(9, 6.5e6, 9, 90) +
             call(1, 6e6, 2, 10) + call(1, 6e6, 2, 10))
    _pmc_csv(tmp_path / "w.csv", call(9, 4.5e6, 9, 90) + call(9, 4.1e6, 9, 90) +
             call(3, 4e6, 4, 5) + call(3, 4e6, 4, 5))
    _pmc_csv(tmp_path / "cf.csv", [(cp, 2 * gib), (cp, 2 * gib + 10)])
    _pmc_csv(tmp_path / "cw.csv", [(cp, gib), (cp, gib)])
    out = tmp_path / "traffic.txt"
    bench.write_traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"),
                                ["rocprofv3 ..."], out=str(out))
    text = out.read_text()
    assert f"kernel_source_sha256_16: {bench.kernel_hash()}" in text
    want = ((1 + 6e6 + 2 + 10) / 2 + (3 + 4e6 + 4 + 5)) * 1024
    assert f"hbm_bytes_per_launch: {want:.0f}" in text
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.measured_traffic() == pytest.approx(want)
    # a profile keyed by another source is not used
    out.write_text(text.replace(bench.kernel_hash(), "0" * 16))
    assert bench.measured_traffic() is None


def test_traffic_summary_of_the_fused_call(tmp_path):
    # the layer's fused call has its own kernels and its own profile file; the
    # headline's counters do not satisfy it
    pre = "void la::(anonymous namespace)::prefill_bf16_kernel<128, true, false, 2, 64>(...)"
    corr = "void la::(anonymous namespace)::cp_correct_kernel<128, 64>(...)"
    prep, fold = "la::split_prep_kernel(...)", "la::split_fold_kernel(...)"
    cp = "__amd_rocclr_copyBuffer"
    gib = 1 << 20
    call = lambda b: [(prep, 2), (pre, b), (fold, 4), (corr, 8)]
    _pmc_csv(tmp_path / "f.csv", call(7e6) + call(6e6) + call(6e6))
    _pmc_csv(tmp_path / "w.csv", call(4e6) + call(4e6) + call(4e6))
    _pmc_csv(tmp_path / "cf.csv", [(cp, 2 * gib)])
    _pmc_csv(tmp_path / "cw.csv", [(cp, gib)])
    out = tmp_path / "fused.txt"
    bench.write_traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"),
                                ["rocprofv3 ..."], out=str(out), call="fused")
    text = out.read_text()
    assert "la_prefill_qk_norm_rope_ws" in text and "--traffic-call fused" in text
    want = ((2 + 6e6 + 4 + 8) / 2 + (2 + 4e6 + 4 + 8)) * 1024
    assert f"hbm_bytes_per_launch: {want:.0f}" in text
    with pytest.raises(SystemExit):
        bench.write_traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                    str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"),
                                    [], out=str(tmp_path / "x.txt"), call="split")


@pytest.mark.parametrize("s", [1.0, 0.5, 2.0 ** -0.125, 2.0 ** -4, 2.0 ** -8, 1e-3])
def test_corrected_tokens_counts_nonzero_fp32_factors(s):
    # the tokens whose factor exp(-s (a+1)) survives in fp32, by brute force
    # over every token of the shard (numpy's fp32 exp; at most one token of
    # difference at the rounding threshold)
    L = 40000
    a = np.arange(L, dtype=np.float64)
    f = np.exp(-(np.float32(s) * (a + 1).astype(np.float32)), dtype=np.float32)
    brute = int(np.count_nonzero(f))
    assert abs(bench.corrected_tokens([s], L) - brute) <= 1


def test_corrected_tokens_special_cases():
    assert bench.corrected_tokens([0.0], 77) == 77              # lambda = 1: every token
    assert bench.corrected_tokens([1e-9], 100) == 100           # nothing underflows in a short shard
    assert bench.corrected_tokens([200.0], 100) == 0            # lambda^1 is already 0
    assert bench.corrected_tokens([1.0, 1.0], 10) == 20         # a sum over heads
