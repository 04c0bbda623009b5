"""Host-side pieces of bench.py: the single-GPU guard and the parsing of the
package power / clock query (no GPU needed)."""
import os
import subprocess
import sys

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
