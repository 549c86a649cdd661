"""Host-side pieces of bench.py (no GPU): the amd-smi clock/power parser and
the --gpus guard."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# The shape of `amd-smi metric -c -p` text output: a POWER block, then one
# GFX_<n> block per XCD with its current clock, then other clock domains.
SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1351 W
        GFX_VOLTAGE: N/A
        POWER_MANAGEMENT: N/A
    CLOCK:
        GFX_0:
            CLK: 1901 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
        GFX_1:
            CLK: 1846 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
        MEM_0:
            CLK: 1900 MHz
            MIN_CLK: 900 MHz
            MAX_CLK: 1900 MHz
        VCLK_0:
            CLK: 29 MHz
"""


def test_parse_smi_metric_takes_gfx_clocks_only():
    clocks, power = bench.parse_smi_metric(SMI_TEXT)
    assert clocks == [1901.0, 1846.0]
    assert power == 1351.0


def test_parse_smi_metric_empty():
    assert bench.parse_smi_metric("") == ([], None)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_child_runs_the_oracle():
    """The CPU baseline leg runs the oracle in a child process and reports its
    throughput with the threads it used (tiny fp32 share: milliseconds)."""
    from synthetic import WORKLOADS
    name = "tiny_fp32_contiguous_cp4_r1"
    res = bench.cpu_baseline(dict(WORKLOADS[name]), name, 1)
    assert res["value"] > 0 and res["cores"] >= 1 and res["kind"] == "oracle", res
    assert "rank 1" in res["sample"] and res["seconds"] > 0
