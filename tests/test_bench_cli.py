"""The benchmark on the CPU: a multi-GPU request exits with a message before
anything touches a GPU (the library has one-GPU kernels only), and the
power-sample parser reads amd-smi's text."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_power_sample_parser_reads_socket_power_and_every_xcd_clock():
    """bench.py --power parses `amd-smi metric -p -c` text: the socket power and
    the CLK line that follows each GFX_<i> header (not MIN_CLK / MAX_CLK, not
    the memory or video clocks)."""
    sys.path.insert(0, ROOT)
    import bench
    text = "\n".join([
        "GPU: 0",
        "    POWER:",
        "        SOCKET_POWER: 1329 W",
        "        GFX_VOLTAGE: N/A",
        "    CLOCK:",
        "        GFX_0:",
        "            CLK: 1877 MHz",
        "            MIN_CLK: 500 MHz",
        "            MAX_CLK: 2400 MHz",
        "            CLK_LOCKED: DISABLED",
        "        GFX_1:",
        "            CLK: 1806 MHz",
        "            MIN_CLK: 500 MHz",
        "        MEM_0:",
        "            CLK: 2000 MHz",
        "        VCLK_0:",
        "            CLK: 59 MHz",
    ])
    assert bench.parse_amd_smi_metric(text) == {"socket_w": 1329.0, "gfx_mhz": [1877.0, 1806.0]}
    assert bench.parse_amd_smi_metric("") == {"socket_w": None, "gfx_mhz": []}
