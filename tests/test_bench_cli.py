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


def test_cpu_baseline_and_parity_report_on_the_tiny_workload():
    """The CPU leg on the host: the oracle runs on a seeded head subset (first
    and last head included), reports the cores it used and the CPU model, and
    the parity report passes outputs equal to the oracle's, counts rows, and
    fails a planted error in O, in LSE and in a mask row."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from block_sparse_attention_ba_amd import workloads as wl
    from oracle import ba_att_oracle as orc

    heads = bench.sample_heads("shift", 2, 32, 16)
    assert len(heads) == 16 and heads[0] == (0, 0) and heads[-1] == (1, 31)
    assert heads == bench.sample_heads("shift", 2, 32, 16)  # seeded
    assert bench.sample_heads("tiny", 1, 1, 16) == [(0, 0)]

    x = wl.make_inputs("tiny")
    w = x["workload"]
    rec, per_head = bench.cpu_baseline(x, w, 0.5, [(0, 0)])
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["heads"] == [[0, 0]]
    assert rec["host_cores_available"] >= 1 and rec["cpu_model"] and rec["affinity_cpus"]
    mask, O, L = per_head[(0, 0)]
    ref = orc.select_oracle(x["q"], x["k"], w.block, 0.5)
    assert np.array_equal(mask, ref["mask"][0, 0])

    gmask = ref["mask"].copy()
    rep = bench.parity_report(x, w, 0.5, gmask, {(0, 0): O.astype(np.float32)},
                              {(0, 0): L.astype(np.float32)}, per_head)
    assert rep["pass"] and rep["bad_rows"] == 0 and rep["o_rows_compared"] == w.N
    assert rep["max_abs_dO"] < 1e-6 and rep["max_abs_dLSE"] < 1e-5

    bad_o = O.copy()
    bad_o[5, 3] += 0.02
    assert not bench.parity_report(x, w, 0.5, gmask, {(0, 0): bad_o}, {(0, 0): L}, per_head)["pass"]
    bad_l = L.copy()
    bad_l[100] += 0.002
    assert not bench.parity_report(x, w, 0.5, gmask, {(0, 0): O}, {(0, 0): bad_l}, per_head)["pass"]
    # a mask row that keeps the wrong blocks outside any near tie
    S = ref["S"][0, 0]
    row = int(np.argmax([np.sort(s)[::-1][ref["keep"] - 1] - np.sort(s)[::-1][ref["keep"]] for s in S]))
    gmask2 = gmask.copy()
    gmask2[0, 0, row] = 1 - gmask2[0, 0, row]
    rep2 = bench.parity_report(x, w, 0.5, gmask2, {(0, 0): O}, {(0, 0): L}, per_head)
    assert not rep2["pass"] and rep2["bad_rows"] == 1
    assert rep2["o_rows_skipped_near_tie"] == w.block  # that row's tokens are not compared


def test_kernel_source_hash_ignores_comments_only():
    """The traffic counters stay valid across comment edits of a kernel's
    sources, and not across code edits."""
    import bench
    code = "int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n"
    assert bench.source_code_text(code) == bench.source_code_text("int f(int x) { return x + 1; }")
    assert bench.source_code_text(code) != bench.source_code_text("int f(int x) { return x + 2; }")
    for kind in bench.KERNEL_SOURCES:
        assert len(bench.kernel_source_hash(kind)) == 16
