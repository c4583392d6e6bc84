"""Benchmark of the BA-Att hot path on one MI355X.

A step is one pass of the whole hot path on one batch of synthetic input:
the selection pass (pool + corrected score + norm sort) followed by the
block-sparse attention pass, at the workload's sparsity.  The default
workload is the largest single-GPU configuration, the distribution-shift
stress (B2 H32 N32768 D128, block 128, 50% sparsity, drifting 16-component
mixture with a local band and planted needle keys).

Prints ONE JSON line: dense-equivalent attention TFLOP/s of the step
(4*B*H*N^2*D per step / step time), the speedup over this library's own
dense kernel, a roofline object for the dominant kernel (the sparse
attention kernel, bf16 MFMA), one for the selection pass (HBM), the same
step on the LLaDA-8B-shaped layer (and, on request, the video-DiT shape),
the long-context sweep, the split key-list measurement, the
selection-quality report (not part of the timed step), the fp64 CPU oracle
timed on a seeded head subset of the same workload, and the benchmark's
own outputs checked against that oracle (mask near-tie counts, max |dO|,
max |dLSE|).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# the sources that fix each kernel's memory traffic: a committed counter
# reading is used only while the hash of its kernel's sources still matches
KERNEL_SOURCES = {
    "attention": ["block_sparse_attention_ba_amd/csrc/attention.hpp",
                  "block_sparse_attention_ba_amd/csrc/common.hpp"],
    "select": ["block_sparse_attention_ba_amd/csrc/select.hpp",
               "block_sparse_attention_ba_amd/csrc/common.hpp"],
}


def source_code_text(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed, so that a
    comment edit leaves the hash of the code unchanged (string literals in
    the kernels hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(source_code_text(f.read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clocks ramp up over the first ~30 ms of sustained work (the
    # sparse step measures ~640 us for its first 25-50 launches, then ~580 us),
    # so the default warm-up covers the ramp and the timed steps see steady state
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="shift")
    ap.add_argument("--sparsity", type=float, default=None)
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU-oracle baseline")
    ap.add_argument("--skip-dense", action="store_true", help="omit the dense comparator")
    ap.add_argument("--skip-peaks", action="store_true",
                    help="omit the machine-peak microbenchmarks (HBM read/copy, bf16 MFMA)")
    ap.add_argument("--skip-flushed", action="store_true",
                    help="omit the step and dense timings with L2 and the MALL flushed before each repetition")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="heads of the seeded subset the CPU oracle runs (and the O/LSE parity covers)")
    ap.add_argument("--extra", default="llada8b",
                    help="comma-separated further workloads timed as a step against dense "
                         "(llada8b, video, long_b64, long_b128, tiny; empty for none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for traffic counters)")
    ap.add_argument("--power", action="store_true",
                    help="also sample socket power and graphics clocks (amd-smi) while the sparse kernel, "
                         "the dense kernel and the bf16 MFMA peak loop each run back to back for a few seconds")
    ap.add_argument("--operand-data", action="store_true",
                    help="also run the sparse and dense kernels, with the workload's own block lists, on "
                         "zeros, ones, normals with 2-bit mantissas, normals and the workload's inputs, "
                         "each back to back for a few seconds with power and clocks sampled")
    ap.add_argument("--skip-split", action="store_true",
                    help="omit the split key-list and external-contribution measurements")
    ap.add_argument("--skip-queued", action="store_true",
                    help="omit the work-queue forward (ba_att_forward_queued) timed against the one-tile forward")
    ap.add_argument("--skip-sweep", action="store_true",
                    help="omit the long-context sweep (16K tokens, block 64/128, sparsity 0/50/75%%)")
    ap.add_argument("--skip-quality", action="store_true",
                    help="omit the selection-quality report (block recall / rank correlation)")
    return ap.parse_args()


def split_kv_measurement(lib, dev, stream, warmup: int, reps: int) -> dict:
    """Split key lists on a shape whose workgroups half-fill the device:
    one head, N = 32768, D = 128, block 64 (512 query blocks in 256 four-wave tiles) at
    50% sparsity.  Times ba_att_forward against ba_att_forward_split."""
    import numpy as np
    import torch
    from block_sparse_attention_ba_amd import api
    B, H, N, D, blk, sp = 1, 1, 32768, 128, 64, 0.5
    g = torch.Generator(device=dev).manual_seed(20260519)
    q, k, v = (torch.randn((B, H, N, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    n = lib.ba_att_num_blocks(N, blk)
    keep = lib.ba_att_keep_count(n, sp)
    ws = torch.empty(api.select_workspace_bytes(B, H, N, D, blk), dtype=torch.uint8, device=dev)
    mask = torch.empty((B, H, n, n), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, H, n, keep), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    sptr = stream.cuda_stream
    assert lib.ba_att_select(B, H, N, D, blk, 0.0, sp, q.data_ptr(), k.data_ptr(), mask.data_ptr(),
                             idx.data_ptr(), cnt.data_ptr(), None, ws.data_ptr(), ws.numel(), sptr) == 0
    splits = (2, 4, 8)
    sws = torch.empty(lib.ba_att_forward_split_workspace_bytes(B, H, N, D, max(splits)), dtype=torch.uint8,
                      device=dev)

    def run(ns):
        if ns == 1:
            return lib.ba_att_forward(B, H, N, D, blk, 0.0, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      idx.data_ptr(), cnt.data_ptr(), keep, o.data_ptr(), 0, lse.data_ptr(), sptr)
        return lib.ba_att_forward_split(B, H, N, D, blk, 0.0, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        idx.data_ptr(), cnt.data_ptr(), keep, ns, o.data_ptr(), 0,
                                        lse.data_ptr(), sws.data_ptr(), sws.numel(), sptr)

    def timed(ns):
        for _ in range(warmup):
            assert run(ns) == 0
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            run(ns)
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    res = {"shape": "B1 H1 N32768 D128 block 64, 50% sparsity (512 query blocks)", "unsplit_ms": timed(1)}
    res["split_ms"] = {str(ns): round(timed(ns), 5) for ns in splits}
    best = min(res["split_ms"].items(), key=lambda kv: kv[1])
    res["unsplit_ms"] = round(res["unsplit_ms"], 5)
    res["best_split"] = int(best[0])
    res["speedup"] = round(res["unsplit_ms"] / best[1], 3)
    # the library's own choice for this shape (ba_att_forward_split_parts)
    res["suggested_split"] = int(lib.ba_att_forward_split_parts(B, H, N, blk, keep))
    return res


def external_measurement(lib, stream, dims, tensors, warmup: int, reps: int) -> dict:
    """ba_att_forward_ext against ba_att_forward on the benchmark's own inputs
    and block lists.  The external part (fp32 O_ext and LSE_ext over another
    key set) is read once per row in the epilogue, so its extra time is priced
    against those bytes: B*H*N*(4*D + 4)."""
    import numpy as np
    import torch
    B, H, N, D, blk, keep, code = dims
    q, k, v, idx, cnt, o, lse = tensors
    dev = q.device
    g = torch.Generator(device=dev).manual_seed(20260520)
    o_ext = torch.randn((B, H, N, D), generator=g, device=dev, dtype=torch.float32)
    lse_ext = torch.randn((B, H, N), generator=g, device=dev, dtype=torch.float32) + 5.0
    sptr = stream.cuda_stream

    def run(ext):
        if ext:
            st = lib.ba_att_forward_ext(B, H, N, D, blk, 0.0, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        idx.data_ptr(), cnt.data_ptr(), keep, o_ext.data_ptr(), lse_ext.data_ptr(),
                                        o.data_ptr(), code, lse.data_ptr(), sptr)
        else:
            st = lib.ba_att_forward(B, H, N, D, blk, 0.0, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    idx.data_ptr(), cnt.data_ptr(), keep, o.data_ptr(), code, lse.data_ptr(), sptr)
        if st:
            raise RuntimeError(lib.ba_att_status_string(st).decode())

    def timed(ext):
        for _ in range(warmup):
            run(ext)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            run(ext)
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    # alternate the two so that clock drift falls on both
    plain, ext = [], []
    for _ in range(3):
        plain.append(timed(False))
        ext.append(timed(True))
    t0, t1 = float(np.median(plain)), float(np.median(ext))
    extra_bytes = B * H * N * (4 * D + 4)
    res = {"forward_ms": round(t0, 5), "forward_ext_ms": round(t1, 5), "extra_ms": round(t1 - t0, 5),
           "extra_bytes": extra_bytes,
           "extra_gbs": round(extra_bytes / ((t1 - t0) * 1e-3) / 1e9, 1) if t1 > t0 else None}
    del o_ext, lse_ext
    return res


def long_context_sweep(dev, stream, warmup: int, reps: int) -> list:
    """The long-context workloads (B1 H32 N16384 D128, block 64 and 128) at each
    of their sparsities: select + sparse step time against the dense kernel,
    all on resident inputs.  Times are means of HIP-event pairs on the stream
    after `warmup` untimed repetitions."""
    import numpy as np
    import torch
    from block_sparse_attention_ba_amd import api, workloads

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # the two long-context workloads share their inputs; only the block differs
    x = workloads.make_inputs("long_b64")
    q, k, v = up(x["q"]), up(x["k"]), up(x["v"])
    del x
    out = []
    for name in ("long_b64", "long_b128"):
        w = workloads.WORKLOADS[name]
        B, H, N, D, blk = w.B, w.H, w.N, w.D, w.block
        assert tuple(q.shape) == (B, H, N, D)
        o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

        def timed(fn):
            for _ in range(warmup):
                fn()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in evs:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([a.elapsed_time(b) for a, b in evs]))

        dense_ms = timed(lambda: api.dense(q, k, v, out_dtype=torch.bfloat16, out=o, lse=lse))
        dense_flops = 4.0 * B * H * N * N * D
        ws = torch.empty(api.select_workspace_bytes(B, H, N, D, blk), dtype=torch.uint8, device=dev)
        for sp in w.sparsities:
            mask, idx, cnt = api.select(q, k, blk, sp, workspace=ws)

            def step():
                _, i2, c2 = api.select(q, k, blk, sp, workspace=ws)
                api.forward(q, k, v, i2, c2, blk, out_dtype=torch.bfloat16, out=o, lse=lse)

            step_ms = timed(step)
            kept = kept_tile_flops(mask.cpu().numpy(), N, D, blk)
            out.append({"workload": name, "shape": f"B{B} H{H} N{N} D{D} b{blk}", "sparsity": sp,
                        "keep": int(idx.shape[-1]), "step_ms": round(step_ms, 5), "dense_ms": round(dense_ms, 5),
                        "speedup_vs_dense": round(dense_ms / step_ms, 4),
                        "dense_equiv_tflops": round(dense_flops / step_ms / 1e9, 1),
                        "kept_tile_tflops": round(kept / step_ms / 1e9, 1)})
        del o, lse, ws
    del q, k, v
    torch.cuda.empty_cache()
    return out


def kept_tile_flops(mask, N: int, D: int, block: int) -> float:
    """4*D*sum over kept (I, J) of |I|*|J| (true sizes of a partial tail)."""
    import numpy as np
    n = mask.shape[-1]
    sizes = np.array([min(block, N - i * block) for i in range(n)], dtype=np.float64)
    m = mask.reshape(-1, n, n).astype(np.float64)
    return float(4.0 * D * np.einsum("bij,i,j->", m, sizes, sizes))


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: the model string with its
    family / model / stepping numbers (a virtualised host may report only a
    generic string), and the number of logical CPUs the host has."""
    fields, logical = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "processor":
                    logical += 1
                elif key in ("model name", "cpu family", "model", "stepping", "microcode") and key not in fields:
                    fields[key] = val.strip()
    except OSError:
        return "unknown host CPU"
    name = fields.get("model name", "unknown host CPU")
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping", "microcode") if k in fields)
    return f"{name} ({ids}; {logical} logical CPUs on the host)" if ids else name


def cpu_ranges(cpus) -> str:
    """Compact form of a CPU set: {0,1,2,3,8} -> '0-3,8'."""
    cpus, out, i = sorted(cpus), [], 0
    while i < len(cpus):
        j = i
        while j + 1 < len(cpus) and cpus[j + 1] == cpus[j] + 1:
            j += 1
        out.append(str(cpus[i]) if i == j else f"{cpus[i]}-{cpus[j]}")
        i = j + 1
    return ",".join(out)


def sample_heads(name: str, B: int, H: int, count: int) -> list:
    """A seeded subset of `count` (batch, head) pairs that holds the first and
    the last head (every head when count >= B*H)."""
    import zlib
    import numpy as np
    every = [(b, h) for b in range(B) for h in range(H)]
    if count >= len(every):
        return every
    rng = np.random.default_rng(zlib.crc32(f"cpu-baseline-{name}".encode()))
    inner = rng.choice(np.arange(1, len(every) - 1), size=count - 2, replace=False)
    return [every[i] for i in sorted({0, len(every) - 1, *(int(i) for i in inner)})]


def cpu_baseline(x, w, sp: float, heads: list) -> tuple:
    """The fp64 oracle as it stands, timed on this host: selection plus
    block-sparse attention of the given heads, one head per host thread
    (BLAS single-threaded inside each).  Returns the baseline record and the
    oracle's (mask, O, LSE) per head for the parity check."""
    from oracle import ba_att_oracle as orc
    from oracle.parity import host_threads, map_heads

    threads = host_threads()
    cpus = os.sched_getaffinity(0)

    def one(bh):
        a = time.perf_counter()
        sel = orc.select_oracle(x["q"], x["k"], w.block, sp, heads=[bh])
        b = time.perf_counter()
        O, L = orc.attention_oracle(x["q"], x["k"], x["v"], sel["mask"], w.block, heads=[bh])[bh]
        return sel["mask"][bh], O, L, b - a, time.perf_counter() - b

    t0 = time.perf_counter()
    res = map_heads(one, heads, threads)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.N * w.N * w.D * len(heads)
    record = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(min(threads, len(heads))),
              "kind": "oracle", "host_cores_available": len(cpus), "affinity_cpus": cpu_ranges(cpus),
              "thread_cap": 16, "cpu_model": cpu_model(), "wall_s": round(dt, 3),
              "select_s_summed": round(sum(r[3] for r in res), 3),
              "attention_s_summed": round(sum(r[4] for r in res), 3),
              "heads": [list(h) for h in heads],
              "sample": f"{len(heads)} of {w.B * w.H} heads of the same workload (seeded subset with the "
                        "first and last head; selection + block-sparse attention, fp64 numpy, one head per "
                        f"thread on {min(threads, len(heads))} threads), {dt:.1f} s; "
                        "dense-equivalent FLOPs of the sampled heads / wall time"}
    return record, {h: r[:3] for h, r in zip(heads, res)}


def parity_report(x, w, sp: float, gmask, o_own, lse_own, oracle_heads: dict) -> dict:
    """The benchmark's own outputs against the oracle.

    Masks: every row of every head against the oracle's selection (the
    near-tie rule: rows whose oracle cut margin is below 1e-4 relative may
    differ inside that band; they are counted).  O and LSE (fp32 output of
    the forward on the GPU's own block lists): every query row of the
    oracle's sampled heads whose mask row equals the oracle's, against the
    oracle's attention."""
    import numpy as np
    from oracle import ba_att_oracle as orc
    from oracle.parity import LSE_TOL, O_TOL, compare_masks, max_abs

    t0 = time.perf_counter()
    ref = orc.select_oracle(x["q"], x["k"], w.block, sp)
    sel_s = time.perf_counter() - t0
    m = compare_masks(gmask, ref["S"], ref["mask"], ref["keep"])
    worst_o = worst_l = 0.0
    rows = skipped = 0
    for (bi, hi), (omask, O, L) in oracle_heads.items():
        eq = np.all(gmask[bi, hi] == omask, axis=-1)
        tok = np.repeat(eq, w.block)[:w.N]
        rows += int(tok.sum())
        skipped += int((~tok).sum())
        worst_o = max(worst_o, max_abs(o_own[(bi, hi)][tok], O[tok]))
        worst_l = max(worst_l, max_abs(lse_own[(bi, hi)][tok], L[tok]))
    ok = not m["bad"] and worst_o <= O_TOL and worst_l <= LSE_TOL
    return {"mask_rows": m["rows"], "mask_exact": m["exact"], "near_tie_rows": m["near_tie_rows"],
            "near_tie_mismatch": m["near_tie_mismatch"], "bad_rows": len(m["bad"]),
            "heads_o_lse": [list(h) for h in oracle_heads], "o_rows_compared": rows,
            "o_rows_skipped_near_tie": skipped, "max_abs_dO": worst_o, "max_abs_dLSE": worst_l,
            "tolerance": {"O": O_TOL, "LSE": LSE_TOL, "near_tie_rel_margin": 1e-4},
            "oracle_select_all_heads_s": round(sel_s, 3), "pass": bool(ok)}


def parse_amd_smi_metric(text: str) -> dict:
    """Socket power (W) and the graphics clock of every XCD (MHz) from the text
    that `amd-smi metric -p -c` prints: `SOCKET_POWER: <W> W` under POWER and
    `GFX_<i>:` followed by `CLK: <MHz> MHz` under CLOCK."""
    import re
    watts = [float(m) for m in re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)]
    gfx = [float(m) for m in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", text)]
    return {"socket_w": watts[0] if watts else None, "gfx_mhz": gfx}


def power_sample(run, stream, seconds: float) -> dict:
    """Runs `run` back to back for about `seconds` while `amd-smi metric -p -c`
    is sampled three times from a thread; returns the socket power (W) and the
    graphics clocks (MHz, one per XCD) it read, with the mean call time."""
    import subprocess
    import threading
    import time
    import torch
    samples = []

    def sampler():
        time.sleep(min(1.0, seconds / 4))
        for _ in range(3):
            try:
                out = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                                     timeout=20).stdout
            except (OSError, subprocess.SubprocessError):
                return
            samples.append(parse_amd_smi_metric(out))
            time.sleep(seconds / 6)

    for _ in range(10):
        run()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    t0 = time.time()
    th.start()
    calls = 0
    while time.time() - t0 < seconds or th.is_alive():
        for _ in range(10):
            run()
        torch.cuda.synchronize()
        calls += 10
    ms = (time.time() - t0) * 1e3 / calls
    return {"mean_ms_per_call": round(ms, 5), "samples": samples}


def mfma_loop_power(dev, stream, seconds: float, random_operands: bool = False) -> dict:
    """Socket power and clocks while a bf16 MFMA peak loop (libba_peaks.so:
    2 waves per SIMD, independent MFMA chains, no memory traffic) runs back to
    back: what the matrix pipes alone draw at full rate, on constant operands
    or on random ones (eight operand pairs cycled per wave)."""
    import torch
    from block_sparse_attention_ba_amd import _lib
    pk = _lib.load_peaks()
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(n_cu * 2 * 256, dtype=torch.float32, device=dev)
    iters, per_iter = (5000, 8) if random_operands else (20000, 4)

    def run():
        rc = (pk.ba_peak_mfma_bf16_random(sink.data_ptr(), n_cu * 2, iters, 12345, stream.cuda_stream)
              if random_operands else
              pk.ba_peak_mfma_bf16(sink.data_ptr(), n_cu * 2, iters, 2.0 ** -10, stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("peak microbenchmark launch failed")

    res = power_sample(run, stream, seconds)
    res["tflops"] = round(n_cu * 2 * 4 * iters * per_iter * 32768 / (res["mean_ms_per_call"] * 1e-3) / 1e12, 1)
    return res


def operand_data(P, dev, stream, seconds: float = 3.0) -> dict:
    """The sparse kernel (the workload's own block lists) and the dense kernel
    on operands of decreasing bit activity: the same instructions, the same
    memory traffic, only the values differ.  Each runs back to back while
    power and clocks are sampled.  Normals are drawn on the GPU from a seeded
    generator; the 2-bit variant keeps sign, exponent and the top two
    mantissa bits of each bf16 normal."""
    import torch
    B, H, N, D, blk = P.dims
    kept = kept_tile_flops(P.mask.cpu().numpy(), N, D, blk)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260)

    def normals(bits_mask=None):
        out = []
        for _ in range(3):
            t = torch.randn((B, H, N, D), generator=gen, device=dev).to(torch.bfloat16)
            if bits_mask is not None:
                t = (t.view(torch.int16) & bits_mask).view(torch.bfloat16)
            out.append(t)
        return out

    own = (P.q, P.k, P.v)
    variants = [("zeros", lambda: [torch.zeros((B, H, N, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]),
                ("ones", lambda: [torch.ones((B, H, N, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]),
                ("normal, 2-bit mantissa", lambda: normals(-32)),   # 0xFFE0
                ("normal", normals),
                ("workload inputs", lambda: list(own))]
    res = {}
    try:
        for name, make in variants:
            P.q, P.k, P.v = make()
            row = {}
            for kname, fn, fl in (("sparse", P.sparse, kept), ("dense", P.dense, P.dense_flops)):
                r = power_sample(fn, stream, seconds)
                ms = r["mean_ms_per_call"]
                clocks = [c for smp in r["samples"] for c in smp["gfx_mhz"]]
                row[kname] = {"ms": ms, "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                              "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                              "socket_w": [smp["socket_w"] for smp in r["samples"]],
                              "gfx_mhz_range": [min(clocks), max(clocks)] if clocks else None}
            res[name] = row
            print(f"[bench] operand data {name}: {row}", file=sys.stderr, flush=True)
            P.q = P.k = P.v = None
            torch.cuda.empty_cache()
    finally:
        P.q, P.k, P.v = own
    return res


def measured_peaks(dev, stream, reps: int = 5) -> dict:
    """HBM read and copy bandwidth and the bf16 MFMA rate measured on this GPU
    (libba_peaks.so), as context for the vendor peaks the rooflines use."""
    import numpy as np
    import torch
    from block_sparse_attention_ba_amd import _lib
    pk = _lib.load_peaks()
    sptr = stream.cuda_stream
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count

    def timed(f):
        if f() != 0:
            raise RuntimeError("peak microbenchmark launch failed")
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            f()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3

    # the best over a few grid sizes (2 workgroups per CU reads fastest: each
    # grid-stride round then covers a compact 2 MB span)
    grids = [2, 8, 32]
    sink = torch.empty(n_cu * max(grids) * 256, dtype=torch.int32, device=dev)
    nbytes = 4 << 30  # far beyond the 256 MB MALL: every byte comes from HBM
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    half = nbytes // 2
    t_read = {g: timed(lambda: pk.ba_peak_read(buf.data_ptr(), nbytes, sink.data_ptr(), n_cu * g, 0, sptr))
              for g in grids}
    t_read_nt = {g: timed(lambda: pk.ba_peak_read(buf.data_ptr(), nbytes, sink.data_ptr(), n_cu * g, 1, sptr))
                 for g in grids}
    t_copy = {g: timed(lambda: pk.ba_peak_copy(buf.data_ptr(), buf.data_ptr() + half, half, n_cu * g, sptr))
              for g in grids}
    del buf, sink
    g_read, g_copy = min(t_read, key=t_read.get), min(t_copy, key=t_copy.get)
    g_read_nt = min(t_read_nt, key=t_read_nt.get)
    mwg, iters = n_cu * 2, 20000  # two waves per SIMD, four independent MFMA chains each
    fsink = torch.empty(mwg * 256, dtype=torch.float32, device=dev)
    t_mfma = timed(lambda: pk.ba_peak_mfma_bf16(fsink.data_ptr(), mwg, iters, 2.0 ** -10, sptr))
    mfma_tfs = mwg * 4 * iters * 4 * 32768 / t_mfma / 1e12
    # random operands: the clock settles lower under their switching power, so
    # the loop runs back to back for about half a second before it is timed
    riters = 5000
    rand = lambda: pk.ba_peak_mfma_bf16_random(fsink.data_ptr(), mwg, riters, 12345, sptr)
    t_end = time.time() + 0.5
    while time.time() < t_end:
        for _ in range(20):
            if rand() != 0:
                raise RuntimeError("peak microbenchmark launch failed")
        torch.cuda.synchronize()
    t_rand = timed(rand)
    del fsink
    rand_tfs = mwg * 4 * riters * 8 * 32768 / t_rand / 1e12
    return {
        "hbm_read_tbs": round(nbytes / t_read[g_read] / 1e12, 3),
        "hbm_read_nontemporal_tbs": round(nbytes / t_read_nt[g_read_nt] / 1e12, 3),
        "hbm_copy_tbs": round(2 * half / t_copy[g_copy] / 1e12, 3),
        "workgroups_per_cu": {"read": g_read, "read_nontemporal": g_read_nt, "copy": g_copy},
        "mfma_bf16_tflops": round(mfma_tfs, 1),
        # v_mfma_f32_32x32x16_bf16: 32768 FLOP per 32 cycles per SIMD, 4 SIMDs per CU
        "implied_clock_ghz": round(mfma_tfs * 1e12 / (n_cu * 4 * 1024) / 1e9, 3),
        # the same loop on random bf16 operands (eight pairs per wave)
        "mfma_bf16_random_operands_tflops": round(rand_tfs, 1),
        "random_operands_implied_clock_ghz": round(rand_tfs * 1e12 / (n_cu * 4 * 1024) / 1e9, 3),
        "vendor": {"hbm_tbs": HBM_PEAK_GBS / 1000.0, "mfma_bf16_tflops": MFMA_BF16_PEAK_TFS},
        "workload": "read 4 GiB with plain and with nontemporal loads and copy 2 GiB (best of 2/8/32 "
                    "workgroups per CU); "
                    "2 waves per SIMD x 20000 rounds of 4 independent MFMAs on constant operands; "
                    "2 waves per SIMD x 5000 rounds of 8 MFMAs over 8 random operand pairs, "
                    "after 0.5 s back to back",
    }


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def time_steps(select, sparse, stream, warmup: int, steps: int) -> tuple:
    """`steps` select + sparse steps back to back with no event between the
    kernels (each event recorded between two kernels leaves about 5 us of idle
    GPU), wall clock between two synchronisations; one event pair around the
    whole loop cross-checks it on the GPU's clock.  Returns (ms, gpu ms) per
    step."""
    import torch
    for _ in range(warmup):
        select()
        sparse()
    torch.cuda.synchronize()
    g0, g1 = _ev(), _ev()
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(steps):
        select()
        sparse()
    g1.record(stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, g0.elapsed_time(g1) / steps


def time_kernels(select, sparse, stream, steps: int) -> tuple:
    """The same steps with HIP events around each kernel on the stream the
    kernels run on: per-call durations (ms) of the select pass and of the
    sparse attention kernel."""
    import numpy as np
    import torch
    ev = [(_ev(), _ev(), _ev()) for _ in range(steps)]
    for e0, e1, e2 in ev:
        e0.record(stream)
        select()
        e1.record(stream)
        sparse()
        e2.record(stream)
    torch.cuda.synchronize()
    return (np.array([a.elapsed_time(b) for a, b, _ in ev]), np.array([b.elapsed_time(c) for _, b, c in ev]))


def time_flushed(fn, stream, warmup: int, reps: int, flush, sink):
    """Per-call durations (ms) of fn, each call after a 1 GiB read that evicts
    L2 and the MALL (a read leaves no dirty lines to write back)."""
    import numpy as np
    import torch
    out = []
    for i in range(warmup + reps):
        torch.sum(flush, dim=0, out=sink)
        a, b = _ev(), _ev()
        a.record(stream)
        fn()
        b.record(stream)
        if i >= warmup:
            out.append((a, b))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in out])


def time_calls(fn, stream, warmup: int, reps: int) -> float:
    """Mean duration (ms) of fn between one event pair per call."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(_ev(), _ev()) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


class Problem:
    """One workload resident on the GPU with its outputs and C-ABI calls."""

    def __init__(self, lib, name: str, sp: float | None, out_dtype: str, dev, stream, x=None):
        import numpy as np
        import torch
        from block_sparse_attention_ba_amd import api, workloads

        self.w = w = workloads.WORKLOADS[name]
        self.sp = sp if sp is not None else (0.5 if 0.5 in w.sparsities else w.sparsities[0])
        self.x = x if x is not None else workloads.make_inputs(name)

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        self.q, self.k, self.v = up(self.x["q"]), up(self.x["k"]), up(self.x["v"])
        B, H, N, D, blk = w.B, w.H, w.N, w.D, w.block
        self.dims = (B, H, N, D, blk)
        self.n = api.num_blocks(N, blk)
        self.keep = api.keep_count(self.n, self.sp)
        self.odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
        self.code = 0 if self.odt == torch.bfloat16 else 1
        self.ws = torch.empty(api.select_workspace_bytes(B, H, N, D, blk), dtype=torch.uint8, device=dev)
        self.mask = torch.empty((B, H, self.n, self.n), dtype=torch.uint8, device=dev)
        self.idx = torch.empty((B, H, self.n, self.keep), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B, H, self.n), dtype=torch.int32, device=dev)
        self.o = torch.empty((B, H, N, D), dtype=self.odt, device=dev)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.lib, self.stream, self.sptr = lib, stream, stream.cuda_stream
        self.dense_flops = 4.0 * B * H * N * N * D
        self.sel_bytes = (2.0 * B * H * N * D * 2 + B * H * self.n * self.n + 4.0 * B * H * self.n * self.keep
                          + 4.0 * B * H * self.n)

    def _check(self, st):
        if st:
            raise RuntimeError(self.lib.ba_att_status_string(st).decode())

    def select(self):
        B, H, N, D, blk = self.dims
        self._check(self.lib.ba_att_select(B, H, N, D, blk, 0.0, self.sp, self.q.data_ptr(), self.k.data_ptr(),
                                           self.mask.data_ptr(), self.idx.data_ptr(), self.cnt.data_ptr(), None,
                                           self.ws.data_ptr(), self.ws.numel(), self.sptr))

    def sparse(self, o=None, code=None):
        B, H, N, D, blk = self.dims
        o = self.o if o is None else o
        self._check(self.lib.ba_att_forward(B, H, N, D, blk, 0.0, self.q.data_ptr(), self.k.data_ptr(),
                                            self.v.data_ptr(), self.idx.data_ptr(), self.cnt.data_ptr(), self.keep,
                                            o.data_ptr(), self.code if code is None else code,
                                            self.lse.data_ptr(), self.sptr))

    def sparse_queued(self, o=None, lse=None):
        """The same forward through ba_att_forward_queued (resident grid, per-XCD work queues)."""
        import torch
        B, H, N, D, blk = self.dims
        if getattr(self, "queue", None) is None:
            self.queue = torch.zeros(16, dtype=torch.int32, device=self.q.device)
        o = self.o if o is None else o
        lse = self.lse if lse is None else lse
        self._check(self.lib.ba_att_forward_queued(B, H, N, D, blk, 0.0, self.q.data_ptr(), self.k.data_ptr(),
                                                   self.v.data_ptr(), self.idx.data_ptr(), self.cnt.data_ptr(),
                                                   self.keep, o.data_ptr(), self.code, lse.data_ptr(),
                                                   self.queue.data_ptr(), self.sptr))

    def dense(self):
        B, H, N, D, blk = self.dims
        self._check(self.lib.ba_att_dense(B, H, N, D, 0.0, self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                          self.o.data_ptr(), self.code, self.lse.data_ptr(), self.sptr))

    def label(self) -> str:
        B, H, N, D, blk = self.dims
        return f"B{B} H{H} N{N} D{D} b{blk}"


def queued_measurement(p, stream, warmup: int, steps: int, rounds: int = 3) -> dict:
    """ba_att_forward_queued against ba_att_forward on a workload's own block
    lists: outputs compared bit for bit, then the select + sparse step timed
    both ways (back to back, alternating rounds so that clock drift falls on
    both), and each sparse kernel alone between event pairs."""
    import numpy as np
    import torch
    p.select()
    o2, l2 = torch.empty_like(p.o), torch.empty_like(p.lse)
    p.sparse()
    p.sparse_queued(o2, l2)
    torch.cuda.synchronize()
    same = bool(torch.equal(o2, p.o) and torch.equal(l2, p.lse))
    del o2, l2
    plain, queued, k_plain, k_queued = [], [], [], []
    for _ in range(rounds):
        plain.append(time_steps(p.select, p.sparse, stream, warmup, steps)[0])
        queued.append(time_steps(p.select, p.sparse_queued, stream, warmup, steps)[0])
        k_plain.append(time_calls(p.sparse, stream, 2, steps))
        k_queued.append(time_calls(p.sparse_queued, stream, 2, steps))
    t0, t1 = float(np.median(plain)), float(np.median(queued))
    return {"workload": p.w.name, "shape": p.label(), "bit_identical": same,
            "step_ms": round(t0, 5), "step_ms_queued": round(t1, 5), "step_speedup": round(t0 / t1, 4),
            "speedup_vs_dense_queued": None,
            "sparse_ms": round(float(np.median(k_plain)), 5), "sparse_ms_queued": round(float(np.median(k_queued)), 5),
            "rounds": rounds, "steps_per_round": steps}


def uneven_lists_measurement(p, stream, reps: int, rounds: int = 3) -> dict:
    """The one-tile and the work-queue forward on block lists whose length
    grows with the head: head i of the B*H keeps n - floor(sp_i * n) blocks,
    sp_i rising linearly from 0 (first head) to 0.875 (last), each row a
    seeded random subset.  The one-tile launch deals each XCD a contiguous
    range of heads, so the XCD holding the first heads holds the most work;
    the queues let the others take part of it.  Outputs compared bit for bit."""
    import numpy as np
    import torch
    B, H, N, D, blk = p.dims
    n, BH = p.n, B * H
    g = torch.Generator(device=p.q.device).manual_seed(20260521)
    idx = torch.argsort(torch.rand((B, H, n, n), generator=g, device=p.q.device), dim=-1).to(torch.int32)
    sp = 0.875 * np.arange(BH) / max(1, BH - 1)
    keep_h = [n - int(np.floor(s * n + 1e-9)) for s in sp]
    cnt = torch.tensor(keep_h, dtype=torch.int32, device=p.q.device).view(B, H, 1).expand(B, H, n).contiguous()
    o2, l2 = torch.empty_like(p.o), torch.empty_like(p.lse)
    if getattr(p, "queue", None) is None:
        p.queue = torch.zeros(16, dtype=torch.int32, device=p.q.device)

    def plain(o=None, lse=None):
        o = p.o if o is None else o
        lse = p.lse if lse is None else lse
        p._check(p.lib.ba_att_forward(B, H, N, D, blk, 0.0, p.q.data_ptr(), p.k.data_ptr(), p.v.data_ptr(),
                                      idx.data_ptr(), cnt.data_ptr(), n, o.data_ptr(), p.code, lse.data_ptr(),
                                      p.sptr))

    def queued(o=None, lse=None):
        o = p.o if o is None else o
        lse = p.lse if lse is None else lse
        p._check(p.lib.ba_att_forward_queued(B, H, N, D, blk, 0.0, p.q.data_ptr(), p.k.data_ptr(), p.v.data_ptr(),
                                             idx.data_ptr(), cnt.data_ptr(), n, o.data_ptr(), p.code,
                                             lse.data_ptr(), p.queue.data_ptr(), p.sptr))

    plain()
    queued(o2, l2)
    torch.cuda.synchronize()
    same = bool(torch.equal(o2, p.o) and torch.equal(l2, p.lse))
    del o2, l2
    tp, tq = [], []
    for _ in range(rounds):
        tp.append(time_calls(plain, stream, 2, reps))
        tq.append(time_calls(queued, stream, 2, reps))
    # kept-tile FLOPs, 4*D*|I|*|J| per kept pair with the tail block at its true size
    size = torch.full((n,), float(blk), device=p.q.device, dtype=torch.float64)
    size[-1] = N - (n - 1) * blk
    on = torch.arange(n, device=p.q.device).view(1, 1, 1, n) < cnt.unsqueeze(-1)
    kj = (size[idx.long()] * on).sum(-1)                     # [B,H,n]: keys attended by a row of block I
    flops = float(4.0 * D * (kj * size.view(1, 1, n)).sum())
    t0, t1 = float(np.median(tp)), float(np.median(tq))
    del idx, cnt, on, kj
    return {"lists": "head i of B*H keeps n - floor(sp_i*n) blocks per row, sp_i = 0.875*i/(B*H-1); "
                     "seeded random subsets",
            "kept_tile_tflop": round(flops / 1e12, 4), "bit_identical": same, "forward_ms": round(t0, 5),
            "forward_queued_ms": round(t1, 5), "speedup": round(t0 / t1, 4),
            "forward_tflops": round(flops / (t0 * 1e-3) / 1e12, 1),
            "forward_queued_tflops": round(flops / (t1 * 1e-3) / 1e12, 1), "rounds": rounds, "reps": reps}


def secondary(lib, name: str, args, dev, stream, flush, sink) -> dict:
    """The step against the dense kernel on another workload: step time,
    per-kernel times, the sparse kernel's and the flushed select pass's
    roofline fractions."""
    import numpy as np
    import torch
    p = Problem(lib, name, None, args.out_dtype, dev, stream)
    step_ms, _ = time_steps(p.select, p.sparse, stream, args.warmup, args.steps)
    sel_t, spa_t = time_kernels(p.select, p.sparse, stream, args.steps)
    sel_f = time_flushed(p.select, stream, 5, max(10, args.steps // 2), flush, sink)
    dense_ms = time_calls(p.dense, stream, max(5, args.warmup // 2), max(5, args.steps // 2))
    kept = kept_tile_flops(p.mask.cpu().numpy(), p.w.N, p.w.D, p.w.block)
    spa_ms, selm = float(spa_t.mean()), float(np.median(sel_f))
    qd = None if args.skip_queued else queued_measurement(p, stream, max(5, args.warmup // 2), args.steps)
    if qd is not None:
        qd["speedup_vs_dense_queued"] = round(dense_ms / qd["step_ms_queued"], 4)
    res = {"workload": p.w.description, "name": name, "shape": p.label(), "sparsity": p.sp,
           "keep": p.keep, "n_blocks": p.n, "ms_per_step": round(step_ms, 5),
           "dense_equiv_tflops": round(p.dense_flops / step_ms / 1e9, 2),
           "dense_ms": round(dense_ms, 5), "speedup_vs_dense": round(dense_ms / step_ms, 4),
           "select_ms": round(float(sel_t.mean()), 5), "sparse_attention_ms": round(spa_ms, 5),
           "sparse_frac_of_mfma_peak": round(kept / (spa_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
           "select_flushed_ms": round(selm, 5),
           "select_frac_of_hbm_peak": round(p.sel_bytes / (selm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "queued": qd}
    del p
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; every head is independent, so a multi-GPU run would shard "
              "(batch, head) pairs with no communication.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_ba_amd import _lib, api

    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_ba_amd import build
        build.build()
    api.load()
    lib = _lib.load()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    P = Problem(lib, args.workload, args.sparsity, args.out_dtype, dev, stream)
    w, sp = P.w, P.sp
    B, H, N, D, blk = P.dims
    n, keep = P.n, P.keep
    print(f"[bench] workload {w.name}: {P.label()} sparsity {sp} keep {keep}/{n}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        # a plain copy of known size in one elementwise dispatch (a uint8 ->
        # int8 cast copy): reads 1 GiB and writes 1 GiB
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(1 << 30, dtype=torch.int8, device=dev)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- the timed hot path
    step_ms, gpu_step_ms = time_steps(P.select, P.sparse, stream, args.warmup, args.steps)
    sel_t, spa_t = time_kernels(P.select, P.sparse, stream, args.steps)
    sel_ms, spa_ms = float(sel_t.mean()), float(spa_t.mean())
    pct = lambda t: [round(float(np.percentile(t, 10)), 5), round(float(np.percentile(t, 90)), 5)]
    print(f"[bench] timed {args.steps} steps: {step_ms:.4f} ms/step ({gpu_step_ms:.4f} ms between GPU events); "
          f"per kernel over {args.steps} more steps: select {sel_ms:.4f} ms, sparse attention {spa_ms:.4f} ms",
          file=sys.stderr, flush=True)

    gmask = P.mask.cpu().numpy()
    kept_flops = kept_tile_flops(gmask, N, D, blk)

    # ---- selection pass with L2 and the MALL flushed before every call
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    sel_flush_t = time_flushed(P.select, stream, args.warmup, args.steps, flush, sink)
    sel_flush_ms = float(np.median(sel_flush_t))

    # ---- the dense comparator
    dense_ms = None
    if not args.skip_dense:
        dense_ms = time_calls(P.dense, stream, args.warmup, max(5, args.steps // 2))
        print(f"[bench] dense {dense_ms:.4f} ms ({P.dense_flops / dense_ms / 1e9:.1f} TFLOP/s)",
              file=sys.stderr, flush=True)

    # ---- the step and the dense comparator again, each repetition after the
    # same flushing read (no input left in L2 or the MALL)
    flushed = None
    if not args.skip_flushed and not args.skip_dense:
        reps = max(10, args.steps // 2)
        f_step = time_flushed(lambda: (P.select(), P.sparse()), stream, 0, reps, flush, sink)
        f_dense = time_flushed(P.dense, stream, 0, reps, flush, sink)
        fs, fd = float(np.median(f_step)), float(np.median(f_dense))
        flushed = {"reps": reps, "flush": "1 GiB read before each repetition",
                   "step_ms": round(fs, 5), "dense_ms": round(fd, 5),
                   "speedup_vs_dense": round(fd / fs, 4),
                   "dense_equiv_tflops": round(P.dense_flops / (fs * 1e-3) / 1e12, 2),
                   "p10_p90_ms": {"step": pct(f_step), "dense": pct(f_dense)}}
        print(f"[bench] flushed: {flushed}", file=sys.stderr, flush=True)

    power = None
    if args.power:
        power = {"sparse": power_sample(P.sparse, stream, 4.0), "dense": power_sample(P.dense, stream, 4.0),
                 "mfma_loop": mfma_loop_power(dev, stream, 4.0),
                 "mfma_loop_random_operands": mfma_loop_power(dev, stream, 4.0, random_operands=True)}
        print(f"[bench] power: {power}", file=sys.stderr, flush=True)
    opdata = operand_data(P, dev, stream) if args.operand_data else None

    # ---- the product path's own outputs for the parity check against the
    # oracle: the forward on the GPU's block lists with fp32 output
    heads = sample_heads(w.name, B, H, args.cpu_heads)
    own_o = own_l = None
    if not args.skip_cpu:
        P.select()
        o32 = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
        P.sparse(o=o32, code=1)
        torch.cuda.synchronize()
        gmask = P.mask.cpu().numpy()
        own_o = {h: o32[h[0], h[1]].cpu().numpy() for h in heads}
        own_l = {h: P.lse[h[0], h[1]].cpu().numpy() for h in heads}
        del o32

    split_kv = external = None
    if not args.skip_split:
        split_kv = split_kv_measurement(lib, dev, stream, args.warmup, max(5, args.steps // 2))
        print(f"[bench] split key lists: {split_kv}", file=sys.stderr, flush=True)
        external = external_measurement(lib, stream, (B, H, N, D, blk, keep, P.code),
                                        (P.q, P.k, P.v, P.idx, P.cnt, P.o, P.lse), 10, max(5, args.steps // 2))
        print(f"[bench] external contribution: {external}", file=sys.stderr, flush=True)

    queued = None
    if not args.skip_queued:
        queued = queued_measurement(P, stream, max(5, args.warmup // 2), args.steps)
        queued["uneven_lists"] = uneven_lists_measurement(P, stream, max(5, args.steps // 5))
        if dense_ms:
            queued["speedup_vs_dense_queued"] = round(dense_ms / queued["step_ms_queued"], 4)
        print(f"[bench] work-queue forward: {queued}", file=sys.stderr, flush=True)

    quality = None
    if not args.skip_quality:
        from block_sparse_attention_ba_amd import quality as qmod
        quality = qmod.measure(P.q, P.k, P.v, blk, sp)
        print(f"[bench] selection quality: {quality}", file=sys.stderr, flush=True)

    extra = []
    for name in [e for e in args.extra.split(",") if e and e != w.name]:
        extra.append(secondary(lib, name, args, dev, stream, flush, sink))
        print(f"[bench] {name}: {extra[-1]}", file=sys.stderr, flush=True)

    sweep = None
    if not args.skip_sweep:
        sweep = long_context_sweep(dev, stream, 5, 10)
        print(f"[bench] long-context sweep: {sweep}", file=sys.stderr, flush=True)
    del flush, sink

    peaks = None
    if not args.skip_peaks:
        peaks = measured_peaks(dev, stream)
        print(f"[bench] measured peaks: {peaks}", file=sys.stderr, flush=True)

    # ---- HBM traffic from the committed counter runs, while the kernels'
    # sources still match the ones the counters were taken on
    traffic = sel_traffic = None
    hashes = {kind: kernel_source_hash(kind) for kind in KERNEL_SOURCES}
    try:
        with open(TRAFFIC_FILE) as f:
            tc = json.load(f)
        entry = tc.get("workloads", {}).get(f"{w.name}:{sp}:{args.out_dtype}") or {}
        if entry.get("attention_source_hash") == hashes["attention"]:
            traffic = entry.get("attention_bytes_per_launch")
        if entry.get("select_source_hash") == hashes["select"]:
            sel_traffic = entry.get("select_bytes_per_call")
    except (OSError, ValueError):
        pass

    achieved = kept_flops / (spa_ms * 1e-3) / 1e12
    value = P.dense_flops / (step_ms * 1e-3) / 1e12
    sel_gbs = P.sel_bytes / (sel_flush_ms * 1e-3) / 1e9
    result = {
        "metric": "dense-equiv attention TFLOP/s + speedup vs own dense kernel @50% sparsity",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "gpu_ms_per_step": round(gpu_step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.description, "name": w.name, "B": B, "H": H, "N": N, "D": D,
                   "block": blk, "sparsity": sp, "keep": keep, "n_blocks": n,
                   "out_dtype": args.out_dtype, "parallelism": "single GPU"},
        "speedup_vs_dense": round(dense_ms / step_ms, 4) if dense_ms else None,
        "dense_ms": round(dense_ms, 5) if dense_ms else None,
        "dense_tflops": round(P.dense_flops / (dense_ms * 1e-3) / 1e12, 2) if dense_ms else None,
        "select_ms": round(sel_ms, 5),
        "sparse_attention_ms": round(spa_ms, 5),
        "p10_p90_ms": {"select": pct(sel_t), "sparse_attention": pct(spa_t), "select_flushed": pct(sel_flush_t)},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel (sparse)",
                     "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4), "traffic": traffic,
                     "work_per_launch": kept_flops,
                     # context: the MFMA-only loop on random operands, measured here
                     "frac_of_random_operand_mfma_loop":
                         round(achieved / peaks["mfma_bf16_random_operands_tflops"], 4) if peaks else None},
        "roofline_select": {"bound": "hbm", "kernel": "pool_stats_kernel + score_topk_kernel",
                            "achieved": round(sel_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(sel_gbs / HBM_PEAK_GBS, 4), "traffic": sel_traffic,
                            "bytes_per_call": P.sel_bytes, "ms_flushed_median": round(sel_flush_ms, 5)},
        "flushed": flushed,
        "other_workloads": extra,
        "long_context_sweep": sweep,
        "measured_peaks": peaks,
        "split_kv": split_kv,
        "external": external,
        "queued": queued,
        "power": power,
        "operand_data": opdata,
        "selection_quality": quality,
        # the pages' only operator-speed figure, as context: it names no hardware,
        # sequence length or sparsity, so it is no target for this measurement
        "paper_context": "up to 6.95x over FlashAttention (hardware, shape and sparsity not stated)",
        "kernel_source_hash": hashes,
    }
    result["cpu_baseline"] = result["parity"] = None
    if not args.skip_cpu:
        print(f"[bench] timing the CPU oracle on {len(heads)} heads ...", file=sys.stderr, flush=True)
        result["cpu_baseline"], oracle_heads = cpu_baseline(P.x, w, sp, heads)
        print(f"[bench] cpu baseline: {result['cpu_baseline']}", file=sys.stderr, flush=True)
        result["parity"] = parity_report(P.x, w, sp, gmask, own_o, own_l, oracle_heads)
        print(f"[bench] parity: {result['parity']}", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
