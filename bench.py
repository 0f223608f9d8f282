#!/usr/bin/env python3
"""Benchmark of the KDA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one kda_prefill_fwd call over the named prefill workload (gate, intra-chunk
products, triangular solve, state pass and outputs all run inside it).  The headline
workload is the largest one, the varlen batch of 64 sequences (about 278K tokens, 32 heads,
initial and final states); the batched (4 x 32768) and single-sequence (4096) workloads are
timed after it and reported under 'prefill_other', each with its own roofline.  The same line also
carries the decode half of the metric: 256 consecutive kda_decode_step calls over
512 sequences x 32 heads, a speculative-decode round, and standalone timings of the output
epilogue, the input prologue and the gate at the batched workload's sizes.  Inputs are seeded
synthetic data resident in HBM before timing.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + MFMA util; decode tokens/s + HBM GB/s"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
CHUNK = 64


def prefill_algorithmic(dk: int, dv: int, elem: int, z_bytes: int = 4):
    """Algorithmic work of the chunkwise prefill per token-head at chunk C = 64 (what the
    method must compute and move; masked, recomputed or dense-padding work excluded):
      flops: per chunk 6 C dk dv (the three state products) + C(C-1) dk (A_kk, strictly
             lower) + 2 C(C+1) dk (A_qk, and W = T K, lower incl.) + 2 C(C+1) dv (T V and
             A_qk U) + C^3/3 (the triangular inverse), divided by C
      bytes: q, k, v, beta and o in the element type, z in fp32 (states amortised)."""
    C = CHUNK
    flops = (6 * C * dk * dv + C * (C - 1) * dk + 2 * C * (C + 1) * dk + 2 * C * (C + 1) * dv
             + C ** 3 / 3) / C
    byts = (2 * dk + dv) * elem + elem + z_bytes * dk + dv * elem
    return flops, byts


def decode_bytes_per_pair(dk: int, dv: int, elem: int):
    """State read + write (fp32) plus one token's inputs and output."""
    return 2 * dk * dv * 4 + prefill_algorithmic(dk, dv, elem)[1]


_COMMON_SOURCES = ("kda_device.h", "kda_launch.h")


def summary_sources(name: str):
    """Kernel source files a profile summary depends on (None: all of them).  A prefill
    summary also depends on the C ABI file, which chooses the prefill's kernels."""
    if name.startswith("prefill_"):
        return ("kda_prefill_split.hip", "kda_api.cpp") + _COMMON_SOURCES
    if name.startswith(("decode_", "spec_decode_")):
        return ("kda_decode.hip",) + _COMMON_SOURCES
    if name.startswith("gate_"):
        return ("kda_gate.hip",) + _COMMON_SOURCES
    if name.startswith("output_gate_"):
        return ("kda_epilogue.hip",) + _COMMON_SOURCES
    if name.startswith("short_conv_"):
        return ("kda_prologue.hip",) + _COMMON_SOURCES
    return None


def kernel_source_hash(files=None) -> str:
    """Hash of the kernel sources (all of them, or the named files) with comments and blank
    space removed, so a stored counter summary stays valid across comment edits and is
    dropped by any code change to the sources it depends on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_chunkwise_amd", "csrc")
    for f in sorted(os.listdir(csrc)) if files is None else sorted(files):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _summary(workload: str, kind: str):
    """Text of profiles/<workload>_<kind>.txt if it was taken for the current sources of the
    kernels it covers, else None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_{kind}.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    if not m_hash or m_hash.group(1) != kernel_source_hash(summary_sources(workload)):
        return None
    return txt


def read_traffic(workload: str):
    """HBM traffic per launch measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each
    scaled by what the same counter reads for a device copy of known size), if a summary for
    the current kernel sources exists under profiles/ (else None)."""
    txt = _summary(workload, "traffic")
    m_bytes = txt and re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    return float(m_bytes.group(1)) if m_bytes else None


def read_mfma(workload: str):
    """Executed MFMA work of one prefill call from rocprofv3 counters, if a summary for the
    current kernel sources exists under profiles/ (else None): bf16 MFMA flops executed
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, including masked tiles and per-slice recompute) and
    the fraction of SIMD cycles the MFMA units were busy over the call's kernels
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs)."""
    txt = _summary(workload, "mfma")
    if txt is None:
        return None
    m_fl = re.search(r"executed_bf16_flops_per_launch:\s*([0-9.eE+]+)", txt)
    m_busy = re.search(r"mfma_busy_frac_per_launch:\s*([0-9.eE+-]+)", txt)
    if not m_fl or not m_busy:
        return None
    return {"executed_bf16_flops_per_launch": float(m_fl.group(1)),
            "mfma_busy_frac": float(m_busy.group(1)),
            "source": f"profiles/{workload}_mfma.txt"}


# --- rocprofv3 summaries under profiles/ ---------------------------------------------------
# The raw rocprofv3 output stays out of the repository; these functions turn it into the short
# text summaries that the readers above use.  The runs they expect, one directory each under
# RAW (R = the repository root; cd /tmp && export TMPDIR=/tmp first):
#   <prefill workload>_kt        rocprofv3 --kernel-trace --stats -d RAW/<dir> -o kt
#                                --output-format csv -- python3 R/bench.py PREFILL_ARGS
#                                --steps 20 --warmup 3
#   <prefill workload>_<C>       rocprofv3 --pmc <C> --kernel-trace -d RAW/<dir> -o p
#                                --output-format csv -- python3 R/bench.py PREFILL_ARGS
#                                --steps 2 --warmup 1 --calibration-copy-mib 1024
#                                for C = FETCH_SIZE, WRITE_SIZE
#   <prefill workload>_mfma      the same with --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
#                                SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE (no calibration copy)
#   others_kt, others_<C>        the same two kinds of runs over OTHER_ARGS (decode, speculative
#                                decode, output epilogue, input prologue and gate), counters
#                                with --decode-steps 4
# where PREFILL_ARGS = --workload <w> --extra-workloads none --no-cpu-baseline --no-decode and
# OTHER_ARGS = --workload prefill_b1_h16_t4096_d128_bf16 --extra-workloads none --no-cpu-baseline.

MFMA_COUNTERS = "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE"
_PRE = "cd /tmp && export TMPDIR=/tmp && "
_PREFILL_KERNELS = ("kda::chunk_table_kernel", "kda::chain_order_kernel", "prefill_intra_kernel",
                    "prefill_state", "prefill_fused_kernel")
# summary name -> (kernel-name filters, what one launch is, filters counted in one launch)
_OTHER_SUMMARIES = {
    "decode_n512_h32_d128_bf16_256steps": (("decode_kernel<",), "decode_kernel (one kda_decode_step)"),
    "spec_decode_n512_h32_d128_bf16_k4": (("decode_multi_kernel",),
                                          "one verify-and-commit round (kda_decode_verify + kda_decode_commit)"),
    "output_gate_rows4194304_dv128_bf16": (("output_gate_kernel",), "output_gate_kernel (one kda_output_gate call)"),
    "short_conv_b4_t32768_c4096_w4_bf16": (("short_conv_kernel", "conv_cache_kernel"),
                                           "one kda_short_conv call (sum over its kernels)"),
    "gate_b4_t32768_h32_d128_f32": (("kda::gate_kernel",), "gate_kernel (one kda_gate call)"),
}


def _profile_commands(tag: str, workload: str):
    if workload == "others":
        args = ("--workload prefill_b1_h16_t4096_d128_bf16 --extra-workloads none --no-cpu-baseline")
        kt = f"{args} --steps 2 --warmup 1"
        pmc = f"{args} --steps 2 --warmup 1 --decode-steps 4 --calibration-copy-mib 1024"
        mf = None
    else:
        args = f"--workload {workload} --extra-workloads none --no-cpu-baseline --no-decode"
        kt = f"{args} --steps 20 --warmup 3"
        pmc = f"{args} --steps 2 --warmup 1 --calibration-copy-mib 1024"
        mf = f"{args} --steps 2 --warmup 1"
    d = "$RAW"  # the directory that collects rocprofv3's raw output
    cmds = {
        "kt": f"{_PRE}rocprofv3 --kernel-trace --stats -d {d}/{tag}_kt -o kt --output-format csv -- "
              f"python3 $R/bench.py {kt}",
        "FETCH_SIZE": f"{_PRE}rocprofv3 --pmc FETCH_SIZE --kernel-trace -d {d}/{tag}_FETCH_SIZE -o p "
                      f"--output-format csv -- python3 $R/bench.py {pmc}",
        "WRITE_SIZE": f"{_PRE}rocprofv3 --pmc WRITE_SIZE --kernel-trace -d {d}/{tag}_WRITE_SIZE -o p "
                      f"--output-format csv -- python3 $R/bench.py {pmc}",
    }
    if mf:
        cmds["mfma"] = (f"{_PRE}rocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace -d {d}/{tag}_mfma -o p "
                        f"--output-format csv -- python3 $R/bench.py {mf}")
    return cmds


def _counter_rows(path: str):
    import csv
    per = {}
    rows = list(csv.DictReader(open(path)))
    for r in rows:
        per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return rows, per


def _short_name(k: str) -> str:
    return k.split("(")[0]


def _write_kernel_trace(name, raw_dir, cmd, filters, hsh, out_dir):
    import csv
    rows = list(csv.DictReader(open(os.path.join(raw_dir, "kt_kernel_stats.csv"))))
    out = [f"# {name}: kernel trace summary (rocprofv3 --kernel-trace --stats)", "",
           "Command (repository root = $R, raw rocprofv3 output under $RAW, run on one MI355X):", "", "    " + cmd, "",
           f"kernel_source_hash: {hsh}", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        if any(f in r["Name"] for f in filters):
            out.append(f"| `{_short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                       f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                       f"{float(r['Percentage']):.1f} |")
    open(os.path.join(out_dir, f"{name}_kernel_trace.txt"), "w").write("\n".join(out) + "\n")


def _write_traffic(name, raw_dirs, cmds, filters, launch, hsh, out_dir):
    out = [f"# {name}: HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
           "Commands (repository root = $R, raw rocprofv3 output under $RAW, one counter per run):", ""]
    out += ["    " + c for c in cmds]
    out += ["", "Each counter is scaled by what it reads for the 1 GiB device copy "
                "(`--calibration-copy-mib 1024`)", "that the same command runs before the timed region.", ""]
    total = 0.0
    for c, d in zip(("FETCH_SIZE", "WRITE_SIZE"), raw_dirs):
        rows, per = _counter_rows(os.path.join(d, "p_counter_collection.csv"))
        cal = sorted((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows
                     if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == c
                     and int(r["Grid_Size"]) == 131072)[0][1]
        fac = (1 << 20) / cal
        kind = "reads" if c == "FETCH_SIZE" else "writes"
        out.append(f"{c}: the 1 GiB calibration copy {kind} {cal:.1f} KiB -> scale factor {fac:.4f}")
        for k, cs in per.items():
            if not any(x in k for x in filters):
                continue
            v = cs[c]
            mean = sum(v) / len(v)
            out.append(f"  {_short_name(k)}: {mean:.1f} KiB per dispatch (mean of {len(v)}) -> "
                       f"{mean * 1024 * fac / 1e6:.2f} MB")
            total += mean * 1024 * fac
    out += ["", f"launch: {launch}", f"kernel_source_hash: {hsh}", f"traffic_bytes_per_launch: {total:.6e}"]
    open(os.path.join(out_dir, f"{name}_traffic.txt"), "w").write("\n".join(out) + "\n")
    return total


def _write_mfma(name, raw_dir, cmd, filters, hsh, out_dir):
    rows, per = _counter_rows(os.path.join(raw_dir, "p_counter_collection.csv"))
    out = [f"# {name}: MFMA counters per launch (rocprofv3 --pmc {MFMA_COUNTERS})", "",
           "Command (repository root = $R, raw rocprofv3 output under $RAW, run on one MI355X):", "", "    " + cmd, "",
           "Executed bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (counts masked tile entries and",
           "per-slice work as executed).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs)",
           "/ (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); GRBM_GUI_ACTIVE is summed over the 8 XCDs.", "",
           "| kernel | dispatches | MFMA flops per dispatch | MFMA busy cycles | GUI active cycles (per XCD) | MFMA busy |",
           "|---|---|---|---|---|---|"]
    fl_tot = busy_tot = gui_tot = 0.0
    for k, cs in per.items():
        if not any(x in k for x in filters):
            continue
        mean = lambda c: sum(cs[c]) / len(cs[c])
        mops, busy, gui = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16"), mean("SQ_VALU_MFMA_BUSY_CYCLES"), mean("GRBM_GUI_ACTIVE") / 8
        fl = mops * 512
        out.append(f"| `{_short_name(k)}` | {len(cs['GRBM_GUI_ACTIVE'])} | {fl:.4e} | {busy:.4e} | {gui:.4e} | "
                   f"{busy / (gui * 1024):.4f} |")
        fl_tot += fl
        busy_tot += busy
        gui_tot += gui
    out += ["", "launch: one kda_prefill_fwd call (sum over its kernels)", f"kernel_source_hash: {hsh}",
            f"executed_bf16_flops_per_launch: {fl_tot:.6e}",
            f"mfma_busy_frac_per_launch: {busy_tot / (gui_tot * 1024):.6f}"]
    open(os.path.join(out_dir, f"{name}_mfma.txt"), "w").write("\n".join(out) + "\n")


def summarize_profiles(raw: str, out_dir: str = None):
    """Write profiles/*.txt from the rocprofv3 runs under `raw` (layout above); every run
    present is summarised, runs that are missing are skipped."""
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    from linear_attention_sequence_chunkwise_amd import workloads
    done = []
    for w in (workloads.PREFILL_VARLEN, workloads.PREFILL_B4, workloads.PREFILL_B1):
        hsh = kernel_source_hash(summary_sources(w))
        cmds = _profile_commands(w, w)
        d = lambda k: os.path.join(raw, f"{w}_{k}")
        if os.path.isdir(d("kt")):
            _write_kernel_trace(w, d("kt"), cmds["kt"], _PREFILL_KERNELS, hsh, out_dir)
            done.append(f"{w}_kernel_trace")
        if os.path.isdir(d("FETCH_SIZE")) and os.path.isdir(d("WRITE_SIZE")):
            _write_traffic(w, [d("FETCH_SIZE"), d("WRITE_SIZE")], [cmds["FETCH_SIZE"], cmds["WRITE_SIZE"]],
                           _PREFILL_KERNELS, "one kda_prefill_fwd call (sum over its kernels)", hsh, out_dir)
            done.append(f"{w}_traffic")
        if os.path.isdir(d("mfma")):
            _write_mfma(w, d("mfma"), cmds["mfma"], _PREFILL_KERNELS, hsh, out_dir)
            done.append(f"{w}_mfma")
    cmds = _profile_commands("others", "others")
    d = lambda k: os.path.join(raw, f"others_{k}")
    for name, (filters, launch) in _OTHER_SUMMARIES.items():
        hsh = kernel_source_hash(summary_sources(name))
        if os.path.isdir(d("kt")):
            _write_kernel_trace(name, d("kt"), cmds["kt"], filters, hsh, out_dir)
            done.append(f"{name}_kernel_trace")
        if os.path.isdir(d("FETCH_SIZE")) and os.path.isdir(d("WRITE_SIZE")):
            _write_traffic(name, [d("FETCH_SIZE"), d("WRITE_SIZE")], [cmds["FETCH_SIZE"], cmds["WRITE_SIZE"]],
                           filters, launch, hsh, out_dir)
            done.append(f"{name}_traffic")
    return done


def cpu_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(inp, budget_s: float = 20.0, min_s: float = 10.0):
    """The oracle, untuned, on the host cores over a bounded sample of the same workload: the
    first whole sequences (all heads) up to about budget_s of estimated CPU time, converted to
    the oracle's fp32 inputs before the clock starts; one oracle call over them is timed.  A
    sample that finishes much sooner (a small workload run whole) is repeated until about
    min_s, so the rate is not a timing of a fraction of a second."""
    import oracle
    orc = oracle.load()
    threads = cpu_threads()
    cu = inp.cu_seqlens.numpy().astype(np.int64)
    f = lambda t: np.ascontiguousarray(t.float().numpy())
    # rate probe: one (sequence, head) pair on one thread
    n0 = next(n for n in range(inp.N) if cu[n + 1] > cu[n])
    s0, e0 = int(cu[n0]), int(cu[n0 + 1])
    probe = [f(inp.q[s0:e0, :1]), f(inp.k[s0:e0, :1]), f(inp.v[s0:e0, :1]), f(inp.beta[s0:e0, :1])]
    t0 = time.perf_counter()
    orc.prefill(*probe, z=inp.z[s0:e0, :1].numpy(), A=inp.A[:1].numpy(), n_threads=1,
                want_state=False)
    per_tok_head = max(time.perf_counter() - t0, 1e-6) / (e0 - s0)
    # whole sequences while the estimate stays within the budget (at least one)
    m = 0
    est = 0.0
    while m < inp.N:
        add = (cu[m + 1] - cu[m]) * inp.H * per_tok_head / threads
        if m > 0 and est + add > budget_s:
            break
        est += add
        m += 1
    end = int(cu[m])
    args = [f(inp.q[:end]), f(inp.k[:end]), f(inp.v[:end]), f(inp.beta[:end])]
    z = np.ascontiguousarray(inp.z[:end].numpy())
    A = np.ascontiguousarray(inp.A.numpy())
    S0 = None if inp.S0 is None else np.ascontiguousarray(inp.S0[:m].numpy())
    cus = np.ascontiguousarray(cu[:m + 1].astype(np.int32))
    reps = int(min(1000, max(1, min_s // max(est, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        orc.prefill(*args, z=z, A=A, S0=S0, cu_seqlens=cus, n_threads=threads, want_state=False)
    secs = time.perf_counter() - t0
    tok_heads = reps * end * inp.H
    tokens_per_s = tok_heads / secs / inp.H   # sequence tokens/s over all H heads
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {m} of {inp.N} sequences, all {inp.H} heads ({m * inp.H} of "
                      f"{inp.N * inp.H} (sequence, head) pairs, {end} of {inp.total} tokens) of "
                      f"the same workload"
                      + (f", run {reps} times" if reps > 1 else "")
                      + f": {tok_heads} token-heads in {secs:.2f} s; fp64 token recurrence, "
                        f"inputs converted before timing"}


def bench_prefill(name: str, steps: int, warmup: int, checkpoint_interval: int = 0) -> dict:
    """Times `steps` back-to-back kda_prefill_fwd calls on the named workload, inputs resident
    in HBM.  Returns the rate over the whole timed region (wall clock, bracketed by device
    synchronisations), the per-call durations from HIP events recorded between the calls on
    the launch stream, and the roofline of one call."""
    import torch
    from linear_attention_sequence_chunkwise_amd import kda, workloads

    inp = workloads.make(name)
    dev = lambda t: None if t is None else t.cuda()
    q, k, v, beta, z, A = map(dev, (inp.q, inp.k, inp.v, inp.beta, inp.z, inp.A))
    s0 = dev(inp.S0)
    cu = None if inp.equal_length else dev(inp.cu_seqlens)
    want_final = name in (workloads.PREFILL_B4, workloads.PREFILL_VARLEN)
    sN = torch.empty((inp.N, inp.H, inp.dk, inp.dv), dtype=torch.float32, device="cuda") \
        if want_final else None
    o = torch.empty((inp.total, inp.H, inp.dv), dtype=q.dtype, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_size(inp.total, inp.N, inp.H, inp.dk, inp.dv, q.dtype),
                     dtype=torch.uint8, device="cuda")

    ck = ck_off = None
    if checkpoint_interval > 0:
        counts = [L // checkpoint_interval for L in inp.lengths]
        offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        ck = torch.empty((max(1, int(offs[-1])), inp.H, inp.dk, inp.dv), dtype=torch.float32,
                         device="cuda")
        ck_off = torch.from_numpy(offs).cuda() if cu is not None else None

    def step():
        kda.kda_prefill_fwd(q, k, v, beta, z, A, initial_state=s0, final_state=sN,
                            cu_seqlens=cu, n_seqs=None if cu is not None else inp.N, o=o,
                            workspace=ws, checkpoints=ck, checkpoint_offsets=ck_off,
                            checkpoint_interval=checkpoint_interval)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    calls = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])  # ms, per call
    ms_avg = float(calls.mean())
    ms_med = float(np.median(calls))
    ms_per_step = wall * 1e3 / steps

    elem = 2 if inp.dtype == "bf16" else 4
    fl, by = prefill_algorithmic(inp.dk, inp.dv, elem)
    tok_heads = inp.total * inp.H
    state_bytes = (0 if s0 is None else s0.numel() * 4) + (0 if sN is None else sN.numel() * 4) \
        + (0 if ck is None else ck.numel() * 4)
    alg_bytes = by * tok_heads + state_bytes
    achieved = alg_bytes / (ms_avg * 1e-3) / 1e9
    mfma_tflops = fl * tok_heads / (ms_avg * 1e-3) / 1e12
    mf = read_mfma(name)
    if mf is not None:
        mf["executed_tflops"] = mf["executed_bf16_flops_per_launch"] / (ms_avg * 1e-3) / 1e12
    warm = inp.total * inp.H * by < 192e6
    return {
        "inp": inp,
        "tokens_per_s": inp.total / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "median_call_ms": ms_med,
        "config": {"workload": name, "sequences": inp.N, "total_tokens": inp.total,
                   "heads": inp.H, "dk": inp.dk, "dv": inp.dv, "chunk": CHUNK,
                   "initial_state": s0 is not None, "final_state": sN is not None,
                   "workspace_bytes": int(ws.numel()),
                   "checkpoint_interval": checkpoint_interval or None,
                   "checkpoint_bytes": 0 if ck is None else int(ck.numel() * 4),
                   "cache": ("warm: back-to-back calls; inputs, outputs and factor blocks fit "
                             "the 256 MB last-level cache") if warm else
                            "back-to-back calls; the working set is many times the 256 MB "
                            "last-level cache"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": read_traffic(name),
                     "kernel": "kda_prefill_fwd (one call: chunk table, intra-chunk and "
                               "state-pass kernels)", "avg_launch_ms": ms_avg,
                     "median_launch_ms": ms_med, "min_launch_ms": float(calls.min()),
                     "max_launch_ms": float(calls.max()), "timed_calls": steps,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "mfma_util": {"useful_tflops": mfma_tflops, "peak_tflops": BF16_PEAK_TFLOPS,
                      "frac": mfma_tflops / BF16_PEAK_TFLOPS,
                      "useful_flops_per_token_head": fl, "rocprof": mf},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="headline prefill workload (default: the varlen batch of 64 sequences)")
    ap.add_argument("--extra-workloads", default=None,
                    help="comma-separated prefill workloads timed after the headline one and "
                         "reported under 'prefill_other' (default: the batched and the "
                         "single-sequence workloads; 'none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--checkpoint-interval", type=int, default=0,
                    help="also write prefix-cache checkpoints every this many tokens "
                         "(kda_prefill_fwd_checkpointed; 0 = off)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB before the timed "
                         "region (a known-size reference for HBM traffic counters)")
    ap.add_argument("--summarize-profiles", metavar="RAW_DIR", default=None,
                    help="write profiles/*.txt from the rocprofv3 runs under RAW_DIR and exit "
                         "(no GPU needed)")
    args = ap.parse_args()

    if args.summarize_profiles:
        for name in summarize_profiles(args.summarize_profiles):
            print(name)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one MI355X only; --gpus above 1 is not supported "
              "(the (sequence, head) chains would shard across GPUs with no communication, "
              "and each GPU would run this single-GPU path on its share).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_sequence_chunkwise_amd import kda, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kda.load_library()
    if args.calibration_copy_mib > 0:
        src = torch.ones(args.calibration_copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    name = args.workload or workloads.PREFILL_VARLEN
    head = bench_prefill(name, args.steps, args.warmup, args.checkpoint_interval)
    inp = head.pop("inp")
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic, seeded (q,k ~N(0,1) L2-normalised per head, q/sqrt(dk); v ~N(0,1); "
                "beta=Sigmoid(N(0,1)); z ~N(0,1); A ~N(0,0.5)"
                + ("; initial states ~N(0,0.02)" if inp.S0 is not None else "") + ")",
        "config": head["config"],
        "median_call_ms": head["median_call_ms"],
        "roofline": head["roofline"],
        "mfma_util": head["mfma_util"],
    }

    extra = args.extra_workloads
    if extra is None:
        extra = ",".join(w for w in (workloads.PREFILL_B4, workloads.PREFILL_B1) if w != name)
    others = {}
    for w in [x for x in extra.split(",") if x and x != "none"]:
        r = bench_prefill(w, args.steps, args.warmup)
        r.pop("inp")
        torch.cuda.empty_cache()
        others[w] = r
    if others:
        out["prefill_other"] = others

    if not args.no_decode:
        out["decode"] = bench_decode(args.decode_steps)
        out["spec_decode"] = bench_spec_decode()
        out["output_gate"] = bench_output_gate()
        out["short_conv"] = bench_short_conv()
        out["gate"] = bench_gate()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


def bench_decode(n_steps: int, distinct: int = 32, repeats: int = 3):
    """256 consecutive decode steps (512 sequences x 32 heads, d = 128, bf16 inputs, fp32
    state in place).  `distinct` step inputs are generated and cycled (each 21 MB, so a
    cycle exceeds the 256 MB last-level cache); the state is restored between repeats
    outside the timed region."""
    import torch
    from linear_attention_sequence_chunkwise_amd import kda, workloads
    d = workloads.decode_inputs(N=512, H=32, dk=128, dv=128, steps=distinct, dtype="bf16",
                                seed=4, name=workloads.DECODE)
    q, k, v, beta, z = (t.cuda() for t in (d.q, d.k, d.v, d.beta, d.z))
    A = d.A.cuda()
    s_init = d.S0.cuda()
    state = s_init.clone()
    o = torch.empty((d.N, d.H, d.dv), dtype=torch.bfloat16, device="cuda")

    def run():
        for t in range(n_steps):
            j = t % distinct
            kda.kda_decode_step(q[j], k[j], v[j], beta[j], z[j], A, state, o=o)

    run()  # warm-up
    times = []
    for _ in range(repeats):
        state.copy_(s_init)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    t = float(np.median(times))
    per_step = t / n_steps
    byts = decode_bytes_per_pair(d.dk, d.dv, 2) * d.N * d.H
    gbps = byts / per_step / 1e9
    return {"workload": workloads.DECODE, "steps": n_steps, "tokens_per_s": d.N * n_steps / t,
            "us_per_step": per_step * 1e6, "hbm_GBps": gbps,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS, "traffic": read_traffic(workloads.DECODE),
                         "kernel": "decode_kernel", "algorithmic_bytes_per_launch": byts},
            "inputs": f"{distinct} distinct seeded steps cycled"}


def bench_spec_decode(K: int = 4, rounds: int = 32, repeats: int = 3):
    """Speculative decode rounds over 512 sequences x 32 heads (d = 128, bf16): each round is
    one kda_decode_verify of K draft tokens from the committed state plus one
    kda_decode_commit of all K (full acceptance), so a round yields K tokens per sequence.
    The state is read once by verify and read and written once by commit (3 x 1 GiB per
    round) instead of 2 x 1 GiB per token.  `rounds` distinct seeded rounds are cycled."""
    import torch
    from linear_attention_sequence_chunkwise_amd import kda, workloads
    d = workloads.decode_inputs(N=512, H=32, dk=128, dv=128, steps=K * 8, dtype="bf16", seed=5,
                                name="spec_decode_n512_h32_d128_bf16")
    nk = lambda x: x.reshape(8, K, *x.shape[1:]).transpose(1, 2).contiguous().cuda()  # [8,N,K,..]
    q, k, v, beta, z = (nk(t) for t in (d.q, d.k, d.v, d.beta, d.z))
    A = d.A.cuda()
    s_init = d.S0.cuda()
    state = s_init.clone()
    acc = torch.full((d.N,), K, dtype=torch.int32, device="cuda")
    o = torch.empty((d.N, K, d.H, d.dv), dtype=torch.bfloat16, device="cuda")

    def run():
        for r in range(rounds):
            j = r % 8
            kda.kda_decode_verify(q[j], k[j], v[j], beta[j], z[j], A, state, o=o)
            kda.kda_decode_commit(k[j], v[j], beta[j], z[j], A, state, acc)

    run()
    times = []
    for _ in range(repeats):
        state.copy_(s_init)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    t = float(np.median(times)) / rounds
    pairs = d.N * d.H
    state = 128 * 128 * 4
    verify = state + K * (3 * 128 * 2 + 2 + 128 * 4) + K * 128 * 2   # q,k,v,beta,z in; o out
    commit = 2 * state + K * (2 * 128 * 2 + 2 + 128 * 4)              # k,v,beta,z in
    byts = pairs * (verify + commit)
    gbps = byts / t / 1e9
    return {"workload": "spec_decode_n512_h32_d128_bf16_k%d" % K, "draft_tokens": K,
            "us_per_round": t * 1e6, "tokens_per_s": d.N * K / t, "hbm_GBps": gbps,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": read_traffic("spec_decode_n512_h32_d128_bf16_k%d" % K),
                         "kernel": "decode_multi_kernel (verify + commit)",
                         "algorithmic_bytes_per_launch": byts},
            "inputs": "8 distinct seeded rounds cycled; full acceptance"}


def bench_output_gate(repeats: int = 10):
    """Fused epilogue y = Sigmoid(gate) * RMSNorm(o) over the readout of the batched prefill
    workload (4 x 32768 tokens x 32 heads, d_v = 128, bf16): 3 x 1.07 GB moved."""
    import torch
    from linear_attention_sequence_chunkwise_amd import kda
    rows, dv = 4 * 32768 * 32, 128
    g = torch.Generator(device="cuda").manual_seed(6)
    o = (torch.randn(rows, dv, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    gate = torch.randn(rows, dv, device="cuda", generator=g).to(torch.bfloat16)
    w = torch.ones(dv, device="cuda")
    y = torch.empty_like(o)
    kda.kda_output_gate(o, gate, w, y=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(repeats):
        kda.kda_output_gate(o, gate, w, y=y)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / repeats
    byts = 3 * rows * dv * 2 + dv * 4
    gbps = byts / t / 1e9
    del o, gate, y
    return {"workload": "output_gate_rows4194304_dv128_bf16", "us_per_call": t * 1e6,
            "hbm_GBps": gbps,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": read_traffic("output_gate_rows4194304_dv128_bf16"),
                         "kernel": "output_gate_kernel", "algorithmic_bytes_per_launch": byts}}


def bench_short_conv(repeats: int = 10):
    """Input prologue y = L2Norm(Swish(ShortConv(x))) (width 4, per-head L2Norm) over the
    q branch of the batched prefill workload: 4 x 32768 tokens x 32 heads x 128 channels,
    bf16, with caches in and out: 2 x 1.07 GB moved."""
    import torch
    from linear_attention_sequence_chunkwise_amd import kda
    N, T, C, width = 4, 32768, 32 * 128, 4
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(N * T, C, device="cuda", generator=g).to(torch.bfloat16)
    w = torch.randn(C, width, device="cuda", generator=g) * 0.5
    cache = torch.zeros(N, C, width - 1, device="cuda")
    cache_out = torch.empty_like(cache)
    y = torch.empty_like(x)
    run = lambda: kda.kda_short_conv(x, w, cache_in=cache, cache_out=cache_out, n_seqs=N,
                                     l2_group=128, y=y)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(repeats):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / repeats
    byts = 2 * N * T * C * 2 + C * width * 4 + 2 * cache.numel() * 4
    gbps = byts / t / 1e9
    del x, y
    return {"workload": "short_conv_b4_t32768_c4096_w4_bf16", "us_per_call": t * 1e6,
            "hbm_GBps": gbps,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": read_traffic("short_conv_b4_t32768_c4096_w4_bf16"),
                         "kernel": "short_conv_kernel", "algorithmic_bytes_per_launch": byts}}


def bench_gate(repeats: int = 10):
    """Standalone gate g = g_min*Sigmoid(e^A z) with its chunk-local cumulative sum, over the
    batched prefill workload's z: 4 x 32768 tokens x 32 heads x 128 channels, fp32 in, g and
    gcum fp32 out: 3 x 2.15 GB moved."""
    import torch
    from linear_attention_sequence_chunkwise_amd import kda
    N, T, H, dk = 4, 32768, 32, 128
    g = torch.Generator(device="cuda").manual_seed(11)
    z = torch.randn(N * T, H, dk, device="cuda", generator=g)
    A = torch.randn(H, dk, device="cuda", generator=g) * 0.5
    gv, gc = torch.empty_like(z), torch.empty_like(z)
    run = lambda: kda.kda_gate(z, A, g=gv, gcum=gc, n_seqs=N)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(repeats):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / repeats
    byts = 3 * z.numel() * 4 + A.numel() * 4
    gbps = byts / t / 1e9
    del z, gv, gc
    return {"workload": "gate_b4_t32768_h32_d128_f32", "us_per_call": t * 1e6,
            "hbm_GBps": gbps,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         "traffic": read_traffic("gate_b4_t32768_h32_d128_f32"),
                         "kernel": "gate_kernel", "algorithmic_bytes_per_launch": byts}}


if __name__ == "__main__":
    main()
