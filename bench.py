"""Paged-attention decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole decode hot path over one batch: pa_cache_write
of the B*Tq new tokens' K/V rows, the split-K decode kernel, and (when there
is more than one partition) the log-sum-exp reduce. Inputs are synthetic and
seeded (workloads.generate) and already resident in HBM when timing starts.
Untimed steps run for --settle-ms (the GPU's clock ramp from idle), then W
warm-up steps. The metric times K eager steps between two device
synchronisations (the host enqueues ahead of the GPU, so this is the GPU's
sustained step throughput); a second pass of K eager steps with HIP events
between the kernels gives the per-kernel breakdown, and K back-to-back
launches of the decode alone its roofline. Replays of the step recorded in a
HIP graph (as decode runs in serving), one and ten steps per graph, are timed
too and reported beside it: each graph launch idles the GPU for a few
microseconds, which ten steps share.
--sparse-top N times the sparse block-selection step instead, and
--graph-interleave R alternates the eager and graph forms (no metric line).
Default workload: long-context decode at 64K tokens per sequence (B=4,
Hq=24, Hkv=4, D=256, bf16 KV).
With --shared-prefix (workloads whose sequences share a prefix) the decode
of a step is one pa_decode_shared_prefix call: a pass over the shared blocks
for the whole batch, a pass over each sequence's own tokens, and their merge.

Printed: ONE JSON line with the metric (algorithmic KV-read GB/s), the step
time, a roofline object for the decode kernel (its algorithmic bytes per
launch over its average launch time, measured with HIP events on the launch
stream) and a CPU baseline (the fp64 oracle timed on this host on a bounded
sample of the same workload). The device's streaming-read ceiling (a 2 GiB
buffer read once per launch with the decode kernels' loads, pa_read_probe) is
measured after the metric and reported beside the vendor peak: the step's
GB/s and the decode's roofline as fractions of both.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "paged-attn decode KV-read GB/s (% of HBM peak) and µs/step at 64K ctx"
DEFAULT_WORKLOAD = "long64k_bf16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w) -> dict:
    """Bytes the method must move per decode step (the split-K workspace is
    implementation overhead and is reported apart)."""
    sp = w.spec
    qelt = 4 if sp.q_dtype == "f32" else 2
    L = w.seq_lens.astype(np.int64)
    if sp.cache_dtype == "nvfp4":  # E2M1 codes and E4M3 block scales (row padding excluded)
        kv = int(L.sum()) * sp.Hkv * 2 * (sp.D // 2 + sp.D // 16)
    else:
        kv = int(L.sum()) * sp.Hkv * sp.D * 2 * {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1}[sp.cache_dtype]
    scales = int(L.sum()) * sp.Hkv * 2 * 4 if sp.cache_dtype in ("i8", "fp8", "nvfp4") else 0
    table = int(((L + 15) // 16).sum()) * 4
    q = sp.B * sp.Tq * sp.Hq * sp.D * qelt
    out = sp.B * sp.Tq * sp.Hq * (sp.D + 1) * 4
    return {"kv": kv, "scales": scales, "table": table, "q": q, "out": out,
            "total": kv + scales + table + q + out}


def algorithmic_flops(w) -> int:
    """Multiply-adds of the attention itself, counted as 2 flops each: QK and
    PV take 2 D each per (query row, visible key), 4 D in all; query token t
    of sequence b sees L_b - Tq + t + 1 keys (the causal rule counted
    exactly, not bounded by L_b)."""
    sp = w.spec
    keys = 0
    for L in w.seq_lens.astype(np.int64):
        for t in range(sp.Tq):
            keys += max(0, int(L) - sp.Tq + t + 1)
    return 4 * sp.D * sp.Hq * keys


_COMMON = ("pa_device.hpp", "pa_internal.hpp")


def unique_bytes(w) -> int:
    """Algorithmic bytes when the shared prefix is read once for the batch
    (the shared-prefix decode): the prefix's tokens once, every sequence's own
    tokens, plus the same table, q and out terms."""
    sp = w.spec
    ab = algorithmic_bytes(w)
    per_tok = ab["kv"] // int(w.seq_lens.astype(np.int64).sum()) + ab["scales"] // int(w.seq_lens.sum())
    return ab["total"] - (sp.B - 1) * sp.shared_prefix * per_tok


_KERNEL_SOURCES = {"decode_valu_kernel": "decode_valu.hip", "decode_mfma_kernel": "decode_mfma.hip",
                   "decode_wave_kernel": "decode_wave.hip", "decode_stream_kernel": "decode_stream.hip"}
_CODES = {"f32": 0, "bf16": 1, "i8": 2, "fp8": 3, "nvfp4": 4}


def decode_kernel(spec) -> tuple:
    """(name, sources) of the decode kernel that runs the workload, as the
    library itself chooses it (pa_decode_kernel_name)."""
    import paged_attention_decode_02_amd as pa

    name = pa.load().pa_decode_kernel_name(spec.Tq, spec.Hq, spec.Hkv, _CODES[spec.cache_dtype]).decode()
    return name, (_KERNEL_SOURCES[name],) + _COMMON


_SHARED_SOURCES = ("decode_mfma.hip", "decode_wave.hip", "splitk_reduce.hip") + _COMMON


def kernel_source_digest(spec, shared: bool = False) -> str:
    """Digest of the decode kernel's sources (ties committed counters to code);
    shared: the kernels of a pa_decode_shared_prefix call."""
    h = hashlib.sha256()
    for f in (_SHARED_SOURCES if shared else decode_kernel(spec)[1]):
        p = os.path.join(ROOT, "paged_attention_decode_02_amd", "csrc", f)
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(spec, shared: bool = False):
    """Per-launch HBM bytes (read + write) from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", "decode_%s%s_hbm_traffic.md" % (spec.name, "_shared" if shared else ""))
    if not os.path.exists(p):
        return None
    text = open(p).read()
    m = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not m or not t or m.group(1) != kernel_source_digest(spec, shared):
        return None
    return int(t.group(1))


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, copy_bytes: int, shared: bool = False) -> str:
    """Markdown summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE).

    Both counters are in KiB per dispatch. Each is scaled by what it reads for
    the plain device copy of copy_bytes bytes that the run also made (the
    largest __amd_rocclr_copyBuffer dispatch), so the figures are bytes.
    """
    import csv
    import collections

    from workloads import SPECS, generate

    def load(path, counter):
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return per

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy_f = max(v for k, vs in fetch.items() if "copyBuffer" in k for v in vs)
    copy_w = max(v for k, vs in write.items() if "copyBuffer" in k for v in vs)
    kib = copy_bytes / 1024.0
    ff, fw = kib / copy_f, kib / copy_w
    spec = SPECS[workload]
    kname = decode_kernel(spec)[0]
    if shared:
        # the pa_decode_shared_prefix call: both decode passes and the merge,
        # each kernel's mean per dispatch (one dispatch of each per call)
        dk = sorted(k for k in fetch if "decode_" in k or "splitk_reduce" in k)
        assert 2 <= len(dk) <= 3, dk
        kname = "pa_decode_shared_prefix (%s)" % ", ".join(k.replace("void ", "").split("(")[0] for k in dk)
    else:
        dk = [k for k in fetch if kname in k]
        assert len(dk) == 1, dk
    f_kib = sum(sum(fetch[k]) / len(fetch[k]) for k in dk)
    w_kib = sum(sum(write[k]) / len(write[k]) for k in dk)
    read_b = int(round(f_kib * ff * 1024))
    write_b = int(round(w_kib * fw * 1024))
    w = generate(spec)
    algo = unique_bytes(w) if shared else algorithmic_bytes(w)["total"]
    extra = " --shared-prefix" if shared else ""
    lines = [
        "# HBM traffic of %s on %s" % (kname, workload), "",
        "Counters from two rocprofv3 runs (one MI355X, repository root as the working directory):", "",
    ] + [
        # the output directory is the one the counter file sits in
        "    rocprofv3 --pmc %s --output-format csv -d %s -o run -- python -u bench.py "
        "--workload %s%s --steps 5 --warmup 1 --no-cpu-baseline --copy-calibration-mb %d" % (
            c, os.path.relpath(os.path.dirname(os.path.abspath(path))), workload, extra, copy_bytes >> 20)
        for c, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))
    ] + [
        "",
        "Both counters are KiB per dispatch; each is scaled by what it reads for a plain device copy of",
        "%d MiB made in the same run (the largest copy dispatch)." % (copy_bytes >> 20), "",
        "| quantity | value |", "|---|---|",
        "| copy kernel (%d MiB) FETCH_SIZE / WRITE_SIZE, KiB | %.1f / %.1f |" % (copy_bytes >> 20, copy_f, copy_w),
        "| scale factors (bytes per counted byte), read / write | %.4f / %.4f |" % (ff, fw),
        "| decode FETCH_SIZE / WRITE_SIZE per %s, KiB (mean of %d) | %.1f / %.1f |" % (
            "call" if shared else "dispatch", len(fetch[dk[0]]), f_kib, w_kib),
        "| decode HBM read / write per %s, bytes (scaled) | %d / %d |" % ("call" if shared else "launch", read_b,
                                                                        write_b),
        "| algorithmic bytes per %s | %d |" % ("call (shared prefix once)" if shared else "launch", algo),
        "| traffic / algorithmic | %.4f |" % ((read_b + write_b) / algo), "",
        "hbm_bytes_per_launch: %d" % (read_b + write_b),
        "kernel_source_digest: %s" % kernel_source_digest(spec, shared), "",
    ]
    return "\n".join(lines)


def summarize_trace(trace_csv: str, workload: str, command: str, tail_cold: int = 20, shared: bool = False) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace CSV of one bench.py run.

    Per kernel: dispatch count and mean / median / min / max duration. The last
    tail_cold dispatches of each library kernel are the bench's cache-flushed
    side steps; the decode kernel is also summarised without them (the
    launches the bench's roofline figure covers).
    """
    import csv
    import collections

    dur = collections.defaultdict(list)
    for r in sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"])):
        dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    total = sum(sum(v) for v in dur.values())

    def short(k):
        if k.startswith("void pa::") or k.startswith("pa::"):
            return k.replace("void ", "").split("(")[0]
        if "copyBuffer" in k:
            return "device copy (bench set-up)"
        return "torch kernel (bench set-up, cache flush): " + k.split("<")[0].replace("void ", "")[:48]

    spec_kernel = decode_kernel(__import__("workloads").SPECS[workload])[0]
    lines = [
        "# Kernel durations of bench.py on %s" % workload, "",
        "Command (one MI355X, repository root as the working directory):", "",
        "    " + command, "",
        "Durations in microseconds from `%s` (kernel begin/end timestamps)." % os.path.basename(trace_csv), "",
        "| kernel | dispatches | mean | median | min | max | share of GPU time |",
        "|---|---:|---:|---:|---:|---:|---:|",
    ]
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(v)
        lines.append("| %s | %d | %.2f | %.2f | %.2f | %.2f | %.1f%% |" % (
            short(k), len(a), a.mean(), np.median(a), a.min(), a.max(), 100.0 * a.sum() / total))
    if shared:
        # one pa_decode_shared_prefix call per step: both passes and the merge
        parts = sorted(k for k in dur if "decode_" in k or "splitk_reduce" in k)
        means = [float(np.mean(dur[k][:-tail_cold])) for k in parts]
        lines += ["", "Without the last %d dispatches of each (the cache-flushed side steps), one "
                  "pa_decode_shared_prefix call:" % tail_cold, "",
                  "| kernel of the call | mean |", "|---|---:|"]
        lines += ["| %s | %.2f |" % (short(k), m) for k, m in zip(parts, means)]
        lines += ["", "shared_prefix_call_mean_us: %.2f" % sum(means), ""]
        return "\n".join(lines)
    dk = [k for k in dur if spec_kernel in k]
    if len(dk) == 1 and len(dur[dk[0]]) > tail_cold:
        a = np.array(dur[dk[0]][:-tail_cold])
        lines += [
            "",
            "Without its last %d dispatches (the cache-flushed side steps), %s: %d dispatches, mean %.2f, "
            "median %.2f, min %.2f, max %.2f." % (tail_cold, short(dk[0]), len(a), a.mean(), np.median(a),
                                                  a.min(), a.max()),
            "",
            "decode_mean_us_warm: %.2f" % a.mean(),
        ]
        # the decode dispatches by bench phase: W warm-up steps, K eager steps
        # (the metric), K eager steps with events between the kernels, K
        # back-to-back decode launches (the roofline), one eager step, W + K
        # one-step graph replays, ten-step graph replays (one warm, K / 10
        # timed), one eager check step, then the cache-flushed steps. The
        # clock-settle steps before the warm-up vary in number, so the
        # phases are placed from the end of the trace.
        m_steps = re.search(r"--steps (\d+)", command)
        m_warm = re.search(r"--warmup (\d+)", command)
        if m_steps and m_warm:
            K, W = int(m_steps.group(1)), int(m_warm.group(1))
            d = np.array(dur[dk[0]])
            graph = "--no-graph" not in command
            n_after = W + 3 * K + 1 + (W + K + 10 + 10 * max(1, K // 10) + 1 if graph else 0) + min(20, K)
            o = len(d) - n_after  # settle steps
            g0 = o + W + 3 * K + 1 + W
            phases = [("eager steps (the metric's timed region)", o + W, o + W + K),
                      ("eager steps with events between the kernels", o + W + K, o + W + 2 * K),
                      ("back-to-back decode launches (the roofline's launches)", o + W + 2 * K, o + W + 3 * K)]
            if graph:
                phases.append(("graph replays, one step per graph", g0, g0 + K))
                phases.append(("graph replays, ten steps per graph", g0 + K + 10, g0 + K + 10 + 10 * max(1, K // 10)))
            if o >= 0:
                lines += ["", "%d clock-settle steps before the warm-up." % o, "",
                          "| decode dispatches by phase | dispatches | mean | median |", "|---|---:|---:|---:|"]
                for name, i0, i1 in phases:
                    x = d[i0:i1]
                    lines.append("| %s | %d | %.2f | %.2f |" % (name, len(x), x.mean(), np.median(x)))
                lines += ["", "decode_mean_us_roofline_launches: %.2f" % d[o + W + 2 * K:o + W + 3 * K].mean()]
    lines.append("")
    return "\n".join(lines)


def summarize_sq(runs, workload: str) -> str:
    """Markdown table of SQ counters per decode dispatch, from one or more
    (label, kernel-name substring, counter CSV, command) runs; counts are
    normalised per 16-token block and kv head of the workload."""
    import csv
    import collections

    from workloads import SPECS, generate

    w = generate(SPECS[workload])
    blocks = int(((w.seq_lens.astype(np.int64) + 15) // 16).sum()) * w.spec.Hkv
    names = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
             "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
             "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT"]
    cols = []
    cmds = []
    for label, kname, paths, cmd in runs:
        vals = collections.defaultdict(list)
        for path in paths:
            for r in csv.DictReader(open(path)):
                if kname in r["Kernel_Name"]:
                    vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
        cols.append((label, {k: sum(v) / len(v) for k, v in vals.items()}))
        cmds += ["    " + c for c in cmd]
    lines = ["# SQ counters of the decode kernel on %s" % workload, "",
             "Counters per decode dispatch (mean over the dispatches of each run), from rocprofv3 runs of at most",
             "8 SQ counters each (one MI355X, repository root as the working directory):", ""] + cmds + [
             "", "Per block: divided by the workload's %d (16-token block, kv head) pairs. Wave-cycle counters "
             "count in units of 4 cycles." % blocks, "",
             "| counter | " + " | ".join("%s: per dispatch | per block" % c[0] for c in cols) + " |",
             "|---|" + "---:|---:|" * len(cols)]
    for n in names:
        row = []
        for _, v in cols:
            x = v.get(n)
            row += ["—", "—"] if x is None else ["%.0f" % x, "%.1f" % (x / blocks)]
        lines.append("| %s | %s |" % (n, " | ".join(row)))
    for label, v in cols:
        if v.get("SQ_WAVE_CYCLES") and v.get("SQ_WAIT_ANY") is not None:
            lines.append("")
            lines.append("%s: waiting %.0f%% of wave time (SQ_WAIT_ANY / SQ_WAVE_CYCLES), VALU active %.0f%%, "
                         "MFMA busy cycles per block %.0f." % (
                             label, 100 * v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"],
                             100 * v.get("SQ_ACTIVE_INST_VALU", 0) / v["SQ_WAVE_CYCLES"],
                             v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / blocks))
    lines.append("")
    return "\n".join(lines)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rows_per_s(w, k, v, ks, vs, threads: int, budget_s: float, tag: str) -> tuple:
    """(rows, seconds) of oracle work on (b, t, h) rows in sequence-major order,
    in chunks of one row per thread, cycling over the step until the budget is
    used (at least one chunk)."""
    import oracle

    sp = w.spec
    rows_total = sp.B * sp.Tq * sp.Hq
    chunk = max(1, min(rows_total, threads))
    done, spent, next_log = 0, 0.0, 1.0
    q = w.q_array()
    while spent < budget_s:
        rows = (np.arange(chunk, dtype=np.int64) + done) % rows_total
        t = time.perf_counter()
        oracle.decode(q, k, v, w.block_table, w.seq_lens, w.softmax_scale, ks, vs, rows=rows, nthreads=threads)
        spent += time.perf_counter() - t
        done += rows.size
        if spent >= next_log:
            log("cpu baseline (%s): %d rows (%.2f steps), %.1f s" % (tag, done, done / rows_total, spent))
            next_log = spent + 1.0
    return done, spent


def run_cpu_baseline(w, bytes_per_step: int, budget_s: float, budget_1t_s: float) -> dict:
    import oracle
    from workloads import BLOCK_SIZE

    sp = w.spec
    t0 = time.time()
    k, v, ks, vs = oracle.alloc_cache(w.num_blocks, BLOCK_SIZE, sp.Hkv, sp.D, sp.cache_dtype)
    oracle.cache_write(w.k_src, w.v_src, w.slot_mapping, k, v, ks, vs)
    log("cpu baseline: oracle cache built in %.1f s" % (time.time() - t0))
    rows_total = sp.B * sp.Tq * sp.Hq
    threads = oracle.max_threads()
    done, spent = _oracle_rows_per_s(w, k, v, ks, vs, threads, budget_s, "%d threads" % threads)
    # the sample covers whole sequences' rows in proportion; scale it to one step
    step_s = spent * rows_total / done
    res = {"value": round(bytes_per_step / step_s / 1e9, 4), "unit": "GB/s", "cores": int(threads),
           "kind": "oracle", "ms_per_step": round(step_s * 1e3, 3), "cpu_model": cpu_model(),
           "sample": "%d (b,t,h) rows of %s (%.2f steps of %d rows) in %.1f s, fp64 oracle, %d OpenMP threads, "
                     "scaled to one step" % (done, sp.name, done / rows_total, rows_total, spent, threads)}
    if budget_1t_s > 0:
        d1, s1 = _oracle_rows_per_s(w, k, v, ks, vs, 1, budget_1t_s, "1 thread")
        step1 = s1 * rows_total / d1
        res["value_1thread"] = round(bytes_per_step / step1 / 1e9, 4)
        res["ms_per_step_1thread"] = round(step1 * 1e3, 3)
        res["sample_1thread"] = "%d rows in %.1f s on one thread, scaled to one step" % (d1, s1)
    return res


def _sysfs_clock(name: str, top: bool = False):
    """Current (or, with top, highest) level in MHz of a DPM clock table in
    sysfs, or None."""
    import glob

    for path in sorted(glob.glob("/sys/class/drm/card*/device/" + name)):
        try:
            levels = []
            for line in open(path):
                m = re.search(r"(\d+)\s*Mhz", line, re.I)
                if m:
                    levels.append(int(m.group(1)))
                    if not top and line.rstrip().endswith("*"):
                        return levels[-1]
            if top and levels:
                return max(levels)
        except OSError:
            continue
    return None


def device_record(pa) -> dict:
    """The device and build the figures were taken on."""
    import torch

    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    info = {}
    bi = os.path.join(os.path.dirname(pa.library_path()), "build_info.json")
    if os.path.exists(bi):
        info = json.load(open(bi))
    return {
        "name": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count, "library_compute_units": pa.device_cu_count(),
        "total_memory_gib": round(props.total_memory / 2**30, 1),
        "sclk_mhz_now": _sysfs_clock("pp_dpm_sclk"), "sclk_mhz_max": _sysfs_clock("pp_dpm_sclk", True),
        "mclk_mhz_now": _sysfs_clock("pp_dpm_mclk"), "mclk_mhz_max": _sysfs_clock("pp_dpm_mclk", True),
        "rocm": rocm, "torch_hip": getattr(torch.version, "hip", None),
        "git_head_at_build": info.get("git_head"), "library_source_digest": info.get("source_digest"),
    }


READ_CEILING_WGS_PER_CU = (8, 32, 64)


def read_ceiling(pa, mib: int, launches: int) -> dict:
    """The device's streaming-read ceiling: pa_read_probe (every byte of a
    mib-MiB buffer read once with the decode kernels' nontemporal 16-byte
    loads) at 8, 32 and 64 workgroups per CU, each launched `launches` times
    back to back between two HIP events on the launch stream; the ceiling is
    the fastest configuration's median launch. The probe's word sums are
    checked against the buffer's first."""
    import torch

    n = mib << 20
    dev = torch.device("cuda:0")
    buf = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    mask = (1 << 32) - 1
    want = int(buf.to(torch.int64).bitwise_and(mask).sum().item()) & mask
    per, ok = {}, True
    for wpc in READ_CEILING_WGS_PER_CU:
        wgs = wpc * pa.device_cu_count()
        sink = torch.zeros(wgs, dtype=torch.int32, device=dev)
        pa.read_probe(buf, sink, stream=stream)
        ok = ok and (int(sink.to(torch.int64).bitwise_and(mask).sum().item()) & mask) == want
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for a, b in ev:
            a.record(stream)
            pa.read_probe(buf, sink, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        per[wpc] = float(np.median([1e3 * a.elapsed_time(b) for a, b in ev]))
    best = min(per, key=per.get)
    gbps = n / (per[best] * 1e-6) / 1e9
    del buf
    return {"gb_per_s": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBS, 4), "bytes": n,
            "launches_per_config": launches, "median_us": round(per[best], 2),
            "median_us_by_workgroups_per_cu": {str(k): round(v, 2) for k, v in per.items()},
            "kernel": "read_probe_kernel: nontemporal 16-byte buffer loads, 4 in flight per thread, "
                      "%d workgroups of 256 per CU" % best,
            "checksum_ok": ok}


def pct(a, q):
    return round(1e3 * float(np.percentile(np.asarray(a), q)), 2)


def sparse_step_bytes(w, sel, SB: int) -> dict:
    """Algorithmic bytes of one sparse step: the mean keys the scores read
    (every block below each length, fp32), the K/V bytes of the selected
    blocks' tokens below each length, the keys the mean refresh re-reads (the
    sparse blocks holding the newest Tq tokens), table entries, q and out."""
    from workloads import kv_bytes_per_token

    sp = w.spec
    per_tok = kv_bytes_per_token(sp) // sp.Hkv  # K + V (+ scales) of one token and kv head
    kv = 0
    for b in range(sp.B):
        L = int(w.seq_lens[b])
        for g in range(sp.Hkv):
            for j in sel[b, g]:
                if j < 0:
                    break
                kv += max(0, min(L, (int(j) + 1) * SB) - int(j) * SB) * per_tok
    nsb = (w.seq_lens.astype(np.int64) + SB - 1) // SB
    mean_read = int(nsb.sum()) * sp.Hkv * sp.D * 4
    refresh = 0
    for b in range(sp.B):
        L = int(w.seq_lens[b])
        if L > 0:
            first = max(L - sp.Tq, 0) // SB
            toks = sum(min(L, (j + 1) * SB) - j * SB for j in range(first, int(nsb[b])))
            refresh += toks * sp.Hkv * (per_tok // 2)
    elt_q = 4 if sp.q_dtype == "f32" else 2
    qo = sp.B * sp.Tq * sp.Hq * sp.D * (elt_q + 4)
    total = kv + mean_read + refresh + qo
    return {"kv_selected": kv, "mean_keys": mean_read, "mean_refresh": refresh, "q_out": qo, "total": total}


INTERLEAVE_FORMS = ("eager_step", "graph_step", "graph_10_steps", "eager_decode", "graph_decode")


def graph_interleave(args, step, dec) -> dict:
    """Graph launches against eager launches, interleaved: each round runs K
    eager steps, K replays of a one-step graph, K / 10 replays of a ten-step
    graph, K eager decodes and K replays of a one-decode graph, each form
    timed between two synchronisations (microseconds per step or decode).
    The three graphs are captured once and replayed once before the rounds,
    so under a kernel trace the decode dispatches follow a fixed layout
    (summarize_interleave)."""
    import torch

    K, R = args.steps, args.graph_interleave
    gs, g10, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs):
        step()
    with torch.cuda.graph(g10):
        for _ in range(10):
            step()
    with torch.cuda.graph(gd):
        dec()
    torch.cuda.synchronize()
    gs.replay()
    g10.replay()
    gd.replay()
    torch.cuda.synchronize()
    forms = {"eager_step": (step, K, 1), "graph_step": (gs.replay, K, 1), "graph_10_steps": (g10.replay, K // 10, 10),
             "eager_decode": (dec, K, 1), "graph_decode": (gd.replay, K, 1)}
    rounds = []
    for _ in range(R):
        rec = {}
        for name in INTERLEAVE_FORMS:
            fn, n, per = forms[name]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            rec[name] = round((time.perf_counter() - t0) * 1e6 / (n * per), 2)
        rounds.append(rec)
        log("interleave round %d: %s" % (len(rounds), rec))
    return {"graph_interleave": {"steps_per_form": K, "rounds": rounds, "unit": "us per step (decode forms: per decode)"}}


def summarize_interleave(trace_csv: str, command: str, K: int, W: int, R: int) -> str:
    """Decode durations and the idle time before each decode, by form and
    round, from a kernel trace of `bench.py --graph-interleave R`."""
    import csv

    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    ks = [(r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
          if r["Kernel_Name"].replace("void ", "").startswith("pa::")]
    dec = [i for i, k in enumerate(ks) if "decode_" in k[0]]
    lines = ["# Graph launches against eager launches, interleaved", "",
             "Command (one MI355X, repository root as the working directory):", "", "    " + command, "",
             "From `%s`: %d warm-up steps, one warm replay of each graph, then %d rounds of the five forms "
             "(%d steps or decodes each; the ten-step graph %d replays). Microseconds, medians over each "
             "phase: the decode kernel's duration, and the idle time between the previous kernel's end and "
             "the decode's start (`gap before`), between the decode's end and the next kernel's start "
             "(`gap after`), and from one decode's start to the next one's (`period`: a step, or a "
             "decode, with every gap)." % (os.path.basename(trace_csv), W, R, K, K // 10), "",
             "| round | form | decodes | decode µs | gap before | gap after | period |",
             "|---|---|---:|---:|---:|---:|---:|"]
    per_round = 4 * K + (K // 10) * 10
    i = len(dec) - R * per_round  # after the clock-settle and warm-up steps and the graphs' warm replays
    for r in range(R):
        for name in INTERLEAVE_FORMS:
            n = (K // 10) * 10 if name == "graph_10_steps" else K
            ids = dec[i:i + n]
            i += n
            if len(ids) < n or not ids:
                lines.append("| %d | %s | trace too short | | | |" % (r + 1, name))
                continue
            d = np.array([(ks[j][2] - ks[j][1]) * 1e-3 for j in ids])
            gb = np.array([(ks[j][1] - ks[j - 1][2]) * 1e-3 for j in ids if j > 0])
            ga = np.array([(ks[j + 1][1] - ks[j][2]) * 1e-3 for j in ids if j + 1 < len(ks)])
            per = np.diff(np.array([ks[j][1] for j in ids])) * 1e-3
            lines.append("| %d | %s | %d | %.2f | %.2f | %.2f | %.2f |" % (
                r + 1, name, n, np.median(d), np.median(gb), np.median(ga), np.median(per) if len(per) else 0.0))
    lines.append("")
    return "\n".join(lines)


def measure(args, spec, partition_size: int, shared: bool, graph: bool, cold: bool, cpu_budget: float,
            cpu_budget_1t: float, sparse=None) -> dict:
    """Time one workload: K eager steps between two synchronisations (the
    metric), K eager steps with HIP events between the kernels (breakdown,
    per-step percentiles, the decode kernel's roofline), optionally K graph
    replays, cache-flushed side steps and the CPU oracle baseline. sparse =
    (sparse_block, top_blocks) times the sparse block-selection step instead
    (cache write, mean-key refresh, pa_decode_sparse)."""
    import torch

    import paged_attention_decode_02_amd as pa
    from workloads import BLOCK_SIZE, generate

    dev = torch.device("cuda:0")
    t0 = time.time()
    w = generate(spec)
    log("generated %s in %.1f s" % (spec.name, time.time() - t0))
    sp = w.spec
    TD = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "fp8": torch.float8_e4m3fn,
          "nvfp4": torch.float4_e2m1fn_x2}

    def up(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    row = sp.D // 2 + sp.D // 16 if sp.cache_dtype == "nvfp4" else sp.D  # nvfp4: bytes per (token, head)
    shape = (w.num_blocks, BLOCK_SIZE, sp.Hkv, row)
    byte_codes = sp.cache_dtype in ("fp8", "nvfp4")
    kc = torch.zeros(shape, dtype=torch.uint8 if byte_codes else TD[sp.cache_dtype], device=dev)
    vc = torch.zeros_like(kc)
    kc, vc = kc.view(TD[sp.cache_dtype]), vc.view(TD[sp.cache_dtype])
    ks = vs = None
    if sp.cache_dtype in ("i8", "fp8", "nvfp4"):
        ks = torch.zeros((shape[0], sp.Hkv, BLOCK_SIZE), dtype=torch.float32, device=dev)  # [nb, Hkv, 16]
        vs = torch.zeros_like(ks)
    N = w.slot_mapping.shape[0]
    step = 1 << 20
    for s in range(0, N, step):
        e = min(N, s + step)
        pa.cache_write(up(w.k_src[s:e], sp.src_dtype), up(w.v_src[s:e], sp.src_dtype),
                       torch.from_numpy(w.slot_mapping[s:e]).to(dev), kc, vc, ks, vs)
    rows = w.step_rows()
    new_k = up(w.k_src[rows], sp.src_dtype)
    new_v = up(w.v_src[rows], sp.src_dtype)
    new_slots = torch.from_numpy(w.slot_mapping[rows]).to(dev)
    q = up(w.q_array(), sp.q_dtype)
    table = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    P = partition_size or pa.choose_partition_size(sp.B, sp.Tq, sp.Hq, sp.Hkv, sp.D, TD[sp.cache_dtype],
                                                   w.max_seq_len)
    ws_bytes = pa.workspace_bytes(sp.B, sp.Tq, sp.Hq, sp.Hkv, sp.D, TD[sp.cache_dtype], w.max_seq_len, P)
    prefix_table = None
    if shared:
        ws_bytes = pa.shared_prefix_workspace_bytes(sp.B, sp.Tq, sp.Hq, sp.Hkv, sp.D, TD[sp.cache_dtype],
                                                    w.max_seq_len, sp.shared_prefix, args.prefix_partition,
                                                    args.tail_partition)
        prefix_table = torch.from_numpy(np.ascontiguousarray(w.block_table[0, : sp.shared_prefix // 16])).to(dev)
    mean_k = sel = None
    if sparse:
        SB, top = sparse
        nsb = (w.max_seq_len + SB - 1) // SB
        ws_bytes = pa.sparse_workspace_bytes(sp.B, sp.Tq, sp.Hq, sp.Hkv, sp.D, TD[sp.cache_dtype], w.max_seq_len,
                                             SB, top, partition_size)
        mean_k = torch.zeros((sp.B, nsb, sp.Hkv, sp.D), dtype=torch.float32, device=dev)
        sel = torch.full((sp.B, sp.Hkv, pa.sparse_max_selected(w.max_seq_len, SB, top)), -1, dtype=torch.int32,
                         device=dev)
        pa.sparse_mean_keys(kc, table, lens, w.max_seq_len, SB, w.max_seq_len, mean_k, ks)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((sp.B, sp.Tq, sp.Hq, sp.D), dtype=torch.float32, device=dev)
    lse = torch.empty((sp.B, sp.Tq, sp.Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    state = {"np": 1}
    # the step's calls checked and marshalled once (buffers at fixed
    # addresses, as in a serving loop): per call only the launch remains
    cw_call = pa.prepare_cache_write(new_k, new_v, new_slots, kc, vc, ks, vs)
    dec_call = red_call = None
    if not (shared or sparse):
        dec_call = pa.prepare_decode_partials(q, kc, vc, table, lens, w.max_seq_len, w.softmax_scale, out, lse, ks,
                                              vs, P, ws)
        state["np"] = dec_call.num_partitions
        if state["np"] > 1:
            red_call = pa.prepare_splitk_reduce(ws, state["np"], P, lens, out, lse)

    def one_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        cw_call()
        if sparse:
            pa.sparse_mean_keys(kc, table, lens, w.max_seq_len, sparse[0], sp.Tq, mean_k, ks)
        if ev is not None:
            ev[1].record(stream)
        if sparse:
            pa.decode_sparse(q, kc, vc, table, lens, w.max_seq_len, w.softmax_scale, mean_k, sparse[0], sparse[1],
                             ks, vs, partition_size, out=out, lse=lse, selected=sel, workspace=ws)
            if ev is not None:
                ev[2].record(stream)
                ev[3].record(stream)
            return
        if shared:
            pa.decode_shared_prefix(q, kc, vc, prefix_table, sp.shared_prefix, table, lens, w.max_seq_len,
                                    w.softmax_scale, ks, vs, args.prefix_partition, args.tail_partition, out=out,
                                    lse=lse, workspace=ws)
            if ev is not None:
                ev[2].record(stream)
                ev[3].record(stream)
            return
        dec_call()
        if ev is not None:
            ev[2].record(stream)
        if red_call is not None:
            red_call()
        if ev is not None:
            ev[3].record(stream)

    # Clock settle: an idle GPU comes back at a low clock and needs ~20 ms of
    # sustained work to reach its decode clock (runs of the same step right
    # after an idle period are 4-6% slower for that long). Untimed steps
    # until settle_ms have passed, then the W warm-up steps, then the timed
    # steps; the step count is reported beside the result.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_ms * 1e-3:
        for _ in range(10):
            one_step()
        torch.cuda.synchronize()
        settle_steps += 10
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    if getattr(args, "graph_interleave", 0):
        if shared or sparse:
            raise SystemExit("--graph-interleave times the plain decode step")
        return graph_interleave(args, one_step, dec_call)

    # ---- timed region for the metric: K eager steps between two synchronisations
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # ---- the same K eager steps again, with HIP events between the kernels of
    # every step (the per-kernel breakdown and the decode kernel's roofline).
    # Back to back like the metric's steps: the GPU keeps the clocks of a
    # sustained run. A kernel shorter than the host's launch interval shows
    # that interval instead (only the smallest workloads).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    cw = [e[0].elapsed_time(e[1]) for e in evs]
    dk = [e[1].elapsed_time(e[2]) for e in evs]
    rk = [e[2].elapsed_time(e[3]) for e in evs]
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]

    # ---- the decode kernel's average launch duration for the roofline: K
    # launches of the decode alone (the pa_decode_shared_prefix call: K
    # calls), back to back between two HIP events on the launch stream. An
    # event between every two kernels adds marker packets that lengthen each
    # interval by a few microseconds; back-to-back launches of one kernel are
    # what a sustained decode runs. The decode leaves its inputs unchanged, so
    # repeating it alone is the same work.
    def decode_only():
        if sparse:
            pa.decode_sparse(q, kc, vc, table, lens, w.max_seq_len, w.softmax_scale, mean_k, sparse[0], sparse[1],
                             ks, vs, partition_size, out=out, lse=lse, selected=sel, workspace=ws)
        elif shared:
            pa.decode_shared_prefix(q, kc, vc, prefix_table, sp.shared_prefix, table, lens, w.max_seq_len,
                                    w.softmax_scale, ks, vs, args.prefix_partition, args.tail_partition, out=out,
                                    lse=lse, workspace=ws)
        else:
            dec_call()

    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for i in range(args.steps):
        decode_only()
    d1.record(stream)
    torch.cuda.synchronize()
    dec_loop_ms = d0.elapsed_time(d1) / args.steps
    one_step()  # leave out/lse as a whole step writes them
    torch.cuda.synchronize()

    # ---- K replays of the step recorded in a HIP graph (decode runs under
    # graph capture in serving; the library allocates and synchronises
    # nothing, so the graph holds exactly the step's kernels)
    graph_ms = graph10_ms = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        g_start = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - g_start) * 1e3 / args.steps
        # the same steps, ten per graph: each graph launch leaves the GPU idle
        # for a few microseconds before its first kernel, which ten steps share
        g10 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g10):
            for _ in range(10):
                one_step()
        torch.cuda.synchronize()
        g10.replay()
        torch.cuda.synchronize()
        n10 = max(1, args.steps // 10)
        g_start = time.perf_counter()
        for _ in range(n10):
            g10.replay()
        torch.cuda.synchronize()
        graph10_ms = (time.perf_counter() - g_start) * 1e3 / (10 * n10)
        del g10
        # the replays must reproduce an eager step bit for bit
        ref_o, ref_l = out.clone(), lse.clone()
        one_step()
        torch.cuda.synchronize()
        if not (torch.equal(ref_o, out) and torch.equal(ref_l, lse)):
            raise RuntimeError("graph replay differs from the eager step")
        del g

    # ---- side measurement: every step after a flush of the caches (not the metric)
    cold_ms = []
    if cold:
        flush = torch.empty(args.flush_mb << 20, dtype=torch.uint8, device=dev)
        for i in range(min(20, args.steps)):
            flush.fill_(i & 0xFF)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            one_step(e)
            torch.cuda.synchronize()
            cold_ms.append(e[1].elapsed_time(e[3]))
        del flush

    ab = algorithmic_bytes(w)
    # the shared-prefix call must read the prefix once: its bytes are the
    # unique ones (the per-sequence total is reported beside them)
    step_bytes = unique_bytes(w) if shared else ab["total"]
    sparse_rec = None
    if sparse:
        # the selection the timed steps made, its bytes, and how far the
        # sparse output lies from the library's full decode of the same step
        seln = sel.cpu().numpy()
        sb = sparse_step_bytes(w, seln, sparse[0])
        step_bytes = sb["total"]
        s_out, s_lse = out.clone(), lse.clone()
        f_out, f_lse = pa.decode(q, kc, vc, table, lens, w.max_seq_len, w.softmax_scale, ks, vs)
        torch.cuda.synchronize()
        dev_out = (s_out - f_out).abs()
        sparse_rec = {
            "sparse_block": sparse[0], "top_blocks": sparse[1],
            "selected_blocks_per_head": [int((seln >= 0).sum(axis=2).min()), int((seln >= 0).sum(axis=2).max())],
            "bytes": sb,
            "full_decode_bytes": ab["total"],
            "vs_full_decode": {"max_abs_out": round(float(dev_out.max()), 6),
                               "mean_abs_out": round(float(dev_out.mean()), 6),
                               "max_abs_lse": round(float((s_lse - f_lse).abs().max()), 6)},
        }
        del f_out, f_lse
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_avg_ms = dec_loop_ms
    achieved = step_bytes / (dec_avg_ms * 1e-3) / 1e9
    ws_traffic = 0
    if state["np"] > 1:
        ws_traffic = 2 * sp.B * sp.Tq * sp.Hq * state["np"] * (sp.D + 1) * 4
    if shared:
        ws_traffic = 2 * ws_bytes
    res = {
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "config": {
            "workload": sp.name, "B": sp.B, "Tq": sp.Tq, "Hq": sp.Hq, "Hkv": sp.Hkv, "D": sp.D,
            "block_size": BLOCK_SIZE, "seq_lens": "%d..%d" % (w.seq_lens.min(), w.seq_lens.max()),
            "kv_dtype": sp.cache_dtype, "q_dtype": sp.q_dtype,
            "partition_size": None if shared else P,
            "num_partitions": None if shared else state["np"],
            "algorithmic_bytes_per_step": step_bytes,
            "per_sequence_bytes_per_step": ab["total"],
            "algorithmic_flops_per_step": None if sparse else algorithmic_flops(w),
            "flop_per_byte": None if sparse else round(algorithmic_flops(w) / step_bytes, 2),
            "shared_prefix": sp.shared_prefix,
            "prefix_partition": args.prefix_partition if shared else None,
            "tail_partition": args.tail_partition if shared else None,
            "splitk_workspace_bytes_per_step": ws_traffic,
        },
        "path": "sparse" if sparse else ("shared_prefix" if shared else "decode"),
        "clock_settle": {"ms": args.settle_ms, "untimed_steps": settle_steps,
                         "note": "untimed steps before the warm-up steps, until the GPU leaves its idle clock"},
        "graph_us_per_step": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
        "graph_10_steps_us_per_step": round(graph10_ms * 1e3, 2) if graph10_ms is not None else None,
        "step_us_event_timed": {"p10": pct(step_ms, 10), "median": pct(step_ms, 50), "p90": pct(step_ms, 90),
                                "min": pct(step_ms, 0), "steps": len(step_ms)},
        "decode_us_back_to_back": round(1e3 * dec_loop_ms, 2),
        "breakdown_us": {
            "note": "per-step HIP events between the kernels (each interval includes a marker packet)",
            "cache_write": round(1e3 * float(np.mean(cw)), 2),
            "decode": round(1e3 * float(np.mean(dk)), 2),
            "decode_p10_median_p90": [pct(dk, 10), pct(dk, 50), pct(dk, 90)],
            "reduce": round(1e3 * float(np.mean(rk)), 2),
            "step_events": round(1e3 * float(np.median(step_ms)), 2),
        },
        "roofline": {
            "kernel": ("pa_decode_sparse: scores, selection, decode and merge, against the bytes of the mean "
                       "keys and the selected blocks" if sparse else
                       "pa_decode_shared_prefix: prefix pass, tail pass and merge, against the bytes with the "
                       "prefix read once" if shared else decode_kernel(sp)[0]),
            "timing": "K back-to-back launches between two HIP events on the launch stream",
            "launch_us": round(1e3 * dec_loop_ms, 2),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            # the committed counters were taken at the library's partition size
            "traffic": None if sparse or partition_size else committed_traffic(sp, shared),
            "kernel_source_digest": kernel_source_digest(sp, shared),
        },
    }
    if sparse_rec:
        res["sparse"] = sparse_rec
        res["breakdown_us"]["note"] += "; sparse: cache_write holds the mean-key refresh, decode the whole call"
        res["config"]["partition_size"] = partition_size or None
        res["config"]["num_partitions"] = None
    if cold_ms:
        res["breakdown_us"]["decode_plus_reduce_after_flush"] = round(1e3 * float(np.median(cold_ms)), 2)
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n
        del src, dst
    del kc, vc, ks, vs, ws
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        res["cpu_baseline"] = run_cpu_baseline(w, ab["total"], cpu_budget, cpu_budget_1t)
    return res


# Side figures of the default run (each its own timed pass, reported under its
# own key): the 250K-token int8 decode, the second workload the >= 70% bar
# applies to, the 64K workload at the 512-token partitions it names, and the
# sparse block-selection step on the 250K int8 cache (512 blocks of 64 tokens
# per kv head, 13% of the context).
EXTRAS = (("int8_250k", "int8_250k", 0, True, None), ("long64k_bf16_p512", "long64k_bf16", 512, False, None),
          ("int8_250k_sparse_top512", "int8_250k", 0, False, (64, 512)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=30.0,
                    help="untimed steps for this long before the warm-up steps (the GPU's clock ramp from idle)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--partition-size", type=int, default=0, help="0 = the library's heuristic")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode through pa_decode_shared_prefix (workloads with a shared prefix)")
    ap.add_argument("--sparse-top", type=int, default=0,
                    help="time the sparse block-selection step (mean-key refresh, pa_decode_sparse) keeping this "
                         "many sparse blocks per (sequence, kv head); 0 = the plain decode")
    ap.add_argument("--sparse-block", type=int, default=64, help="--sparse-top: tokens per sparse block")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's B (0 = as named)")
    ap.add_argument("--lengths", default="", help="override the workload's sequence lengths, LO:HI")
    ap.add_argument("--prefix", type=int, default=-1, help="override the workload's shared prefix (tokens)")
    ap.add_argument("--prefix-partition", type=int, default=0, help="--shared-prefix: prefix pass partition (0 = "
                    "the library's choice)")
    ap.add_argument("--tail-partition", type=int, default=0, help="--shared-prefix: tail pass partition (0 = the "
                    "library's choice)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--cpu-budget-1thread", type=float, default=3.0,
                    help="seconds of single-thread oracle work for the CPU baseline's 1-thread figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay side measurement")
    ap.add_argument("--read-ceiling-mb", type=int, default=2048,
                    help="buffer of the streaming-read ceiling measurement (MiB; 0 skips it)")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run: skip the side workloads (int8 250K, 64K at 512-token partitions)")
    ap.add_argument("--flush-mb", type=int, default=512, help="flush buffer for the cold-cache side measurement")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after the benchmark, run 3 plain device copies of this many MiB (a kernel of known "
                         "traffic for scaling rocprofv3's FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM-traffic summary of two rocprofv3 --pmc counter CSVs and exit")
    ap.add_argument("--graph-interleave", type=int, default=0, metavar="ROUNDS",
                    help="instead of the benchmark: ROUNDS rounds of eager steps, one-step graph replays, "
                         "ten-step graph replays, eager decodes and one-decode graph replays, K each (a JSON line)")
    ap.add_argument("--summarize-interleave", nargs=2, metavar=("TRACE_CSV", "COMMAND"),
                    help="print the per-form summary of a kernel trace of --graph-interleave and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "COMMAND"),
                    help="print the kernel-duration summary of a rocprofv3 --kernel-trace CSV made by COMMAND "
                         "and exit")
    args = ap.parse_args()
    explicit_workload = any(a == "--workload" or a.startswith("--workload=") for a in sys.argv[1:])

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace[0], args.workload, args.summarize_trace[1],
                              shared=args.shared_prefix))
        return
    if args.summarize_interleave:
        print(summarize_interleave(args.summarize_interleave[0], args.summarize_interleave[1], args.steps,
                                   args.warmup, args.graph_interleave or 2))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.workload,
                                 (args.copy_calibration_mb or 512) << 20, shared=args.shared_prefix))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this decode library runs on a single MI355X "
              "(multi-GPU sharding is not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_attention_decode_02_amd as pa
    from workloads import SPECS, scaled

    if not os.path.exists(pa.library_path()):
        import __graft_entry__

        __graft_entry__.build()
    pa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = SPECS[args.workload]
    changes = {}
    if args.batch:
        changes["B"] = args.batch
    if args.lengths:
        lo, hi = (int(x) for x in args.lengths.split(":"))
        changes["seq_lens"] = (lo, hi)
    if args.prefix >= 0:
        changes["shared_prefix"] = args.prefix
    if changes:  # a workload of its own: no committed counters apply
        spec = scaled(spec, name=spec.name + "_custom", **changes)
    if args.shared_prefix and args.sparse_top:
        print("--shared-prefix and --sparse-top are separate paths", file=sys.stderr)
        sys.exit(2)
    if args.shared_prefix and not spec.shared_prefix:
        print("--shared-prefix needs a workload whose sequences share a prefix", file=sys.stderr)
        sys.exit(2)

    cpu = 0.0 if args.no_cpu_baseline else args.cpu_budget
    cpu1 = 0.0 if args.no_cpu_baseline else args.cpu_budget_1thread
    if args.graph_interleave:
        r = measure(args, spec, args.partition_size, False, True, False, 0.0, 0.0)
        r.update({"workload": spec.name, "device": device_record(pa)})
        print(json.dumps(r), flush=True)
        return
    sparse = (args.sparse_block, args.sparse_top) if args.sparse_top else None
    main_res = measure(args, spec, args.partition_size, args.shared_prefix, not args.no_graph, not sparse,
                       0.0 if sparse else cpu, 0.0 if sparse else cpu1, sparse)
    result = {
        "metric": METRIC,
        "value": main_res.pop("value"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res.pop("ms_per_step"),
        "us_per_step": main_res.pop("us_per_step"),
        "pct_hbm_peak": main_res.pop("pct_hbm_peak"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.cache_dtype,
        "data": "synthetic",
        "config": main_res.pop("config"),
        "timing": "eager launches, K steps between two device synchronisations",
    }
    cpu_res = main_res.pop("cpu_baseline", None)
    roof = main_res.pop("roofline")
    result.update(main_res)
    result["roofline"] = roof
    if cpu_res is not None:
        result["cpu_baseline"] = cpu_res
    result["device"] = device_record(pa)
    if args.read_ceiling_mb > 0:
        log("streaming-read ceiling (%d MiB)" % args.read_ceiling_mb)
        rc = read_ceiling(pa, args.read_ceiling_mb, 20)
        result["read_ceiling"] = rc
        result["pct_of_read_ceiling"] = round(100.0 * result["value"] / rc["gb_per_s"], 1)
        roof["frac_of_read_ceiling"] = round(roof["achieved"] / rc["gb_per_s"], 4)
    if not explicit_workload and not args.no_extras and not changes and not args.partition_size and not sparse:
        for key, name, P, with_cpu, sp_sel in EXTRAS:
            log("side workload %s (%s, P=%s)" % (key, name, P or "heuristic"))
            r = measure(args, SPECS[name], P, False, False, False, cpu if with_cpu else 0.0,
                        cpu1 if with_cpu else 0.0, sp_sel)
            r["dtype"] = SPECS[name].cache_dtype
            result[key] = r
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
