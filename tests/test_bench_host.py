"""bench.py's host-side pieces (CPU only): the byte counts behind its metric and
its refusal to run on more than one GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import bench
from workloads import SPECS, generate, scaled

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_64k_workload():
    # 4 x 65536 tokens x 4 kv heads x 256 x 2 (K, V) x 2 bytes, the table, q and out
    w = generate(scaled("long64k_bf16", D=8, Hq=2, Hkv=1, seq_lens=(100, 100)))
    ab = bench.algorithmic_bytes(w)
    L = int(w.seq_lens.sum())
    assert ab["kv"] == L * 1 * 8 * 2 * 2
    assert ab["table"] == int(((w.seq_lens + 15) // 16).sum()) * 4
    assert ab["total"] == ab["kv"] + ab["scales"] + ab["table"] + ab["q"] + ab["out"]
    full = SPECS["long64k_bf16"]
    assert 4 * 65536 * full.Hkv * full.D * 2 * 2 == 1073741824


def test_algorithmic_flops_count_each_query_tokens_visible_keys():
    # one decode token: 4 D Hq flops per key of every sequence; the 64K
    # workload's 4 x 65536 keys x 24 heads x 256 x 4 = 6.44 GFLOP
    w = generate(scaled("long64k_bf16", D=8, Hq=2, Hkv=1, seq_lens=(100, 130)))
    assert bench.algorithmic_flops(w) == 4 * 8 * 2 * int(w.seq_lens.sum())
    full = SPECS["long64k_bf16"]
    assert 4 * full.D * full.Hq * 4 * 65536 == 6442450944
    # Tq query tokens: token t sees L - Tq + t + 1 keys (L - 3, L - 2, L - 1, L for Tq = 4)
    w = generate(scaled("verify_bf16", B=2, Tq=4, Hq=4, Hkv=2, D=16, seq_lens=(50, 60), shared_prefix=0))
    keys = sum(4 * int(L) - 6 for L in w.seq_lens)
    assert bench.algorithmic_flops(w) == 4 * 16 * 4 * keys


def test_unique_bytes_count_the_shared_prefix_once():
    for kv in ("bf16", "i8", "nvfp4"):
        spec = scaled("verify_bf16", B=3, Tq=2, Hq=4, Hkv=2, D=64, seq_lens=(300, 400), shared_prefix=256,
                      cache_dtype=kv, src_dtype="f32")
        w = generate(spec, seed=1)
        ab = bench.algorithmic_bytes(w)
        per_token = (ab["kv"] + ab["scales"]) // int(w.seq_lens.sum())
        assert (ab["kv"] + ab["scales"]) % int(w.seq_lens.sum()) == 0
        assert bench.unique_bytes(w) == ab["total"] - 2 * 256 * per_token


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_names_the_kernel_the_library_launches():
    import paged_attention_decode_02_amd as pa

    for name, spec in SPECS.items():
        kname, srcs = bench.decode_kernel(spec)
        assert kname == pa.decode_kernel_name(spec.Tq, spec.Hq, spec.Hkv, bench_dtype(spec.cache_dtype)), name
        assert srcs[0] == kname.replace("_kernel", ".hip"), (kname, srcs)
    assert bench.decode_kernel(SPECS["long64k_bf16"])[0] == "decode_wave_kernel"
    assert bench.decode_kernel(SPECS["int8_250k"])[0] == "decode_stream_kernel"
    assert bench.decode_kernel(SPECS["verify_i8"])[0] == "decode_mfma_kernel"
    assert bench.decode_kernel(SPECS["tiny_f32"])[0] == "decode_valu_kernel"


def bench_dtype(name):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "fp8": torch.float8_e4m3fn,
            "nvfp4": torch.float4_e2m1fn_x2}[name]


def test_sparse_step_bytes_with_every_block_selected():
    # every sparse block of every (sequence, kv head) selected: the K/V bytes
    # are the full decode's; the mean keys add one fp32 row per block and head
    for kv in ("bf16", "i8", "nvfp4"):
        spec = scaled("int8_250k", B=3, Tq=2, Hq=4, Hkv=2, D=64, seq_lens=(100, 300), cache_dtype=kv,
                      src_dtype="f32")
        w = generate(spec, seed=3)
        SB = 32
        nsb = (w.seq_lens + SB - 1) // SB
        sel = np.full((spec.B, spec.Hkv, int(nsb.max())), -1, dtype=np.int32)
        for b in range(spec.B):
            sel[b, :, :nsb[b]] = np.arange(nsb[b])
        sb = bench.sparse_step_bytes(w, sel, SB)
        ab = bench.algorithmic_bytes(w)
        assert sb["kv_selected"] == ab["kv"] + ab["scales"]
        assert sb["mean_keys"] == int(nsb.sum()) * spec.Hkv * spec.D * 4
        # the refresh re-reads the keys of the blocks holding the last Tq tokens
        per_key = (ab["kv"] + ab["scales"]) // int(w.seq_lens.sum()) // 2
        refresh = sum(min(int(L), (j + 1) * SB) - j * SB for L in w.seq_lens
                      for j in range((int(L) - spec.Tq) // SB, (int(L) + SB - 1) // SB))
        assert sb["mean_refresh"] == refresh * per_key
        # half the blocks: half-ish the K/V bytes, never more than the full set
        sel2 = sel.copy()
        sel2[:, :, 1::2] = -1
        sel2 = np.sort(np.where(sel2 < 0, 1 << 30, sel2), axis=2)
        sel2[sel2 == 1 << 30] = -1
        assert bench.sparse_step_bytes(w, sel2, SB)["kv_selected"] < sb["kv_selected"]


def test_interleave_summary_splits_the_trace_by_form(tmp_path):
    # a synthetic kernel trace in the layout of --graph-interleave: W warm-up
    # steps, one warm replay of each graph (1 + 10 + 1 decodes), then rounds
    # of the five forms; the decode of form f in round r lasts 100 + 10 f + r us
    K, W, R = 20, 3, 2
    rows, t = [], 0

    def kern(name, dur, gap=0.0):
        nonlocal t
        t += int(gap * 1000)
        rows.append({"Kernel_Name": "void pa::%s(pa::P)" % name, "Start_Timestamp": t, "End_Timestamp": t + int(dur * 1000)})
        t += int(dur * 1000)

    for _ in range(W + 12):
        kern("decode_wave_kernel<1, 256, 6, 4>", 50.0)
    for r in range(R):
        for f, name in enumerate(bench.INTERLEAVE_FORMS):
            n = (K // 10) * 10 if name == "graph_10_steps" else K
            for _ in range(n):
                if "step" in name:
                    kern("cache_write_kernel<1, 256, true>", 2.0, gap=8.0 if name == "graph_step" else 0.0)
                kern("decode_wave_kernel<1, 256, 6, 4>", 100.0 + 10 * f + r, gap=5.0 if name == "graph_decode" else 0.0)
                if "step" in name:
                    kern("splitk_reduce_kernel<4>", 4.0)
    path = tmp_path / "run_kernel_trace.csv"
    with open(path, "w") as fh:
        fh.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for rw in rows:
            fh.write('"%s",%d,%d\n' % (rw["Kernel_Name"], rw["Start_Timestamp"], rw["End_Timestamp"]))
    md = bench.summarize_interleave(str(path), "cmd", K, W, R)
    for r in range(R):
        for f, name in enumerate(bench.INTERLEAVE_FORMS):
            n = (K // 10) * 10 if name == "graph_10_steps" else K
            gap_before = 5.0 if name == "graph_decode" else 0.0
            assert "| %d | %s | %d | %.2f | %.2f |" % (r + 1, name, n, 100.0 + 10 * f + r, gap_before) in md, (r, name)
            # period: the decode plus the step's other kernels and gaps
            period = 100.0 + 10 * f + r + gap_before + (14.0 if name == "graph_step" else 6.0 if "step" in name else 0.0)
            line = [ln for ln in md.splitlines() if ln.startswith("| %d | %s |" % (r + 1, name))][0]
            assert line.endswith("| %.2f |" % period), (line, period)


def test_trace_summary_places_phases_after_any_number_of_settle_steps(tmp_path):
    # decode durations by phase in the layout of one bench.py run: S clock-settle
    # steps (any S), W warm-up, K eager, K with events, K back-to-back decodes,
    # one eager step, W + K one-step graph replays, 10 + 10 (K / 10) ten-step
    # graph decodes, one check step, 20 cache-flushed steps
    K, W = 50, 5
    phases = [("settle", 37, 300.0), ("warm", W, 290.0), ("eager", K, 171.0), ("events", K, 163.0), ("b2b", K, 162.0),
              ("one", 1, 280.0), ("gwarm", W, 280.0), ("graph", K, 176.0), ("g10warm", 10, 280.0),
              ("g10", 10 * (K // 10), 165.0), ("check", 1, 280.0), ("cold", 20, 200.0)]
    path = tmp_path / "run_kernel_trace.csv"
    t = 0
    with open(path, "w") as fh:
        fh.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for _, n, dur in phases:
            for _ in range(n):
                fh.write('"void pa::decode_wave_kernel<1, 256, 6, 4>(pa::DecodeParams)",%d,%d\n' % (t, t + int(dur * 1000)))
                t += int(dur * 1000) + 1000
    cmd = "rocprofv3 -- python -u bench.py --workload long64k_bf16 --steps %d --warmup %d --no-cpu-baseline" % (K, W)
    md = bench.summarize_trace(str(path), "long64k_bf16", cmd)
    assert "37 clock-settle steps before the warm-up." in md
    for label, dur in (("eager steps (the metric's timed region)", 171.0),
                       ("eager steps with events between the kernels", 163.0),
                       ("back-to-back decode launches (the roofline's launches)", 162.0),
                       ("graph replays, one step per graph", 176.0), ("graph replays, ten steps per graph", 165.0)):
        assert "| %s | 50 | %.2f | %.2f |" % (label, dur, dur) in md, label
    assert "decode_mean_us_roofline_launches: 162.00" in md


def test_sq_summary_normalises_per_block_and_skips_other_kernels(tmp_path):
    # two counter passes of a synthetic rocprofv3 CSV: two decode dispatches
    # per counter (their mean is reported), a reduce dispatch that must be
    # ignored; per-block values divide by the workload's (16-token block, kv
    # head) pairs
    w = generate(SPECS["verify_i8"])
    blocks = int(((w.seq_lens.astype(np.int64) + 15) // 16).sum()) * w.spec.Hkv
    a, b = tmp_path / "a.csv", tmp_path / "b.csv"
    hdr = "Kernel_Name,Counter_Name,Counter_Value\n"
    # kernel names hold commas: quoted, as rocprofv3 writes them
    a.write_text(hdr + "".join('"pa::decode_mfma_kernel<2, 256, 3, 1>(pa::DecodeParams)",%s,%d\n' % (n, v)
                               for n, vals in (("SQ_WAVE_CYCLES", (1000 * blocks, 3000 * blocks)),
                                               ("SQ_INSTS_VALU", (500 * blocks, 500 * blocks)))
                               for v in vals)
                 + '"pa::splitk_reduce_rows_kernel<256>(pa::ReduceParams)",SQ_INSTS_VALU,999999999\n')
    b.write_text(hdr + "".join('"pa::decode_mfma_kernel<2, 256, 3, 1>(pa::DecodeParams)",SQ_WAIT_ANY,%d\n' % v
                               for v in (800 * blocks, 800 * blocks)))
    md = bench.summarize_sq([("k", "decode_mfma_kernel", [str(a), str(b)], ["cmd a", "cmd b"])], "verify_i8")
    assert "| SQ_WAVE_CYCLES | %d | 2000.0 |" % (2000 * blocks) in md
    assert "| SQ_INSTS_VALU | %d | 500.0 |" % (500 * blocks) in md
    assert "| SQ_INSTS_MFMA | — | — |" in md  # not collected
    assert "waiting 40% of wave time" in md  # 800 / 2000
    assert "    cmd a" in md and "    cmd b" in md
