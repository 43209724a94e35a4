"""rocprofv3 passes over bench.py for one workload, and their summary.

    python3 bench_profile.py run --workload csa64k --out $OUT

runs, as child processes from /tmp (TMPDIR=/tmp), each under its own time
limit:

  1. rocprofv3 --kernel-trace --stats  -- python3 bench.py --workload W --only ...
  2. rocprofv3 --pmc FETCH_SIZE        -- python3 bench.py --workload W --only ...
  3. rocprofv3 --pmc WRITE_SIZE        -- python3 bench.py --workload W --only ...
  4. rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
                     SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE
                                       -- python3 bench.py --workload W --only ...

then writes profiles/<unit>_<workload>.md (per-kernel durations, per-dispatch
byte counters scaled by the calibration kernel, MFMA and LDS counters, the
dominant unit's duration next to the one bench.py measured in the same run)
and the workload's record in profiles/counters.json, which bench.py reads
for the ``traffic`` field of its roofline.

The byte counters are scaled by what they read for the calibration kernel
(bench.py's bitwise_not over 512 MiB: 512 MiB read, 512 MiB written).  A
record carries a hash of the dominant unit's sources; bench.py ignores it
once they change.  MFMA utilisation is the busy-cycle count over the
dispatch's active cycles (GRBM_GUI_ACTIVE, which reads the sum over the 8
XCDs, divided by 8) times the 1,024 SIMDs (256 CUs x 4): the fraction of the
MFMA peak at the clock the kernel ran at; the bf16 MFMA operation count is
SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops.

``summarize`` re-runs only the summary step on existing output directories.
This script never touches the GPU itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shlex
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CAL_BYTES = 512 << 20
CAL_KERNEL = "bitwise_not"
SIMDS = 256 * 4
# GRBM_GUI_ACTIVE comes back summed over the 8 XCDs (per dispatch it reads
# about 8 x 2.1 GHz x the traced duration), so one XCD's active cycles are a
# eighth of it
XCDS = 8
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"]
# device kernels of each dominant unit (substrings of rocprof kernel names)
UNIT_KERNELS = {
    # CSA decode: the step's first launch, compressors + scoring
    "index_decode_fresh": ["index_decode<true,"],
    # prefill: the scoring kernel of the step's index_topk call
    "index_scores": ["index_prefill"],
    "hca_step": ["attn_hs<false,", "attn_combine"],
    "swa_step": ["attn_hs<false,", "attn_combine"],
    "sparse_attn": ["attn_hs<true,", "attn_combine"],
    "output_proj": ["proj_rows<", "proj_gemm<"],
    "compress": ["compress_rows_kernel<"],
}
DOMINANT = {"hca1m": "hca_step", "hca1m_fp8": "hca_step", "swa": "swa_step",
            "oproj": "output_proj", "oproj_prefill": "output_proj", "prefill": "index_scores"}
WORKLOAD_NAME = {"csa64k": "csa_decode_64k", "csa1m": "csa_decode_1m",
                 "hca1m": "hca_decode_1m", "prefill": "csa_prefill_4k_on_60k",
                 "csa64k_pro": "csa_decode_64k_v4pro",
                 "csa64k_fp4": "csa_decode_64k_mxfp4_keys",
                 "csa1m_fp4": "csa_decode_1m_mxfp4_keys",
                 "swa": "swa_decode_1m", "oproj": "output_proj_decode",
                 "oproj_prefill": "output_proj_prefill_4k",
                 "csa64k_stream": "csa_decode_64k_streaming",
                 "compress_stream": "compress_stream_1m",
                 "csa64k_fp8": "csa_decode_64k_fp8_kv", "csa1m_fp8": "csa_decode_1m_fp8_kv",
                 "hca1m_fp8": "hca_decode_1m_fp8_kv"}


def dominant(workload):
    return DOMINANT.get(workload, "compress" if workload == "compress_stream"
                        else "index_decode_fresh")


def bench_cmd(workload, steps):
    return ["python3", os.path.join(ROOT, "bench.py"), "--workload", workload, "--only",
            "--steps", str(steps), "--warmup", str(steps), "--no-cpu"]


def passes(workload, out, steps):
    w = workload
    return [
        ("stats", ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
                   "-d", os.path.join(out, f"{w}_stats"), "-o", "run", "--"] + bench_cmd(w, steps)),
        ("fetch", ["rocprofv3", "--pmc", "FETCH_SIZE", "--output-format", "csv",
                   "-d", os.path.join(out, f"{w}_fetch"), "-o", "run", "--"] + bench_cmd(w, 10)),
        ("write", ["rocprofv3", "--pmc", "WRITE_SIZE", "--output-format", "csv",
                   "-d", os.path.join(out, f"{w}_write"), "-o", "run", "--"] + bench_cmd(w, 10)),
        ("mfma", ["rocprofv3", "--pmc", *MFMA_COUNTERS, "--output-format", "csv",
                  "-d", os.path.join(out, f"{w}_mfma"), "-o", "run", "--"] + bench_cmd(w, 10)),
    ]


def run(args):
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    logs = {}
    for name, cmd in passes(args.workload, out, args.steps):
        log = os.path.join(out, f"{args.workload}_{name}.log")
        print(f"[bench_profile] {args.workload} {name}: {' '.join(cmd)}", flush=True)
        with open(log, "w") as fh:
            try:
                rc = subprocess.run(["timeout", "-s", "KILL", str(args.timeout)] + cmd, cwd="/tmp",
                                    env=env, stdout=fh, stderr=subprocess.STDOUT).returncode
            except OSError as e:
                print(f"[bench_profile] could not start: {e}", flush=True)
                return 1
        logs[name] = log
        if rc != 0:
            # rocprofv3 may itself end with a fault after a complete run
            tail = open(log).read().splitlines()[-5:]
            done = any(line.startswith("{\"metric\"") for line in open(log))
            print(f"[bench_profile] {name} exited {rc}; bench line printed: {done}", flush=True)
            print("\n".join(tail), flush=True)
            if not done:
                return rc
        print(f"[bench_profile] {args.workload} {name} done", flush=True)
    return summarize_dirs(args.workload, out, logs, args.steps)


def _find(d, suffix):
    f = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not f:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return f[0]


def _short(name):
    n = name.replace("void ", "")
    return n.split("(")[0] if "(" in n else n


def _bench_line(log):
    for line in open(log):
        if line.startswith("{\"metric\""):
            return json.loads(line)
    return None


def _counter(d, counter):
    per = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def _match(names, pattern):
    return [n for n in names if pattern in n]


def summarize_dirs(workload, out, logs, steps):
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (constants and the source hash; no GPU work on import)

    stats_dir = os.path.join(out, f"{workload}_stats")
    rows = list(csv.DictReader(open(_find(stats_dir, "kernel_stats.csv"))))
    stats = {r["Name"]: (int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])) for r in rows}
    fetch = _counter(os.path.join(out, f"{workload}_fetch"), "FETCH_SIZE")
    write = _counter(os.path.join(out, f"{workload}_write"), "WRITE_SIZE")
    mdir = os.path.join(out, f"{workload}_mfma")
    mf = {c: _counter(mdir, c) for c in MFMA_COUNTERS} if os.path.isdir(mdir) else None
    cal_f = _match(fetch, CAL_KERNEL)
    cal_w = _match(write, CAL_KERNEL)
    if not cal_f or not cal_w:
        raise RuntimeError("calibration kernel missing from the counter runs")
    f_kib = statistics.median(fetch[cal_f[0]])
    w_kib = statistics.median(write[cal_w[0]])
    f_scale = CAL_BYTES / (f_kib * 1024.0)
    w_scale = CAL_BYTES / (w_kib * 1024.0)

    line = _bench_line(logs["stats"]) if logs.get("stats") else None
    dom = dominant(workload)
    dom_us, dom_bytes, comp = 0.0, 0.0, []
    for pat in UNIT_KERNELS[dom]:
        sk = _match(stats, pat)
        if not sk:
            continue
        fk = _match(fetch, pat)
        wk = _match(write, pat)
        if not (fk and wk):
            raise RuntimeError(f"kernel {pat} missing from the counter runs")
        for name in sk:
            us = stats[name][1]
            f_n = [n for n in fk if _short(n) == _short(name)]
            w_n = [n for n in wk if _short(n) == _short(name)]
            fb = statistics.median(fetch[f_n[0]]) * 1024.0 * f_scale if f_n else float("nan")
            wb = statistics.median(write[w_n[0]]) * 1024.0 * w_scale if w_n else float("nan")
            dom_us += us
            dom_bytes += fb + wb
            comp.append((_short(name), us, fb, wb))
    if not comp:
        raise RuntimeError(f"no kernel of unit {dom} in the profiles")

    rec = {
        "kernel": dom,
        "device_kernels": [c[0] for c in comp],
        "hbm_bytes_per_launch": int(round(dom_bytes)),
        "fetch_bytes_per_launch": int(round(sum(c[2] for c in comp))),
        "write_bytes_per_launch": int(round(sum(c[3] for c in comp))),
        "avg_launch_us_rocprof": round(dom_us, 2),
        "avg_launch_us_bench": None if line is None else line["roofline"]["avg_launch_us"],
        "algorithmic_bytes_per_launch": None if line is None else
        line["roofline"]["algorithmic_bytes_per_launch"],
        "calibration": {"kernel": _short(cal_f[0]), "bytes": CAL_BYTES,
                        "fetch_kib": f_kib, "fetch_scale": round(f_scale, 4),
                        "write_kib": w_kib, "write_scale": round(w_scale, 4)},
        "source_sha256": bench.kernel_source_hash(dom),
        "summary": f"profiles/{dom}_{WORKLOAD_NAME[workload]}.md",
    }
    os.makedirs(PROFILES, exist_ok=True)
    cpath = os.path.join(PROFILES, "counters.json")
    allrec = json.load(open(cpath)) if os.path.exists(cpath) else {}
    allrec[workload] = rec
    with open(cpath, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
        fh.write("\n")

    # markdown summary
    cmds = [" ".join(shlex.quote(x) for x in c).replace(out, "$OUT").replace(ROOT, "$REPO")
            for _, c in passes(workload, out, steps)]
    md = [f"# {dom} — {WORKLOAD_NAME[workload]} (rocprofv3)", "",
          "Commands (from /tmp with TMPDIR=/tmp; $REPO is the repository root, $OUT any "
          "output directory):", "", "```"]
    md += cmds
    md += [f"python3 $REPO/bench_profile.py summarize --workload {workload} --out $OUT "
           f"--steps {steps}", "```", "",
           "All of it at once: `python3 $REPO/bench_profile.py run "
           f"--workload {workload} --out $OUT --steps {steps}`.", "",
           "## Kernel durations (kernel trace, whole bench run)", "",
           "| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---|---|---|---|---|"]
    for name, (calls, avg, mn, mx, pct) in sorted(stats.items(), key=lambda kv: -kv[1][4]):
        if "spin_kernel" in name:
            continue
        md.append(f"| `{_short(name)}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.1f} |")
    md += ["", "## HBM byte counters per dispatch (median), scaled by the calibration", "",
           f"Calibration `{_short(cal_f[0])}` over {CAL_BYTES >> 20} MiB: FETCH_SIZE reads "
           f"{f_kib:.0f} KiB (scale {f_scale:.4f}), WRITE_SIZE {w_kib:.0f} KiB "
           f"(scale {w_scale:.4f}).", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes | written bytes |",
           "|---|---|---|---|---|"]
    for name in sorted(set(fetch) | set(write)):
        if CAL_KERNEL in name or "spin_kernel" in name:
            continue
        fk = statistics.median(fetch[name]) if name in fetch else float("nan")
        wk = statistics.median(write[name]) if name in write else float("nan")
        md.append(f"| `{_short(name)}` | {fk:.1f} | {wk:.1f} | {fk * 1024 * f_scale:.0f} | "
                  f"{wk * 1024 * w_scale:.0f} |")
    if mf is not None:
        md += ["", "## MFMA and LDS counters per dispatch (median)", "",
               "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1,024 SIMDs), "
               "the fraction of the MFMA peak at the clock the kernel ran at (GRBM_GUI_ACTIVE "
               "reads the sum over the 8 XCDs; the clock column is that sum / 8 over the traced "
               "duration; a value above the 2.4 GHz peak clock means the counter window ran longer "
               "than the kernel, which happens for kernels of tens of microseconds, and their "
               "busy % is then a lower bound); bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x "
               "512, their rate over "
               "the kernel's traced average duration, against the published 2.5 PFLOP/s; LDS bank "
               "conflicts per access = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - "
               "SQ_LDS_BANK_CONFLICT).", "",
               "| kernel | MFMA busy % | clock GHz | bf16 MFMA flops | bf16 MFMA TFLOP/s "
               "| % of 2.5 PFLOP/s | LDS conflict cycles | LDS conflicts / access |",
               "|---|---|---|---|---|---|---|---|"]
        names = sorted(mf["GRBM_GUI_ACTIVE"])
        for name in names:
            if CAL_KERNEL in name or "spin_kernel" in name or "elementwise" in name \
                    or "copyBuffer" in name:
                continue
            med = {c: statistics.median(mf[c][name]) if name in mf[c] else float("nan")
                   for c in MFMA_COUNTERS}
            active = med["GRBM_GUI_ACTIVE"] / XCDS
            busy = 100.0 * med["SQ_VALU_MFMA_BUSY_CYCLES"] / max(active * SIMDS, 1)
            flops = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            st = [v for k, v in stats.items() if _short(k) == _short(name)]
            us = st[0][1] if st else float("nan")
            tf = flops / (us * 1e-6) / 1e12 if us > 0 else float("nan")
            ghz = active / (us * 1e3) if us > 0 else float("nan")
            acc = med["SQ_LDS_IDX_ACTIVE"] - med["SQ_LDS_BANK_CONFLICT"]
            cpa = med["SQ_LDS_BANK_CONFLICT"] / acc if acc > 0 else float("nan")
            md.append(f"| `{_short(name)}` | {busy:.1f} | {ghz:.2f} | {flops:.4g} | {tf:.1f} | "
                      f"{100 * tf / 2500:.1f} | {med['SQ_LDS_BANK_CONFLICT']:.4g} | {cpa:.4f} |")
    md += ["", "## Dominant unit", "",
           f"- unit: `{dom}` = " + " + ".join(f"`{c[0]}`" for c in comp),
           f"- average duration per launch, rocprofv3: {dom_us:.2f} µs"
           + ("" if line is None else
              f"; bench.py (HIP events, same run): {line['roofline']['avg_launch_us']:.2f} µs"),
           f"- HBM traffic per launch (counters): {dom_bytes:.0f} bytes"
           + ("" if line is None else
              f"; algorithmic bytes per launch: {line['roofline']['algorithmic_bytes_per_launch']}"),
           f"- kernel source hash: `{rec['source_sha256']}`"]
    if line is not None:
        md += ["", "bench.py line of the kernel-trace run:", "", "```", json.dumps(line), "```"]
    path = os.path.join(PROFILES, f"{dom}_{WORKLOAD_NAME[workload]}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(f"[bench_profile] wrote {path} and the {workload} record of {cpath}", flush=True)
    return 0


def summarize(args):
    out = os.path.abspath(args.out)
    logs = {"stats": os.path.join(out, f"{args.workload}_stats.log")}
    if not os.path.exists(logs["stats"]):
        logs = {}
    return summarize_dirs(args.workload, out, logs, args.steps)


def main():
    p = argparse.ArgumentParser()
    p.add_argument("action", choices=["run", "summarize"])
    p.add_argument("--workload", default="csa64k", choices=sorted(WORKLOAD_NAME))
    p.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "prof"))
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--timeout", type=int, default=240)
    a = p.parse_args()
    sys.exit(run(a) if a.action == "run" else summarize(a))


if __name__ == "__main__":
    main()
