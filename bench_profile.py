"""rocprofv3 passes over bench.py for one workload, and their summary.

    python3 -m long_context_sparse_11_amd.profsum run --workload csa64k --out _prof

runs, as child processes from /tmp (TMPDIR=/tmp):

  1. rocprofv3 --kernel-trace --stats  -- python3 bench.py --workload W ...
  2. rocprofv3 --pmc FETCH_SIZE        -- python3 bench.py --workload W ...
  3. rocprofv3 --pmc WRITE_SIZE        -- python3 bench.py --workload W ...

(each counter in a run of its own), then writes profiles/<kernel>_<workload>.md
(per-kernel durations, per-dispatch byte counters, the calibration, the
dominant kernel's duration next to the one bench.py measured in the same run)
and the workload's record in profiles/counters.json, which bench.py reads
for the ``traffic`` field of its roofline.

The byte counters are scaled by what they read for the calibration kernel
(bench.py's bitwise_not over 512 MiB: 512 MiB read, 512 MiB written).  A
record carries a hash of the dominant kernel's sources; bench.py ignores it
once they change.

``summarize`` re-runs only the summary step on existing output directories.
This module never touches the GPU itself.
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

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
CAL_BYTES = 512 << 20
CAL_KERNEL = "bitwise_not"
# device kernels of each dominant unit (substrings of rocprof kernel names)
UNIT_KERNELS = {
    # decode: the scoring kernel as the bench times it (csa_index_scores); the
    # step runs its variant with the fresh-entry workgroups, index_decode<true>
    "index_scores": {"decode": ["index_decode<false,"], "prefill": ["index_prefill"]},
    "hca_attn": {"decode": ["attn_hs<false, true, 4>", "attn_combine"]},
    "sparse_attn": {"decode": ["attn_hs<true,", "attn_combine"]},
    "output_proj": {"decode": ["proj_rows<4>", "proj_rows<8>"],
                    "prefill": ["proj_gemm<0>", "proj_gemm<1>"]},
}
WORKLOAD_NAME = {"csa64k": "csa_decode_64k", "csa1m": "csa_decode_1m",
                 "hca1m": "hca_decode_1m", "prefill": "csa_prefill_4k_on_60k",
                 "csa64k_pro": "csa_decode_64k_v4pro",
                 "csa64k_fp4": "csa_decode_64k_mxfp4_keys",
                 "csa1m_fp4": "csa_decode_1m_mxfp4_keys",
                 "swa": "swa_decode_1m", "oproj": "output_proj_decode",
                 "oproj_prefill": "output_proj_prefill_4k",
                 "csa64k_stream": "csa_decode_64k_streaming"}


def bench_cmd(workload, steps):
    return ["python3", os.path.join(ROOT, "bench.py"), "--workload", workload,
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
    ]


def run(args):
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    logs = {}
    for name, cmd in passes(args.workload, out, args.steps):
        log = os.path.join(out, f"{args.workload}_{name}.log")
        print(f"[profsum] {args.workload} {name}: {' '.join(cmd)}", flush=True)
        with open(log, "w") as fh:
            try:
                rc = subprocess.run(["timeout", "-s", "KILL", str(args.timeout)] + cmd, cwd="/tmp",
                                    env=env, stdout=fh, stderr=subprocess.STDOUT).returncode
            except OSError as e:
                print(f"[profsum] could not start: {e}", flush=True)
                return 1
        logs[name] = log
        if rc != 0:
            # rocprofv3 may itself end with a fault after a complete run
            tail = open(log).read().splitlines()[-5:]
            done = any(line.startswith("{\"metric\"") for line in open(log))
            print(f"[profsum] {name} exited {rc}; bench line printed: {done}", flush=True)
            print("\n".join(tail), flush=True)
            if not done:
                return rc
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
    cal_f = _match(fetch, CAL_KERNEL)
    cal_w = _match(write, CAL_KERNEL)
    if not cal_f or not cal_w:
        raise RuntimeError("calibration kernel missing from the counter runs")
    f_kib = statistics.median(fetch[cal_f[0]])
    w_kib = statistics.median(write[cal_w[0]])
    f_scale = CAL_BYTES / (f_kib * 1024.0)
    w_scale = CAL_BYTES / (w_kib * 1024.0)

    line = _bench_line(logs["stats"]) if logs.get("stats") else None
    dom = {"hca1m": "hca_attn", "swa": "sparse_attn", "oproj": "output_proj",
           "oproj_prefill": "output_proj"}.get(workload, "index_scores")
    phase = "prefill" if workload in ("prefill", "oproj_prefill") else "decode"
    parts = UNIT_KERNELS[dom][phase]
    dom_us, dom_bytes, comp = 0.0, 0.0, []
    for pat in parts:
        sk = _match(stats, pat)
        fk = _match(fetch, pat)
        wk = _match(write, pat)
        if not (sk and fk and wk):
            raise RuntimeError(f"kernel {pat} missing from the profiles")
        us = stats[sk[0]][1]
        fb = statistics.median(fetch[fk[0]]) * 1024.0 * f_scale
        wb = statistics.median(write[wk[0]]) * 1024.0 * w_scale
        dom_us += us
        dom_bytes += fb + wb
        comp.append((_short(sk[0]), us, fb, wb))

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
    md += [f"python3 -m long_context_sparse_11_amd.profsum summarize --workload {workload} "
           f"--out $OUT --steps {steps}", "```", "",
           "All of it at once: `python3 -m long_context_sparse_11_amd.profsum run "
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
    md += ["", "## Dominant kernel", "",
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
    print(f"[profsum] wrote {path} and the {workload} record of {cpath}", flush=True)
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
    p.add_argument("--out", default=os.path.join(ROOT, "_prof"))
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--timeout", type=int, default=300)
    a = p.parse_args()
    sys.exit(run(a) if a.action == "run" else summarize(a))


if __name__ == "__main__":
    main()
