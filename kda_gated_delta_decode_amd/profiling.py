"""Turn rocprofv3 CSV output into the short text summaries kept with the
benchmark (kernel durations, HBM traffic per launch).

    python -m kda_gated_delta_decode_amd.profiling trace --stats S.csv --trace T.csv \
        --kernel SUBSTR --timed N --command "..." --title "..." --out FILE.md
    python -m kda_gated_delta_decode_amd.profiling pmc --run LABEL FETCH.csv WRITE.csv \
        [--run ...] --command "..." --out FILE.json

`pmc` calibrates the counters on the copy kernels of the same runs: the
nontemporal copy (kda_bw_probe_kernel, the hint the decode's state traffic
carries) and the plain one (kda_copy_probe_kernel) each copy one 16-byte
vector per work-item, so a dispatch of grid G work-items reads and writes
16 G bytes.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by
(16 G) / (1024 * counter), averaged over the nontemporal copy's dispatches,
then applied to each decode kernel's mean per dispatch.

Reads only the CSV files it is given; runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import shlex
import statistics
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "kda_decode.hip")
COPY_KERNEL = "kda_copy_probe_kernel"
DECODE_KERNEL = "kda_decode_tile"


# headers a kernel's code and launch shapes also come from
KERNEL_HEADERS = ("kda_launch.h", "kda_device.h", "kda_internal.h")


def kernel_hash(src: str = KERNEL_SRC) -> str:
    """sha256[:16] of a kernel source file and the csrc headers it is built
    with (device helpers, launch-shape defaults): a summary taken on other
    sources no longer describes the kernel that runs."""
    h = hashlib.sha256()
    for path in [src] + [os.path.join(HERE, "csrc", n) for n in KERNEL_HEADERS]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _counter_by_dispatch(path, counter):
    """{kernel name: [(grid size, value), ...]} for one counter, one entry per
    dispatch (values of several agents / dimensions of a dispatch summed)."""
    per = defaultdict(float)
    meta = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter:
            continue
        key = int(r["Dispatch_Id"])
        per[key] += float(r["Counter_Value"])
        meta[key] = (r["Kernel_Name"], int(r["Grid_Size"]))
    out = defaultdict(list)
    for key in sorted(per):
        name, grid = meta[key]
        out[name].append((grid, per[key]))
    return out


# Calibration kernels: each dispatch of grid G work-items copies 16 G bytes
# (one 16-byte vector per work-item), plain or with the nontemporal hint.
CALIBRATION = {
    "plain": ("kda_copy_probe_kernel",),
    "nontemporal": ("kda_bw_probe_kernel<0, 1, true>", "kda_bw_probe_kernelILi0ELi1ELb1E"),
}
# Kernels whose traffic is summarised: (label suffix, name substrings, workload)
SUMMARISED = (
    ("", ("kda_decode_tile",), None),
    ("_spec_verify_8x8", ("kda_rows_mfma8_kernel",), "spec_verify_f16"),
)


def _calibrate(fe, wr, label, calib):
    """Counter-to-bytes factors of each calibration kernel found in one run."""
    out = {}
    for kind, subs in CALIBRATION.items():
        for name in fe:
            if not any(sub in name for sub in subs):
                continue
            by_f, by_w = defaultdict(list), defaultdict(list)
            for grid, v in fe[name]:
                by_f[16 * grid].append(v)
            for grid, v in wr.get(name, []):
                by_w[16 * grid].append(v)
            for nbytes in sorted(by_f):
                ff = nbytes / (statistics.mean(by_f[nbytes]) * 1024)
                wf = nbytes / (statistics.mean(by_w[nbytes]) * 1024)
                out.setdefault(kind, []).append((ff, wf))
                calib["%s/%s/%d" % (label, kind, nbytes)] = {
                    "kernel": name, "bytes_copied": nbytes,
                    "FETCH_SIZE_KiB": round(statistics.mean(by_f[nbytes]), 1),
                    "WRITE_SIZE_KiB": round(statistics.mean(by_w[nbytes]), 1),
                    "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}
    return out


def pmc(args):
    import kda_inputs
    factors = defaultdict(list)
    calib, runs = {}, {}
    for label, fpath, wpath in args.run:
        fe = _counter_by_dispatch(fpath, "FETCH_SIZE")
        wr = _counter_by_dispatch(wpath, "WRITE_SIZE")
        for kind, fw in _calibrate(fe, wr, label, calib).items():
            factors[kind].extend(fw)
        for suffix, subs, workload in SUMMARISED:
            names = [n for n in fe if any(sub in n for sub in subs)]
            if not names:
                continue
            if len(names) != 1:
                raise SystemExit("run %s: expected one %s kernel, found %r" % (label, subs, names))
            runs[label + suffix] = (names[0], fe[names[0]], wr[names[0]], label.split("_")[0], workload)
    if "nontemporal" not in factors:
        raise SystemExit("no nontemporal copy dispatch to calibrate on")
    fac = {kind: (statistics.mean(f for f, _ in v), statistics.mean(w for _, w in v))
           for kind, v in factors.items()}
    ff, wf = fac["nontemporal"]
    launches = {}
    for key, (name, fe, wr, dtype, workload) in runs.items():
        if workload is not None:
            inp = getattr(kda_inputs, workload)(0)
        else:
            inp = kda_inputs.batched_f32(0) if dtype == "f32" else kda_inputs.batched_f16(0)
        fk = statistics.mean(v for _, v in fe)
        wk = statistics.mean(v for _, v in wr)
        rd, wt = fk * 1024 * ff, wk * 1024 * wf
        alg = inp.state_bytes() + inp.io_bytes()
        launches[key] = {"kernel": name, "dispatches": len(fe),
                         "FETCH_SIZE_KiB": round(fk, 1), "WRITE_SIZE_KiB": round(wk, 1),
                         "hbm_read_bytes": int(rd), "hbm_write_bytes": int(wt),
                         "hbm_bytes_per_launch": int(rd + wt),
                         "algorithmic_bytes_per_launch": alg,
                         "hbm_over_algorithmic": round((rd + wt) / alg, 4),
                         "hbm_bytes_with_plain_copy_factors": int(fk * 1024 * fac["plain"][0] +
                                                                  wk * 1024 * fac["plain"][1])
                         if "plain" in fac else None}
    doc = {"what": "HBM traffic of the decode kernels from rocprofv3 --pmc FETCH_SIZE and "
                   "WRITE_SIZE (KiB per dispatch), each scaled by the factor that maps the same "
                   "counter to the known bytes of the nontemporal copy kernel (kda_bw_probe_kernel, "
                   "one 16-byte vector per work-item) in the same runs: the decode's state loads "
                   "and stores carry the nontemporal hint.  The plain copy's factors are listed "
                   "beside them",
           "commands": args.command, "summary_command": self_command(),
           "kernel_source_sha256_16": kernel_hash(),
           "calibration_copies": calib,
           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
           "plain_copy_factors": [round(x, 4) for x in fac["plain"]] if "plain" in fac else None,
           "launches": launches}
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


def self_command() -> str:
    """This summary's own invocation, in full."""
    return "python -m kda_gated_delta_decode_amd.profiling " + shlex.join(sys.argv[1:])


def trace(args):
    stats = _rows(args.stats)
    lines = ["# %s" % args.title, "",
             "Command (from the repository root, `TMPDIR=/tmp`):", "", "```"]
    lines += args.command + ["```", "", "Summary written by (from the repository root):", "", "```",
                             self_command(), "```", "",
                             "Kernel sources (%s with %s) sha256[:16] at the time: `%s`." % (
                                 args.source, ", ".join(KERNEL_HEADERS),
                                 kernel_hash(os.path.join(HERE, "csrc", args.source))), "",
                             "## rocprofv3 kernel stats (all dispatches of the run)", "",
                             "| Kernel | Calls | Average µs | Min µs | Max µs |", "|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"][:100]
        lines.append("| `%s` | %s | %.3f | %.3f | %.3f |" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3))
    tr = [r for r in _rows(args.trace) if args.kernel in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = sorted({r["Kernel_Name"] for r in tr})
    timed = tr[-args.timed:]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
    span = (int(timed[-1]["End_Timestamp"]) - int(timed[0]["Start_Timestamp"])) / 1e3
    gaps = [(int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) / 1e3
            for a, b in zip(timed, timed[1:])]
    q = statistics.quantiles(dur, n=10)
    lines += ["", "## The timed launches (the last %d dispatches of `%s`)" % (args.timed, args.kernel), "",
              "- kernel(s): %s" % ", ".join("`%s`" % n for n in names),
              "- kernel duration mean %.3f µs, median %.3f µs, p10 %.3f µs, p90 %.3f µs" % (
                  statistics.mean(dur), statistics.median(dur), q[0], q[-1]),
              "- first start to last end / %d = %.3f µs; median gap between launches %.3f µs" % (
                  args.timed, span / args.timed, statistics.median(gaps) if gaps else 0.0)]
    if args.algorithmic_bytes:
        m = statistics.mean(dur)
        lines.append("- %d algorithmic bytes / %.3f µs = %.0f GB/s = %.1f%% of 8 TB/s" % (
            args.algorithmic_bytes, m, args.algorithmic_bytes / m / 1e3,
            100 * args.algorithmic_bytes / m / 1e3 / 8000))
    if args.algorithmic_flops:
        m = statistics.mean(dur)
        tf = args.algorithmic_flops / m / 1e6
        lines.append("- %d algorithmic flops / %.3f µs = %.1f TFLOP/s = %.1f%% of %.1f TFLOP/s" % (
            args.algorithmic_flops, m, tf, 100 * tf / args.peak_tflops, args.peak_tflops))
    for note in args.note or []:
        lines += ["", note]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("--run", nargs=3, action="append", required=True,
                   metavar=("LABEL", "FETCH_CSV", "WRITE_CSV"))
    p.add_argument("--command", action="append", required=True)
    p.add_argument("--out", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--trace", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--timed", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, default=0)
    t.add_argument("--algorithmic-flops", type=int, default=0)
    t.add_argument("--source", default="kda_decode.hip", help="kernel source file under csrc/")
    t.add_argument("--peak-tflops", type=float, default=157.3)
    t.add_argument("--command", action="append", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--note", action="append")
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    (pmc if a.cmd == "pmc" else trace)(a)


if __name__ == "__main__":
    main()
