"""Short text summaries of rocprofv3 output, and the reader of the HBM byte counts they record.

    python -m gemv_wq_gemm_amd.rocprof_summary trace STATS_CSV OUT_MD --command CMD [--top N]
    python -m gemv_wq_gemm_amd.rocprof_summary counters OUT_MD --run FETCH_CSV WRITE_CSV [--run ...] \\
        --command CMD --kernel LABEL=[RUN:]SUBSTRING [...] --copy SUBSTRING --copy-bytes N
    python -m gemv_wq_gemm_amd.rocprof_summary pmc OUT_MD CSV [CSV ...] --command CMD --title T \\
        --kernel LABEL=SUBSTRING [...]

``trace`` condenses a ``--kernel-trace --stats`` kernel statistics file into a table of
per-kernel call counts and durations.

``pmc`` tabulates the mean per dispatch of every counter in one or more ``--pmc`` runs
for the labelled kernels.

``counters`` condenses two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of the same
command into HBM bytes per launch for the kernels named by ``--kernel``. The raw
counters are scaled by what they read for a plain copy kernel of known size in the
same run (``--copy``, which reads and writes ``--copy-bytes`` each). The summary ends
with machine-readable ``traffic LABEL BYTES`` lines and the digest of the kernel
sources the counters were taken with; :func:`read_traffic` returns a label's bytes
only while the sources still have that digest.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))

# The files the kernels are built from (and the flags they are built with): counters taken with
# other sources no longer describe the library.
KERNEL_SOURCES = ["csrc/wq_matvec_sliced.hip", "csrc/wq_matvec_mfma.hip", "csrc/wq_matvec.hip", "csrc/wq_gemm.hip",
                  "csrc/wq_decode.hpp", "csrc/wq_internal.hpp", "csrc/wq_lds_dma.hpp", "csrc/wq_moe_sched.hpp",
                  "csrc/wq_tile_math.hpp", "csrc/wq_encoder.hip", "csrc/wq_matvec_q4k.hip", "build.py"]


def source_digest(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _short(name: str, width: int = 88) -> str:
    name = re.sub(r"^void ", "", name)
    name = name.replace("wq::(anonymous namespace)::", "").replace("at::native::", "")
    return name if len(name) <= width else name[: width - 3] + "..."


def trace_summary(stats_csv: str, command: str, out: str, top: int = 16) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        "# Kernel trace statistics",
        "",
        f"Command: `{command}`",
        "",
        "| kernel | calls | mean us | min us | max us | share of GPU time |",
        "|---|---:|---:|---:|---:|---:|",
    ]
    for r in rows[:top]:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as fh:
        fh.write(text)
    return text


def _per_kernel(path: str, counter: str) -> dict[str, list[float]]:
    acc: dict[str, list[float]] = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return acc


def _pick(acc: dict[str, list[float]], sub: str) -> tuple[str, list[float]]:
    hits = [(k, v) for k, v in acc.items() if sub in k]
    if len(hits) != 1:
        raise SystemExit(f"'{sub}' matches {len(hits)} kernels: {[k[:80] for k, _ in hits]}")
    return hits[0]


def counter_summary(runs: list[tuple[str, str]], command: str, out: str, kernels: dict[str, str],
                    copy_sub: str, copy_bytes: int) -> str:
    """HBM bytes per launch of the labelled kernels, from one or more profiled runs (each a FETCH_SIZE
    CSV and a WRITE_SIZE CSV of the same command, each with its own copy calibration). A kernel is
    named ``RUN:SUBSTRING`` (RUN the index of its run, 0 if omitted)."""
    lines = [
        "# HBM bytes per launch (FETCH_SIZE, WRITE_SIZE)",
        "",
        f"Command (each run once with `--pmc FETCH_SIZE`, once with `--pmc WRITE_SIZE`): `{command}`",
        "",
    ]
    scales = []
    data = []
    for i, (fetch_csv, write_csv) in enumerate(runs):
        fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
        write = _per_kernel(write_csv, "WRITE_SIZE")
        _, cf = _pick(fetch, copy_sub)
        _, cw = _pick(write, copy_sub)
        cf_kib, cw_kib = sum(cf) / len(cf), sum(cw) / len(cw)
        f_scale = copy_bytes / (cf_kib * 1024)
        w_scale = copy_bytes / (cw_kib * 1024)
        scales.append((f_scale, w_scale))
        data.append((fetch, write))
        lines.append(f"Run {i} calibration: the copy kernel `{_short(_pick(fetch, copy_sub)[0], 70)}` reads and "
                     f"writes {copy_bytes} bytes; it counts FETCH_SIZE {cf_kib:.1f} KiB and WRITE_SIZE {cw_kib:.1f} "
                     f"KiB per dispatch, so read bytes = {f_scale:.3f} x FETCH_SIZE x 1024 and written bytes = "
                     f"{w_scale:.3f} x WRITE_SIZE x 1024.")
        lines.append("")
    lines += ["| label | run | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes |",
              "|---|---:|---|---:|---:|---:|---:|---:|"]
    tail = []
    for label, spec in kernels.items():
        run, sub = (int(spec.split(":", 1)[0]), spec.split(":", 1)[1]) if ":" in spec and spec.split(":", 1)[0].isdigit() \
            else (0, spec)
        fetch, write = data[run]
        f_scale, w_scale = scales[run]
        name, fv = _pick(fetch, sub)
        _, wv = _pick(write, sub)
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        rd, wr = f_kib * 1024 * f_scale, w_kib * 1024 * w_scale
        lines.append(f"| {label} | {run} | `{_short(name, 60)}` | {len(fv)} | {f_kib:.1f} | {w_kib:.1f} | "
                     f"{rd:.0f} | {wr:.0f} |")
        tail.append(f"traffic {label} {rd + wr:.0f}")
    tail.append(f"source_digest {source_digest()}")
    text = "\n".join(lines) + "\n\n```\n" + "\n".join(tail) + "\n```\n"
    with open(out, "w") as fh:
        fh.write(text)
    return text


def pmc_summary(csvs: list[str], command: str, out: str, kernels: dict[str, str], title: str) -> str:
    """Mean per dispatch of every counter in the ``--pmc`` CSVs, for the labelled kernels."""
    names: list[str] = []
    values: dict[str, dict[str, float]] = {}
    for path in csvs:
        rows = list(csv.DictReader(open(path)))
        for counter in dict.fromkeys(r["Counter_Name"] for r in rows):
            if counter not in names:
                names.append(counter)
            acc: dict[str, list[float]] = defaultdict(list)
            for r in rows:
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
            for label, sub in kernels.items():
                _, vals = _pick(acc, sub)
                values.setdefault(label, {})[counter] = sum(vals) / len(vals)
    lines = [f"# {title}", "", f"Command (one run per pass): `{command}`", "",
             "Mean per dispatch. " + ", ".join(names) + ".", "",
             "| label | kernel | " + " | ".join(names) + " |", "|---|---|" + "---:|" * len(names)]
    for label, sub in kernels.items():
        lines.append(f"| {label} | `{_short(sub, 60)}` | " +
                     " | ".join(f"{values[label][c]:.4g}" for c in names) + " |")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as fh:
        fh.write(text)
    return text


def read_traffic(path: str, label: str) -> float | None:
    """Bytes per launch recorded for ``label``, or None if absent or the kernel sources changed."""
    if not os.path.exists(path):
        return None
    found, digest = None, None
    for line in open(path):
        parts = line.split()
        if len(parts) == 3 and parts[0] == "traffic" and parts[1] == label:
            found = float(parts[2])
        elif len(parts) == 2 and parts[0] == "source_digest":
            digest = parts[1]
    if found is None or digest != source_digest():
        return None
    return found


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--top", type=int, default=16, help="kernels listed, by total time")
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("--run", nargs=2, action="append", required=True, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="one profiled run: its FETCH_SIZE and WRITE_SIZE CSVs (repeat for more runs)")
    c.add_argument("--command", required=True)
    c.add_argument("--kernel", action="append", required=True,
                   help="LABEL=[RUN:]SUBSTRING of the kernel name (RUN: index of its --run, default 0)")
    c.add_argument("--copy", required=True, help="substring of the calibration copy kernel's name")
    c.add_argument("--copy-bytes", type=int, required=True)
    q = sub.add_parser("pmc")
    q.add_argument("out")
    q.add_argument("csvs", nargs="+")
    q.add_argument("--command", required=True)
    q.add_argument("--title", required=True)
    q.add_argument("--kernel", action="append", required=True, help="LABEL=SUBSTRING of the kernel name")
    a = ap.parse_args()
    if a.what == "trace":
        print(trace_summary(a.stats_csv, a.command, a.out, a.top))
    elif a.what == "pmc":
        print(pmc_summary(a.csvs, a.command, a.out, dict(kv.split("=", 1) for kv in a.kernel), a.title))
    else:
        kernels = dict(kv.split("=", 1) for kv in a.kernel)
        print(counter_summary([tuple(r) for r in a.run], a.command, a.out, kernels, a.copy, a.copy_bytes))


if __name__ == "__main__":
    main()
