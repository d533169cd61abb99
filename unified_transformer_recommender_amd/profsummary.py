"""Summaries of rocprofv3 result databases for the three OneTrans kernels.

Reads the SQLite databases rocprofv3 writes (`-d DIR -o run` gives DIR/run_results.db):
  * a `--kernel-trace --stats` run: calls, average and total duration per kernel;
  * two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of the same command: KiB per dispatch;
  * the same two counters for a plain elementwise copy of known size (bench.py
    --copy-calibration), which gives the factor from counter reading to bytes.

`python -m unified_transformer_recommender_amd.profsummary --help` lists the inputs; it prints
one markdown summary per kernel class into --out-dir and a traffic record per kernel class that
bench.py reads back (with the sha256 of the kernel's source file, so that a record taken on a
different kernel version is ignored).
"""

from __future__ import annotations

import argparse
import collections
import hashlib
import os
import sqlite3
from typing import Dict, List, Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# kernel class -> (substring of the kernel symbol, source file)
KERNELS = {
    "qkv": ("qkv_kernel", "qkv.hip"),
    "attn": ("attn_kernel", "attn.hip"),
    "post": ("post_kernel", "post.hip"),
    "lin": ("lin_kernel", "tok.hip"),
}
COPY_KERNEL = "neg"


def classify(name: str) -> Optional[str]:
    for k, (sub, _) in KERNELS.items():
        if sub in name:
            return k
    return None


def source_sha256(kernel: str) -> str:
    """Hash of the kernel's source file together with the shared device header."""
    h = hashlib.sha256()
    for f in (KERNELS[kernel][1], "common.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_stats(db: str) -> Dict[str, Tuple[int, float, float]]:
    """kernel class -> (calls, average ns, total ns) from the kernel-trace run."""
    c = sqlite3.connect(db)
    out: Dict[str, List[float]] = collections.defaultdict(list)
    for name, dur in c.execute("select name, duration from kernels"):
        k = classify(name)
        if k:
            out[k].append(float(dur))
    return {k: (len(v), sum(v) / len(v), sum(v)) for k, v in out.items()}


def counter_avg(db: str, counter: str, match) -> Tuple[float, int]:
    """Average per dispatch of `counter` over dispatches whose kernel name satisfies `match`."""
    c = sqlite3.connect(db)
    per: Dict[int, float] = collections.defaultdict(float)
    for disp, name, cname, val in c.execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        if cname == counter and match(name):
            per[disp] += float(val)
    if not per:
        return float("nan"), 0
    return sum(per.values()) / len(per), len(per)


def write_traffic(path: str, kernel: str, workload: str, fetch_kib: float, write_kib: float,
                  f_fetch: float, f_write: float, command: str) -> None:
    with open(path, "w") as f:
        f.write(f"# HBM traffic per launch of {kernel}_kernel, workload {workload}\n")
        f.write(f"# from: {command}\n")
        f.write(f"kernel = {kernel}\n")
        f.write(f"workload = {workload}\n")
        f.write(f"source_sha256 = {source_sha256(kernel)}\n")
        f.write(f"fetch_kib_per_launch = {fetch_kib:.3f}\n")
        f.write(f"write_kib_per_launch = {write_kib:.3f}\n")
        f.write(f"fetch_scale = {f_fetch:.6f}\n")
        f.write(f"write_scale = {f_write:.6f}\n")
        f.write(f"traffic_bytes_per_launch = {1024.0 * (fetch_kib * f_fetch + write_kib * f_write):.0f}\n")


def read_traffic(path: str) -> Optional[Dict[str, str]]:
    """The record at `path` if it exists and matches the current kernel source, else None."""
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
    k = rec.get("kernel")
    if k not in KERNELS or rec.get("source_sha256") != source_sha256(k):
        return None
    return rec


def main() -> None:
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--stats", required=True, help="results db of the --kernel-trace --stats run")
    p.add_argument("--fetch", help="results db of the --pmc FETCH_SIZE run")
    p.add_argument("--write", help="results db of the --pmc WRITE_SIZE run")
    p.add_argument("--copy-fetch", help="results db of FETCH_SIZE over bench.py --copy-calibration")
    p.add_argument("--copy-write", help="results db of WRITE_SIZE over bench.py --copy-calibration")
    p.add_argument("--copy-mib", type=int, default=1024, help="MiB the copy calibration read and wrote")
    p.add_argument("--workload", default="onetrans_s")
    p.add_argument("--command", required=True, help="the profiled command line, recorded in the summaries")
    p.add_argument("--out-dir", required=True)
    a = p.parse_args()

    stats = kernel_stats(a.stats)
    total = sum(v[2] for v in stats.values())
    f_fetch = f_write = None
    if a.copy_fetch and a.copy_write:
        known_kib = a.copy_mib * 1024.0
        cf, _ = counter_avg(a.copy_fetch, "FETCH_SIZE", lambda n: COPY_KERNEL in n)
        cw, _ = counter_avg(a.copy_write, "WRITE_SIZE", lambda n: COPY_KERNEL in n)
        f_fetch, f_write = known_kib / cf, known_kib / cw
    os.makedirs(a.out_dir, exist_ok=True)
    for k, (calls, avg, tot) in sorted(stats.items(), key=lambda kv: -kv[1][2]):
        lines = [f"# {k}_kernel — workload {a.workload}", "",
                 "Command (rocprofv3 kernel trace with statistics):", "",
                 "```", a.command, "```", "",
                 "| kernel | calls | average duration (us) | total (ms) | share of traced kernel time |",
                 "|---|---|---|---|---|",
                 f"| {k}_kernel | {calls} | {avg / 1e3:.2f} | {tot / 1e6:.3f} | {100.0 * tot / total:.1f} % |", ""]
        if a.fetch and a.write:
            fk, nf = counter_avg(a.fetch, "FETCH_SIZE", lambda n, k=k: KERNELS[k][0] in n)
            wk, nw = counter_avg(a.write, "WRITE_SIZE", lambda n, k=k: KERNELS[k][0] in n)
            lines += ["Counters (separate `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE` runs of the same command):", "",
                      f"- FETCH_SIZE: {fk:.1f} KiB per dispatch ({nf} dispatches)",
                      f"- WRITE_SIZE: {wk:.1f} KiB per dispatch ({nw} dispatches)"]
            if f_fetch is not None:
                byts = 1024.0 * (fk * f_fetch + wk * f_write)
                lines += [f"- copy-kernel scale factors (known bytes / counter bytes): fetch {f_fetch:.4f}, write {f_write:.4f}",
                          f"- HBM traffic per launch: {byts / 1e6:.2f} MB",
                          f"- traffic over average launch duration: {byts / (avg * 1e-9) / 1e9:.1f} GB/s"]
                write_traffic(os.path.join(a.out_dir, f"traffic_{k}_{a.workload}.txt"), k, a.workload,
                              fk, wk, f_fetch, f_write, a.command)
            lines.append("")
        with open(os.path.join(a.out_dir, f"{k}_kernel_{a.workload}.md"), "w") as f:
            f.write("\n".join(lines))
        print("\n".join(lines))


if __name__ == "__main__":
    main()
