"""Summaries of rocprofv3 result databases for the three OneTrans kernels.

Reads the SQLite databases rocprofv3 writes (`-d DIR -o run` gives DIR/run_results.db):
  * a `--kernel-trace --stats` run: calls, average and total duration per kernel;
  * two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of the same command: KiB per dispatch;
  * the same two counters for a plain elementwise copy of known size (bench.py
    --copy-calibration), which gives the factor from counter reading to bytes;
  * a `--pmc MfmaUtil VALUBusy SQ_INSTS_VALU_MFMA_MOPS_BF16` (or `_F32`) run: the matrix units'
    busy share per dispatch (rocprofv3's MfmaUtil: MFMA-busy SIMD cycles over the dispatch's GPU
    cycles times the SIMD count), the vector ALUs' busy share, and the MFMA operations executed
    (the counter counts 512 flops per unit).

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

# kernel class -> (substrings of the kernel symbols, source files)
KERNELS = {
    "qkv": (("qkv_kernel",), ("qkv.hip",)),
    "attn": (("attn_kernel", "attn_split_kernel", "attn_pair_kernel"), ("attn.hip",)),
    "post": (("post_kernel", "post_reduce_kernel", "post_f32w_kernel", "post_pair_kernel"),
             ("post.hip", "post_f32w.hip", "post_pair.hip")),
    "lin": (("lin_kernel",), ("tok.hip",)),
    "bwd_gemm": (("gemm_kernel", "reduce_kernel"), ("gemm.hip",)),
    "bwd_attn": (("attn_dkdv_kernel", "attn_dq_kernel"), ("attn_bwd.hip",)),
    "bwd_rows": (("rows_kernel", "colsum_kernel", "transpose_kernel", "fill_kernel"), ("rows.hip",)),
}
COPY_KERNEL = "neg"
MFMA_COUNTERS = ("MfmaUtil", "VALUBusy")
MOPS_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32")


def classify(name: str) -> Optional[str]:
    for k, (subs, _) in KERNELS.items():
        if any(sub in name for sub in subs):
            return k
    return None


def source_sha256(kernel: str) -> str:
    """Hash of the kernel class's source files together with the shared device header."""
    h = hashlib.sha256()
    for f in (*KERNELS[kernel][1], "common.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# Dispatches to leave out, per kernel class: the first SKIP[k] of the run (set-up work that runs
# before the measured steps, e.g. the Stage I that builds an append benchmark's cache).
SKIP: Dict[str, int] = {}


def _kept(dispatches: Dict[int, object], kernel: str) -> Dict[int, object]:
    n = SKIP.get(kernel, 0)
    return {d: dispatches[d] for d in sorted(dispatches)[n:]}


def kernel_stats(db: str) -> Dict[str, Tuple[int, float, float]]:
    """kernel class -> (calls, average ns, total ns) from the kernel-trace run."""
    c = sqlite3.connect(db)
    out: Dict[str, Dict[int, float]] = collections.defaultdict(dict)
    for i, (name, dur) in enumerate(c.execute("select name, duration from kernels order by start")):
        k = classify(name)
        if k:
            out[k][i] = float(dur)
    kept = {k: list(_kept(v, k).values()) for k, v in out.items()}
    return {k: (len(v), sum(v) / len(v), sum(v)) for k, v in kept.items() if v}


def counter_avg(db: str, counter: str, kernel: str) -> Tuple[float, int]:
    """Average per dispatch of `counter` over the dispatches of a kernel class."""
    c = sqlite3.connect(db)
    per: Dict[int, float] = collections.defaultdict(float)
    for disp, name, cname, val in c.execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        if cname == counter and classify(name) == kernel:
            per[disp] += float(val)
    per = _kept(per, kernel)
    if not per:
        return float("nan"), 0
    return sum(per.values()) / len(per), len(per)


def copy_counter(db: str, counter: str) -> Tuple[float, int]:
    """Average per dispatch of `counter` over the calibration copy kernel's dispatches."""
    c = sqlite3.connect(db)
    vals = [float(v) for name, cname, v in c.execute(
        "select kernel_name, counter_name, value from counters_collection") if cname == counter and COPY_KERNEL in name]
    return (sum(vals) / len(vals), len(vals)) if vals else (float("nan"), 0)


def mfma_summary(db: str, kernel: str) -> Optional[Dict[str, float]]:
    """Per kernel class from the MFMA counter run: MfmaUtil and VALUBusy averaged over dispatches
    weighted by duration (percent), executed MFMA flops per dispatch, dispatch count."""
    c = sqlite3.connect(db)
    per: Dict[int, Dict[str, float]] = collections.defaultdict(dict)
    for disp, name, cname, val, dur in c.execute(
            "select dispatch_id, kernel_name, counter_name, value, duration from counters_collection"):
        if classify(name) == kernel:
            per[disp][cname] = float(val)
            per[disp]["_dur"] = float(dur)
    per = _kept(per, kernel)
    if not per:
        return None
    tot = sum(d["_dur"] for d in per.values())
    out = {"dispatches": float(len(per))}
    for cn in MFMA_COUNTERS:
        out[cn] = sum(d.get(cn, 0.0) * d["_dur"] for d in per.values()) / tot
    out["mfma_flops_per_dispatch"] = 512.0 * sum(sum(d.get(cn, 0.0) for cn in MOPS_COUNTERS)
                                                 for d in per.values()) / len(per)
    return out


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
    p.add_argument("--mfma", help="results db of the --pmc MfmaUtil VALUBusy SQ_INSTS_VALU_MFMA_MOPS_* run")
    p.add_argument("--alg-flops", nargs="*", default=[], metavar="CLASS=FLOPS",
                   help="algorithmic flops per dispatch of a kernel class, printed beside the executed ones")
    p.add_argument("--skip", nargs="*", default=[], metavar="CLASS=N",
                   help="leave out the first N dispatches of a kernel class (set-up work before the measured steps)")
    p.add_argument("--workload", default="onetrans_s")
    p.add_argument("--command", required=True, help="the profiled command line, recorded in the summaries")
    p.add_argument("--out-dir", required=True)
    a = p.parse_args()
    SKIP.update({k: int(v) for k, v in (x.split("=") for x in a.skip)})

    stats = kernel_stats(a.stats)
    total = sum(v[2] for v in stats.values())
    f_fetch = f_write = None
    if a.copy_fetch and a.copy_write:
        known_kib = a.copy_mib * 1024.0
        cf, _ = copy_counter(a.copy_fetch, "FETCH_SIZE")
        cw, _ = copy_counter(a.copy_write, "WRITE_SIZE")
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
            fk, nf = counter_avg(a.fetch, "FETCH_SIZE", k)
            wk, nw = counter_avg(a.write, "WRITE_SIZE", k)
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
        if a.mfma:
            mf = mfma_summary(a.mfma, k)
            if mf is not None:
                alg = dict(x.split("=") for x in a.alg_flops).get(k)
                lines += ["Counters (separate `--pmc MfmaUtil VALUBusy SQ_INSTS_VALU_MFMA_MOPS_*` run of the same command):",
                          "",
                          f"- MfmaUtil (matrix units busy, duration-weighted over {int(mf['dispatches'])} dispatches): "
                          f"{mf['MfmaUtil']:.1f} %",
                          f"- VALUBusy (vector ALUs busy): {mf['VALUBusy']:.1f} %",
                          f"- MFMA flops executed per dispatch: {mf['mfma_flops_per_dispatch'] / 1e9:.2f} GFLOP"]
                if alg and float(alg) > 0:
                    lines.append(f"- algorithmic flops per dispatch: {float(alg) / 1e9:.2f} GFLOP "
                                 f"(executed / algorithmic = {mf['mfma_flops_per_dispatch'] / float(alg):.3f})")
                lines.append("")
        with open(os.path.join(a.out_dir, f"{k}_kernel_{a.workload}.md"), "w") as f:
            f.write("\n".join(lines))
        print("\n".join(lines))


if __name__ == "__main__":
    main()
