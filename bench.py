"""Benchmark of the OneTrans hot path on one MI355X.

Default workload: the OneTransS-shaped forward (6 blocks, d=256, 8 heads, FFN 1024, L_S=1190,
L_NS=16, pyramid 1190 -> 12, batch 256, bf16 storage with fp32 accumulation). One step is one
onetrans_forward call over the whole batch: every block's norm, mixed Q/K/V projection, causal
pyramid attention, output projection and mixed FFN. The metric is candidates scored per second
(each batch row is one candidate carrying its own user sequence) plus the fraction of bf16 MFMA
peak that the algorithmic FLOPs reach.

Other workloads (--workload two_stage | append | append_ragged | onetrans_l | tokenize_s) print their
own line; they are parity cases of the same kernels (tokenize_s: the tokenizers that build X(0)) and
are measured for the design notes, not as the headline.

Timing: W untimed warm-up steps, then K timed steps between a device synchronisation on both
sides (one GPU, so no barrier is needed). Inputs and weights are resident in HBM before the
timed region starts. The library runs large batches as two concurrent halves on two streams
(--streams 2, the default), so per-kernel device time comes from a separate pass after the timed
region with one stream, from hipEvents the library records around each launch (--streams 1 times
and traces the same single-stream run). The CPU baseline times the fp64 oracle on a bounded sample
of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 (matrix and packed vector)
PEAK_HBM_GBS = 8000.0
METRIC = "candidates scored/sec at 1 GPU (OneTransS shape) + % bf16 MFMA peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="onetrans_s",
                   choices=["onetrans_s", "two_stage", "append", "append_ragged", "append_pyramid", "onetrans_l",
                            "train_s", "tokenize_s", "tokenize_s_time"])
    p.add_argument("--dtype", default=None, choices=[None, "bf16", "f32"])
    p.add_argument("--no-trace", action="store_true", help="no per-kernel events in the timed region")
    p.add_argument("--streams", type=int, default=2, choices=[1, 2, 4],
                   help="streams of the batched calls: 2 runs a forward batch / an append's users as two "
                        "concurrent halves (per-kernel timing then comes from a separate one-stream pass); 1 "
                        "runs everything on one stream")
    p.add_argument("--separate-append", action="store_true",
                   help="append workloads: time the append and Stage II as two calls, not the fused call")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline (0: skip)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain elementwise copy of MIB MiB (fp32 negate: reads and writes MIB MiB "
                        "once each), to scale the FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    return p.parse_args()


def copy_calibration(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch neg (fp32, elementwise)", "launches": 3,
                                           "read_bytes_per_launch": n * 4, "write_bytes_per_launch": n * 4}}))


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def host_info() -> dict:
    """CPU model (from /proc/cpuinfo) and the BLAS library NumPy calls (vendor, version, threads)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', 'threads')}, " \
                   f"{i.get('num_threads')} threads, {i.get('architecture')})"
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


def roofline_entry(name, work, ms, launches, peak, unit, bound):
    achieved = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    return {"kernel": name, "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None, "avg_launch_us": round(1e3 * ms / max(launches, 1), 2),
            "launches": launches}


def kernel_table(classes, timing, steps, n_units, peak_tflops):
    """Per class: algorithmic flops per step over measured device time per step."""
    out = {}
    for k, (ms, cnt) in timing.items():
        if cnt == 0:
            continue
        ms_step = ms / steps
        tf = classes[k] * n_units / (ms_step * 1e-3) / 1e12
        out[k] = {"ms_per_step": round(ms_step, 4), "TFLOP/s": round(tf, 2), "frac_mfma": round(tf / peak_tflops, 4),
                  "launches_per_step": cnt // steps}
    return out


def dominant(classes, timing, steps, n_units, peak_tflops, workload):
    k = max((c for c in timing if timing[c][1] > 0), key=lambda c: timing[c][0])
    ms, cnt = timing[k]
    entry = roofline_entry(k, classes[k] * n_units * steps, ms, cnt, peak_tflops, "TFLOP/s", "mfma")
    # HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this
    # kernel and workload, scaled by the copy-kernel calibration; null when that record was taken
    # on a different version of the kernel source.
    from unified_transformer_recommender_amd import profsummary
    rec = profsummary.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{k}_{workload}.txt"))
    if rec is not None:
        entry["traffic"] = float(rec["traffic_bytes_per_launch"])
    return entry


def bench_tokenize(a):
    """The tokenizers ahead of block 1 (behaviour MLPs, [SEP] merge, Auto-Split): samples/s, HBM-bound."""
    from dataclasses import replace

    import numpy as np
    import torch

    import synth
    from unified_transformer_recommender_amd import binding as ob
    from unified_transformer_recommender_amd import costmodel as cm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = synth.tok_workload(a.workload, a.dtype)
    m = w.model
    store_bytes = 2 if m.dtype == "bf16" else 4
    t_setup = time.time()
    one = replace(m, n_blocks=1)
    model = ob.Model.from_host(one, (w.l_s,), synth.make_weights(one), device=dev)
    ob.set_streams(a.streams)
    tw = synth.tokenizer_weights(w)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev, dtype=model.torch_dtype)
    tok = ob.Tokenizer(model, w.seq_lens, [{k: up(v) for k, v in p.items()} for p in tw["seq"]], up(tw["sep"]),
                       {k: up(v) for k, v in tw["ns"].items()} if tw["ns"] is not None else None, merge=w.merge)
    ev, ns = synth.tokenizer_batch(w)
    evd, nsd = [up(e) for e in ev], up(ns)
    tmd = [torch.from_numpy(t).to(dev) for t in synth.tokenizer_times_batch(w)] if w.merge == "time" else None
    x0 = torch.empty((w.batch, w.l_s + m.l_ns, m.d_model), dtype=model.torch_dtype, device=dev)
    wsp = tok.workspace(w.batch)
    stream = torch.cuda.current_stream(dev)

    def step():
        ob.onetrans_tokenize(tok, evd, nsd, x0, wsp, times=tmd)

    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ob.timing_read()
    ob.timing_enable(not a.no_trace)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    ob.timing_enable(False)
    timing = ob.timing_read()
    ms_step = e0.elapsed_time(e1) / a.steps
    flops, act, wts = cm.tokenize_work(m.d_model, m.l_ns, w.seq_lens, w.seq_dims, w.seq_hidden, w.ns_dim,
                                       w.ns_hidden, store_bytes, w.merge)
    lin_ms, lin_n = timing["lin"]
    lin_bytes = (act * w.batch + wts) * a.steps           # every linear launch of the timed steps
    roof = roofline_entry("lin", lin_bytes, lin_ms, lin_n, PEAK_HBM_GBS, "GB/s", "hbm") if lin_n else None
    if roof is not None:
        from unified_transformer_recommender_amd import profsummary
        rec = profsummary.read_traffic(os.path.join(ROOT, "profiles", f"traffic_lin_{w.key}.txt"))
        if rec is not None:
            roof["traffic"] = float(rec["traffic_bytes_per_launch"])
        roof["tflops"] = round(flops * w.batch * a.steps / (lin_ms * 1e-3) / 1e12, 2)
    cpu = None
    if a.cpu_seconds > 0:
        import oracle as O
        t0 = time.perf_counter()
        done = 0
        while done < 256 and (time.perf_counter() - t0 < a.cpu_seconds or done < 2):
            e_b, n_b = synth.tokenizer_sample(w, done)
            O.tokenize(e_b, n_b, tw, m.l_ns, times=synth.tokenizer_times(w, done) if w.merge == "time" else None)
            done += 1
        cpu_s = time.perf_counter() - t0
        cpu = {"value": round(done / cpu_s, 4), "unit": "samples/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"{done} samples of the same workload, one at a time (input generation included)",
               "seconds": round(cpu_s, 2), **host_info()}
    kernels = {k: {"ms_per_step": round(ms / a.steps, 4), "launches_per_step": n // a.steps}
               for k, (ms, n) in timing.items() if n}
    print(json.dumps({
        "metric": f"samples tokenized/sec at 1 GPU ({w.key})",
        "value": round(w.batch / (ms_step * 1e-3), 2),
        "unit": "samples/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": m.dtype,
        "data": "synthetic (seeded N(0,1) raw events and NS features, N(0,1/fan_in) MLP weights)",
        "config": {"workload": w.description, "batch": w.batch, "seq_lens": list(w.seq_lens),
                   "seq_dims": list(w.seq_dims), "seq_hidden": list(w.seq_hidden), "ns_dim": w.ns_dim,
                   "ns_hidden": w.ns_hidden, "l_ns": m.l_ns, "d_model": m.d_model},
        "tflops": round(flops * w.batch / (ms_step * 1e-3) / 1e12, 2),
        "hbm_GB/s": round((act * w.batch + wts) / (ms_step * 1e-3) / 1e9, 1),
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
        "trace_in_timed_region": not a.no_trace, "setup_s": round(t_setup, 1),
        "wall_ms_per_step": round(wall / a.steps, 4),
    }))


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {a.gpus}); samples are independent, "
              "so N GPUs would each run this same per-GPU step on their own share of the batch.", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.workload.startswith("tokenize_s"):
        bench_tokenize(a)
        return

    import numpy as np
    import torch

    import synth
    from unified_transformer_recommender_amd import binding as ob
    from unified_transformer_recommender_amd import costmodel as cm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = synth.workload(a.workload, a.dtype)
    m = w.model
    store_bytes = 2 if m.dtype == "bf16" else 4
    peak = PEAK_BF16_TFLOPS if m.dtype == "bf16" else PEAK_FP32_TFLOPS
    t_setup = time.time()
    host_w = synth.make_weights(m)
    # append workloads: the schedule the cached rows were prefilled with (the plain append caches
    # are unpyramided; append_pyramid keeps the OneTransS pyramid over its 1158 cached rows)
    pyramid_append = w.kind == "append" and w.s_queries[0] == w.l_old and len(set(w.s_queries)) > 1
    sched = w.s_queries if w.kind != "append" or pyramid_append else (w.l_old,) * m.n_blocks
    model = ob.Model.from_host(m, sched, host_w, device=dev)
    ob.set_streams(a.streams)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev, dtype=model.torch_dtype)

    stream = torch.cuda.current_stream(dev)
    extra = {}
    if w.kind == "forward":
        x0 = up(synth.forward_batch(w))
        out = torch.empty((w.batch, w.s_queries[-1] + m.l_ns, m.d_model), dtype=torch.float32, device=dev)
        wsp = model.workspace(ob.L.OP_FORWARD, w.batch, w.l_s)
        n_units = w.batch
        classes = cm.forward_classes(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries, store_bytes)

        def step():
            ob.onetrans_forward(model, x0, out, wsp)
    elif w.kind == "train":
        x0 = up(synth.forward_batch(w))
        d_out = torch.from_numpy(synth.grad_out_batch(w)).to(dev)
        out = torch.empty((w.batch, w.s_queries[-1] + m.l_ns, m.d_model), dtype=torch.float32, device=dev)
        dx0 = torch.empty((w.batch, w.l_s + m.l_ns, m.d_model), dtype=torch.float32, device=dev)
        grads = ob.grad_buffers(model)
        wsp = ob.backward_workspace(model, w.batch, w.l_s)
        n_units = w.batch
        classes = cm.train_classes(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries)
        extra["workspace_GiB"] = round(wsp.numel() / 2**30, 2)

        def step():
            ob.onetrans_backward(model, x0, d_out, grads=grads, ws=wsp, out=out, dx0=dx0)
    elif w.kind == "two_stage":
        xs = up(synth.user_sequences(w))
        xn = up(synth.candidate_batch(w))
        cache = ob.KVCache(model, w.n_users, w.l_s)
        out = torch.empty((w.n_users, w.n_cand, m.l_ns, m.d_model), dtype=torch.float32, device=dev)
        ws1 = model.workspace(ob.L.OP_PREFILL, w.n_users, w.l_s)
        ws2 = model.workspace(ob.L.OP_SCORE, w.n_users, n_cand=w.n_cand)
        n_units = w.n_users * w.n_cand
        pre = cm.prefill_classes(m.d_model, m.d_ff, w.l_s, w.s_queries, store_bytes)
        sc = cm.score_classes(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries, store_bytes)
        classes = {k: (pre[k] * w.n_users + sc[k] * n_units) / n_units for k in sc}

        def step(mark=None):   # mark: an event recorded between Stage I and Stage II
            ob.onetrans_prefill_user(model, xs, cache, None, ws1)
            if mark is not None:
                mark.record(stream)
            ob.onetrans_score_candidates(model, cache, xn, out, ws2)
    else:   # append: restore the pristine cache (untimed), then append + score the user's NS tokens
        old, new = synth.append_batch(w)
        xo, xnw = up(old), up(new)
        xn = up(np.stack([synth.candidate_tokens(w, u, 0) for u in range(w.n_users)])[:, None])
        # ragged users: user u's cached rows are the first lens[u] rows (the rest of `old` pads)
        lens = synth.user_cached_lengths(w) if w.l_old_min else None
        pristine = ob.KVCache(model, w.n_users, w.l_s, user_len=lens, x_tail=pyramid_append)
        ob.onetrans_prefill_user(model, xo, pristine)
        cache = ob.KVCache(model, w.n_users, w.l_s, user_len=lens, x_tail=pyramid_append)
        n_units = w.n_users
        classes = {}
        if pyramid_append:
            grown = cm.grown_schedule(w.l_old, sched, w.d_l)
            q_final = min(w.d_l, grown[-1])
            ap = cm.pyramid_append_classes(m.d_model, m.d_ff, w.l_old, w.d_l, sched, store_bytes, out_rows=q_final)
            sc = cm.score_classes(m.d_model, m.d_ff, m.l_ns, w.l_old + w.d_l, grown, store_bytes)
            classes = {k: ap[k] + sc[k] for k in sc}
        else:
            q_final = w.d_l
            for l_old in (lens or [w.l_old]):   # per-user work, averaged over the users
                ap = cm.append_classes(m.d_model, m.d_ff, m.n_blocks, l_old, w.d_l, store_bytes)
                sc = cm.score_classes(m.d_model, m.d_ff, m.l_ns, l_old + w.d_l, (l_old + w.d_l,) * m.n_blocks,
                                      store_bytes)
                for k in sc:
                    classes[k] = classes.get(k, 0.0) + (ap[k] + sc[k]) / len(lens or [w.l_old])
        out_new = torch.empty((w.n_users, q_final, m.d_model), dtype=torch.float32, device=dev)
        out = torch.empty((w.n_users, 1, m.l_ns, m.d_model), dtype=torch.float32, device=dev)
        # one call for both (each block's attention reads the cache once) where it applies: no pyramid,
        # at most 32 new rows and 32 NS rows per user
        fused = not pyramid_append and not a.separate_append and w.d_l <= 32 and m.l_ns <= 32
        extra["append_call"] = "append_score" if fused else "append_events + score_candidates"
        if fused:
            ws1 = model.workspace(ob.L.OP_APPEND_SCORE, w.n_users, n_cand=1, d_l=w.d_l)
        else:
            ws1 = model.workspace(ob.L.OP_APPEND, w.n_users, l_s=pristine.append_window(), d_l=w.d_l)
            ws2 = model.workspace(ob.L.OP_SCORE, w.n_users, n_cand=1)
        restore_ms = []

        def step():
            if fused:
                ob.onetrans_append_score(model, cache, xnw, xn, out_new, out, ws1)
                return
            ob.onetrans_append_events(model, cache, xnw, out_new, ws1)
            ob.onetrans_score_candidates(model, cache, xn, out, ws2)

        def restore():
            cache.copy_(pristine)

    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    # warm-up
    for _ in range(a.warmup):
        if w.kind == "append":
            restore()
        step()
    torch.cuda.synchronize()
    ob.timing_read()                        # drop anything recorded so far

    # timed region. With two forward streams a launch's duration overlaps the other half's kernels,
    # so the per-kernel table (and the roofline) comes from a separate one-stream pass.
    trace_in = not a.no_trace and a.streams == 1
    ob.timing_enable(trace_in)
    total_ms = 0.0
    per_step = []   # each step's own event interval (ms)
    if w.kind == "append":
        # the cache restore between steps is outside the timed intervals
        for _ in range(a.steps):
            restore()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            per_step.append(e0.elapsed_time(e1))
        total_ms = sum(per_step)
    else:
        # one event between consecutive steps (recording it adds no work to the stream)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
        mids = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)] if w.kind == "two_stage" else None
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(a.steps):
            if mids is not None:
                step(mids[i])
            else:
                step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        total_ms = max(evs[0].elapsed_time(evs[-1]), 0.0)
        per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps)]
        extra["wall_ms_per_step"] = round(wall / a.steps, 4)
        if mids is not None:
            extra["stage_ms_per_step"] = {
                "prefill_user": round(sum(evs[i].elapsed_time(mids[i]) for i in range(a.steps)) / a.steps, 4),
                "score_candidates": round(sum(mids[i].elapsed_time(evs[i + 1]) for i in range(a.steps)) / a.steps, 4)}
    q = np.percentile(np.asarray(per_step, np.float64), [10, 50, 90])
    extra["ms_step_p10_median_p90"] = [round(float(v), 4) for v in q]
    ob.timing_enable(False)
    timing = ob.timing_read()
    ms_step = total_ms / a.steps
    if not trace_in:
        # per-kernel table from a separate traced pass (one stream) after the timed region
        ob.set_streams(1)
        ob.timing_enable(True)
        for _ in range(a.steps):
            if w.kind == "append":
                restore()
            step()
        torch.cuda.synchronize()
        ob.timing_enable(False)
        timing = ob.timing_read()
        ob.set_streams(a.streams)
    value = n_units / (ms_step * 1e-3)

    flops_unit = sum(classes.values())
    mfma_frac = flops_unit * n_units / (ms_step * 1e-3) / 1e12 / peak
    kernels = kernel_table(classes, timing, a.steps, n_units, peak)
    roof = dominant(classes, timing, a.steps, n_units, peak, w.key)

    # CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if a.cpu_seconds > 0:
        import oracle as O
        t0 = time.perf_counter()
        done = 0
        if w.kind == "forward":
            while done < 64 and (time.perf_counter() - t0 < a.cpu_seconds or done < 2):
                O.forward(synth.forward_sample(w, done), host_w, m, w.s_queries)
                done += 1
            sample = f"{done} samples of the same workload, one at a time"
            units = done
        elif w.kind == "train":
            while done < 16 and (time.perf_counter() - t0 < a.cpu_seconds or done < 1):
                O.backward(synth.forward_sample(w, done), host_w, m, w.s_queries, synth.grad_out_sample(w, done))
                done += 1
            sample = f"{done} samples' forward and backward, one at a time"
            units = done
        elif w.kind == "two_stage":
            cache_o, _ = O.prefill_user(synth.user_sequence(w, 0), host_w, m, w.s_queries)
            while done < 2048 and (time.perf_counter() - t0 < a.cpu_seconds or done < 4):
                O.score_candidate(cache_o, synth.candidate_tokens(w, 0, done), host_w, m)
                done += 1
            sample = f"Stage I of user 0 plus Stage II of {done} of its candidates, both timed"
            units = done
        elif pyramid_append:
            # the oracle's definition: Stage I of the longer sequence under the grown pyramid
            t_app = 0.0
            while done < min(64, w.n_users) and (time.perf_counter() - t0 < a.cpu_seconds or done < 2):
                o, nw = synth.append_rows(w, done)
                t1 = time.perf_counter()
                O.append_recompute(o, nw, host_w, m, sched)
                t_app += time.perf_counter() - t1
                done += 1
            sample = f"{done} users' appends, each recomputed as the oracle defines it"
            units = done
        else:
            t_app = 0.0
            ul = synth.user_cached_lengths(w)
            while done < min(64, w.n_users) and (time.perf_counter() - t0 < a.cpu_seconds or done < 2):
                o, nw = synth.append_rows(w, done)
                o = o[: ul[done]]
                co, _ = O.prefill_user(o, host_w, m, (ul[done],) * m.n_blocks)
                t1 = time.perf_counter()
                O.append_events(co, nw, host_w, m)
                t_app += time.perf_counter() - t1
                done += 1
            sample = f"{done} users' appends (their Stage I prefill runs untimed)"
            units = done
        cpu_s = time.perf_counter() - t0 if w.kind != "append" else t_app
        cpu = {"value": round(units / cpu_s, 4),
               "unit": {"append": "users/s", "train": "samples/s"}.get(w.kind, "candidates/s"),
               "cores": blas_threads(), "kind": "oracle", "sample": sample, "seconds": round(cpu_s, 2),
               **host_info()}

    unit = {"append": "user appends/s", "train": "training samples/s"}.get(w.kind, "candidates/s")
    metric = METRIC if w.key == "onetrans_s" else f"{unit} at 1 GPU ({w.key})"
    if w.kind == "train":
        metric = f"{unit} at 1 GPU ({w.key}: forward keeping block inputs + backward with recomputation)"
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m.dtype,
        "data": "synthetic (seeded N(0,1) inputs with shared [SEP] rows, N(0,0.02^2) weights)",
        "config": {"workload": w.description, "batch": w.batch or None, "n_users": w.n_users or None,
                   "n_cand": w.n_cand or None, "l_s": w.l_s, "l_ns": m.l_ns, "s_queries": list(sched),
                   "n_blocks": m.n_blocks, "d_model": m.d_model, "n_heads": m.n_heads, "d_ff": m.d_ff},
        "mfma_frac": round(mfma_frac, 4),
        "tflops": round(flops_unit * n_units / (ms_step * 1e-3) / 1e12, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "trace_in_timed_region": trace_in,
        "streams": a.streams,
        "kernel_table": "timed region" if trace_in else "separate one-stream pass",
        "setup_s": round(t_setup, 1),
        **extra,
    }
    if w.kind == "append" and not pyramid_append:
        byts = sum(cm.append_cache_bytes(m.d_model, m.n_blocks, l_old, w.d_l, store_bytes)
                   for l_old in (synth.user_cached_lengths(w)))
        line["cache_GB/s"] = round(byts / (ms_step * 1e-3) / 1e9, 1)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
