#!/usr/bin/env python3
"""Benchmark of the verify + E2E-TV-loss hot path on one MI355X.

One step = one pass of the whole hot path at V = 151936:
  * spec_verify on the B=64, K=7, V=151936 bf16 Zipf workload at T = 0, 0.6
    and 1.0 (three calls, 3 x 512 verified vocab-rows), and
  * e2e_tv_loss_fwd_bwd on N=512 branches x W=7 positions, V=151936
    (3584 vocab-rows).
Inputs are synthetic (seeded generators), resident in HBM before the timed
region. Each temperature's call reads its own copy of the logits, and the
4.4 GB loss pass runs between them, so no call is served from the 256 MB
last-level cache by the previous one.

Prints one JSON line: the metric (verified vocab-rows/s over the step), the
roofline of the dominant kernel (the loss), timed live inside the timed steps
with a pair of HIP events around the loss call on the stream the kernels run
on, and the CPU oracle timed on the step's own inputs.

Per-call times (the step's components, the variants, the small workloads,
and a sweep of the loss and the sampling verify over three other
vocabularies, one of them not a multiple of 8) are medians over many calls, each call bracketed by its own pair of events
with a 1 GiB write between calls outside the brackets, so that no call is
served from the 256 MB last-level cache by the one before it. The step's
components also carry batched times: the median over 5 batches of
back-to-back calls of the batch time per call, the verify inputs rotated
over 4 copies (4 x 292 MB) for the same reason.

``python bench.py --trace-summary <kernel_trace.csv>`` prints per-kernel
launch statistics from a rocprofv3 kernel trace, and the per-launch medians
of the bench steps found in it (no GPU needed).
``python bench.py --traffic <fetch.csv> <write.csv>`` writes
profiles/traffic.json from two rocprofv3 --pmc runs of this script
(FETCH_SIZE, then WRITE_SIZE, with --copy-calibration; no GPU needed).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
VOCAB = 151936
VERIFY_B, VERIFY_K = 64, 7
LOSS_N, LOSS_W = 512, 7
TEMPS = (0.0, 0.6, 1.0)


def kernel_source_hash():
    """Hash of the HIP sources: traffic counters are only reported for the
    kernel build they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lossless_verify_tv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def verify_bytes(k_per_req, vocab, elem=2):
    return int(sum((2 * int(k) + 1) * vocab * elem for k in k_per_req))


def loss_bytes(n, w, vocab):
    return 8 * n * w * vocab


_POOL = {}


def _verify_task(task):
    """Worker: the oracle on requests [b0, b1) of verify case ci."""
    from oracle import verify as ov
    ci, b0, b1 = task
    case = _POOL["vcases"][ci]
    out = []
    for b in range(b0, b1):
        r = ov.verify_request(ov.decode_rows(case.target[b], case.dtype),
                              ov.decode_rows(case.draft[b], case.dtype), case.tokens[b],
                              case.k[b], case.temperature[b], int(case.seed[b]), b,
                              case.shape[1])
        out.append((ci, b, r["accepted_len"], r["tokens"], r["accept_margin"],
                    r["draw_margin"], r["greedy"]))
    return out


def _loss_task(task):
    """Worker: the oracle on loss branches [n0, n1)."""
    from oracle import bf16 as obf16
    from oracle import loss as ol
    n0, n1 = task
    lc = _POOL["lcase"]
    for n in range(n0, n1):
        ol.branch(obf16.decode(lc.draft_logits[n]), lc.target_probs[n], LOSS_N)
    return n1 - n0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(verify_cases, loss_case, gpu_verify, workers):
    """Time the fp64 oracle, as it stands, on the step's own inputs (every
    request of each temperature's verify call and every branch of the loss
    call, about 30 s of single-thread work), in two ways: one process with
    one thread, and a pool of `workers` processes over requests and branches
    (the arrays reach the workers by fork). The headline value is the pool's
    (every core the host gives); the single-thread rate is reported beside
    it. The pool's verify results are also compared with the GPU outputs of
    the same calls: differing requests whose oracle decision margin is below
    1e-6 are counted as excused, any other difference as a mismatch."""
    from concurrent.futures import ProcessPoolExecutor

    sys.path.insert(0, ROOT)
    from oracle import bf16 as obf16
    from oracle import loss as ol
    from oracle import verify as ov

    rows_v = sum(int(k) + 1 for c in verify_cases for k in c.k)
    rows_l = LOSS_N * LOSS_W
    # one process, one thread
    t0 = time.perf_counter()
    for case in verify_cases:
        for b in range(case.shape[0]):
            ov.verify_request(ov.decode_rows(case.target[b], case.dtype),
                              ov.decode_rows(case.draft[b], case.dtype), case.tokens[b],
                              case.k[b], case.temperature[b], int(case.seed[b]), b,
                              case.shape[1])
    t_v1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    for n in range(LOSS_N):
        ol.branch(obf16.decode(loss_case.draft_logits[n]), loss_case.target_probs[n], LOSS_N)
    t_l1 = time.perf_counter() - t0
    # a pool of processes
    _POOL["vcases"], _POOL["lcase"] = verify_cases, loss_case
    try:
        with ProcessPoolExecutor(max_workers=workers) as pool:
            t0 = time.perf_counter()
            vres = [r for part in pool.map(
                _verify_task, [(ci, b, b + 1) for ci, c in enumerate(verify_cases)
                               for b in range(c.shape[0])]) for r in part]
            t_vp = time.perf_counter() - t0
            t0 = time.perf_counter()
            done = sum(pool.map(_loss_task, [(n, min(LOSS_N, n + 4))
                                             for n in range(0, LOSS_N, 4)]))
            t_lp = time.perf_counter() - t0
    finally:
        _POOL.clear()
    assert done == LOSS_N
    # parity of the step's verify outputs against the pool's oracle results
    par = {"requests": 0, "identical": 0, "excused_accept": 0, "excused_draw": 0,
           "mismatched": 0}
    for ci, b, j_o, t_o, am, dm, greedy in vres:
        acc, toks = gpu_verify[ci]
        j_g, t_g = int(acc[b]), np.asarray(toks[b])
        par["requests"] += 1
        if j_g == j_o and np.array_equal(t_g, t_o):
            par["identical"] += 1
        elif not greedy and j_g != j_o and 0 <= min(j_g, j_o) < len(am) \
                and am[min(j_g, j_o)] < 1e-6:
            par["excused_accept"] += 1
        elif not greedy and j_g == j_o and dm < 1e-6:
            par["excused_draw"] += 1
        else:
            par["mismatched"] += 1

    def rate(tv, tl):
        step_rows_v = len(verify_cases) * VERIFY_B * (VERIFY_K + 1)
        return (step_rows_v + rows_l) / (step_rows_v * tv / rows_v + rows_l * tl / rows_l)

    return {
        "value": rate(t_vp, t_lp),
        "unit": "vocab-rows/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"the step's own inputs: every request of the {len(verify_cases)} verify "
                   f"calls ({rows_v} vocab-rows) and all {LOSS_N} loss branches ({rows_l} "
                   f"vocab-rows), fp64 numpy; a pool of {workers} processes took "
                   f"{t_vp:.1f} s + {t_lp:.1f} s, one process {t_v1:.1f} s + {t_l1:.1f} s; "
                   f"scaled to the step's row mix"),
        "single_thread_value": rate(t_v1, t_l1),
        "verify_rows_per_s": rows_v / t_vp,
        "loss_rows_per_s": rows_l / t_lp,
        "cpu_model": _cpu_model(),
        "host_cpus": os.cpu_count(),
        "numpy": np.__version__,
        "verify_parity": par,
    }


def trace_summary(path, timed_steps=None):
    """Per-kernel launch statistics from a rocprofv3 kernel-trace CSV: calls,
    mean, median, min and max duration in microseconds, and the mean over
    the last half of the launches (after any warm-up). Then the bench steps
    found in the trace (the verify row kernel and finalize at T = 0, 0.6,
    1.0, then clear_words, loss_halves and loss_finish, with no other launch
    in between): per-launch medians over the steps."""
    import csv
    rows = {}
    seq = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("KernelName") or r.get("Name")
            t0 = int(r.get("Start_Timestamp") or r.get("BeginNs"))
            t1 = int(r.get("End_Timestamp") or r.get("EndNs"))
            rows.setdefault(name, []).append((t0, (t1 - t0) * 1e-3))
            seq.append((t0, t1, name))
    print("| kernel | calls | mean µs | median µs | min µs | max µs | mean of last half µs |")
    print("|---|---|---|---|---|---|---|")
    for name, v in sorted(rows.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        d = np.array([x for _, x in sorted(v)])
        short = name if len(name) < 90 else name[:87] + "..."
        print(f"| {short} | {d.size} | {d.mean():.1f} | {np.median(d):.1f} | {d.min():.1f} | "
              f"{d.max():.1f} | {d[d.size // 2:].mean():.1f} |")
    seq.sort()
    pattern = ["rows", "finalize"] * 3 + ["clear", "loss", "loss_finish"]
    steps = []
    for i in range(len(seq) - len(pattern) + 1):
        win = seq[i:i + len(pattern)]
        if all(_TRAFFIC_KERNELS[k] in n for k, (_, _, n) in zip(pattern, win)):
            steps.append([(t1 - t0) * 1e-3 for t0, t1, _ in win] +
                         [(win[-1][1] - win[-3][0]) * 1e-3])
    if steps:
        st = np.array(steps)
        head = ("| steps | T=0 rows | T=0 finalize | T=0.6 rows | T=0.6 finalize | T=1.0 rows | "
                "T=1.0 finalize | clear_words | loss_halves | loss_finish | loss call span |")
        print()
        print(f"Bench steps found in the trace: {len(steps)} (warm-up and timed); µs per launch:")
        print()
        print(head)
        print("|---|---|---|---|---|---|---|---|---|---|---|")
        print(f"| median of all {len(steps)} | " +
              " | ".join(f"{x:.1f}" for x in np.median(st, axis=0)) + " |")
        if timed_steps and timed_steps <= len(steps):
            print(f"| mean of the last {timed_steps} (the timed steps) | " +
                  " | ".join(f"{x:.1f}" for x in st[-timed_steps:].mean(axis=0)) + " |")


# Kernels whose per-launch HBM bytes traffic.json records, by the part of
# the demangled name that identifies them.
_TRAFFIC_KERNELS = {
    "rows": "verify_rows_bf16<true, false>",
    "finalize": "verify_finalize<1>",
    "clear": "clear_words",
    # loss_halves<vector loads, logits target, debug, CE/KL, row mode (1: two
    # workgroups a row, every group used)>
    "loss": "loss_halves<true, false, false, false, 1>",
    "loss_finish": "loss_finish<true, false, false, false>",
    "loss_logits": "loss_halves<true, true, false, false, 1>",
    "loss_xent": "loss_halves<true, false, false, true, 1>",
    "trunc": "trunc_rows<1, true>",
    "rows_trunc": "verify_rows_bf16<true, true>",
}


def _counter_dispatches(path, counter):
    """[(kernel name, value)] per dispatch, in dispatch order, of one counter
    of a rocprofv3 --pmc CSV (values summed over the CSV's rows of a
    dispatch)."""
    import csv
    disp = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            if d not in disp:
                disp[d] = [r["Kernel_Name"], 0.0]
            disp[d][1] += float(r["Counter_Value"])
    return [tuple(disp[d]) for d in sorted(disp)]


def traffic_from_counters(fetch_csv, write_csv):
    """HBM bytes per launch of the step's kernels from two rocprofv3 --pmc
    runs of `bench.py --steps 1 --warmup 0 --calls 3 --no-cpu-baseline
    --copy-calibration`: FETCH_SIZE in one, WRITE_SIZE in the other (KiB per
    dispatch). Each counter is scaled by 1 GiB over its median reading for
    the three plain 1 GiB device copies the calibration runs first. The
    step's kernels are the first launches after the calibration: the
    verify row kernel and finalize of T = 0, 0.6, 1.0 in that order, then
    the loss call; the logits-target loss and the top-k/top-p kernels are
    the first launches of theirs (top-p alone: the fifth)."""
    out = {"kernel_source_hash": kernel_source_hash(),
           "method": ("rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (separate runs) of "
                      "bench.py --steps 1 --warmup 0 --calls 3 --no-cpu-baseline "
                      "--copy-calibration; each counter scaled by (1 GiB / the counter's "
                      "median reading for the plain 1 GiB device copies in the same run); "
                      "derived by bench.py --traffic")}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"),
                               ("write", write_csv, "WRITE_SIZE")):
        disp = _counter_dispatches(path, counter)
        first = next(i for i, (n, _) in enumerate(disp) if _TRAFFIC_KERNELS["rows"] in n)
        copies = sorted((v for n, v in disp[:first] if "copy" in n.lower()), reverse=True)[:3]
        if len(copies) < 3 or copies[-1] <= 0:
            raise SystemExit(f"{path}: no 1 GiB copy calibration before the step")
        scale = float(1 << 30) / (float(np.median(copies)) * 1024.0)
        out[f"{key}_scale"] = scale
        after = disp[first:]

        def nth(tag, k=0):
            hits = [v for n, v in after if _TRAFFIC_KERNELS[tag] in n]
            return hits[k] * 1024.0 * scale if len(hits) > k else None

        for i, t in enumerate(TEMPS):
            out[f"verify_T{t}_rows_{key}"] = nth("rows", i)
            out[f"verify_T{t}_finalize_{key}"] = nth("finalize", i)
        out[f"loss_{key}_bytes"] = nth("loss")
        out[f"loss_finish_{key}_bytes"] = nth("loss_finish")
        out[f"clear_words_{key}_bytes"] = nth("clear")
        out[f"loss_logits_T1.0_{key}_bytes"] = nth("loss_logits")
        out[f"loss_ce_{key}_bytes"] = nth("loss_xent")
        out[f"trunc_topk50_{key}_bytes"] = nth("trunc")
        out[f"rows_topk50_{key}_bytes"] = nth("rows_trunc")
        # top-p alone follows the top-k 50 calls (one untimed and 3 timed)
        out[f"trunc_topp_{key}_bytes"] = nth("trunc", 4)
        out[f"rows_topp_{key}_bytes"] = nth("rows_trunc", 4)
    out["loss_bytes_per_launch"] = out["loss_fetch_bytes"] + out["loss_write_bytes"]
    for t in TEMPS:
        rows = out[f"verify_T{t}_rows_fetch"] + out[f"verify_T{t}_rows_write"]
        fin = out[f"verify_T{t}_finalize_fetch"] + out[f"verify_T{t}_finalize_write"]
        out[f"verify_T{t}_rows_kernel_bytes"] = rows
        out[f"verify_T{t}_bytes_per_launch"] = rows + fin
    return out


def load_traffic(src_hash):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    scaled by the copy-kernel calibration, if they were taken on this kernel
    build (profiles/traffic.json); else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_source_hash") != src_hash:
        return None
    return data


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run three plain 1 GiB device-to-device copies, whose HBM "
                         "bytes are known, so a counter profile of this run can be scaled")
    ap.add_argument("--calls", type=int, default=100,
                    help="calls per median for the per-call times (loss calls: a third)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-kernel statistics of a rocprofv3 kernel trace and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of this script and exit")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps)
        return
    if args.traffic:
        data = traffic_from_counters(*args.traffic)
        with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
            json.dump(data, f, indent=1)
            f.write("\n")
        print(json.dumps(data, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this hot path has no "
              "multi-GPU leg to measure", file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, ROOT)
    import lossless_verify_tv_amd as lv
    from lossless_verify_tv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lv.load_library()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    log("generating inputs")
    base = synth.verify_case(3, temperature=1.0)
    vcases = [synth.redraw_tokens(base, t) if t != 1.0 else base for t in TEMPS]
    lcase = synth.loss_case(workers=min(16, os.cpu_count() or 1))

    def bf16_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    vin = []
    for c in vcases:   # one copy of the logits per temperature
        vin.append(dict(
            target_logits=bf16_dev(c.target), draft_logits=bf16_dev(c.draft),
            draft_tokens=torch.from_numpy(c.tokens).to(dev),
            k_per_req=torch.from_numpy(c.k).to(dev),
            temperature=torch.from_numpy(c.temperature).to(dev),
            seed=torch.from_numpy(c.seed.view(np.int64)).to(dev)))
    z = bf16_dev(lcase.draft_logits)
    p = torch.from_numpy(lcase.target_probs).to(dev)
    vouts = [(torch.empty(VERIFY_B, dtype=torch.int32, device=dev),
              torch.empty(VERIFY_B, VERIFY_K + 1, dtype=torch.int32, device=dev),
              torch.empty(VERIFY_B, VERIFY_K, dtype=torch.float32, device=dev),
              torch.empty(VERIFY_B, dtype=torch.int32, device=dev)) for _ in TEMPS]
    lout = (torch.empty(1, dtype=torch.float32, device=dev),
            torch.empty(LOSS_N, LOSS_W, dtype=torch.float32, device=dev),
            torch.empty(LOSS_N, LOSS_W, VOCAB, dtype=torch.bfloat16, device=dev))
    vws = lv.new_workspace(lv.spec_verify_workspace_bytes(VERIFY_B, VERIFY_K, VOCAB), dev)
    lws = lv.new_workspace(lv.e2e_tv_loss_workspace_bytes(LOSS_N, LOSS_W, VOCAB), dev)
    torch.cuda.synchronize()
    log("inputs resident")

    if args.copy_calibration:
        src_c = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst_c = torch.empty_like(src_c)
        for _ in range(3):
            dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
        log("copy calibration done (3 x 1 GiB device copies)")

    stream = torch.cuda.current_stream(dev)

    def step(loss_events=None):
        for i in range(len(TEMPS)):
            lv.spec_verify(**vin[i], workspace=vws, out=vouts[i])
        if loss_events:
            loss_events[0].record(stream)
        lv.e2e_tv_loss_fwd_bwd(z, p, workspace=lws, out=lout)
        if loss_events:
            loss_events[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # The timed region holds the K steps and nothing else; inside each step
    # a pair of events brackets the loss call (the roofline's kernel).
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    loss_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step(loss_evs[s])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    loss_step_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in loss_evs]))
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall:.2f} s)")
    gpu_verify = [(o[0].cpu().numpy(), o[1].cpu().numpy()) for o in vouts]

    # Per-call times: each call between its own two events, a 1 GiB write
    # between calls (outside the events) so that nothing a call reads is
    # left in the last-level cache by the previous one; medians over calls.
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def per_call(fn, n):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for e0, e1 in evs:
            flush_buf.fill_(1.0)
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
        return {"ms": float(np.median(ms)), "ms_mean": float(ms.mean()),
                "ms_min": float(ms.min()), "calls": n}

    n_v = max(args.calls, 1)
    n_l = max(args.calls // 3, 1)
    verify_t = [per_call(lambda i=i: lv.spec_verify(**vin[i], workspace=vws, out=vouts[i]), n_v)
                for i in range(len(TEMPS))]
    loss_t = per_call(lambda: lv.e2e_tv_loss_fwd_bwd(z, p, workspace=lws, out=lout), n_l)
    verify_ms = [t["ms"] for t in verify_t]
    loss_ms = loss_t["ms"]
    log("per-call medians: " + ", ".join(f"verify T={t} {m * 1e3:.1f} us"
                                          for t, m in zip(TEMPS, verify_ms)) +
        f", loss {loss_ms:.3f} ms")

    # Batched per-call times: 5 batches of back-to-back calls, each batch
    # between two events (a 1 GiB write before each batch, outside them);
    # the verify calls rotate over 4 copies of their inputs (4 x 292 MB,
    # beyond the 256 MB last-level cache), the loss reads 4.4 GB per call.
    # Median over the batches of the batch time per call.
    def batched(fns, n, nb=5):
        flush_buf.fill_(1.0)  # also keeps these calls from reading as a bench step in a trace
        for fn in fns:
            fn()
        torch.cuda.synchronize()
        per = []
        for _ in range(nb):
            flush_buf.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for c in range(n):
                fns[c % len(fns)]()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n)
        return {"ms": float(np.median(per)), "batches": nb, "calls_per_batch": n,
                "ms_per_batch": [float(x) for x in per]}

    verify_b = []
    for i in range(len(TEMPS)):
        copies = [vin[i]] + [dict(vin[i], target_logits=vin[i]["target_logits"].clone(),
                                  draft_logits=vin[i]["draft_logits"].clone()) for _ in range(3)]
        verify_b.append(batched([lambda v=v, i=i: lv.spec_verify(**v, workspace=vws, out=vouts[i])
                                 for v in copies], n_v))
        del copies
    loss_b = batched([lambda: lv.e2e_tv_loss_fwd_bwd(z, p, workspace=lws, out=lout)], n_l)
    log("batched per-call times: " + ", ".join(f"verify T={t} {b['ms'] * 1e3:.1f} us"
                                               for t, b in zip(TEMPS, verify_b)) +
        f", loss {loss_b['ms']:.3f} ms")

    rows_step = len(TEMPS) * sum(int(k) + 1 for k in base.k) + LOSS_N * LOSS_W
    vb = verify_bytes(base.k, VOCAB)
    lb = loss_bytes(LOSS_N, LOSS_W, VOCAB)
    loss_gbs = lb / (loss_ms * 1e-3) / 1e9
    roof_gbs = lb / (loss_step_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash)
    result = {
        "metric": "verified vocab-rows/s + achieved HBM GB/s (% of peak), V=151936, 1 GPU",
        "value": rows_step / (ms_step * 1e-3),
        "unit": "vocab-rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Zipf-prior logits; no model, no dataset)",
        "config": {
            "workload": ("spec_verify B=64 K=7 V=151936 bf16 at T=0,0.6,1.0 + "
                         "e2e_tv_loss_fwd_bwd N=512 W=7 V=151936 (bf16 logits, fp32 probs)"),
            "vocab": VOCAB,
            "verify_rows_per_step": len(TEMPS) * VERIFY_B * (VERIFY_K + 1),
            "loss_rows_per_step": LOSS_N * LOSS_W,
            "algorithmic_bytes_per_step": len(TEMPS) * vb + lb,
        },
        "achieved_hbm_gbs": (len(TEMPS) * vb + lb) / (ms_step * 1e-3) / 1e9,
        "timing": (f"value and ms_per_step: {args.steps} back-to-back steps between two events; "
                   f"roofline: mean over those steps of the loss call between its own two "
                   f"events; per-call ms: median of {n_v} calls ({n_l} for the loss) each "
                   f"between its own two events, a 1 GiB write between calls outside them; "
                   f"'batched': median over 5 batches of {n_v} back-to-back calls ({n_l} "
                   f"for the loss) of the batch time per call, verify inputs rotated over 4 "
                   f"copies"),
        "roofline": {
            "kernel": ("loss_halves, timed as the e2e_tv_loss_fwd_bwd call inside each timed "
                       "step (one pair of events on the call's stream: clear_words + "
                       "loss_halves + loss_finish, the two small kernels about 11 us)"),
            "bound": "hbm",
            "achieved": roof_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": roof_gbs / HBM_PEAK_GBS,
            "traffic": (traffic or {}).get("loss_bytes_per_launch"),
            "ms_per_launch": loss_step_ms,
            "algorithmic_bytes_per_launch": lb,
        },
        "components": {
            f"spec_verify_T{t}": {
                **verify_t[i],
                "rows_per_s": VERIFY_B * (VERIFY_K + 1) / (verify_ms[i] * 1e-3),
                "gbs": vb / (verify_ms[i] * 1e-3) / 1e9,
                "frac": vb / (verify_ms[i] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes": vb,
                "traffic": (traffic or {}).get(f"verify_T{t}_bytes_per_launch"),
                "batched": verify_b[i],
            } for i, t in enumerate(TEMPS)
        },
        "kernel_source_hash": src_hash,
    }
    def traffic_of(*prefixes):
        """Counter bytes (FETCH_SIZE + WRITE_SIZE, scaled) of one launch of
        each named kernel, summed; None without counters for this build."""
        if not traffic:
            return None
        tot = 0.0
        for pre in prefixes:
            f, w = traffic.get(f"{pre}_fetch_bytes"), traffic.get(f"{pre}_write_bytes")
            if f is None or w is None:
                return None
            tot += f + w
        return tot

    result["components"]["e2e_tv_loss_fwd_bwd"] = {
        **loss_t, "rows_per_s": LOSS_N * LOSS_W / (loss_ms * 1e-3), "gbs": loss_gbs,
        "frac": loss_gbs / HBM_PEAK_GBS, "algorithmic_bytes": lb,
        "traffic": traffic_of("loss", "clear_words", "loss_finish"), "batched": loss_b}
    # The per-position comparators of the loss on the same inputs, outside
    # the step.
    variants = {}
    for name in ("step_tv", "ce", "kl"):
        t = per_call(lambda: lv.draft_loss_fwd_bwd(z, p, name, workspace=lws, out=lout),
                     max(n_l // 3, 1))
        ms = t["ms"]
        variants[f"draft_loss_{name}"] = {
            **t, "gbs": lb / (ms * 1e-3) / 1e9,
            "frac": lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": lb,
            "traffic": traffic_of("loss_ce") if name == "ce" else None}
    # The loss with the target given as bf16 logits (target softmax fused;
    # algorithmic bytes 6 per token: z 2 + t 2 read, dz 2 written).
    lgc = synth.loss_logits_case(workers=min(16, os.cpu_count() or 1))
    tl = bf16_dev(lgc.target_logits)
    del lgc
    lb6 = 6 * LOSS_N * LOSS_W * VOCAB
    for name, temp in (("e2e_tv", 1.0), ("e2e_tv", 0.7)):
        t = per_call(lambda: lv.draft_loss_logits_fwd_bwd(z, tl, temp, name, workspace=lws,
                                                          out=lout), max(n_l // 3, 1))
        ms = t["ms"]
        variants[f"draft_loss_logits_{name}_T{temp}"] = {
            **t, "gbs": lb6 / (ms * 1e-3) / 1e9,
            "frac": lb6 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": lb6,
            "traffic": traffic_of("loss_logits_T1.0") if temp == 1.0 else None}
    del tl
    result["loss_variants"] = variants
    log("loss variants: " + ", ".join(f"{k} {v['ms']:.3f} ms" for k, v in variants.items()))
    # Verify variants, outside the step, each timed over as many calls as the
    # step count: top-k / top-p truncation on the step's T = 1 inputs, and the
    # ragged confidence-scheduled workload (B = 256, K_b in 1..8, V = 129280,
    # half greedy) in the padded and the packed layouts.
    vvar = {}

    def time_calls(fn):
        return per_call(fn, n_v)

    tk = torch.full((VERIFY_B,), 50, dtype=torch.int32, device=dev)
    tp = torch.full((VERIFY_B,), 0.9, dtype=torch.float32, device=dev)
    tws = lv.new_workspace(lv.spec_verify_topkp_workspace_bytes(VERIFY_B, VERIFY_K, VOCAB), dev)
    t = time_calls(lambda: lv.spec_verify_topkp(**vin[2], top_k=tk, top_p=tp, workspace=tws,
                                                out=vouts[2]))
    ms = t["ms"]
    vvar["spec_verify_topkp_T1.0_k50_p0.9"] = {
        **t, "rows_per_s": VERIFY_B * (VERIFY_K + 1) / (ms * 1e-3),
        "gbs": vb / (ms * 1e-3) / 1e9, "frac": vb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": vb, "traffic": traffic_of("trunc_topk50", "rows_topk50")}
    tk0 = torch.zeros((VERIFY_B,), dtype=torch.int32, device=dev)
    t = time_calls(lambda: lv.spec_verify_topkp(**vin[2], top_k=tk0, top_p=tp, workspace=tws,
                                                out=vouts[2]))
    ms = t["ms"]
    vvar["spec_verify_topkp_T1.0_p0.9"] = {
        **t, "rows_per_s": VERIFY_B * (VERIFY_K + 1) / (ms * 1e-3),
        "gbs": vb / (ms * 1e-3) / 1e9, "frac": vb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": vb, "traffic": traffic_of("trunc_topp", "rows_topp")}
    del tws
    rc = synth.verify_case(5)
    rvocab = rc.target.shape[2]
    rb = verify_bytes(rc.k, rvocab)
    rrows = int(sum(int(k) + 1 for k in rc.k))
    rin = dict(target_logits=bf16_dev(rc.target), draft_logits=bf16_dev(rc.draft),
               draft_tokens=torch.from_numpy(rc.tokens).to(dev),
               k_per_req=torch.from_numpy(rc.k).to(dev),
               temperature=torch.from_numpy(rc.temperature).to(dev),
               seed=torch.from_numpy(rc.seed.view(np.int64)).to(dev))
    t = time_calls(lambda: lv.spec_verify(**rin))
    ms = t["ms"]
    vvar["spec_verify_ragged_padded"] = {
        **t, "rows_per_s": rrows / (ms * 1e-3), "gbs": rb / (ms * 1e-3) / 1e9,
        "frac": rb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": rb, "requests": int(rc.k.size), "rows": rrows, "vocab": rvocab}
    kk = np.asarray(rc.k, dtype=np.int64)
    off = np.zeros(kk.size + 1, dtype=np.int32)
    off[1:] = np.cumsum(kk + 1)
    pt = bf16_dev(np.concatenate([rc.target[b, :kk[b] + 1] for b in range(kk.size)]))
    pdr = bf16_dev(np.concatenate([rc.draft[b, :kk[b]] for b in range(kk.size)]))
    ptok = torch.from_numpy(np.concatenate([rc.tokens[b, :kk[b]]
                                            for b in range(kk.size)]).astype(np.int32)).to(dev)
    del rin
    offd = torch.from_numpy(off).to(dev)
    rtemp = torch.from_numpy(rc.temperature).to(dev)
    rseed = torch.from_numpy(rc.seed.view(np.int64)).to(dev)
    t = time_calls(lambda: lv.spec_verify_packed(pt, pdr, ptok, offd, rtemp, rseed))
    ms = t["ms"]
    vvar["spec_verify_ragged_packed"] = {
        **t, "rows_per_s": rrows / (ms * 1e-3), "gbs": rb / (ms * 1e-3) / 1e9,
        "frac": rb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": rb, "requests": int(rc.k.size), "rows": rrows, "vocab": rvocab}
    del pt, pdr, ptok, rc
    result["verify_variants"] = vvar
    log("verify variants: " + ", ".join(f"{k} {v['ms'] * 1e3:.1f} us" for k, v in vvar.items()))
    # Confidence-scheduled verify lengths for 256 requests x 16 positions
    # (one workgroup; latency-bound, reported as time per call).
    srng = np.random.default_rng([7, 1])
    sR, sL = 256, 16
    conf = torch.from_numpy(srng.uniform(0.05, 1.0, (sR, sL)).astype(np.float32)).to(dev)
    Bs = np.arange(sR * (sL + 1) + 1, dtype=np.float64)
    sps = torch.from_numpy((4000.0 / (1.0 + np.floor(Bs / 128.0))).astype(np.float32)).to(dev)
    sout = (torch.empty(sR, dtype=torch.int32, device=dev),
            torch.empty(2, dtype=torch.float64, device=dev))
    lv.dspark_schedule(conf, sps, out=sout)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 100
    e0.record(stream)
    for _ in range(reps):
        lv.dspark_schedule(conf, sps, out=sout)
    e1.record(stream)
    torch.cuda.synchronize()
    result["dspark_schedule"] = {"us": e0.elapsed_time(e1) / reps * 1e3, "requests": sR,
                                 "positions": sL}
    log(f"dspark_schedule R={sR} L={sL}: {result['dspark_schedule']['us']:.1f} us")
    # The two small workloads (latency-bound; reported as time per call):
    # B=1 K=4 V=4096 fp32 at T = 1 and T = 0, and B=32 K=4 V=32000 bf16.
    small = {}
    for tag, sc in (("B1_K4_V4096_f32_T1.0", synth.verify_case(1, temperature=1.0)),
                    ("B1_K4_V4096_f32_T0.0", synth.verify_case(1, temperature=0.0)),
                    ("B32_K4_V32000_bf16_T1.0", synth.verify_case(2))):
        conv = bf16_dev if sc.dtype == "bf16" else (
            lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev))
        sin = dict(target_logits=conv(sc.target), draft_logits=conv(sc.draft),
                   draft_tokens=torch.from_numpy(sc.tokens).to(dev),
                   k_per_req=torch.from_numpy(sc.k).to(dev),
                   temperature=torch.from_numpy(sc.temperature).to(dev),
                   seed=torch.from_numpy(sc.seed.view(np.int64)).to(dev))
        t = per_call(lambda: lv.spec_verify(**sin), n_v)
        sb = verify_bytes(sc.k, sc.shape[2], 2 if sc.dtype == "bf16" else 4)
        rows = int(sum(int(k) + 1 for k in sc.k))
        small[tag] = {**t, "us": t["ms"] * 1e3, "rows_per_s": rows / (t["ms"] * 1e-3),
                      "gbs": sb / (t["ms"] * 1e-3) / 1e9, "algorithmic_bytes": sb}
    result["small_workloads"] = small
    log("small workloads: " + ", ".join(f"{k} {v['us']:.1f} us" for k, v in small.items()))
    # Other vocabularies (seeded random logits drawn on the device; one V not
    # a multiple of 8, so its rows are not 16-byte aligned): the loss at
    # N=512 W=7 and the sampling verify at B=64 K=7 T=1, time per call.
    sweep = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    for sv in (32000, 50257, 128256):
        zs = (torch.randn(LOSS_N, LOSS_W, sv, device=dev, generator=gen) * 2).to(torch.bfloat16)
        ps = torch.softmax(torch.randn(LOSS_N, LOSS_W, sv, device=dev, generator=gen) * 2, dim=-1)
        t = per_call(lambda: lv.e2e_tv_loss_fwd_bwd(zs, ps), max(n_l // 3, 3))
        lbs = LOSS_N * LOSS_W * sv * 8
        sweep[f"loss_N{LOSS_N}_W{LOSS_W}_V{sv}"] = {
            **t, "us": t["ms"] * 1e3, "gbs": lbs / (t["ms"] * 1e-3) / 1e9,
            "algorithmic_bytes": lbs}
        del zs, ps
        vt = (torch.randn(VERIFY_B, VERIFY_K + 1, sv, device=dev, generator=gen) * 2).to(
            torch.bfloat16)
        vd = (torch.randn(VERIFY_B, VERIFY_K, sv, device=dev, generator=gen) * 2).to(
            torch.bfloat16)
        tok = torch.randint(0, sv, (VERIFY_B, VERIFY_K), device=dev, dtype=torch.int32,
                            generator=gen)
        kk = torch.full((VERIFY_B,), VERIFY_K, device=dev, dtype=torch.int32)
        temp = torch.ones(VERIFY_B, device=dev, dtype=torch.float32)
        seed = torch.arange(VERIFY_B, device=dev, dtype=torch.int64)
        t = per_call(lambda: lv.spec_verify(vt, vd, tok, kk, temp, seed), max(n_v // 5, 5))
        vbs = VERIFY_B * (2 * VERIFY_K + 1) * sv * 2
        sweep[f"verify_B{VERIFY_B}_K{VERIFY_K}_V{sv}_T1.0"] = {
            **t, "us": t["ms"] * 1e3, "gbs": vbs / (t["ms"] * 1e-3) / 1e9,
            "algorithmic_bytes": vbs}
        del vt, vd
    result["vocab_sweep"] = sweep
    log("vocabulary sweep: " + ", ".join(f"{k} {v['us']:.1f} us" for k, v in sweep.items()))
    del flush_buf
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the step's inputs (one process, then a pool)")
        result["cpu_baseline"] = cpu_baseline(vcases, lcase, gpu_verify,
                                              workers=min(16, os.cpu_count() or 1))
        log(f"cpu baseline {result['cpu_baseline']['value']:.0f} vocab-rows/s on "
            f"{result['cpu_baseline']['cores']} processes; verify parity "
            f"{result['cpu_baseline']['verify_parity']}")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
