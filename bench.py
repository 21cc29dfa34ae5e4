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
roofline of the dominant kernel (the loss), timed live with HIP events on
the stream the kernels run on, and the CPU oracle timed on a bounded sample.
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


def cpu_baseline(verify_cases, loss_case, verify_passes=2, n_branches=LOSS_N):
    """Time the fp64 oracle, as it stands, on a bounded sample of the same
    workload (10-15 s of CPU work on the GPU host): every request of each
    temperature's verify inputs, `verify_passes` times, and the first
    `n_branches` branches of the loss inputs. Single process, one thread
    (numpy elementwise work is single-threaded)."""
    sys.path.insert(0, ROOT)
    from oracle import bf16 as obf16
    from oracle import loss as ol
    from oracle import verify as ov

    rows_v = 0
    t0 = time.perf_counter()
    for _ in range(verify_passes):
        for case in verify_cases:
            for b in range(case.shape[0]):
                ov.verify_request(ov.decode_rows(case.target[b], case.dtype),
                                  ov.decode_rows(case.draft[b], case.dtype), case.tokens[b],
                                  case.k[b], case.temperature[b], int(case.seed[b]), b,
                                  case.shape[1])
                rows_v += int(case.k[b]) + 1
    t_v = time.perf_counter() - t0
    t0 = time.perf_counter()
    for n in range(n_branches):
        ol.branch(obf16.decode(loss_case.draft_logits[n]), loss_case.target_probs[n], LOSS_N)
    t_l = time.perf_counter() - t0
    rows_l = n_branches * LOSS_W
    step_rows_v = len(verify_cases) * VERIFY_B * (VERIFY_K + 1)
    step_rows_l = LOSS_N * LOSS_W
    step_seconds = step_rows_v * t_v / rows_v + step_rows_l * t_l / rows_l
    return {
        "value": (step_rows_v + step_rows_l) / step_seconds,
        "unit": "vocab-rows/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{verify_passes} passes over all requests x {len(verify_cases)} "
                   f"temperatures of the verify workload ({rows_v} vocab-rows, {t_v:.1f} s) "
                   f"and {n_branches} branches of the loss workload ({rows_l} vocab-rows, "
                   f"{t_l:.1f} s), fp64 numpy, one process; scaled to the step's row mix"),
        "verify_rows_per_s": rows_v / t_v,
        "loss_rows_per_s": rows_l / t_l,
        "host_cpus": os.cpu_count(),
    }


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
    args = ap.parse_args()
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

    def step(events=None):
        for i in range(len(TEMPS)):
            if events is not None:
                events[2 * i].record(stream)
            lv.spec_verify(**vin[i], workspace=vws, out=vouts[i])
            if events is not None:
                events[2 * i + 1].record(stream)
        if events is not None:
            events[6].record(stream)
        lv.e2e_tv_loss_fwd_bwd(z, p, workspace=lws, out=lout)
        if events is not None:
            events[7].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # The timed region holds the K steps and nothing else: an event recorded
    # between two calls costs the stream several microseconds, so the
    # per-call breakdown comes from a second, separate run of K steps.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    per_step = [[torch.cuda.Event(enable_timing=True) for _ in range(8)]
                for _ in range(args.steps)]
    for s in range(args.steps):
        step(per_step[s])
    torch.cuda.synchronize()
    verify_ms = [np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for ev in per_step])
                 for i in range(len(TEMPS))]
    loss_ms = float(np.mean([ev[6].elapsed_time(ev[7]) for ev in per_step]))
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall:.2f} s)")

    rows_step = len(TEMPS) * sum(int(k) + 1 for k in base.k) + LOSS_N * LOSS_W
    vb = verify_bytes(base.k, VOCAB)
    lb = loss_bytes(LOSS_N, LOSS_W, VOCAB)
    loss_gbs = lb / (loss_ms * 1e-3) / 1e9
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
        "roofline": {
            "kernel": "loss_halves (e2e_tv_loss_fwd_bwd)",
            "bound": "hbm",
            "achieved": loss_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": loss_gbs / HBM_PEAK_GBS,
            "traffic": (traffic or {}).get("loss_bytes_per_launch"),
        },
        "components": {
            f"spec_verify_T{t}": {
                "ms": verify_ms[i],
                "rows_per_s": VERIFY_B * (VERIFY_K + 1) / (verify_ms[i] * 1e-3),
                "gbs": vb / (verify_ms[i] * 1e-3) / 1e9,
                "frac": vb / (verify_ms[i] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes": vb,
                "traffic": (traffic or {}).get(f"verify_T{t}_bytes_per_launch"),
            } for i, t in enumerate(TEMPS)
        },
        "kernel_source_hash": src_hash,
    }
    result["components"]["e2e_tv_loss_fwd_bwd"] = {
        "ms": loss_ms, "rows_per_s": LOSS_N * LOSS_W / (loss_ms * 1e-3), "gbs": loss_gbs,
        "frac": loss_gbs / HBM_PEAK_GBS, "algorithmic_bytes": lb}
    # The per-position comparators of the loss on the same inputs, outside
    # the step: each timed over as many calls as the step count.
    variants = {}
    for name in ("step_tv", "ce", "kl"):
        lv.draft_loss_fwd_bwd(z, p, name, workspace=lws, out=lout)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            lv.draft_loss_fwd_bwd(z, p, name, workspace=lws, out=lout)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        variants[f"draft_loss_{name}"] = {
            "ms": ms, "gbs": lb / (ms * 1e-3) / 1e9,
            "frac": lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": lb}
    # The loss with the target given as bf16 logits (target softmax fused;
    # algorithmic bytes 6 per token: z 2 + t 2 read, dz 2 written).
    lgc = synth.loss_logits_case(workers=min(16, os.cpu_count() or 1))
    tl = bf16_dev(lgc.target_logits)
    del lgc
    lb6 = 6 * LOSS_N * LOSS_W * VOCAB
    for name, temp in (("e2e_tv", 1.0), ("e2e_tv", 0.7)):
        lv.draft_loss_logits_fwd_bwd(z, tl, temp, name, workspace=lws, out=lout)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            lv.draft_loss_logits_fwd_bwd(z, tl, temp, name, workspace=lws, out=lout)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        variants[f"draft_loss_logits_{name}_T{temp}"] = {
            "ms": ms, "gbs": lb6 / (ms * 1e-3) / 1e9,
            "frac": lb6 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": lb6}
    del tl
    result["loss_variants"] = variants
    log("loss variants: " + ", ".join(f"{k} {v['ms']:.3f} ms" for k, v in variants.items()))
    # Verify variants, outside the step, each timed over as many calls as the
    # step count: top-k / top-p truncation on the step's T = 1 inputs, and the
    # ragged confidence-scheduled workload (B = 256, K_b in 1..8, V = 129280,
    # half greedy) in the padded and the packed layouts.
    vvar = {}

    def time_calls(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    tk = torch.full((VERIFY_B,), 50, dtype=torch.int32, device=dev)
    tp = torch.full((VERIFY_B,), 0.9, dtype=torch.float32, device=dev)
    tws = lv.new_workspace(lv.spec_verify_topkp_workspace_bytes(VERIFY_B, VERIFY_K, VOCAB), dev)
    ms = time_calls(lambda: lv.spec_verify_topkp(**vin[2], top_k=tk, top_p=tp, workspace=tws,
                                                 out=vouts[2]))
    vvar["spec_verify_topkp_T1.0_k50_p0.9"] = {
        "ms": ms, "rows_per_s": VERIFY_B * (VERIFY_K + 1) / (ms * 1e-3),
        "gbs": vb / (ms * 1e-3) / 1e9, "algorithmic_bytes": vb}
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
    ms = time_calls(lambda: lv.spec_verify(**rin))
    vvar["spec_verify_ragged_padded"] = {
        "ms": ms, "rows_per_s": rrows / (ms * 1e-3), "gbs": rb / (ms * 1e-3) / 1e9,
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
    ms = time_calls(lambda: lv.spec_verify_packed(pt, pdr, ptok, offd, rtemp, rseed))
    vvar["spec_verify_ragged_packed"] = {
        "ms": ms, "rows_per_s": rrows / (ms * 1e-3), "gbs": rb / (ms * 1e-3) / 1e9,
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
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(vcases, lcase)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
