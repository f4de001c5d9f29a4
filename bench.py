"""Throughput of the error-feedback Top-k compress step on one MI355X.

One step = one pass of the whole hot path over one gradient: (momentum,) EF add, exact
per-segment Top-k select, ordered compaction into (value, index), residual write (and, for
the hybrid workload, the int8 stage).  Inputs are seeded synthetic gradients resident in
HBM before the timed region; a pool of four gradient buffers cycles so that every step sees a fresh
gradient.  Prints one JSON line.

value = GB/s of fp32 input gradient (4 N bytes per step / step time), whole job.
roofline = the streaming EF pass (the dominant kernel): algorithmic bytes per launch
(12 N: read g, read e, write e; 20 N with momentum) / its average HIP-event duration,
against the 8 TB/s HBM3E peak; traffic = the HBM bytes the committed rocprofv3 counters
measured for it (null once its code has changed since).
cpu_baseline = the CPU oracle on a bounded sample of the same workload's segments.

--codec selects the threshold, Random-k, sign or QSGD codec instead of Top-k (the same
fields, their own pass bytes).  The default run also reports, as context: every workload
(`all_configs`: single 1M segment, ResNet-50, BERT-large, hybrid int8, the 7B shape with
momentum, and the headline 7B plain step) with its step time, effective fraction of peak
and streaming-pass time; the plan's first (cold) call; local gradient clipping; the
receiver-side sum of eight workers' payloads; and three reference streams in the pass's tile
layout (`reference_streams`: a pure read, a copy, and a bare y += x with the pass's memory
instructions and none of its selection work).  They are measured references, not ceilings:
the pass streams faster than the bare y += x.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EF-Top-k compress GB/s of fp32 gradient (1 GPU) and % of HBM peak"
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "c5p_llama2_7b_plain"
# HBM bytes per launch of the streaming pass, from rocprofv3 FETCH_SIZE/WRITE_SIZE runs
# scaled by the same counters on the copy kernel (see the summaries next to it)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the code the Top-k streaming pass is built from (its source file, the capture
    and device helpers it includes and the plan layout): comments dropped and whitespace
    collapsed, so that only a change of that code invalidates counters taken on it."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "gradient_compression_amd", "csrc")
    code = []
    for f in ("gc_pass.hip", "gc_capture.h", "gc_device.h", "gc_internal.h"):
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        code.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch of the streaming pass from the committed rocprofv3 counters, or
    None when they are missing or were taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f).get(name)
    if not tr or tr.get("source_sha256_16") != kernel_source_hash():
        return None
    return tr["bytes_per_launch"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--codec", choices=("topk", "sign", "qsgd", "threshold", "randk"),
                    default="topk",
                    help="topk: EF-Top-k (default); sign: 1-bit sign with error feedback; "
                         "qsgd: QSGD with 127 levels and error feedback; threshold: keep "
                         "|acc| >= tau_s (at most k_s) with error feedback; randk: Random-k "
                         "with error feedback")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-configs", "--no-momentum-variant", dest="no_all_configs",
                    action="store_true",
                    help="skip the other workloads (timed in the default run as context)")
    ap.add_argument("--no-receiver", action="store_true",
                    help="skip the receiver-side sum of 8 workers' payloads (context figure)")
    return ap.parse_args()


def bytes_per_element(wl, codec="topk"):
    """Algorithmic HBM bytes per element of the timed streaming passes."""
    if codec == "sign":   # pass 1: g, e (u) in, e (u) out; pass 2: e in, e out, one bit
        return (20 if wl.momentum is not None else 12) + 8 + 1 / 8
    if codec == "qsgd":   # pass 1 as for sign; pass 2: e in, e out, one int8 code
        return (20 if wl.momentum is not None else 12) + 8 + 1
    return 20 if wl.momentum is not None else 12


def run_step(plan, wl, codec, g, e, u, outs, t):
    """One step of the codec on gradient g (error feedback state e, velocity u)."""
    vals, idx, codes, scales = outs
    m = wl.momentum or 0.0
    if codec == "threshold":   # the thresholds ride in the scales slot
        plan.threshold_compress(g, e, scales, vals, idx, u=u, momentum=m)
    elif codec == "randk":
        plan.randk_compress(g, vals, idx, e=e, u=u, momentum=m, seed=0, step=t)
    elif codec == "sign":
        plan.sign_compress(g, e, codes, scales, u=u, momentum=m)
    elif codec == "qsgd":
        plan.qsgd_compress(g, codes, scales, levels=127, e=e, u=u, momentum=m, seed=0, step=t)
    elif wl.int8:   # compress and int8 (error feedback of the quantisation error) in one call
        plan.compress_int8(g, e, idx, codes, scales, out_vals=vals, u=u, momentum=m, seed=0,
                           step=t)
    else:
        plan.compress(g, e, vals, idx, u=u, momentum=m)


def time_steps(plan, wl, gbufs, e, u, outs, steps, warmup, codec="topk"):
    """(ms per step, ms per streaming pass, passes timed, first call ms): warmup steps (the
    first one timed alone), then `steps` timed steps with no event between them, then as many
    again with events around each pass and after each step for the pass time, the median
    step (time_steps.median_ms) and the mean step of that run (time_steps.events_ms), from
    which the time after the pass is taken (both from the same steps)."""
    import torch

    def step(t):
        run_step(plan, wl, codec, gbufs[t % len(gbufs)], e, u, outs, t)

    cold = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for t in range(warmup):
        if t == 0:
            cold[0].record()
        step(t)
        if t == 0:
            cold[1].record()
    torch.cuda.synchronize()
    cold_ms = cold[0].elapsed_time(cold[1]) if warmup > 0 else None
    plan.timing()                       # drop the warm-up events
    # the timed steps: nothing between them but the steps (an event record per step costs a
    # few microseconds of GPU time, which shows on the small shapes)
    ends = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ends[0].record()
    for t in range(warmup, warmup + steps):
        step(t)
    ends[1].record()
    torch.cuda.synchronize()
    total_ms = ends[0].elapsed_time(ends[1])
    # the same number of steps again with events: the streaming pass's own time (the library's
    # events on the stream it launches on, around each pass) and the median step (an event
    # after every step)
    plan.set_timing(True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for j, t in enumerate(range(warmup + steps, warmup + 2 * steps)):
        step(t)
        marks[j + 1].record()
    torch.cuda.synchronize()
    plan.set_timing(False)
    per_step = [marks[j].elapsed_time(marks[j + 1]) for j in range(steps)]
    time_steps.median_ms = float(np.median(per_step)) if per_step else None
    time_steps.events_ms = marks[0].elapsed_time(marks[-1]) / steps if steps else None
    k1_ms, launches = plan.timing()
    return total_ms / steps, k1_ms / max(launches, 1), launches, cold_ms


def gradient_fingerprint(g, n_max=1 << 24):
    """SHA-256 (first 16 hex digits) of the first min(N, 2^24) fp32 gradient elements of the
    first timed buffer: a record of the synthetic bytes (they depend on the generator's
    library, so they are recorded rather than predicted)."""
    import hashlib
    return hashlib.sha256(g[:n_max].cpu().numpy().tobytes()).hexdigest()[:16]


def setup(wl, n_gbufs=4, codec="topk"):
    import torch
    import gradient_compression_amd as gca
    from synth import gen
    plan = gca.Plan(wl.offsets(),
                    ratio=wl.ratio if codec in ("topk", "threshold", "randk") else 0.0)
    dev = torch.device("cuda")
    gbufs = []
    for t in range(n_gbufs):
        g = torch.empty(wl.n, dtype=torch.float32, device=dev)
        gen.fill_gradient(g, wl, t)
        gbufs.append(g)
    e = torch.zeros(wl.n, dtype=torch.float32, device=dev)
    u = torch.zeros(wl.n, dtype=torch.float32, device=dev) if wl.momentum is not None else None
    vals = torch.empty(plan.total_k, dtype=torch.float32, device=dev)
    idx = torch.empty(plan.total_k, dtype=torch.int32, device=dev)
    codes = torch.empty(plan.total_k, dtype=torch.int8, device=dev) if wl.int8 else None
    scales = torch.empty(wl.n_seg, dtype=torch.float32, device=dev) if wl.int8 else None
    if codec == "sign":   # sign bits in place of codes, one scale per segment
        codes = torch.empty(plan.total_words, dtype=torch.int32, device=dev)
        scales = torch.empty(wl.n_seg, dtype=torch.float32, device=dev)
    if codec == "qsgd":   # one int8 code per element, one norm per segment
        codes = torch.empty(wl.n, dtype=torch.int8, device=dev)
        scales = torch.empty(wl.n_seg, dtype=torch.float32, device=dev)
    if codec == "threshold":
        # tau_s = |k_s-th largest acc| after 8 EF-Top-k steps (the residual's steady state),
        # then fixed: about k_s entries reach it per step, the cap k_s binding when more do
        for t in range(8):
            plan.compress(gbufs[t % n_gbufs], e, vals, idx, u=u, momentum=wl.momentum or 0.0)
        kth = torch.from_numpy(plan.last_stats()["kth_key"].astype(np.uint32).view(np.float32))
        scales = kth.to(dev)   # the thresholds ride in the scales slot
    torch.cuda.synchronize()
    return plan, gbufs, e, u, (vals, idx, codes, scales)


def copy_stream(n_bytes=8 << 30):
    """Reference: the library's dwordx4 copy kernel, GB/s of read + write."""
    import torch
    import gradient_compression_amd as gca
    n = n_bytes // 4
    a = torch.zeros(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        gca.copy_f32(a, b)
    torch.cuda.synchronize()
    s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        gca.copy_f32(a, b)
    t.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(t) / 10
    del a, b
    return 2 * n * 4 / ms / 1e6


def read_stream(n_bytes=16 << 30):
    """Reference: a pure read stream in the pass's tile layout (non-temporal dwordx4 loads),
    GB/s read."""
    import torch
    import gradient_compression_amd as gca
    n = n_bytes // 4
    x = torch.zeros(n, dtype=torch.float32, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    for _ in range(2):
        gca.read_f32(x, sink)
    torch.cuda.synchronize()
    s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        gca.read_f32(x, sink)
    t.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(t) / 10
    del x, sink
    return n * 4 / ms / 1e6


def add_stream(n_bytes=8 << 30):
    """Reference for the streaming pass: the library's y += x kernel (the pass's tile layout
    and non-temporal loads and stores, nothing else), GB/s of its two reads and one write."""
    import torch
    import gradient_compression_amd as gca
    n = n_bytes // 4
    x = torch.zeros(n, dtype=torch.float32, device="cuda")
    y = torch.zeros(n, dtype=torch.float32, device="cuda")
    for _ in range(2):
        gca.add_f32(x, y)
    torch.cuda.synchronize()
    s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        gca.add_f32(x, y)
    t.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(t) / 10
    del x, y
    return 3 * n * 4 / ms / 1e6


def _ulp(x):
    return float(np.spacing(np.float32(abs(x))))


def host_threads():
    """The oracle's threads: the host cores this process may use, at most 16 (the CPU share
    of one GPU on the machines this runs on)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def cpu_baseline(plan, wl, gbuf, e, u, outs, codec="topk", t=0):
    """Time the CPU oracle for the codec on a bounded sample of the workload's segments (from
    segment 1 on, at least one per host thread and at least a budget of elements: 800M for
    the sorting codecs, about four layers of the 7B shape, some 10 s on 16 threads; 3.2G for
    sign and QSGD, which do not sort), in a thread pool over segments; check it against the
    GPU's output of the same step on the same state.  For sign and QSGD the scale / norm is a
    double sum in an unspecified order (one ulp); their bits, codes and residual are compared
    where the two agree."""
    import concurrent.futures as cf
    import torch
    import oracle
    off = wl.offsets()
    segs = list(range(1, wl.n_seg)) if wl.n_seg > 9 else list(range(wl.n_seg))
    threads = host_threads()
    budget = 3_200_000_000 if codec in ("sign", "qsgd") else 800_000_000
    total = 0
    pick = []
    for s in segs:
        if len(pick) >= threads and total >= budget:
            break
        pick.append(s)
        total += int(off[s + 1] - off[s])
    host = {}
    for s in pick:
        a, b = int(off[s]), int(off[s + 1])
        host[s] = dict(g=gbuf[a:b].cpu().numpy(), e=e[a:b].cpu().numpy(),
                       u=u[a:b].cpu().numpy() if u is not None else None)
    vals, idx, codes, scales = outs
    tau = scales.cpu().numpy() if codec == "threshold" else None
    if codec == "topk" and wl.int8:   # the bounded sample times the sparsifier alone
        codec_run = "topk-no-int8"
        plan.compress(gbuf, e, vals, idx, u=u, momentum=wl.momentum or 0.0)
    else:
        codec_run = codec
        run_step(plan, wl, codec, gbuf, e, u, outs, t)
    torch.cuda.synchronize()
    oracle.lib()
    m = wl.momentum or 0.0

    def run(s):
        h = host[s]
        a = int(off[s])
        k = int(plan.k[s])
        if codec in ("topk",):
            r = oracle.topk_ef_segment(h["g"], h["e"], k, u=h["u"], momentum=m)
        elif codec == "threshold":
            r = oracle.threshold_ef_segment(h["g"], h["e"], k, float(tau[s]), u=h["u"], momentum=m)
        elif codec == "randk":
            r = oracle.randk_segment(h["g"], k, e=h["e"], u=h["u"], momentum=m, seed=0, step=t,
                                     seg_base=a)
        elif codec == "sign":
            r = oracle.sign_ef_segment(h["g"], h["e"], u=h["u"], momentum=m)
        else:
            r = oracle.qsgd_segment(h["g"], h["e"], u=h["u"], momentum=m, levels=127, seed=0,
                                    step=t, seg_base=a)
        return s, r

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        res = dict(ex.map(run, pick))
    dt = time.perf_counter() - t0
    ok = True
    for s in pick:
        a, b = int(off[s]), int(off[s + 1])
        e_ok = e[a:b].cpu().numpy().tobytes() == host[s]["e"].tobytes()
        if codec in ("topk", "threshold", "randk"):
            hv, hi = res[s]
            ka = int(plan.out_off[s])
            ok &= vals[ka:ka + hv.size].cpu().numpy().tobytes() == hv.tobytes()
            ok &= np.array_equal(idx[ka:ka + hi.size].cpu().numpy(), hi)
            ok &= e_ok
        elif codec == "sign":
            hb, hs = res[s]
            wa, wb = int(plan.word_off[s]), int(plan.word_off[s + 1])
            ok &= np.array_equal(codes[wa:wb].cpu().numpy().view(np.uint32), hb)
            sd = float(scales[s])
            ok &= abs(sd - float(hs)) <= _ulp(hs)
            ok &= e_ok or sd != hs
        else:
            hc, hn = res[s]
            nd = float(scales[s])
            ok &= abs(nd - float(hn)) <= _ulp(hn)
            if nd == hn:
                ok &= np.array_equal(codes[a:b].cpu().numpy(), hc) and e_ok
    what = {"topk": "EF-Top-k step, full sort per segment",
            "topk-no-int8": "EF-Top-k step (the sparsifier alone), full sort per segment",
            "threshold": "threshold-EF step, count then full sort per segment",
            "randk": "Random-k EF step, Philox key per element and full sort per segment",
            "sign": "1-bit sign EF step",
            "qsgd": "QSGD-127 EF step, Philox draw per element"}[codec_run]
    return {
        "value": round(4.0 * total / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "host_affinity_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"one {what} on segments {pick[0]}..{pick[-1]} ({len(pick)} tensors, "
                   f"{total} fp32 elements) of {wl.name}, {dt:.2f} s wall on {threads} threads "
                   f"(the host cores this process may use, at most 16)"),
        "parity_with_gpu_on_sample": bool(ok),
    }


def clip_bench(plan, wl, g, reps=8):
    """Local gradient clipping of every segment on one resident gradient: call t clips to
    norm0 * 2^-(t+1), so each call scales every segment (read 4 B in the norm pass, read and
    write 4 B in the scaling pass: 12 B per element)."""
    import torch
    norms = torch.empty(wl.n_seg, device="cuda")
    plan.clip_by_norm(g, torch.full((wl.n_seg,), float("inf"), device="cuda"), norms)
    n0 = norms.clone()
    caps = [n0 * 2.0 ** -(t + 1) for t in range(reps + 1)]
    plan.clip_by_norm(g, caps[0])
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for t in range(reps):
        plan.clip_by_norm(g, caps[t + 1])
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / reps
    return {"ms_per_call": round(ms, 4), "bytes_per_element": 12,
            "achieved_GBps": round(12 * wl.n / ms / 1e6, 1),
            "hbm_peak_frac": round(12 * wl.n / ms / 1e6 / HBM_PEAK_GBPS, 4)}


def clip_fused_bench(plan, wl, codec, gbufs, e, u, outs, steps, warmup):
    """The codec's step with local gradient clipping folded into its loads: the norm pass
    (gc_clip_factors, reads g) then the codec with the per-segment scale set (every segment
    clipped to half its norm)."""
    import torch
    norms = torch.empty(wl.n_seg, device="cuda")
    caps = []
    for g in gbufs:
        plan.clip_factors(g, torch.full((wl.n_seg,), float("inf"), device="cuda"),
                          torch.empty(wl.n_seg, device="cuda"), norms_out=norms)
        caps.append(norms * 0.5)
    factors = torch.empty(wl.n_seg, device="cuda")
    plan.set_gradient_scale(factors)

    def step(t):
        i = t % len(gbufs)
        plan.clip_factors(gbufs[i], caps[i], factors)
        run_step(plan, wl, codec, gbufs[i], e, u, outs, t)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for t in range(warmup, warmup + steps):
        step(t)
    s1.record()
    torch.cuda.synchronize()
    plan.set_gradient_scale(None)
    ms = s0.elapsed_time(s1) / steps
    bpe = bytes_per_element(wl, codec) + 4
    return {"ms_per_step": round(ms, 4), "bytes_per_element": bpe,
            "effective_GBps": round(bpe * wl.n / ms / 1e6, 1),
            "hbm_peak_frac": round(bpe * wl.n / ms / 1e6 / HBM_PEAK_GBPS, 4)}


def randk_plain_bench(plan, wl, gbufs, outs, steps):
    """Random-k without error feedback or momentum: the pass draws a Philox key per element
    and reads nothing; the k kept values are gathered from g and scaled by n/k."""
    import torch
    vals, idx, _, _ = outs
    for t in range(2):
        plan.randk_compress(gbufs[t % len(gbufs)], vals, idx, seed=0, step=t)
    torch.cuda.synchronize()
    plan.timing()
    plan.set_timing(True)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for t in range(steps):
        plan.randk_compress(gbufs[t % len(gbufs)], vals, idx, seed=0, step=t + 2)
    s1.record()
    torch.cuda.synchronize()
    plan.set_timing(False)
    ms = s0.elapsed_time(s1) / steps
    k1_ms, n = plan.timing()
    k1 = k1_ms / max(n, 1)
    # Philox4x32-10 per 4 elements: 10 rounds of two 32x32->64 products (v_mad_u64_u32)
    blocks = wl.n / 4
    return {"ms_per_step": round(ms, 4), "key_pass_ms": round(k1, 4),
            "G_keys_per_s": round(wl.n / k1 / 1e6, 1),
            "philox_blocks_per_s_G": round(blocks / k1 / 1e6, 1)}


# Every other workload, timed in the same run as the headline step (steps per workload: at
# least these, so that the short steps are timed over a few milliseconds).
ALL_CONFIGS = {"c1_single_1m": 200, "c2_resnet50": 100, "c3_bert_large": 30,
               "c4_hybrid_int8": 12, "c5_llama2_7b": 8}


def config_record(wl, ms, pass_ms, median_ms, st, total_k, steps, events_ms=None):
    """Step and streaming-pass figures of one workload: effective bytes per element are 12
    (read g, read e, write e), 20 with momentum (u read and written too).  The time after the
    pass: for steps of a millisecond or more, the mean step of the run with events minus its
    mean pass (events_ms - pass_ms: the pass varies by about 0.1 ms between runs, so both
    figures come from the same steps); for shorter steps, the event-free mean step minus the
    pass (the event records would add about 10 us a step)."""
    bpe = bytes_per_element(wl)
    rec = {"n_elements": wl.n, "segments": wl.n_seg, "k_ratio": wl.ratio,
           "total_k": int(total_k), "momentum": wl.momentum, "int8": wl.int8,
           "steps": steps, "ms_per_step": round(ms, 4),
           "median_ms_per_step": round(median_ms, 4) if median_ms else None,
           "GBps_gradient": round(4.0 * wl.n / ms / 1e6, 2),
           "bytes_per_element": bpe,
           "hbm_peak_frac_effective": round(bpe * wl.n / ms / 1e6 / HBM_PEAK_GBPS, 4),
           "pass_ms": round(pass_ms, 4),
           "pass_achieved_GBps": round(bpe * wl.n / pass_ms / 1e6, 1),
           "pass_hbm_peak_frac": round(bpe * wl.n / pass_ms / 1e6 / HBM_PEAK_GBPS, 4),
           "after_pass_ms": round((events_ms if events_ms and ms >= 1.0 else ms) - pass_ms, 4),
           "candidates_per_k": round(float(st["candidates"].sum()) / max(total_k, 1), 3)}
    if wl.momentum is not None:   # also on the 12 B/elt basis of the metric
        rec["hbm_peak_frac_effective_12B"] = round(12.0 * wl.n / ms / 1e6 / HBM_PEAK_GBPS, 4)
    if wl.n * 12 < 512e6:
        rec["note"] = "fits the 256 MB on-package cache: not an HBM measurement"
    return rec


def bench_config(name, steps, warmup):
    """One workload's Top-k step (int8 fused for the hybrid one), on its own plan and
    buffers, freed afterwards."""
    import torch
    from synth import workload
    w = workload(name)
    steps = max(steps, ALL_CONFIGS[name])
    plan, gbufs, e, u, outs = setup(w)
    ms, pass_ms, _, _ = time_steps(plan, w, gbufs, e, u, outs, steps, warmup)
    rec = config_record(w, ms, pass_ms, time_steps.median_ms, plan.last_stats(), plan.total_k,
                        steps, time_steps.events_ms)
    plan.close()
    del gbufs, e, u, outs
    torch.cuda.empty_cache()
    return rec


def receiver_bench(wl, n_workers=8, reps=5):
    """Receiver side of an n_workers data-parallel exchange on one GPU: the gathered payloads
    (synthetic, the plan's layout) added into a resident dense gradient in worker order."""
    import torch
    import gradient_compression_amd as gca
    import synth
    off = wl.offsets()
    plan = gca.Plan(off, ratio=wl.ratio)
    kk = plan.total_k
    dev = torch.device("cuda")
    vals = torch.empty(n_workers * kk, device=dev)
    idx = torch.empty(n_workers * kk, dtype=torch.int32, device=dev)
    synth.fill_payloads(vals, idx, off, plan.k, n_workers, seed=7)
    dense = torch.zeros(wl.n, device=dev)
    plan.decompress_gathered(n_workers, idx, dense, vals=vals, accumulate=True)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        plan.decompress_gathered(n_workers, idx, dense, vals=vals, accumulate=True)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / reps
    plan.close()
    entries = n_workers * kk
    return {"workers": n_workers, "entries": entries, "ms_scatter_add": round(ms, 4),
            "G_entries_per_s": round(entries / ms / 1e6, 2),
            "note": "payloads read 8 B/entry sequentially, one scattered 4 B read-modify-write "
                    "per entry; dense zero fill (4 B/elt) not included"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (--gpus {args.gpus} "
              "requested). Compression is worker-local; run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import gradient_compression_amd as gca
    from synth import workload
    gca.lib()  # fails loudly when the HIP library is not built
    wl = workload(args.workload)
    log(f"[bench] workload {wl.name}: N={wl.n} segments={wl.n_seg} ratio={wl.ratio}")
    codec = args.codec
    plan, gbufs, e, u, outs = setup(wl, codec=codec)
    log(f"[bench] inputs resident ({len(gbufs)} gradient buffers); warmup {args.warmup}, "
        f"timing {args.steps} steps, codec {codec}")
    ms, k1_ms, launches, cold_ms = time_steps(plan, wl, gbufs, e, u, outs, args.steps,
                                              args.warmup, codec)
    st = plan.last_stats()
    bpe = bytes_per_element(wl, codec)
    value = 4.0 * wl.n / ms / 1e6                     # GB/s of fp32 gradient
    eff = bpe * wl.n / ms / 1e6
    k1_ach = bpe * wl.n / k1_ms / 1e6
    log(f"[bench] {ms:.3f} ms/step, {value:.1f} GB/s gradient, effective {eff:.1f} GB/s "
        f"({eff / HBM_PEAK_GBPS:.1%} of peak); EF pass {k1_ms:.3f} ms ({k1_ach:.1f} GB/s)")
    traffic = measured_traffic(wl.name) if codec in ("topk", "threshold") else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name if codec == "topk" else f"{wl.name}+{codec}",
            "codec": codec,
            "n_elements": wl.n,
            "segments": wl.n_seg,
            "k_ratio": wl.ratio,
            "total_k": int(plan.total_k),
            "momentum": wl.momentum,
            "int8": wl.int8,
            "gradient_dist": f"{wl.scale} * Student-t({wl.df})" if wl.dist == "t" else wl.dist,
        },
        "elements_per_s": round(wl.n / ms * 1e3, 1),
        # the plan's first call (no threshold estimate yet; warm-up, not in the timed steps)
        "first_call_ms": round(cold_ms, 4) if cold_ms is not None else None,
        "median_ms_per_step": round(time_steps.median_ms, 4) if time_steps.median_ms else None,
        "gradient_sha256_16": gradient_fingerprint(gbufs[0]),
        "effective_GBps": round(eff, 1),
        "hbm_peak_frac_effective": round(eff / HBM_PEAK_GBPS, 4),
        "candidates_per_k": round(float(st["candidates"].sum()) / max(plan.total_k, 1), 3),
        "full_path_segments_last_step": int((st["mode"] == gca.MODE_FULL).sum()),
        "roofline": {
            "bound": "hbm",
            "kernel": {"topk": "k_ef_capture (EF add + key + candidate capture)",
                       "threshold": "k_ef_capture (EF add + key + capture at tau)",
                       "randk": "k_randk_capture (EF add + Philox key + capture)",
                       "sign": "k_sign_pass1 + k_sign_scale + k_sign_pass2",
                       "qsgd": "k_qsgd_pass1 + k_qsgd_norm + k_qsgd_pass2"}[codec],
            "achieved": round(k1_ach, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(k1_ach / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_element": bpe,
            "avg_launch_ms": round(k1_ms, 4),
            "launches": launches,
        },
    }
    if codec == "qsgd" or (codec == "topk" and wl.name == DEFAULT_WORKLOAD
                           and not args.no_receiver):
        # local gradient clipping before compression (a context figure, not in the step)
        result["clip_all_segments"] = clip_bench(plan, wl, gbufs[-1])
        gen_mod = __import__("synth").gen
        gen_mod.fill_gradient(gbufs[-1], wl, len(gbufs) - 1)   # restore the clipped buffer
        if codec == "qsgd":
            result["with_clipping_fused"] = clip_fused_bench(
                plan, wl, codec, gbufs, e, u, outs, max(args.steps // 2, 3), args.warmup)
            log(f"[bench] QSGD with clipping folded in: "
                f"{result['with_clipping_fused']['ms_per_step']:.3f} ms/step")
        log(f"[bench] clipping: {result['clip_all_segments']['ms_per_call']:.3f} ms")
    if codec == "randk":
        result["without_error_feedback"] = randk_plain_bench(plan, wl, gbufs, outs,
                                                             max(args.steps // 2, 3))
        log(f"[bench] Random-k without feedback: "
            f"{result['without_error_feedback']['ms_per_step']:.3f} ms/step")
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline: oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(plan, wl, gbufs[0], e, u, outs, codec,
                                              t=args.warmup + args.steps)
    if codec != "topk":
        name = {"sign": "1-bit sign EF", "qsgd": "QSGD-127 EF", "threshold": "threshold EF",
                "randk": "Random-k EF"}[codec]
        result["metric"] = f"{name} compress GB/s of fp32 gradient (1 GPU) and % of HBM peak"
        print(json.dumps(result), flush=True)
        return
    del gbufs, e, u, outs
    plan.close()
    torch.cuda.empty_cache()
    try:
        add = add_stream()
        result["reference_streams"] = {
            "note": "measured streams in the pass's tile layout with non-temporal dwordx4 "
                    "accesses; references, not ceilings (the pass streams faster than the "
                    "bare 2-read/1-write kernel)",
            "read_GBps": round(read_stream(), 1),
            "copy_1r1w_GBps": round(copy_stream(), 1),
            "add_2r1w_GBps": round(add, 1),
            # the pass against the same 2-read/1-write stream without its selection work
            "pass_vs_add_2r1w": round(result["roofline"]["achieved"] / add, 4),
        }
    except Exception as ex:  # noqa: BLE001 - context figures only
        log(f"[bench] reference streams skipped: {ex}")
    if not args.no_all_configs and wl.name == DEFAULT_WORKLOAD:
        result["all_configs"] = {DEFAULT_WORKLOAD: config_record(
            wl, ms, k1_ms, time_steps.median_ms, st, plan.total_k, args.steps,
            time_steps.events_ms)}
        for name in ALL_CONFIGS:
            rec = bench_config(name, args.steps, args.warmup)
            result["all_configs"][name] = rec
            log(f"[bench] {name}: {rec['ms_per_step']:.4f} ms/step, "
                f"{rec['hbm_peak_frac_effective']:.1%} effective, pass {rec['pass_ms']:.4f} ms")
    if not args.no_receiver and wl.name == DEFAULT_WORKLOAD:
        result["receiver_8_workers"] = receiver_bench(wl)
        log(f"[bench] receiver: {result['receiver_8_workers']['ms_scatter_add']:.3f} ms")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
