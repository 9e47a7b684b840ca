#!/usr/bin/env python3
"""Throughput of the selective-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]

A step is one ssm_scan_fwd call over the whole workload (every pass of the
hot path: chunk summaries, carry combine, output pass) on inputs already
resident in HBM.  W untimed steps, then exactly K timed steps between two
device synchronizations, each step right after a 1 GiB write that evicts L2
and the Infinity Cache (so every step streams its inputs from HBM); the
headline (value, ms_per_step, hbm_gbps) is the median of those K flushed
steps.  K more steps run back to back afterwards and are reported as the
warm figures (warm_ms_per_step, ...).  Prints one JSON line.

The default workload is the largest scan: batch=1, L=1,048,576, D=512, N=16,
bf16 x, Delta, B, C and y with fp32 state (x, B, C ~ N(0,1), Delta =
softplus(0.5 N(0,1) - 4), A_log[d,n] = log(n+1), D_skip = 1).  The others:
tiny, fp32 (8 x 2048 x 1536 x 16 fp32), conv (4 x 8192 x 2560 x 16 bf16 with
the conv prologue and exact ZOH) and decode (512 consecutive ssm_step calls
on 256 x 5120 x 16 timed as one step).

Roofline of the dominant kernel (the output pass k_scan_out, or k_scan_wave
where the plan is the one-pass lane scan): its duration is measured per launch with HIP events that the library records around that
kernel on the launch stream.  Two roofs are evaluated:
  hbm  algorithmic bytes of the call / duration vs 8000 GB/s;
  alu  algorithmic VALU lane-slots / duration vs 256 CU x 4 SIMD x 16 lanes
       x 2.4 GHz = 39.3 T lane-slots/s, where an element costs 5 issue slots
       for Delta*B (v_mul, v_exp, v_mul, v_fma, v_fma) or 7 for ZOH, plus 2
       slots per (b, t, d) (Delta*u and the skip term).  A transcendental
       (v_exp, v_log, v_rcp) counts one issue slot: its unit works at half
       rate, but beside other VALU work that second cycle overlaps (the long
       scan's output pass retires 6.6e12 elements/s, more than 6 slots per
       element would allow even at 2.4 GHz).
The reported bound is the roof with the higher utilisation.

--backward times ssm_scan_bwd instead: the gradients of the same workload's
scan for upstream gradients dy ~ N(0, 1) and dh_last ~ N(0, 1); the roofline
entry is that of the main backward kernel k_bwd_main (VALU lane-slots per
element: 18 for Delta*B, 26 for ZOH -- the forward recompute plus the
adjoint step, its four gradient products and the channel-sum adds).  The
backward starts from the states the forward scan kept every 16 steps
(h_saved, written by one forward call before the timed region, as in
training); --recompute-states times the backward that computes them itself.
--train times forward (keeping the states) plus backward as one step.

--fused runs the same workload with every fused step on: the step size from
its pre-activation (softplus(delta + bias[d])), the gate y * silu(z) and, with
a conv, the conv window read from and handed back to a state buffer; the
decode workload then also runs a 4-tap conv over its rolling window.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "scan elems (B·L·D·N)/s and achieved HBM GB/s vs MI355X peak, 1 GPU"
HBM_PEAK_GBS = 8000.0
FUSED_DECODE_CONV_K = 4                    # conv taps of the fused decode run
SLOT_PEAK = 256 * 4 * 16 * 2.4e9          # VALU lane-slots per second
KERNEL_SRC = os.path.join(ROOT, "selective_state_space_83_amd", "csrc", "ssm_kernels.hpp")
BWD_SRC = os.path.join(ROOT, "selective_state_space_83_amd", "csrc", "ssm_bwd.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# HIP events through the runtime's C API (for the library's event hooks)
# ---------------------------------------------------------------------------

class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def algorithmic_bytes(w, h0=False, h_last=False, fused=False) -> int:
    s_in = 2 if w.in_dtype == "bf16" else 4
    s_out = 2 if w.out_dtype == "bf16" else 4
    Bt, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    n = Bt * L * (D * (2 * s_in + s_out) + N * 2 * s_in) + 4 * D * N + 4 * D
    if w.conv_k:
        n += 4 * D * w.conv_k + 4 * D
    n += 4 * Bt * D * N * (int(h0) + int(h_last))
    if fused:
        n += Bt * L * D * s_in + 4 * D                 # z, delta_bias
        if w.conv_k:
            n += 2 * 4 * Bt * D * (w.conv_k - 1)        # conv window in and out
    return n


def decode_bytes(w, fused=False) -> int:
    """Algorithmic bytes of one decode step: h read and written (fp32), x,
    Delta and y, the B and C rows, A and D; fused also z, delta_bias, the conv
    weights and bias and the fp32 window read and written."""
    s_in = 2 if w.in_dtype == "bf16" else 4
    n = (2 * 4 * w.batch * w.dim * w.dstate + w.batch * w.dim * 3 * s_in
         + 2 * w.batch * w.dstate * s_in + 4 * w.dim * (w.dstate + 1))
    if fused:
        K = FUSED_DECODE_CONV_K
        n += (w.batch * w.dim * s_in + 4 * w.dim * (2 + K)
              + 2 * 4 * w.batch * w.dim * (K - 1))
    return n


# VALU issue slots per (b, t, d) of the fused steps: softplus (bias add,
# scale, exp, 1 + e, compare + select, log, 2 muls, sub, rcp) and the gate
# (scale, exp, add, rcp, 2 muls); a transcendental counts one slot
SLOTS_BWD_ELEM = {False: 18.0, True: 26.0}   # k_bwd_main, keyed by ZOH
SLOTS_SOFTPLUS = 12.0
SLOTS_GATE = 6.0


def algorithmic_slots(w, fused=False) -> float:
    per_elem = 7.0 if w.zoh else 5.0
    per_btd = 2.0
    if w.conv_k:
        per_btd += 4 + 1 + 1 + 2   # 4 taps, exp, rcp, add + mul of SiLU
    if fused:
        per_btd += SLOTS_SOFTPLUS + SLOTS_GATE
    Bt, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    return Bt * L * D * (N * per_elem + per_btd)


def traffic_record(workload: str, kernel: str = "k_scan_out"):
    """HBM traffic per launch of `kernel` from committed rocprofv3 --pmc
    summaries, valid only if the kernel sources are unchanged since they were
    taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src_hash = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != src_hash:
        return None
    if "bwd_source_sha256" in rec:
        bwd_hash = hashlib.sha256(open(BWD_SRC, "rb").read()).hexdigest()
        if rec["bwd_source_sha256"] != bwd_hash:
            return None
    return rec.get("bytes_per_launch")


def copy_bandwidth(torch, nbytes=1 << 30, reps=10) -> float:
    """Achievable streaming rate in GB/s (bytes read + written) of a plain
    elementwise kernel, dst = src + 1 over fp32, on buffers large enough
    (1 GiB each) to stream from HBM rather than the 256 MB Infinity Cache:
    the practical ceiling an HBM-bound kernel is held to.  (The runtime's own
    copy kernel streams more slowly than torch's elementwise kernels here.)"""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.add(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


# ---------------------------------------------------------------------------
# runs
# ---------------------------------------------------------------------------

def to_dev(a, dtype, torch):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def bench_scan(w, steps, warmup, torch, ssm, chunk_len=0, fused=False):
    import ssm_inputs as SI
    inp = SI.scan_inputs(w)
    t = {k: to_dev(inp[k], w.in_dtype, torch) for k in ("x", "delta", "B", "C")}
    for k in ("A", "D", "conv_w", "conv_b"):
        t[k] = to_dev(inp[k], "f32", torch)
    odt = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
    y = torch.empty(t["x"].shape, dtype=odt, device="cuda")
    kw = {}
    if fused:
        ex = SI.fused_inputs(w)
        t["delta"] = to_dev(ex["delta_raw"], w.in_dtype, torch)
        kw = dict(delta_bias=to_dev(ex["delta_bias"], "f32", torch), delta_softplus=True,
                  z=to_dev(ex["z"], w.in_dtype, torch))
        if w.conv_k:
            kw["conv_state_in"] = to_dev(ex["conv_state"], "f32", torch)
            kw["conv_state_out"] = torch.empty_like(kw["conv_state_in"])
    # arguments are checked and marshalled once, so the timed loop measures
    # the library's launches rather than Python argument handling
    prep, y, _ = ssm.prepare_scan(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                  conv_w=t["conv_w"], conv_b=t["conv_b"], zoh=w.zoh, y=y,
                                  chunk_len=chunk_len, **kw)
    ws_bytes = ssm.workspace_size(prep.args)
    chunk = ssm.plan_chunk_len(prep.args)
    lane_scan = ssm.plan_lane_scan(prep.args)
    hip = HipEvents()
    evs = hip.create(4 * steps)       # the output pass of every timed step, both loops
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def call(i=None):
        ev = (evs[2 * i], evs[2 * i + 1]) if i is not None else None
        prep.run(stream=stream, events=ev)

    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # timed region: K steps, each right after a cache-evicting write (the
    # write is outside each step's event pair)
    t0 = time.perf_counter()
    pairs = [ev_pair() for _ in range(steps)]
    for i in range(steps):
        flush.fill_(1)
        pairs[i][0].record(stream)
        call(i)
        pairs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flushed_ms = [a.elapsed_time(b) for a, b in pairs]
    out_ms = [hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)]
    # warm: K more steps back to back
    e0, e1 = ev_pair()
    e0.record(stream)
    for i in range(steps):
        call(steps + i)
    e1.record(stream)
    torch.cuda.synchronize()
    warm_total_ms = e0.elapsed_time(e1)
    out_ms_warm = [hip.elapsed_ms(evs[2 * (steps + i)], evs[2 * (steps + i) + 1])
                   for i in range(steps)]
    hip.destroy(evs)
    del flush
    return dict(inp=inp, flushed_ms=flushed_ms, wall_s=wall, out_ms=out_ms,
                warm_ms=warm_total_ms / steps, out_ms_warm=out_ms_warm,
                chunk_len=chunk, chunks=-(-w.seqlen // chunk), workspace=ws_bytes,
                kernel="k_scan_wave" if lane_scan else "k_scan_out")


def bench_decode(w, steps, warmup, torch, ssm, fused=False):
    """One step = `w.steps` consecutive ssm_step calls (a 512-token decode)."""
    import ssm_inputs as SI
    n = w.steps
    inp = SI.decode_inputs(w)
    h = to_dev(inp["h"], "f32", torch)
    A, Dv = to_dev(inp["A"], "f32", torch), to_dev(inp["D"], "f32", torch)
    xs, ds_, Bs, Cs = (to_dev(inp[k], w.in_dtype, torch) for k in ("x", "delta", "B", "C"))
    y = torch.empty((w.batch, w.dim), dtype=torch.bfloat16, device="cuda")
    per_tok = [{} for _ in range(n)]
    if fused:
        ex = SI.fused_inputs(w.with_(conv_k=FUSED_DECODE_CONV_K), steps=n)
        ds_ = to_dev(ex["delta_raw"], w.in_dtype, torch)
        zs = to_dev(ex["z"], w.in_dtype, torch)
        common = dict(delta_bias=to_dev(ex["delta_bias"], "f32", torch), delta_softplus=True,
                      conv_w=to_dev(ex["conv_w"], "f32", torch),
                      conv_b=to_dev(ex["conv_b"], "f32", torch),
                      conv_state=to_dev(ex["conv_state"], "f32", torch))
        per_tok = [dict(common, z=zs[s]) for s in range(n)]
    # arguments marshalled once per token; the timed loop only launches
    calls = [ssm.prepare_step(h, xs[s], ds_[s], A, Bs[s], Cs[s], Dv, y=y, **per_tok[s])[0]
             for s in range(n)]
    stream = torch.cuda.current_stream()

    def run():
        for s in range(n):
            calls[s].run(stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # k_step launches run back to back on the stream (the host enqueues them
    # faster than they execute), so the timed region over the launch count is
    # the average launch duration, inter-launch gap included; events around
    # each launch would add their own overhead to every launch instead.
    launch_us = e0.elapsed_time(e1) * 1e3 / (steps * n)
    # one more decode of all the tokens right after a 1 GiB write that evicts
    # L2 and the Infinity Cache (state and inputs start in HBM)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush.fill_(1)
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    run()
    f1.record(stream)
    torch.cuda.synchronize()
    del flush
    return dict(total_ms=e0.elapsed_time(e1), wall_s=wall, launch_us=launch_us,
                flushed_ms=f0.elapsed_time(f1), inp=inp)


def bench_bwd(w, steps, warmup, torch, ssm, kept=True, train=False):
    """Backward (train=False) or forward + backward (train=True) steps; with
    kept=True the backward starts from the forward's kept states."""
    import ssm_inputs as SI
    inp = SI.scan_inputs(w, h0=True)
    gi = SI.grad_inputs(w)
    t = {k: to_dev(inp[k], w.in_dtype, torch) for k in ("x", "delta", "B", "C")}
    A, Dv, h0 = (to_dev(inp[k], "f32", torch) for k in ("A", "D", "h0"))
    dy = to_dev(gi["dy"], w.in_dtype, torch)
    dhl = to_dev(gi["dh_last"], "f32", torch)
    hs = None
    if kept or train:
        hs = torch.empty(ssm.saved_states_shape(w.batch, w.seqlen, w.dim, w.dstate),
                         dtype=torch.float32, device="cuda")
    fwd, _, _ = ssm.prepare_scan(t["x"], t["delta"], A, t["B"], t["C"], Dv, h0=h0, zoh=w.zoh,
                                 h_saved=hs)
    prep, _ = ssm.prepare_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0,
                              dh_last=dhl, zoh=w.zoh, h_saved=hs)
    hip = HipEvents()
    evs = hip.create(2 * steps)
    stream = torch.cuda.current_stream()
    if hs is not None:
        fwd.run(stream)          # the states the backward starts from
    for _ in range(warmup):
        if train:
            fwd.run(stream)
        prep.run(stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        if train:
            fwd.run(stream)
        prep.run(stream, events=(evs[2 * i], evs[2 * i + 1]))
    e1.record(stream)
    torch.cuda.synchronize()
    main_ms = [hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)]
    hip.destroy(evs)
    return dict(total_ms=e0.elapsed_time(e1), main_ms=main_ms,
                super_chunk=None, inp=inp, gi=gi)


def cpu_baseline(w, inp, budget_s=20.0, min_s=10.0):
    """The oracle, untuned, on this host's cores, over a bounded sample of the
    same workload: whole batch rows when a row takes at most half the budget
    (whole passes over the batch repeated until min_s has elapsed when the
    whole workload is quicker than that), otherwise consecutive 64-channel
    blocks of the batch rows (wrapping around) until min_s has elapsed."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    orc = oracle.default()

    def run(r0, r1, d0=0, d1=None):
        d1 = w.dim if d1 is None else d1
        sl = lambda a: a[r0:r1, :, d0:d1]
        ch = lambda a: None if a is None else a[d0:d1]
        t = time.perf_counter()
        orc.scan(sl(inp["x"]), sl(inp["delta"]), ch(inp["A"]), inp["B"][r0:r1],
                 inp["C"][r0:r1], ch(inp["D"]), conv_w=ch(inp.get("conv_w")),
                 conv_b=ch(inp.get("conv_b")), zoh=w.zoh, want_h_last=False, nthreads=cores)
        return time.perf_counter() - t

    blk = min(64, w.dim)
    dt = run(0, 1, 0, blk)          # probe: one block of row 0
    per_row = dt * w.dim / blk
    if per_row <= budget_s / 2:
        dt = run(0, 1)
        rows = 1
        extra = int(min(w.batch - 1, max(0, budget_s / max(dt, 1e-6) - 1)))
        if extra > 0:
            dt += run(1, 1 + extra)
            rows += extra
        passes = 1
        if rows == w.batch:
            while dt < min_s:
                dt += run(0, w.batch)
                passes += 1
        elems = (rows + (passes - 1) * w.batch) * w.seqlen * w.dim * w.dstate
        if passes > 1:
            what = "%d passes over the whole workload (%d batch row%s" % (
                passes, w.batch, "s" if w.batch > 1 else "")
        else:
            what = "%d of %d batch rows (" % (rows, w.batch)
        sample = "%s of %d x %d x %d elems)" % (what, w.seqlen, w.dim, w.dstate)
    else:
        nblk = 1
        k = 1
        nb = -(-w.dim // blk)
        while dt < min_s:
            r, j = divmod(k, nb)
            d0 = j * blk
            dt += run(r % w.batch, r % w.batch + 1, d0, min(w.dim, d0 + blk))
            nblk += 1
            k += 1
        elems = nblk * w.seqlen * blk * w.dstate
        sample = ("%d consecutive blocks of %d channels of a batch row (1 x %d x %d x %d "
                  "elems each)" % (nblk, blk, w.seqlen, blk, w.dstate))
    return {"value": elems / dt, "unit": "elem/s", "cores": cores, "kind": "oracle",
            "sample": "%s, fp64 sequential recurrence, %.1f s wall" % (sample, dt),
            "single_thread": cpu_single_thread(w, inp, orc)}


def cpu_baseline_bwd(w, inp, gi, train, budget_s=20.0, min_s=10.0):
    """The oracle's backward (after its forward when `train`) on this host's
    cores: whole batch rows of the same workload, as many as fit the budget
    (at least one), whole passes repeated until min_s has elapsed."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    orc = oracle.default()

    def run(lo, hi):
        t = time.perf_counter()
        if train:
            orc.scan(inp["x"][lo:hi], inp["delta"][lo:hi], inp["A"], inp["B"][lo:hi],
                     inp["C"][lo:hi], inp["D"], h0=inp["h0"][lo:hi], zoh=w.zoh,
                     nthreads=cores)
        orc.scan_bwd(inp["x"][lo:hi], inp["delta"][lo:hi], inp["A"], inp["B"][lo:hi],
                     inp["C"][lo:hi], gi["dy"][lo:hi], D=inp["D"], h0=inp["h0"][lo:hi],
                     dh_last=gi["dh_last"][lo:hi], zoh=w.zoh, nthreads=cores)
        return time.perf_counter() - t

    dt = run(0, 1)
    rows = 1
    extra = int(min(w.batch - 1, max(0, budget_s / max(dt, 1e-6) - 1)))
    if extra > 0:
        dt += run(1, 1 + extra)
        rows += extra
    passes = 1
    if rows == w.batch:
        while dt < min_s:
            dt += run(0, w.batch)
            passes += 1
    what = ("%d passes over all %d batch rows" % (passes, w.batch) if passes > 1
            else "%d of %d batch rows" % (rows, w.batch))
    return {"value": (rows + (passes - 1) * w.batch) * w.seqlen * w.dim * w.dstate / dt,
            "unit": "elem/s", "cores": cores, "kind": "oracle",
            "sample": "%s (%d x %d x %d elems each), fp64 %s, %.1f s wall"
                      % (what, w.seqlen, w.dim, w.dstate,
                         "forward + reverse sweep" if train else "reverse-mode sweep", dt)}


def cpu_baseline_decode(w, inp, min_s=10.0):
    """The oracle's decode step on this host's cores over the workload's
    tokens in order (whole passes over all of them repeated until min_s has
    elapsed)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    orc = oracle.default()
    dt, tokens = 0.0, 0
    while dt < min_s:
        h = inp["h"]
        for s in range(w.steps):
            t = time.perf_counter()
            _, h = orc.step(h, inp["x"][s], inp["delta"][s], inp["A"], inp["B"][s],
                            inp["C"][s], inp["D"], nthreads=cores)
            dt += time.perf_counter() - t
            tokens += 1
            if dt >= min_s and tokens >= 8:
                break
    per_token = w.batch * w.dim * w.dstate
    return {"value": tokens * per_token / dt, "unit": "elem/s", "cores": cores, "kind": "oracle",
            "sample": "%d decode steps of %d x %d x %d elems in order, fp64, %.1f s wall"
                      % (tokens, w.batch, w.dim, w.dstate, dt)}


def cpu_single_thread(w, inp, orc, min_s=1.0):
    """The same oracle on one thread over 1/64 of the channels of one batch
    row (whole passes repeated until min_s has elapsed): a per-core figure
    beside the all-cores baseline."""
    import numpy as np
    nd = max(1, w.dim // 64)
    part = {k: np.ascontiguousarray(inp[k][:1, :, :nd]) for k in ("x", "delta")}
    for k in ("A", "D", "conv_w", "conv_b"):
        part[k] = None if inp.get(k) is None else np.ascontiguousarray(inp[k][:nd])
    dt, passes = 0.0, 0
    while dt < min_s:
        t = time.perf_counter()
        orc.scan(part["x"], part["delta"], part["A"], inp["B"][:1], inp["C"][:1], part["D"],
                 conv_w=part["conv_w"], conv_b=part["conv_b"], zoh=w.zoh, want_h_last=False,
                 nthreads=1)
        dt += time.perf_counter() - t
        passes += 1
    return {"value": passes * w.seqlen * nd * w.dstate / dt, "unit": "elem/s",
            "sample": "%d passes over %d channels of one batch row, one thread, %.1f s wall"
                      % (passes, nd, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward scan (ssm_scan_bwd) of the workload")
    ap.add_argument("--recompute-states", action="store_true",
                    help="with --backward: the backward computes the forward states itself")
    ap.add_argument("--train", action="store_true",
                    help="time forward (keeping the states) + backward as one step")
    ap.add_argument("--fused", action="store_true",
                    help="run with the fused steps on (softplus step size, gate, conv window)")
    ap.add_argument("--chunk-len", type=int, default=0,
                    help="force the scan's chunk length (0 = the library's plan)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times); "
                         "its FETCH_SIZE / WRITE_SIZE counters calibrate HBM traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the scan is not sharded across GPUs by this "
              "library; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return
    import selective_state_space_83_amd as ssm
    import ssm_inputs as SI

    ssm.load_library()
    w = SI.WORKLOADS[args.workload]
    torch.cuda.init()
    log("bench: workload %s, %d warmup + %d timed steps" % (w, args.warmup, args.steps))

    if w.steps:
        r = bench_decode(w, args.steps, args.warmup, torch, ssm, fused=args.fused)
        ms = r["total_ms"] / args.steps
        elems = w.elems
        per_launch = decode_bytes(w, fused=args.fused)
        bytes_ = w.steps * per_launch
        ach = per_launch / (r["launch_us"] * 1e-6) / 1e9
        copy = copy_bandwidth(torch)
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS,
                "traffic": None if args.fused else traffic_record(w.name, "k_step"),
                "kernel": "k_step", "kernel_us": r["launch_us"],
                "copy_gbps": copy, "frac_of_copy": ach / copy}
        out = {"metric": METRIC, "value": elems / (ms * 1e-3), "unit": "elem/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": "f32", "data": "synthetic",
               "config": {"workload": "decode", "batch": w.batch, "dim": w.dim,
                          "dstate": w.dstate, "tokens_per_step": w.steps,
                          "in_dtype": w.in_dtype, "state": "f32",
                          "fused": "softplus+gate+conv4" if args.fused else None},
               "hbm_gbps": bytes_ / (ms * 1e-3) / 1e9,
               "flushed_ms_per_step": r["flushed_ms"],
               "roofline": roof,
               "cpu_baseline": (None if args.no_cpu_baseline or args.fused
                                else cpu_baseline_decode(w, r["inp"]))}
        print(json.dumps(out), flush=True)
        return

    if args.backward or args.train:
        kept = not args.recompute_states
        r = bench_bwd(w, args.steps, args.warmup, torch, ssm, kept=kept, train=args.train)
        ms = r["total_ms"] / args.steps
        main_us = float(np.mean(r["main_ms"])) * 1e3
        slots = w.elems * SLOTS_BWD_ELEM[w.zoh]
        alu = slots / (main_us * 1e-6) / 1e12
        roof = {"bound": "alu", "achieved": alu, "peak": SLOT_PEAK / 1e12,
                "unit": "T lane-slot/s", "frac": alu / (SLOT_PEAK / 1e12),
                "traffic": traffic_record(w.name, "k_bwd_main") if kept and not args.train
                else None,
                "kernel": "k_bwd_main", "kernel_us": main_us}
        out = {"metric": METRIC, "value": w.elems / (ms * 1e-3), "unit": "elem/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": "f32", "data": "synthetic",
               "config": {"workload": w.name,
                          "pass": "forward+backward" if args.train else "backward",
                          "states": "kept by the forward" if (kept or args.train)
                          else "recomputed",
                          "batch": w.batch,
                          "seqlen": w.seqlen, "dim": w.dim, "dstate": w.dstate,
                          "in_dtype": w.in_dtype, "disc": "zoh" if w.zoh else "delta_b"},
               "roofline": roof,
               "cpu_baseline": (None if args.no_cpu_baseline
                                else cpu_baseline_bwd(w, r["inp"], r["gi"], args.train))}
        print(json.dumps(out), flush=True)
        return

    r = bench_scan(w, args.steps, args.warmup, torch, ssm, args.chunk_len, fused=args.fused)
    ms = float(np.median(r["flushed_ms"]))
    elems = w.elems
    out_us = float(np.mean(r["out_ms"])) * 1e3
    out_us_warm = float(np.mean(r["out_ms_warm"])) * 1e3
    abytes = algorithmic_bytes(w, fused=args.fused)
    slots = algorithmic_slots(w, fused=args.fused)
    hbm_ach = abytes / (out_us * 1e-6) / 1e9
    alu_ach = slots / (out_us * 1e-6) / 1e12
    hbm_frac = hbm_ach / HBM_PEAK_GBS
    alu_frac = alu_ach / (SLOT_PEAK / 1e12)
    traffic = None if args.fused else traffic_record(w.name, r["kernel"])
    if alu_frac > hbm_frac:
        roof = {"bound": "alu", "achieved": alu_ach, "peak": SLOT_PEAK / 1e12,
                "unit": "T lane-slot/s", "frac": alu_frac, "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": hbm_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": hbm_frac, "traffic": traffic}
    roof["kernel"] = r["kernel"]
    roof["kernel_us"] = out_us
    roof["kernel_us_warm"] = out_us_warm
    copy = copy_bandwidth(torch)
    roof["hbm_view"] = {"achieved_gbps": hbm_ach, "frac": hbm_frac, "copy_gbps": copy,
                        "frac_of_copy": hbm_ach / copy}
    roof["alu_view"] = {"achieved_tslots": alu_ach, "frac": alu_frac}
    whole_gbps = abytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline and not args.fused:
        log("bench: timing the oracle on the host")
        cpu = cpu_baseline(w, r["inp"])
    dtype = "f32"   # arithmetic and state are fp32 for every storage dtype
    out = {"metric": METRIC, "value": elems / (ms * 1e-3), "unit": "elem/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dtype, "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                      "dstate": w.dstate, "in_dtype": w.in_dtype, "out_dtype": w.out_dtype,
                      "disc": "zoh" if w.zoh else "delta_b", "conv_k": w.conv_k,
                      "chunk_len": r["chunk_len"], "chunks": r["chunks"],
                      "timing": "median of K steps, each after a 1 GiB cache-evicting write",
                      "fused": ("softplus+gate" + ("+conv_state" if w.conv_k else ""))
                      if args.fused else None},
           "hbm_gbps": whole_gbps, "hbm_frac": whole_gbps / HBM_PEAK_GBS,
           "warm_ms_per_step": r["warm_ms"], "warm_value": elems / (r["warm_ms"] * 1e-3),
           "warm_hbm_gbps": abytes / (r["warm_ms"] * 1e-3) / 1e9,
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
