#!/usr/bin/env python3
"""Attention-forward throughput of one MI355X on a seeded synthetic workload.

Default workload: one rank's share of an 8-way zigzag ring at 128K context
(B=1, H=32, d=128, bf16, causal, RoPE base 10000): 16384 local query rows
against 131072 keys in ring order, 17 attention sub-calls (those of each query
half run up to sixteen to a launch of the chained kernel, which carries the
softmax state across them: 3 launches per step, the last launch of each half
writing the bf16 output).  One step is one whole
share (attn_ring_fwd), inputs resident in HBM.  `--workload N` selects another
workload (workloads.py: 0-4 the forward configurations, 5 one decoding step,
6 the same 128K sequence's share under the head-parallel layout).

value  = algorithmic TFLOP/s of the step: 4 d FLOPs per allowed (query, key)
         pair (two contractions, 2 FLOPs per multiply-add); masked work that
         tiles skip is not counted.
roofline = the attention kernel alone: the same algorithmic FLOPs divided by
         the kernel's own time, measured with HIP events recorded around every
         launch on the launch's stream over K further steps run after the
         timed ones (so the events add no gaps to the step time), against the
         MI355X dense bf16 MFMA peak (2516.6 TFLOP/s).
cpu_baseline = the fp64 oracle timed on the host cores on a bounded sample
         of the same workload (rank 0, one GPU only).
clock  = the shader clock and board power sampled from sysfs over the timing.
warmup = untimed steps before the timed ones: --warmup W runs exactly W; by
         default at least 5 and at least 0.2 s of them, since the clock climbs
         from idle over the first tens of milliseconds of load (on the encoder
         workload five warm-up steps left the first timed steps 5-15% slow).

--pass bwd times the backward of the same share instead (attn_ring_bwd, or
attn_bwd for a single call): 8 d algorithmic FLOPs per allowed pair (dP, dV,
dQ, dK; the recomputed scores are not counted), and the roofline takes the dQ
and dK/dV kernels of one sub-call together as one launch.

step_ms  = median, min and max wall time of single steps, from one HIP event
         at each step boundary over K more steps (a third pass; value and
         ms_per_step come from the first, which has no events inside it).
targets = the default run (workload 4, forward) also times workloads 2 (the
         8K ring share) and 3 (the encoder), the other configurations of the
         >= 50 % of peak target, by the same method, each in a child process
         started before this one initialises the GPU: step and kernel-only
         TFLOP/s with their fractions of the peak.  --no-targets skips them.
mfma_sustained = the default run also runs the matrix-core rate probe
         (probe/mfma_rate, built with the library) first: a stream of
         independent bf16 MFMAs with no memory traffic, held for a few
         seconds, once with standard-normal and once with zero operands.  Under
         sustained load the board holds its power cap by lowering the shader
         clock, so this is the rate a kernel doing nothing but matrix work
         sustains on this board; the attention kernel's rate is also given as
         a fraction of it.  The roofline's peak stays the published one.
         --no-yardstick skips it.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import blockwise_online_softmax_attn_amd as bosa  # noqa: E402
import workloads  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of MFMA bf16 peak (causal, d=128) on 1 MI355X"
METRIC_BWD = "attention bwd TFLOP/s and % of MFMA bf16 peak (causal, d=128) on 1 MI355X"
METRIC_DECODE = "attention decode step GB/s over the key/value cache (bf16, d=128) on 1 MI355X"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6      # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_F32_TFLOPS = 157.3
TRAFFIC_FILES = {"fwd": os.path.join(ROOT, "profiles", "attn_fwd_bf16_traffic.json"),
                 "bwd": os.path.join(ROOT, "profiles", "attn_bwd_bf16_traffic.json"),
                 "decode": os.path.join(ROOT, "profiles", "attn_decode_bf16_traffic.json")}
KERNEL_SOURCES = {
    "fwd": ["blockwise_online_softmax_attn_amd/csrc/fwd_bf16.hip",
            "blockwise_online_softmax_attn_amd/csrc/tile_io.h",
            "blockwise_online_softmax_attn_amd/csrc/common.h"],
    "bwd": ["blockwise_online_softmax_attn_amd/csrc/bwd_bf16.hip",
            "blockwise_online_softmax_attn_amd/csrc/tile_io.h",
            "blockwise_online_softmax_attn_amd/csrc/common.h"],
    "decode": ["blockwise_online_softmax_attn_amd/csrc/decode.hip",
               "blockwise_online_softmax_attn_amd/csrc/common.h"],
}
# kernels whose counters make up one attention "launch" of each pass: the
# forward kernel alone; for the backward the dQ and dK/dV kernels of one
# sub-call together
TRAFFIC_KERNELS = {"fwd": ("attn_fwd_bf16_chain_kernel<128",),
                   "bwd": ("bwd_dq_kernel<128", "bwd_dkdv_kernel<128"),
                   "decode": ("decode_chunk_kernel<unsigned short, 128",)}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources_sha(which: str = "fwd") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ---------------------------------------------------------------- pair counts
def causal_pairs(q_pos0: int, nq: int, kv_pos0: int, nk: int, valid=None) -> int:
    """Allowed pairs of a contiguous query block against a contiguous key
    block under causal order, optionally restricted to keys with valid=True."""
    i = np.arange(nq, dtype=np.int64)
    lim = np.clip(q_pos0 + i - kv_pos0 + 1, 0, nk)          # keys [0, lim) are not in the future
    if valid is None:
        return int(lim.sum())
    prefix = np.concatenate([[0], np.cumsum(valid.astype(np.int64))])
    return int(prefix[lim].sum())


def step_pairs(w, plan, kpm) -> int:
    """Allowed (query, key) pairs of one step, summed over batch and heads."""
    total = 0
    for b in range(w.B):
        valid = None if kpm is None else (kpm[b].numpy() == 0)
        if plan is None:
            if w.causal:
                total += causal_pairs(0, w.T, 0, w.T, valid)
            else:
                total += w.T * (w.T if valid is None else int(valid.sum()))
        else:
            for c in plan:
                vb = None if valid is None else valid[c.kv_pos0:c.kv_pos0 + c.kv_rows]
                if w.causal:
                    total += causal_pairs(c.q_pos0, c.q_rows, c.kv_pos0, c.kv_rows, vb)
                else:
                    total += c.q_rows * (c.kv_rows if vb is None else int(vb.sum()))
    return total * w.H


# ---------------------------------------------------------------- inputs
def build_inputs(w):
    dev = torch.device("cuda:0")
    kpm = workloads.key_padding_mask(w)
    if w.ring_P > 1:
        plan = bosa.attn_ring_plan(w.T, w.ring_P, w.ring_rank, w.zigzag, w.causal)
        # the rank's local query chunks, in local order
        firsts = {}
        for c in plan:
            firsts.setdefault(c.q_row0, c.q_pos0)
        chunks = [firsts[r] // w.chunk for r in sorted(firsts)]
        q = workloads.draw_tokens(w, 0, chunks)
        qpos = np.concatenate([np.arange(firsts[r], firsts[r] + plan[0].q_rows) for r in sorted(firsts)])
    else:
        plan = None
        q = workloads.draw_tokens(w, 0, range(w.n_chunks))
        qpos = np.arange(w.T)
    k = workloads.draw_tokens(w, 1, range(w.n_chunks))
    v = workloads.draw_tokens(w, 2, range(w.n_chunks))
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    dkpm = None if kpm is None else kpm.to(dev)
    return plan, (q, k, v, kpm, qpos), (dq, dk, dv, dkpm)


def make_step(w, plan, dev_inputs):
    dq, dk, dv, dkpm = dev_inputs
    out = torch.empty_like(dq)
    Tq = dq.shape[1]
    lse = torch.empty((w.B, w.H, Tq), dtype=torch.float32, device=dq.device)
    if plan is not None:
        acc = out if dq.dtype == torch.float32 else torch.empty(dq.shape, dtype=torch.float32, device=dq.device)

        def step():
            bosa.attn_ring_fwd(dq, dk, dv, P=w.ring_P, rank=w.ring_rank, zigzag=w.zigzag, causal=w.causal,
                               kpm=dkpm, rope_base=w.rope_base, out=out, lse=lse, acc=acc)
        step.outputs = (out, lse)
        return step, len(plan)

    def step():
        bosa.attn_fwd(dq, dk, dv, out, lse, causal=w.causal, kpm=dkpm, rope_base=w.rope_base)
    step.outputs = (out, lse)
    return step, 1


def make_bwd_step(w, plan, dev_inputs):
    """The backward of the same share: forward once (untimed) for out and lse,
    then each step runs attn_ring_bwd (or attn_bwd) on a fixed dout."""
    dq, dk, dv, dkpm = dev_inputs
    chunks = None
    if plan is not None:
        firsts = {}
        for c in plan:
            firsts.setdefault(c.q_row0, c.q_pos0)
        chunks = [firsts[r] // w.chunk for r in sorted(firsts)]
    dout = workloads.draw_tokens(w, 4, chunks if chunks is not None else range(w.n_chunks)).to(dq.device)
    if plan is not None:
        out, lse = bosa.attn_ring_fwd(dq, dk, dv, P=w.ring_P, rank=w.ring_rank, zigzag=w.zigzag, causal=w.causal,
                                      kpm=dkpm, rope_base=w.rope_base)
        g = [torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)]

        def step():
            bosa.attn_ring_bwd(dq, dk, dv, out, dout, lse, P=w.ring_P, rank=w.ring_rank, zigzag=w.zigzag,
                               causal=w.causal, kpm=dkpm, rope_base=w.rope_base, dq=g[0], dk=g[1], dv=g[2])
        return step, 2 * len(plan), dout.cpu()
    out, lse = bosa.attn_fwd(dq, dk, dv, causal=w.causal, kpm=dkpm, rope_base=w.rope_base)
    g = [torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)]

    def step():
        bosa.attn_bwd(dq, dk, dv, out, dout, lse, g[0], g[1], g[2], causal=w.causal, kpm=dkpm,
                      rope_base=w.rope_base)
    return step, 2, dout.cpu()


# ---------------------------------------------------------------- CPU baseline
def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class ClockSampler:
    """The shader clock and the board power while a block runs: a thread reads
    the driver's current sclk level (the line of pp_dpm_sclk marked '*') and
    hwmon power1_input every `period` seconds.  Reading these files starts no
    program and makes no GPU call.  With no such files (or more than one GPU's)
    the summary is None."""

    def __init__(self, period: float = 0.01):
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.sclk_file = cards[0] if len(cards) == 1 else None
        pw = sorted(glob.glob(os.path.join(os.path.dirname(cards[0]), "hwmon", "hwmon*", "power1_input"))) \
            if self.sclk_file else []
        self.power_file = pw[0] if pw else None
        self.period = period
        self.mhz, self.watts = [], []
        self._stop = threading.Event()
        self._thread = None

    def _read(self):
        try:
            with open(self.sclk_file) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        self.mhz.append(float(line.split(":", 1)[1].strip().split("Mhz")[0]))
                        break
            if self.power_file:
                with open(self.power_file) as f:
                    self.watts.append(int(f.read().strip()) / 1e6)
        except (OSError, ValueError, IndexError):
            pass

    def _run(self):
        while not self._stop.wait(self.period):
            self._read()

    def __enter__(self):
        if self.sclk_file:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.mhz:
            return None
        m = np.asarray(self.mhz)
        out = {"sclk_mhz": {"mean": float(m.mean()), "min": float(m.min()), "max": float(m.max()),
                            "samples": int(m.size)},
               "source": "pp_dpm_sclk current level, sampled every %g s over the timed steps and the "
                         "per-launch timing" % self.period}
        if self.watts:
            p = np.asarray(self.watts)
            out["power_w"] = {"mean": float(p.mean()), "max": float(p.max())}
        return out


WARMUP_MIN_S = 0.2


def warm_up(step, n) -> int:
    """Run n untimed steps; with n None, at least 5 steps and at least
    WARMUP_MIN_S seconds of them (the clock climbs from its idle level over
    the first tens of milliseconds of load).  Returns the number run."""
    if n is not None:
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        return n
    done, t0 = 0, time.perf_counter()
    while done < 5 or time.perf_counter() - t0 < WARMUP_MIN_S:
        step()
        torch.cuda.synchronize()
        done += 1
    return done


def graph_pass(step, n: int, outputs) -> dict:
    """One step captured into a HIP graph (torch.cuda.CUDAGraph) and replayed:
    each of three checked replays, with eager work between them, must give
    the eager step's outputs bit for bit; then n replays are timed."""
    try:
        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outputs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for _ in range(3):
            for t in outputs:
                t.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(outputs, ref)):
                return {"error": "a graph replay differs from the eager step"}
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(n):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        return {"ms_per_step": start.elapsed_time(end) / n, "steps": n, "replays_checked": 3}
    except RuntimeError as e:   # capture refused by the runtime or the library
        torch.cuda.synchronize()
        return {"error": str(e)[:300]}


def step_stats(step, n: int) -> dict:
    """Wall time of each of n further steps: one HIP event at every step
    boundary on the current stream (a separate pass, after the timed one)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.asarray([ev[i].elapsed_time(ev[i + 1]) for i in range(n)], dtype=np.float64)
    return {"median": float(np.median(t)), "min": float(t.min()), "max": float(t.max()), "steps": n}


def cpu_baseline(w, host_inputs, rows: int, heads: int, dout=None):
    """The fp64 oracle, as it stands, on the heaviest `rows` local query rows
    of the first `heads` heads against every key (bounded sample); the
    backward oracle instead when dout is given."""
    import threadpoolctl

    import oracle
    q, k, v, kpm, qpos = host_inputs
    sel = np.arange(q.shape[1] - rows, q.shape[1])
    qs = q[:, sel, :heads].double().numpy()
    ks = k[:, :, :heads].double().numpy()
    vs = v[:, :, :heads].double().numpy()
    info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    t0 = time.perf_counter()
    if dout is None:
        oracle.sdpa(qs, ks, vs, qpos[sel], np.arange(w.T), causal=w.causal,
                    kpm=None if kpm is None else kpm.numpy(), rope_base=w.rope_base, dtype=w.dtype)
    else:
        oracle.sdpa_backward(qs, ks, vs, dout[:, sel, :heads].double().numpy(), qpos[sel], np.arange(w.T),
                             causal=w.causal, kpm=None if kpm is None else kpm.numpy(), rope_base=w.rope_base,
                             dtype=w.dtype)
    dt = time.perf_counter() - t0
    pairs = 0
    for b in range(w.B):
        valid = None if kpm is None else (kpm[b].numpy() == 0)
        for p in qpos[sel]:
            lim = min(int(p) + 1, w.T) if w.causal else w.T
            pairs += lim if valid is None else int(valid[:lim].sum())
    flops = (8.0 if dout is not None else 4.0) * w.d * pairs * heads
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{rows} query rows (local rows {sel[0]}..{sel[-1]}, positions {int(qpos[sel[0]])}.."
                   f"{int(qpos[sel[-1]])}) x {heads} of {w.H} heads x B={w.B} against all {w.T} keys, "
                   f"{'causal' if w.causal else 'non-causal'}{', RoPE' if w.rope_base else ''}"
                   f"{' (backward: dq, dk, dv)' if dout is not None else ''}: "
                   f"{flops:.3e} algorithmic FLOPs in {dt:.2f} s (float64 numpy, BLAS threads={blas_threads}, "
                   f"host cpus={os.cpu_count()})"),
    }


def time_steps(step, launches: int, flops: float, steps: int, per_launch: int = 1):
    """Time `steps` steps (HIP events on the current stream around them all),
    then the attention kernels alone (HIP events the library records around
    every launch on the launch's stream, over `steps` further steps, so they
    add no gaps to the step time), then per-step wall times (a third pass).
    Returns ms per step, step TFLOP/s, kernel-only TFLOP/s, the per-launch
    times, the per-step statistics and the clock sampler."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {steps} steps")
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        start.record()
        for _ in range(steps):
            step()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        with bosa.KernelTimer(max_launches=steps * launches * per_launch + 16) as kt:
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
    stats = step_stats(step, steps)
    kms = np.asarray(kt.ms, dtype=np.float64)
    kern_ms = float(kms.sum())
    achieved = flops * steps / (kern_ms * 1e-3) / 1e12 if kern_ms > 0 else None
    return ms, flops / (ms * 1e-3) / 1e12, achieved, kms, stats, clk


# the other forward workloads of the >= 50 % of peak target, timed by the
# default run with the same method and reported under "targets"
TARGET_WORKLOADS = (2, 3)


def target_lines(args) -> dict:
    """Forward workloads 2 and 3, each timed by this script in a child process
    of its own (fresh device state, as a separate run would see it), started
    before this process touches the GPU.  Returns a summary per workload."""
    import subprocess
    out = {}
    for wi in TARGET_WORKLOADS:
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", str(wi), "--steps", str(args.steps),
               "--no-cpu-baseline", "--no-targets"]
        log(f"target workload {wi}: {' '.join(cmd[1:])}")
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            out[f"workload{wi}"] = {"error": f"exit status {r.returncode}"}
            continue
        t = json.loads(lines[-1])
        ro = t["roofline"]
        out[f"workload{wi}"] = {
            "workload": t["config"]["workload"], "steps": t["steps"], "warmup": t["warmup"],
            "ms_per_step": t["ms_per_step"], "step_ms": t["step_ms"], "value": t["value"], "unit": t["unit"],
            "frac": t["value"] / PEAK_BF16_TFLOPS,
            "kernel": {"name": ro["kernel"], "achieved": ro["achieved"], "frac": ro["frac"],
                       "launches_per_step": t["config"]["attention_launches_per_step"],
                       "avg_launch_ms": ro["avg_launch_ms"]},
            "algorithmic_flops_per_step": t["config"]["algorithmic_flops_per_step"], "clock": t["clock"]}
    return out


def mfma_yardstick() -> dict:
    """The sustained matrix-core rate probe, run as a child process before
    this process initialises the GPU."""
    import subprocess
    from blockwise_online_softmax_attn_amd import _build
    if not os.path.exists(_build.PROBE):
        return {"error": "probe not built (run __graft_entry__.build())"}
    log(f"matrix-core rate probe: {_build.PROBE}")
    r = subprocess.run([_build.PROBE], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    if r.returncode != 0 or not lines:
        return {"error": f"exit status {r.returncode}: {r.stderr.strip()[-200:]}"}
    return json.loads(lines[-1])


# ---------------------------------------------------------------- decoding
def run_decode(args, w) -> dict:
    """One decoding step per iteration over a static cache of w.T slots per
    row (filled lengths from the workload's length range): attn_kv_append of
    the new token, then attn_decode of its query.  Algorithmic bytes: every
    visible cached key and value row read once (the append and the query are
    a few KiB)."""
    dev = torch.device("cuda:0")
    lens0 = workloads.kpm_lengths(w)
    log(f"workload {w.name}: drawing a {w.B}x{w.T}x{w.H}x{w.d} cache")
    kc = workloads.draw_tokens(w, 1, range(w.n_chunks)).to(dev)
    vc = workloads.draw_tokens(w, 2, range(w.n_chunks)).to(dev)
    q = workloads.random_normal((w.B, w.H, w.d), workloads.seed_for(w, 0, 0), w.torch_dtype).to(dev)
    kn = workloads.random_normal((w.B, w.H, w.d), workloads.seed_for(w, 0, 1), w.torch_dtype).to(dev)
    vn = workloads.random_normal((w.B, w.H, w.d), workloads.seed_for(w, 0, 2), w.torch_dtype).to(dev)
    ln = lens0.to(torch.int32).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    esize = 2 if w.dtype == "bf16" else 4

    def step():
        bosa.attn_kv_append(kn, vn, kc, vc, ln, rope_base=w.rope_base)
        bosa.attn_decode(q, kc, vc, ln, out=out, lse=lse, rope_base=w.rope_base)

    args.warmup = warm_up(step, args.warmup)
    L_start = ln.cpu().to(torch.int64)
    # the s-th timed step sees L_start + s + 1 slots per row
    nbytes = sum(int((L_start + s + 1).sum()) for s in range(args.steps)) * w.H * w.d * 2 * esize
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} decode steps")
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        start.record()
        for _ in range(args.steps):
            step()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        gbs = nbytes / args.steps / (ms * 1e-3) / 1e9
        # the decode kernel alone, timed with events around each launch over K
        # further steps (kept out of the step time above)
        L2 = ln.cpu().to(torch.int64)
        nbytes_k = sum(int((L2 + s + 1).sum()) for s in range(args.steps)) * w.H * w.d * 2 * esize
        with bosa.KernelTimer(max_launches=args.steps + 16) as kt:
            for _ in range(args.steps):
                step()
            torch.cuda.synchronize()
    kms = np.asarray(kt.ms, dtype=np.float64)
    achieved = nbytes_k / (kms.sum() * 1e-3) / 1e9 if kms.sum() > 0 else None
    stats = step_stats(step, args.steps)
    log(f"{ms:.4f} ms/step, {gbs:.0f} GB/s; decode kernel {achieved:.0f} GB/s over {len(kms)} launches "
        f"(avg {kms.mean():.4f} ms)")
    traffic = None
    if os.path.exists(TRAFFIC_FILES["decode"]):
        with open(TRAFFIC_FILES["decode"]) as f:
            tr = json.load(f)
        if tr.get("kernel_sources_sha256") == kernel_sources_sha("decode") and tr.get("workload") == w.name:
            traffic = tr.get("bytes_per_launch")
    cpu = None
    if not args.no_cpu_baseline:
        import threadpoolctl

        import oracle
        info = threadpoolctl.threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        kh = kc.cpu().double().numpy()
        vh = vc.cpu().double().numpy()
        qh = q.cpu().double().numpy()
        lh = ln.cpu().numpy()
        # the whole decoding step (every row and head), repeated until about 10 s of host time
        reps, dt = 0, 0.0
        while dt < 10.0 and reps < 200:
            t0 = time.perf_counter()
            oracle.decode(qh, kh, vh, lh, rope_base=w.rope_base, dtype=w.dtype)
            dt += time.perf_counter() - t0
            reps += 1
        cb = reps * int(lh.sum()) * w.H * w.d * 2 * esize
        cpu = {"value": cb / dt / 1e9, "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": (f"oracle.decode of the whole step ({w.B} rows x {w.H} heads, {int(lh.sum())} visible "
                          f"slots) {reps} times: {cb:.3e} algorithmic bytes in {dt:.2f} s (float64 numpy, BLAS "
                          f"threads={blas_threads}, host cpus={os.cpu_count()})")}
        log(f"cpu baseline {cpu['value']:.3f} GB/s")
    return {
        "metric": METRIC_DECODE, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "step_ms": stats, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "pct_of_peak": 100.0 * gbs / PEAK_HBM_GBS,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "cache_slots": w.T, "d": w.d,
                   "filled_range": w.kpm_len_range, "rope_base": w.rope_base, "pass": "decode",
                   "algorithmic_bytes_per_step": nbytes / args.steps},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS if achieved else None, "traffic": traffic,
                     "kernel": f"decode_chunk_kernel<bf16,{w.d}>", "launches": int(len(kms)),
                     "avg_launch_ms": float(kms.mean()) if len(kms) else None,
                     "bytes_per_launch": nbytes_k / max(len(kms), 1)},
        "cpu_baseline": cpu,
        "clock": clk.summary(),
    }


# ---------------------------------------------------------------- HBM traffic
COPY_KERNEL_HINT = "copy_f32_kernel"   # the library's plain float32 copy (calibration of the byte counters)


def pmc_per_dispatch(csv_path: str, counter: str, which: str):
    """Mean value of `counter` per dispatch of each attention kernel of the
    pass, summed over those kernels (one attention launch), and of the
    calibration copy kernel, from a rocprofv3 --pmc counter_collection.csv."""
    import csv
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        kind = next((kn for kn in TRAFFIC_KERNELS[which] if kn in name), None)
        if kind is None and COPY_KERNEL_HINT in name:
            kind = "copy"
        if kind:
            vals[kind][r["Dispatch_Id"]] += float(r["Counter_Value"])
    means = {k: float(np.mean(list(v.values()))) for k, v in vals.items()}
    means["attn"] = sum(means[kn] for kn in TRAFFIC_KERNELS[which])
    return means


def write_traffic(fetch_csv: str, write_csv: str, copy_mib: int, workload: str, which: str) -> dict:
    """Scale the attention kernels' FETCH_SIZE / WRITE_SIZE (KiB per dispatch)
    by what the same counters read for a copy of known size, and record the
    kernel source hash they were taken with."""
    f = pmc_per_dispatch(fetch_csv, "FETCH_SIZE", which)
    wv = pmc_per_dispatch(write_csv, "WRITE_SIZE", which)
    nbytes = copy_mib * 2 ** 20
    scale_f = nbytes / (f["copy"] * 1024.0)
    scale_w = nbytes / (wv["copy"] * 1024.0)
    out = {
        "workload": workload,
        "pass": which,
        "kernels": list(TRAFFIC_KERNELS[which]),
        "kernel_sources_sha256": kernel_sources_sha(which),
        "fetch_kib_per_dispatch": f["attn"], "write_kib_per_dispatch": wv["attn"],
        "per_kernel_kib": {kn: {"fetch": f[kn], "write": wv[kn]} for kn in TRAFFIC_KERNELS[which]},
        "copy_bytes": nbytes, "copy_fetch_kib": f["copy"], "copy_write_kib": wv["copy"],
        "scale_fetch": scale_f, "scale_write": scale_w,
        "fetch_bytes_per_launch": f["attn"] * 1024.0 * scale_f,
        "write_bytes_per_launch": wv["attn"] * 1024.0 * scale_w,
    }
    out["bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    with open(TRAFFIC_FILES[which], "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 5 and at least %g s of them, which lets the "
                         "shader clock ramp up from idle)" % WARMUP_MIN_S)
    ap.add_argument("--workload", type=int, default=4, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward share (default, the headline metric) or its backward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-targets", action="store_true",
                    help="skip the extra forward workloads (2 and 3) the default run times in child processes")
    ap.add_argument("--no-yardstick", action="store_true",
                    help="skip the sustained matrix-core rate probe the default run starts with")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--cpu-heads", type=int, default=4)
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured into a HIP graph (forward passes; reported as 'graph')")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (byte-counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of a calibrated bench into "
                         "the traffic record bench.py reports, then exit")
    args = ap.parse_args()
    if args.write_traffic:
        w = workloads.WORKLOADS[args.workload]
        print(json.dumps(write_traffic(*args.write_traffic, args.copy_calibration_mib or 1024, w.name,
                                       "decode" if w.decode else args.which)))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the ring on a single GPU (the ring itself is emulated "
              "on that GPU); the library has no multi-GPU path (the ring's transfers are design only). Use --gpus 1.",
              file=sys.stderr)
        return 2
    # the default run also times workloads 2 and 3, in child processes started
    # before this process initialises the GPU
    targets = None
    yardstick = None
    if args.which == "fwd" and args.workload == 4 and not args.no_yardstick:
        yardstick = mfma_yardstick()
    if args.which == "fwd" and args.workload == 4 and not args.no_targets:
        targets = target_lines(args)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    bosa.load()
    w = workloads.WORKLOADS[args.workload]
    if w.decode:
        if args.copy_calibration_mib:
            src = torch.zeros(args.copy_calibration_mib * 2 ** 18, dtype=torch.float32, device="cuda:0")
            bosa.attn_cast(src, torch.empty_like(src))
            torch.cuda.synchronize()
            del src
        print(json.dumps(run_decode(args, w)), flush=True)
        return 0
    log(f"workload {w.name}: drawing inputs")
    plan, host, dev = build_inputs(w)
    bwd = args.which == "bwd"
    if bwd and w.dtype != "bf16":
        print("the backward pass takes bf16 inputs", file=sys.stderr)
        return 2
    dout_host = None
    if bwd:
        step, launches, dout_host = make_bwd_step(w, plan, dev)
    else:
        step, launches = make_step(w, plan, dev)
    pairs = step_pairs(w, plan, host[3])
    # algorithmic FLOPs: forward S = Q K^T and P V, 2 d each per allowed pair;
    # backward dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q (the scores
    # the kernels recompute are not counted)
    flops = (8.0 if bwd else 4.0) * w.d * pairs
    log(f"{pairs} allowed pairs/step = {flops:.4e} FLOPs; {launches} attention sub-calls/step")
    if args.copy_calibration_mib:
        # a plain copy of known size through the library's float32 copy kernel:
        # reads and writes copy_calibration_mib MiB once each
        src = torch.zeros(args.copy_calibration_mib * 2 ** 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        bosa.attn_cast(src, dst)
        torch.cuda.synchronize()
        del src, dst
    args.warmup = warm_up(step, args.warmup)
    per_launch = 2 if bwd else 1
    ms, tflops, achieved, kms, stats, clk = time_steps(step, launches, flops, args.steps, per_launch)
    graph = None
    if args.graph and not bwd:
        graph = graph_pass(step, args.steps, step.outputs)
        if "ms_per_step" in graph:
            graph["value"] = flops / (graph["ms_per_step"] * 1e-3) / 1e12
            log(f"graph replay: {graph['ms_per_step']:.4f} ms/step, {graph['value']:.1f} TFLOP/s")
        else:
            log(f"graph: {graph['error']}")
    kern_ms = float(kms.sum())
    n_launch = len(kms) // per_launch
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    log(f"{ms:.3f} ms/step, {tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of peak); kernel-only "
        f"{achieved:.1f} TFLOP/s over {n_launch} launches (avg {kern_ms / max(n_launch, 1):.4f} ms)")

    traffic = None
    tfile = TRAFFIC_FILES[args.which]
    if w.dtype == "bf16" and os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_sources_sha256") == kernel_sources_sha(args.which) and tr.get("workload") == w.name:
            traffic = tr.get("bytes_per_launch")
    roofline = {
        "bound": "mfma",
        "achieved": achieved,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": (achieved / peak) if achieved else None,
        "traffic": traffic,
        "kernel": (f"bwd_dq_kernel<{w.d}> + bwd_dkdv_kernel<{w.d}>" if bwd else
                   (f"attn_fwd_bf16_chain_kernel<{w.d}>" if plan is not None else f"attn_fwd_bf16_kernel<{w.d}>")
                   if w.dtype == "bf16" else f"attn_fwd_f32_kernel<{w.d}>"),
        "launches": n_launch,
        "avg_launch_ms": kern_ms / max(n_launch, 1),
        "flops_per_launch": flops * args.steps / max(n_launch, 1),
    }
    if bwd and len(kms) >= 2:
        roofline["avg_ms_per_kernel"] = {f"bwd_dq_kernel<{w.d}>": float(kms[0::2].mean()),
                                         f"bwd_dkdv_kernel<{w.d}>": float(kms[1::2].mean())}
    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_rows // 2 if bwd else args.cpu_rows} rows x {args.cpu_heads} heads")
        cpu = cpu_baseline(w, host, args.cpu_rows // 2 if bwd else args.cpu_rows, args.cpu_heads, dout_host)
        log(f"cpu baseline {cpu['value']:.3e} TFLOP/s")
    line = {
        "metric": METRIC_BWD if bwd else METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_ms": stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_peak": 100.0 * tflops / peak,
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "Tq_local": int(dev[0].shape[1]), "d": w.d,
            "causal": w.causal, "rope_base": w.rope_base, "kpm_len_range": w.kpm_len_range,
            "ring_P": w.ring_P, "ring_rank": w.ring_rank, "zigzag": w.zigzag,
            "attention_subcalls_per_step": launches, "attention_launches_per_step": n_launch // args.steps,
            "algorithmic_flops_per_step": flops,
            "pass": args.which,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "clock": clk.summary(),
    }
    if graph is not None:
        line["graph"] = graph
    if targets is not None:
        line["targets"] = targets
    if yardstick is not None:
        rate = yardstick.get("normal_operands_tflops")
        if rate and achieved:
            yardstick["kernel_frac_of_normal_operand_rate"] = achieved / rate
        line["mfma_sustained"] = yardstick
    clock = line["clock"]
    if clock and w.dtype == "bf16":
        # the same MFMA rate per clock at the clock the work ran at
        clock["bf16_peak_at_mean_sclk_tflops"] = peak * clock["sclk_mhz"]["mean"] / 2400.0
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
