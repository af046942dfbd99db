"""The scratch a call needs (rotated copies of q and k, tables, live-tile
lists) comes from a buffer the library keeps per (device, stream) and reuses,
so a call only enqueues work and returns: freeing device memory after every
call waited for the stream's pending work, which made each call synchronous
with the one before it.  These tests check that calls run ahead of the GPU,
that two streams with their own buffers give the same bits as one stream,
that a graph captured with the library's calls replays correctly between
eager calls, that releasing the buffers leaves later calls correct, and that
calls on the per-thread default stream, which keep no buffer, are correct.
"""
import time

import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import workloads
from gpu_helpers import DEV, note

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _qkv(T, H, seed, d=128):
    return tuple(workloads.random_normal((1, T, H, d), seed + i, BF).to(DEV) for i in range(3))


def _same(a, b):
    return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_calls_return_before_the_gpu_finishes():
    """Five back-to-back calls of a causal forward with RoPE (16384 rows, 32
    heads, about 2 ms of GPU work each, scratch for the rotated copies) are
    enqueued in less than half the GPU time they take."""
    q, k, v = _qkv(16384, 32, 7100)
    bosa.attn_fwd(q, k, v, causal=True, rope_base=10000.0)   # the stream's buffer exists from here on
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    t0 = time.perf_counter()
    for _ in range(5):
        bosa.attn_fwd(q, k, v, causal=True, rope_base=10000.0)
    host_ms = (time.perf_counter() - t0) * 1e3
    end.record()
    torch.cuda.synchronize()
    gpu_ms = start.elapsed_time(end)
    note(f"five calls: enqueued in {host_ms:.2f} ms, GPU {gpu_ms:.2f} ms")
    assert host_ms < 0.5 * gpu_ms, f"calls waited for the GPU: host {host_ms:.2f} ms, GPU {gpu_ms:.2f} ms"


def test_two_streams_with_their_own_buffers():
    """Calls alternating between two streams (each with its own kept buffer,
    running concurrently) give the bits of the same calls made one at a time
    on the default stream; the second input is larger, so its stream's
    buffer is replaced while the other stream's work is in flight."""
    a = _qkv(3000, 4, 7200)
    b = _qkv(5000, 4, 7300)
    ref_a = bosa.attn_fwd(*a, causal=True, rope_base=10000.0)
    ref_b = bosa.attn_fwd(*b, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    res = []
    for i in range(4):
        ra = bosa.attn_fwd(*a, causal=True, rope_base=10000.0, stream=s1)
        rb = bosa.attn_fwd(*(b if i >= 1 else a), causal=True, rope_base=10000.0, stream=s2)
        res.append((ra, rb, i))
    torch.cuda.synchronize()
    for ra, rb, i in res:
        assert _same(ra, ref_a), f"stream 1, call {i}"
        assert _same(rb, ref_b if i >= 1 else ref_a), f"stream 2, call {i}"


def test_graph_replays_between_eager_calls():
    """A forward with RoPE captured into a graph (its scratch becomes the
    graph's own allocation) replays with the eager result's bits three times,
    with eager calls of a larger input in between (which grow the default
    stream's kept buffer)."""
    a = _qkv(2048, 8, 7400)
    big = _qkv(6000, 8, 7500)
    ref = bosa.attn_fwd(*a, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    out = torch.empty_like(ref[0])
    lse = torch.empty_like(ref[1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bosa.attn_fwd(*a, out=out, lse=lse, causal=True, rope_base=10000.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bosa.attn_fwd(*a, out=out, lse=lse, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        lse.zero_()
        bosa.attn_fwd(*big, causal=True, rope_base=10000.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same((out, lse), ref), f"replay {r}"


def test_release_then_call_again():
    """attn_release_scratch frees the kept buffers; the next calls allocate
    again and give the same bits."""
    a = _qkv(1000, 4, 7600)
    ref = bosa.attn_fwd(*a, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    bosa.release_scratch()
    bosa.release_scratch()   # nothing kept: still fine
    again = bosa.attn_fwd(*a, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    assert _same(again, ref)


def test_two_host_threads_on_one_stream():
    """Two host threads calling on the same stream at once (ctypes releases
    the interpreter lock during a call, so the library's host code runs
    concurrently): each call holds the stream's buffer while it enqueues, so
    its kernels never share the scratch with the other thread's, and every
    result has the bits of the same call made alone."""
    import threading
    a = _qkv(2500, 4, 7700)
    b = _qkv(4000, 4, 7800)
    ref_a = bosa.attn_fwd(*a, causal=True, rope_base=10000.0)
    ref_b = bosa.attn_fwd(*b, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    results = {0: [], 1: []}
    errors = []

    def worker(idx, x):
        try:
            for _ in range(12):
                results[idx].append(bosa.attn_fwd(*x, causal=True, rope_base=10000.0, stream=stream))
        except Exception as e:   # surfaced below
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(0, a)), threading.Thread(target=worker, args=(1, b))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for r in results[0]:
        assert _same(r, ref_a)
    for r in results[1]:
        assert _same(r, ref_b)


class _PerThreadStream:
    cuda_stream = 2   # hipStreamPerThread: a different stream in every host thread


def test_per_thread_default_stream():
    """Calls on the per-thread default stream allocate and free their scratch
    per call, since a buffer kept for that one handle could pass from a host
    thread that ended with work queued to the next thread that reuses its id.
    Three threads in turn, each making three calls and ending without waiting
    for them, give the bits of the same call on torch's stream."""
    import threading
    a = _qkv(2500, 4, 7900)
    ref = bosa.attn_fwd(*a, causal=True, rope_base=10000.0)
    torch.cuda.synchronize()
    results, errors = [], []

    def worker():
        try:
            for _ in range(3):
                results.append(bosa.attn_fwd(*a, causal=True, rope_base=10000.0, stream=_PerThreadStream))
        except Exception as e:   # surfaced below
            errors.append(e)

    for _ in range(3):
        t = threading.Thread(target=worker)
        t.start()
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    assert len(results) == 9
    for i, r in enumerate(results):
        assert _same(r, ref), f"call {i}"
