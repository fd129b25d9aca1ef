"""Benchmark of the fused HATA decode step on one MI355X.

Workload: one decode step of a Llama-3.1-8B-shaped attention layer at 128K
context -- batch 1, 32 query heads over 8 KV heads (GQA 4), head dim 128,
N = 131072 cached tokens, 128-bit codes, budget k = 512 -- on seeded
synthetic inputs (bf16 q/K/V ~ N(0,1) with 4 outlier key channels x8 per KV
head, W_H ~ N(0, 1/128) per KV head).

A step is one hata_decode_step call: encode the 32 new queries, encode and
append the 8 new keys, Hamming + GQA sum over the 8 x 131072 cached codes,
top-512 per KV head, gather + exact attention.  The caches of `--layers`
distinct layers live in HBM and consecutive steps walk through them, as a
model's layers would, so no step finds its working set in the 256 MB
Infinity Cache.  The K timed steps are captured in one HIP graph and timed
with HIP events on the stream they run on.

Printed: one JSON line (steps/s, the roofline object of the fused kernel,
the oracle's CPU baseline, the dense flash-decode baseline on the same
caches and the prefill bulk encode).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(B: int, Hq: int, Hkv: int, N: int, k: int, d: int = 128, r: int = 128) -> int:
    """Algorithmic HBM bytes of one step: per unit N*r/8 code bytes plus
    2*k*d*2 gathered K/V bytes, plus q (bf16) and out (fp32)."""
    units = B * Hkv
    return units * (N * r // 8 + 2 * min(k, N) * d * 2) + B * Hq * d * 2 + B * Hq * d * 4


def dense_bytes(B: int, Hq: int, Hkv: int, N: int, d: int = 128) -> int:
    return B * Hkv * 2 * N * d * 2 + B * Hq * d * 2 + B * Hq * d * 4


def bulk_bytes(B: int, Hkv: int, N: int, d: int = 128, r: int = 128) -> int:
    return B * Hkv * N * (d * 2 + r // 8) + Hkv * d * r * 4


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_step_128k_hbm_traffic.md")
KERNEL_SOURCES = ("hash_top_sparse_amd/csrc/decode_step.hip", "hash_top_sparse_amd/csrc/hata_device.hpp")


def profiled_traffic():
    """HBM bytes per fused-step launch from the committed counter summary,
    or None when the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        txt = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in txt.splitlines() if ": " in line and line[:1].isalpha())
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("kernel_source_sha256_16", "").strip() != h.hexdigest()[:16]:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, budget_s: float) -> dict:
    """Time the oracle's whole decode step on the host (OpenMP over units)."""
    import oracle

    oracle.build()
    B, Hq, d = inp.q.shape
    _, Hkv, cap, _ = inp.K.shape
    threads = oracle.max_threads()
    log(f"oracle: building the code cache on {threads} host threads (not timed)")
    codes = np.zeros((B, Hkv, cap, 2), np.uint64)
    jobs = [(b, h) for b in range(B) for h in range(Hkv)]

    def enc(bh):
        b, h = bh
        n = int(inp.seq_lens[b])
        codes[b, h, :n - 1] = oracle.encode(inp.K[b, h, :n - 1], inp.W[h])

    with cf.ThreadPoolExecutor(max_workers=max(1, min(threads, len(jobs)))) as ex:
        list(ex.map(enc, jobs))
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.decode_step(inp.q, inp.K, inp.V, inp.W, codes, inp.seq_lens, inp.k, inp.scale,
                           nthreads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 50:
            break
    med = float(np.median(times))
    # the same step on one host thread (two runs), and the oracle's encode of
    # 16384 cached keys of one KV head (the prefill bulk encode's work per row)
    t1 = []
    for _ in range(2):
        t0 = time.perf_counter()
        oracle.decode_step(inp.q, inp.K, inp.V, inp.W, codes, inp.seq_lens, inp.k, inp.scale,
                           nthreads=1)
        t1.append(time.perf_counter() - t0)
    rows = min(16384, cap)
    t0 = time.perf_counter()
    oracle.encode(inp.K[0, 0, :rows], inp.W[0])
    enc_s = time.perf_counter() - t0
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": 1.0 / med, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"the whole step of this workload (all {B * Hkv} units, N={cap}, k={inp.k}); "
                       f"median of {len(times)} runs, {med * 1e3:.1f} ms each; code cache prebuilt "
                       f"by the oracle outside the timing"),
            "single_thread_steps_per_s": 1.0 / float(np.median(t1)),
            "encode_keys_per_s_one_thread": rows / enc_s,
            "cpu_model": cpu_model}


# Device-side delay put ahead of the start event of a timed graph replay
# (torch's spin kernel, about 1 ms): the host has finished submitting the
# graph's launches when the start event is reached, so the time the host
# takes to submit them is not counted as time of the kernels.
GRAPH_LEAD_CYCLES = 2_000_000


def replay_ms(g, n: int) -> float:
    """Milliseconds per launch of one replay of graph `g` holding `n`
    launches, by HIP events on the replay stream."""
    import torch

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(GRAPH_LEAD_CYCLES)
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n


def read_peak(gib: int = 4, reps: int = 5) -> float:
    """HBM read rate (GB/s) of the library's streaming-read kernel over a
    `gib` GiB buffer: best of `reps` passes, HIP events on the launch stream."""
    import torch

    from hash_top_sparse_amd import binding

    src = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    src.fill_(7)
    sink = torch.zeros(1024, dtype=torch.int64, device="cuda")
    binding.stream_read(src, sink)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(reps):
        ev0.record()
        binding.stream_read(src, sink)
        ev1.record()
        torch.cuda.synchronize()
        best = max(best, src.numel() / (ev0.elapsed_time(ev1) * 1e-3) / 1e9)
    del src
    torch.cuda.empty_cache()
    return best


def code_stream_alone(layer_bufs, L: int, n: int) -> dict | None:
    """The code cache read on its own: the library's plain streaming kernel
    (one workgroup of 256 threads per CU, 16 loads of 16 bytes in flight per
    thread, as many workgroups as the fused step launches at 128K) over each
    layer's code cache in the same rotation as the step, timed as a captured
    graph of n launches; and the same kernel over only the first 16 bytes per
    thread of each cache (one load per thread), which times the launch and
    the first access.  A bound for the step's scan phase, which cannot end
    before its code rows have arrived."""
    import torch

    from hash_top_sparse_amd import binding

    if n <= 0:
        return None
    sink = torch.zeros(1024, dtype=torch.int64, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    first = min(cus, 1024) * 256 * 16
    out = {}
    for name, nbytes in (("whole", None), ("one_load_per_thread", first)):
        views = []
        for i in range(L):
            c = layer_bufs[i][2].view(-1).view(torch.uint8)
            views.append(c if nbytes is None else c[: min(nbytes, c.numel())])
        for i in range(4):
            binding.stream_read(views[i % L], sink)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                binding.stream_read(views[i % L], sink)
        g.replay()
        torch.cuda.synchronize()
        ms = replay_ms(g, n)
        out[name] = {"ms_per_launch": ms, "bytes": int(views[0].numel()),
                     "GBs": views[0].numel() / (ms * 1e-3) / 1e9}
        del g
    log(f"code cache read alone: {out['whole']['ms_per_launch'] * 1e3:.2f} us "
        f"({out['whole']['bytes'] / 1e6:.1f} MB); one load per thread: "
        f"{out['one_load_per_thread']['ms_per_launch'] * 1e3:.2f} us")
    out["timing"] = "graph of the launches, HIP events"
    return out


def measure(cfg_id: int, steps: int, warmup: int, dense_steps: int, layers: int, use_graph: bool,
            with_bulk: bool, with_qk: bool = True, r: int = 128, read_rate: float | None = None):
    """Time the fused step (and the dense baseline) on one workload; returns
    (result dict, inputs)."""
    import torch

    from hash_top_sparse_amd import binding, synth

    import dataclasses

    dev = torch.device("cuda:0")
    shape = synth.CONFIGS[cfg_id]
    if r != shape.r:
        shape = dataclasses.replace(shape, r=r, name=f"{shape.name}-r{r}")
    B, Hq, Hkv, N, k = shape.B, shape.Hq, shape.Hkv, shape.N, shape.k
    per_step = step_bytes(B, Hq, Hkv, N, k, r=r)
    L = layers or max(2, min(64, int(np.ceil(1.5e9 / per_step))))
    log(f"workload {shape.name}: B={B} Hq={Hq} Hkv={Hkv} N={N} k={k}; {L} layer caches")
    t0 = time.perf_counter()
    inp = synth.make_inputs(shape)
    log(f"inputs drawn in {time.perf_counter() - t0:.1f} s")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    q0, K0, V0 = bf(inp.q), bf(inp.K), bf(inp.V)
    W = torch.from_numpy(inp.W).to(dev)
    seq = torch.from_numpy(inp.seq_lens).to(dev)
    codes0 = binding.new_codes(B, Hkv, N, r=r, device=dev)
    binding.encode_append(K0, W, codes0, n_new=N)
    torch.cuda.synchronize()
    layer_bufs = []
    for l in range(L):
        layer_bufs.append((K0.clone() if l else K0, V0.clone() if l else V0,
                           codes0.clone() if l else codes0))
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    bulk = None
    if with_bulk:
        nb = min(L, 16)
        scratch = [torch.empty_like(codes0) for _ in range(2)]
        for i in range(4):
            binding.encode_append(layer_bufs[i % L][0], W, scratch[i % 2], n_new=N)
        ev0.record()
        for i in range(nb):
            binding.encode_append(layer_bufs[i][0], W, scratch[i % 2], n_new=N)
        ev1.record()
        torch.cuda.synchronize()
        bulk_ms = ev0.elapsed_time(ev1) / nb
        bulk = {"ms": bulk_ms, "keys_per_s": B * Hkv * N / (bulk_ms * 1e-3),
                "GBs": bulk_bytes(B, Hkv, N) / (bulk_ms * 1e-3) / 1e9,
                "TFLOPs": 2.0 * B * Hkv * N * 128 * 128 / (bulk_ms * 1e-3) / 1e12}
        del scratch
        log(f"bulk encode: {bulk_ms * 1e3:.1f} us per layer")

    ws = binding.alloc_workspace(binding.OP_DECODE_STEP, B, Hq, Hkv, N, k, device=dev, r=r)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device=dev)

    def step(i):
        Kl, Vl, cl = layer_bufs[i % L]
        binding.decode_step(q0, Kl, Vl, W, cl, seq, N, k, inp.scale, out, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if not use_graph:
        ev0.record()
        for i in range(steps):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        ms_step = ev0.elapsed_time(ev1) / steps
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ms_step = replay_ms(g, steps)
    # spread of single eagerly launched steps (launch gap included), events
    # around each step on the launch stream
    nsp = min(200, steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsp + 1)]
    evs[0].record()
    for i in range(nsp):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(nsp)])
    spread = {"steps": nsp, "median_us": float(np.median(per)), "p10_us": float(np.percentile(per, 10)),
              "p90_us": float(np.percentile(per, 90))}
    # the same step with a separate key encoder (an equal-valued copy of W_H
    # at another address, so the separate-encoder kernel instance runs)
    Wk = W.clone()
    qk = None

    def step_qk(i):
        Kl, Vl, cl = layer_bufs[i % L]
        binding.decode_step_qk(q0, Kl, Vl, W, Wk, cl, seq, N, k, inp.scale, out, ws)

    if with_qk and use_graph:
        nqk = min(steps, 1024)
        for i in range(8):
            step_qk(i)
        torch.cuda.synchronize()
        gq = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gq):
            for i in range(nqk):
                step_qk(i)
        gq.replay()
        torch.cuda.synchronize()
        qk_ms = replay_ms(gq, nqk)
        del gq
        qk = {"ms_per_step": qk_ms, "steps_per_s": 1000.0 / qk_ms}
        log(f"fused step, separate key encoder: {qk_ms * 1e3:.2f} us/step")
    err = binding.workspace_check(ws)
    if err:
        raise RuntimeError(f"workspace error word {err}: a cross-workgroup wait timed out")
    stream = code_stream_alone(layer_bufs, L, min(steps, 1024) if use_graph else 0) if use_graph else None
    achieved = per_step / (ms_step * 1e-3) / 1e9
    log(f"fused step: {ms_step * 1e3:.2f} us/step, {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBS:.1%})")

    dense = None
    if dense_steps > 0:
        dws = binding.alloc_workspace(binding.OP_DENSE_DECODE, B, Hq, Hkv, N, 1, device=dev)
        dout = torch.zeros_like(out)

        def dstep(i):
            Kl, Vl, _ = layer_bufs[i % L]
            binding.dense_decode(q0, Kl, Vl, seq, N, inp.scale, dout, dws)

        for i in range(4):
            dstep(i)
        torch.cuda.synchronize()
        # timed like the fused step: a captured graph of the steps (eagerly
        # when the fused step is timed eagerly)
        if use_graph:
            gd = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gd):
                for i in range(dense_steps):
                    dstep(i)
            gd.replay()
            torch.cuda.synchronize()
        if use_graph:
            d_ms = replay_ms(gd, dense_steps)
        else:
            ev0.record()
            for i in range(dense_steps):
                dstep(i)
            ev1.record()
            torch.cuda.synchronize()
            d_ms = ev0.elapsed_time(ev1) / dense_steps
        dgb = dense_bytes(B, Hq, Hkv, N) / (d_ms * 1e-3) / 1e9
        dense = {"ms_per_step": d_ms, "GBs": dgb, "frac_of_peak": dgb / PEAK_HBM_GBS,
                 "speedup_of_hata": d_ms / ms_step,
                 "timing": "graph of the steps, HIP events" if use_graph else "eager, HIP events"}
        if read_rate:
            # a dense pass that moved its bytes at the measured read rate
            floor_ms = dense_bytes(B, Hq, Hkv, N) / (read_rate * 1e9) * 1e3
            dense["floor_ms_at_measured_read_rate"] = floor_ms
            dense["speedup_of_hata_vs_floor"] = floor_ms / ms_step
            dense["frac_of_measured_read_rate"] = dgb / read_rate
        log(f"dense: {d_ms * 1e3:.1f} us/step, {dgb:.0f} GB/s, hata speedup {d_ms / ms_step:.2f}x")
    res = {"workload": shape.name, "code_bits": r, "ms_per_step": ms_step, "steps_per_s": 1000.0 / ms_step,
           "tokens_per_s": B * 1000.0 / ms_step,
           "GBs": achieved, "frac_of_peak": achieved / PEAK_HBM_GBS, "bytes_per_step": per_step,
           "layers": L, "eager_step_spread": spread, "separate_key_encoder": qk, "dense": dense,
           "bulk_encode": bulk, "code_stream_alone": stream}
    del layer_bufs
    torch.cuda.empty_cache()
    return res, inp


def model_sweep(layers: int = 32, ctxs=(32768, 65536, 131072), reps: int = 10) -> list:
    """Multi-layer decode: for each context length, `layers` layers of a
    Llama-3.1-8B-shaped attention (B=1, 32 query / 8 KV heads, d=128, k=512),
    each with its own q, K, V, W_H and code cache, decoded one token as one
    captured graph of `layers` fused steps, against a graph of `layers` dense
    flash-decodes over the same caches.  Attention only (no projections or
    MLP): the shape of a whole-model decode speed table, not its values."""
    import torch

    from hash_top_sparse_amd import binding

    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, k = 1, 32, 8, 128, 512
    scale = 1.0 / np.sqrt(d)
    gen = torch.Generator(device=dev)
    res = []
    for N in ctxs:
        gen.manual_seed(6000 + N // 1024)
        bf = lambda *shp: torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
        qs = [bf(B, Hq, d) for _ in range(layers)]
        Ks = [bf(B, Hkv, N, d) for _ in range(layers)]
        Vs = [bf(B, Hkv, N, d) for _ in range(layers)]
        Ws = [torch.randn((Hkv, d, 128), generator=gen, device=dev) / np.sqrt(128.0) for _ in range(layers)]
        codes = [torch.zeros((B, Hkv, N, 2), dtype=torch.int64, device=dev) for _ in range(layers)]
        for l in range(layers):
            binding.encode_append(Ks[l], Ws[l], codes[l], n_new=N)
        seq = torch.full((B,), N, dtype=torch.int32, device=dev)
        outs = [torch.zeros((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(layers)]
        ws = binding.alloc_workspace(binding.OP_DECODE_STEP, B, Hq, Hkv, N, k, device=dev)
        dws = binding.alloc_workspace(binding.OP_DENSE_DECODE, B, Hq, Hkv, N, 1, device=dev)
        torch.cuda.synchronize()

        def timed(one_layer):
            for l in range(layers):  # warm-up, eager
                one_layer(l)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for l in range(layers):
                    one_layer(l)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        h_ms = timed(lambda l: binding.decode_step(qs[l], Ks[l], Vs[l], Ws[l], codes[l], seq, N, k, scale,
                                                   outs[l], ws))
        err = binding.workspace_check(ws)
        if err:
            raise RuntimeError(f"workspace error word {err}: a cross-workgroup wait timed out")
        d_ms = timed(lambda l: binding.dense_decode(qs[l], Ks[l], Vs[l], seq, N, scale, outs[l], dws))
        r = {"ctx": N, "layers": layers, "hata_ms_per_token": h_ms, "dense_ms_per_token": d_ms,
             "speedup": d_ms / h_ms, "hata_tokens_per_s": 1000.0 / h_ms,
             "hata_GBs": layers * step_bytes(B, Hq, Hkv, N, k) / (h_ms * 1e-3) / 1e9}
        log(f"model sweep {N // 1024}K x {layers} layers: hata {h_ms * 1e3:.1f} us/token, dense "
            f"{d_ms * 1e3:.1f} us/token, speedup {d_ms / h_ms:.2f}x")
        res.append(r)
        del qs, Ks, Vs, Ws, codes, outs, ws, dws
        torch.cuda.empty_cache()
    return res


def prefill_bench(N: int = 32768, B: int = 1, Hq: int = 32, Hkv: int = 8, r: int = 128, reps: int = 5,
                  paged: bool = True) -> dict:
    """Time hata_prefill on one Llama-3.1-8B-shaped layer (bf16 N(0,1) q/K/V
    and fp32 N(0, 1/128) W_H drawn on the device; parity is in the tests):
    causal attention over an N-token prompt with the prompt keys' codes
    written to the cache.  Algorithmic work: 4 d per visible (query, key)
    pair and query head (the two products), i.e. 2 d Hq N (N + 1) flops, plus
    the encode.  Beside it, the separate bulk encode of the same keys
    (hata_encode_append), the pass that the fused encode replaces, and (paged)
    hata_prefill_paged on the same data in pools of 256-row pages."""
    import torch

    from hash_top_sparse_amd import binding

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7300)
    q = torch.randn((B, Hq, N, 128), generator=g, device=dev).to(torch.bfloat16)
    K = torch.randn((B, Hkv, N, 128), generator=g, device=dev).to(torch.bfloat16)
    V = torch.randn((B, Hkv, N, 128), generator=g, device=dev).to(torch.bfloat16)
    W = torch.randn((Hkv, 128, r), generator=g, device=dev) / np.sqrt(128.0)
    out = torch.empty((B, Hq, N, 128), dtype=torch.float32, device=dev)
    codes = binding.new_codes(B, Hkv, N, r=r, device=dev)
    seq = torch.full((B,), N, dtype=torch.int32, device=dev)
    scale = 1.0 / np.sqrt(128.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    binding.prefill(q, K, V, W, codes, seq, N, scale, out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        binding.prefill(q, K, V, W, codes, seq, N, scale, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    binding.encode_append(K, W, codes, n_new=N)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        binding.encode_append(K, W, codes, n_new=N)
    e1.record()
    torch.cuda.synchronize()
    enc_ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * 128 * Hq * B * N * (N + 1)
    enc_flops = 2.0 * 128 * r * B * Hkv * N
    tf = (flops + enc_flops) / (ms * 1e-3) / 1e12
    log(f"prefill {N} tokens x {Hq}/{Hkv} heads: {ms:.2f} ms ({tf:.0f} TFLOP/s, {tf / 2500:.1%} of bf16 peak); "
        f"separate bulk encode of the keys {enc_ms * 1e3:.0f} us")
    # the same prompt into K/V/code pools of 256-row pages in shuffled order
    paged_ms = None
    if paged:
        P = 256
        mp = (N + P - 1) // P
        num_pages = B * mp
        bt = torch.randperm(num_pages, generator=g, device=dev).to(torch.int32).view(B, mp)
        idx = bt.reshape(-1).long()

        def pool(x):
            c = x.shape[-1]
            xp = torch.zeros((B, Hkv, mp * P, c), dtype=x.dtype, device=dev)
            xp[:, :, :N] = x
            pl = torch.empty((num_pages, Hkv, P, c), dtype=x.dtype, device=dev)
            pl[idx] = xp.view(B, Hkv, mp, P, c).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, c)
            return pl

        Kp, Vp, Cp = pool(K), pool(V), pool(codes)
        binding.prefill_paged(q, Kp, Vp, W, Cp, bt, seq, N, scale, out)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            binding.prefill_paged(q, Kp, Vp, W, Cp, bt, seq, N, scale, out)
        e1.record()
        torch.cuda.synchronize()
        paged_ms = e0.elapsed_time(e1) / reps
        log(f"paged prefill ({P}-row pages in shuffled order): {paged_ms:.2f} ms")
        del Kp, Vp, Cp
    del q, K, V, out
    torch.cuda.empty_cache()
    return {"workload": f"Llama-3.1-8B-shaped layer prefill, B={B}, {Hq}/{Hkv} heads, d=128, r={r}",
            "tokens": B * N, "ms": ms, "tokens_per_s": B * N / (ms * 1e-3),
            "flops": flops + enc_flops, "TFLOPs": tf, "peak_TFLOPs": 2500.0, "frac_of_peak": tf / 2500.0,
            "encode_flops_share": enc_flops / (flops + enc_flops),
            "separate_bulk_encode_ms": enc_ms, "paged_256_row_pages_ms": paged_ms}


def paged_bench(config: int = 4, pages=(16, 256), steps: int = 200) -> dict:
    """Time hata_decode_step_paged on the workload's shape with K/V/code
    pools of fixed-size pages in shuffled order, against hata_decode_step on
    the same data laid out contiguously (bf16 N(0,1) K/V, random codes,
    fp32 N(0, 1/128) W_H drawn on the device; one layer, no cache rotation;
    parity is in the tests).  Eager launches timed with HIP events."""
    import torch

    from hash_top_sparse_amd import binding, synth

    shape = synth.CONFIGS[config]
    B, Hq, Hkv, N, k = shape.B, shape.Hq, shape.Hkv, shape.N, shape.k
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7400)
    q = torch.randn((B, Hq, 128), generator=g, device=dev).to(torch.bfloat16)
    W = torch.randn((Hkv, 128, 128), generator=g, device=dev) / np.sqrt(128.0)
    seq = torch.full((B,), N, dtype=torch.int32, device=dev)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device=dev)
    K = torch.randn((B, Hkv, N, 128), generator=g, device=dev).to(torch.bfloat16)
    V = torch.randn((B, Hkv, N, 128), generator=g, device=dev).to(torch.bfloat16)
    C = torch.randint(-(1 << 62), 1 << 62, (B, Hkv, N, 2), generator=g, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(step):
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    cws = binding.alloc_workspace(binding.OP_DECODE_STEP, B, Hq, Hkv, N, k)
    cms = timed(lambda: binding.decode_step(q, K, V, W, C, seq, N, k, 1.0 / np.sqrt(128.0), out, cws))
    res = {"workload": shape.name, "contiguous_ms_per_step": cms}
    log(f"contiguous step on the same data ({shape.name}): {cms * 1e3:.1f} us/step")
    for P in pages:
        mp = (N + P - 1) // P
        num_pages = B * mp
        bt = torch.randperm(num_pages, generator=g, device=dev).to(torch.int32).view(B, mp)
        idx = bt.reshape(-1).long()

        def pool(x):
            c = x.shape[-1]
            xp = torch.zeros((B, Hkv, mp * P, c), dtype=x.dtype, device=dev)
            xp[:, :, :N] = x
            p = torch.empty((num_pages, Hkv, P, c), dtype=x.dtype, device=dev)
            p[idx] = xp.view(B, Hkv, mp, P, c).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, c)
            return p

        Kp, Vp, Cp = pool(K), pool(V), pool(C)
        ws = binding.alloc_workspace(binding.OP_DECODE_STEP_PAGED, B, Hq, Hkv, N, k)
        ms = timed(lambda: binding.decode_step_paged(q, Kp, Vp, W, Cp, bt, seq, N, k, 1.0 / np.sqrt(128.0),
                                                     out, ws))
        res[f"page_rows_{P}"] = {"ms_per_step": ms, "steps_per_s": 1000.0 / ms}
        log(f"paged step ({shape.name}, {P}-row pages): {ms * 1e3:.1f} us/step")
        del Kp, Vp, Cp
        torch.cuda.empty_cache()
    return res


def train_bench(J: int = 512, n: int = 8192, r: int = 128, steps: int = 20) -> dict:
    """Time the hash-weight training step for one head (synthetic bf16 N(0,1)
    Q/K drawn on the device, J sampled queries at random positions of an
    n-key sequence): the label kernel and one gradient step, HIP events over
    `steps` eager calls each, and the step again as a captured graph of
    `steps` steps.  FLOP count of the step: the two projections, the two
    J x n x r label-weighted pair products, the two gradient products and
    the W^T W terms (the causal-mask sums, O((n + J) r) adds, are not
    counted)."""
    import torch

    from hash_top_sparse_amd import binding

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7100)
    q = torch.randn((J, 128), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((n, 128), generator=g, device=dev).to(torch.bfloat16)
    pos = torch.sort(torch.randperm(n, generator=torch.Generator().manual_seed(7101))[:J]).values
    pos = pos.to(torch.int32).to(dev)
    W = torch.randn((128, r), generator=g, device=dev) / np.sqrt(128.0)
    S = torch.zeros((J, n), dtype=torch.float32, device=dev)
    loss = torch.zeros(4, dtype=torch.float32, device=dev)
    ws = binding.hash_train_workspace(J, n, r)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    binding.hash_labels(q, k, pos, S)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        binding.hash_labels(q, k, pos, S)
    e1.record()
    torch.cuda.synchronize()
    lab_ms = e0.elapsed_time(e1) / steps
    binding.hash_train_step(q, k, pos, S, W, 1.0, 1e-3, 1e-4, 0.1, 1e-3, loss, ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        binding.hash_train_step(q, k, pos, S, W, 1.0, 1e-3, 1e-4, 0.1, 1e-3, loss, ws)
    e1.record()
    torch.cuda.synchronize()
    st_eager_ms = e0.elapsed_time(e1) / steps
    # the same steps from a captured graph, like the decode step (each replay
    # continues the training: every step updates W in place)
    gtr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gtr):
        for _ in range(steps):
            binding.hash_train_step(q, k, pos, S, W, 1.0, 1e-3, 1e-4, 0.1, 1e-3, loss, ws)
    gtr.replay()
    torch.cuda.synchronize()
    st_ms = replay_ms(gtr, steps)
    del gtr
    flops = 4.0 * J * n * r + 4.0 * (J + n) * 128 * r + 4.0 * 128 * r * r
    tf = flops / (st_ms * 1e-3) / 1e12
    log(f"hash training, J={J} n={n} r={r}: labels {lab_ms * 1e3:.1f} us, step {st_ms * 1e3:.1f} us "
        f"from a graph, {st_eager_ms * 1e3:.1f} us eager ({tf:.2f} TFLOP/s fp32)")
    return {"J": J, "n": n, "r": r, "labels_ms": lab_ms, "step_ms": st_ms, "step_ms_eager": st_eager_ms,
            "timing": "graph of the steps, HIP events (step_ms); eager launches (step_ms_eager)",
            "step_flops": flops, "step_TFLOPs": tf, "frac_of_fp32_peak": tf / 157.3,
            "loss_after": loss.cpu().tolist()}


TRACE_POINTS = ("start", "qcodes", "scanned", "hist", "published", "wait1", "windows", "threshold",
                "compacted", "attended", "record", "wait2", "end", "qrows", "search_loop", "round1", "search", "gathered", "accumulated")
# the boundaries in the order a workgroup passes them (indices into TRACE_POINTS)
TRACE_ORDER = (0, 13, 1, 2, 3, 4, 5, 6, 14, 15, 16, 7, 8, 17, 18, 9, 10, 11, 12)
TRACE_SLOTS = 24  # timestamps stored per workgroup


def phase_trace(cfg_id: int = 4, steps: int = 200, layers: int = 0, r: int = 128) -> dict:
    """Per-phase timeline of the fused step, from the phase-trace build of the
    library (libhata_trace.so: thread 0 of every workgroup reads the 100 MHz
    real-time counter at each phase boundary and stores the readings in the
    workspace, past the plain build's layout).  Eager steps over rotated
    layer caches as in the headline measurement; after each step the trace
    area is copied aside on the stream.  Reported per phase boundary: the
    median over steps of the median and of the latest workgroup's time since
    the step's first workgroup started, and the median time each workgroup
    spends in each phase."""
    import torch

    from hash_top_sparse_amd import binding, synth

    import dataclasses

    binding.load(binding.TRACE_LIB_PATH)
    dev = torch.device("cuda:0")
    shape = synth.CONFIGS[cfg_id]
    if r != shape.r:
        shape = dataclasses.replace(shape, r=r, name=f"{shape.name}-r{r}")
    B, Hq, Hkv, N, k = shape.B, shape.Hq, shape.Hkv, shape.N, shape.k
    U = B * Hkv
    L = layers or max(2, min(64, int(np.ceil(1.5e9 / step_bytes(B, Hq, Hkv, N, k)))))
    inp = synth.make_inputs(shape)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    q0, K0, V0 = bf(inp.q), bf(inp.K), bf(inp.V)
    W = torch.from_numpy(inp.W).to(dev)
    seq = torch.from_numpy(inp.seq_lens).to(dev)
    codes0 = binding.new_codes(B, Hkv, N, r=r, device=dev)
    binding.encode_append(K0, W, codes0, n_new=N)
    bufs = [(K0.clone() if l else K0, V0.clone() if l else V0, codes0.clone() if l else codes0)
            for l in range(L)]
    ws = binding.alloc_workspace(binding.OP_DECODE_STEP, B, Hq, Hkv, N, k, device=dev, r=r)
    # workgroups per unit as the library plans them for these sizes (a
    # fused step within the LDS limit); the trace area is the workspace's
    # last ceil(U * Wg * 8 * TRACE_SLOTS / 256) * 256 bytes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Wg = max(1, min(cus // U, 64, -(-N // 256)))
    if Hq // Hkv <= 4 and r <= 128 and Wg > 1:  # two workgroups per compute unit when that gives more of them
        Wg2 = min(2 * cus // U, 32, -(-N // 256))
        if Wg2 > Wg and -(-N // Wg2) <= 32768 and U * Wg2 <= 2 * cus:
            Wg = Wg2
    assert -(-N // Wg) <= 32768, "the phase trace covers shapes of at most 32768 tokens per workgroup"
    nbytes = -(-U * Wg * TRACE_SLOTS * 8 // 256) * 256
    off = ws.numel() - nbytes
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device=dev)
    rec = torch.zeros((steps, nbytes), dtype=torch.uint8, device=dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(16):
        Kl, Vl, cl = bufs[i % L]
        binding.decode_step(q0, Kl, Vl, W, cl, seq, N, k, inp.scale, out, ws)
    torch.cuda.synchronize()
    for i in range(steps):
        Kl, Vl, cl = bufs[i % L]
        evs[2 * i].record()
        binding.decode_step(q0, Kl, Vl, W, cl, seq, N, k, inp.scale, out, ws)
        evs[2 * i + 1].record()
        rec[i].copy_(ws[off:])
    torch.cuda.synchronize()
    if binding.workspace_check(ws):
        raise RuntimeError("workspace error word set during the phase trace")
    ev_us = np.array([evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e3 for i in range(steps)])
    ts = rec.cpu().numpy().view(np.uint64).reshape(steps, -1, TRACE_SLOTS).astype(np.int64)[:, :U * Wg]
    nwg = int((ts[0, :, 0] != 0).sum())
    assert nwg == U * Wg, f"{nwg} workgroups left timestamps, {U * Wg} expected"
    ts = ts[:, :, :len(TRACE_POINTS)]
    tick_ns = 10.0  # s_memrealtime runs at 100 MHz
    t0 = ts[:, :, 0].min(axis=1)[:, None]
    valid = ts != 0
    rel = np.where(valid, (ts - t0[:, :, None]) * tick_ns / 1e3, np.nan)  # us since the first start
    med_rel = np.nanmedian(np.nanmedian(rel, axis=1), axis=0)
    max_rel = np.nanmedian(np.nanmax(rel, axis=1), axis=0)
    phases = {}
    prev = None
    for j in TRACE_ORDER:
        name = TRACE_POINTS[j]
        col = rel[:, :, j]
        if np.isnan(col).all():
            continue
        entry = {"median_since_first_start_us": float(med_rel[j]), "latest_since_first_start_us": float(max_rel[j])}
        if prev is not None:
            dur = rel[:, :, j] - rel[:, :, prev]
            entry["median_phase_us"] = float(np.nanmedian(dur))
            entry["p90_phase_us"] = float(np.nanpercentile(dur, 90))
        phases[name] = entry
        prev = j
    # values the traced build records in slots 20..23 (search rounds, window
    # base, smallest own k-th score, threshold | kept rows << 16)
    vals = rec.cpu().numpy().view(np.uint64).reshape(steps, -1, TRACE_SLOTS).astype(np.int64)[:, :U * Wg, 20:24]
    kept = vals[:, :, 3] >> 16
    search = {"rounds_median": float(np.median(vals[:, :, 0])), "rounds_max": int(vals[:, :, 0].max()),
              "window_base_median": float(np.median(vals[:, :, 1])),
              "min_kth_median": float(np.median(vals[:, :, 2])),
              "threshold_median": float(np.median(vals[:, :, 3] & 0xFFFF)),
              "kept_rows_per_workgroup_median": float(np.median(kept)),
              "kept_rows_per_workgroup_max_median_over_steps": float(np.median(kept.max(axis=1)))}
    log(f"search: {search}")
    res = {"workload": shape.name, "workgroups": nwg, "units": U, "steps": steps, "layers": L, "search": search,
           "kernel_us_hip_events_median": float(np.median(ev_us)),
           "span_first_start_to_last_end_us_median": float(max_rel[TRACE_POINTS.index("end")]),
           "start_spread_us_median": float(max_rel[0]), "phases": phases}
    log(f"phase trace {shape.name}: {nwg} workgroups, {steps} eager steps, events {np.median(ev_us):.2f} us/step")
    log(f"{'boundary':>10} {'median':>8} {'latest':>8} {'phase':>8} {'p90':>8}  (us)")
    for name, e in phases.items():
        log(f"{name:>10} {e['median_since_first_start_us']:8.2f} {e['latest_since_first_start_us']:8.2f} "
            f"{e.get('median_phase_us', 0.0):8.2f} {e.get('p90_phase_us', 0.0):8.2f}")
    del bufs
    torch.cuda.empty_cache()
    return res


def bulk_run(cfg_id: int = 4, calls: int = 20) -> None:
    """Short run for counter passes on the bulk encode: `calls` encodes of
    the workload's whole key cache (every KV head, all N rows) over rotating
    key tensors, then one plain device copy of 1 GiB as the byte-counter
    reference."""
    import torch

    from hash_top_sparse_amd import binding, synth

    shape = synth.CONFIGS[cfg_id]
    B, Hkv, N = shape.B, shape.Hkv, shape.N
    g = torch.Generator(device="cuda").manual_seed(5)
    keys = [torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(4)]
    W = torch.randn((Hkv, 128, 128), generator=g, device="cuda") / 128 ** 0.5
    codes = torch.zeros((B, Hkv, N, 2), dtype=torch.int64, device="cuda")
    for i in range(calls):
        binding.encode_append(keys[i % len(keys)], W, codes, n_new=N)
    torch.cuda.synchronize()
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)  # reference: reads and writes exactly 1 GiB
    torch.cuda.synchronize()
    log(f"bulk run done: {calls} encodes of {B * Hkv * N} keys; reference copy of 1073741824 bytes")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--config", type=int, default=4, help="workload id in hash_top_sparse_amd.synth.CONFIGS")
    ap.add_argument("--layers", type=int, default=0, help="distinct layer caches to rotate through (0 = auto)")
    ap.add_argument("--dense-steps", type=int, default=256)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch the timed steps eagerly")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the other workloads (32K batch 1, 64K batch 4, 32K MHA batch 8, 4K tiny)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 32K-token prefill measurement")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache step measurement")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the hash-weight training step (labels + one gradient step, one head)")
    ap.add_argument("--no-width-sweep", action="store_true",
                    help="skip the workload with 32-, 64- and 256-bit codes")
    ap.add_argument("--no-model-sweep", action="store_true",
                    help="skip the 32-layer decode (one graph per token) at 32K/64K/128K against dense")
    ap.add_argument("--prefill-run", action="store_true",
                    help="short run for hardware-counter passes on the prefill: one 32K-token prefill")
    ap.add_argument("--bulk-run", action="store_true",
                    help="short run for hardware-counter passes on the bulk encode (20 encodes of the "
                         "workload's key cache, then a 1 GiB reference copy)")
    ap.add_argument("--train-run", action="store_true",
                    help="only the training step, 20 calls (for kernel traces)")
    ap.add_argument("--r", type=int, default=128, help="code width for --phase-trace (32, 64, 128, 256)")
    ap.add_argument("--phase-trace", action="store_true",
                    help="only the per-phase timeline of the fused step (phase-trace build of the library)")
    ap.add_argument("--pmc-run", action="store_true",
                    help="short run for hardware-counter passes: 32 eager fused steps over the layer "
                         "caches, then one plain device copy of 1 GiB as the byte-counter reference")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2

    import torch

    from hash_top_sparse_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.phase_trace:
        for c in ((args.config,) if args.config != 4 or args.r != 128 else (4, 2, 1)):
            print(json.dumps({"phase_trace": phase_trace(c, steps=200, r=args.r)}), flush=True)
        return 0
    binding.load()
    if args.prefill_run:
        prefill_bench(reps=1, paged=False)
        log("prefill run done")
        return 0
    if args.bulk_run:
        bulk_run(args.config)
        return 0
    if args.train_run:
        train_bench(steps=20)
        log("train run done")
        return 0
    if args.pmc_run:
        measure(args.config, 32, 8, 0, args.layers, False, with_bulk=False, with_qk=False)
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)  # reference: reads and writes exactly 1 GiB
        torch.cuda.synchronize()
        log("pmc run done: reference copy of 1073741824 bytes")
        return 0
    peak_meas = read_peak()
    log(f"streaming read of 4 GiB: {peak_meas:.0f} GB/s")
    head, inp = measure(args.config, args.steps, args.warmup, 0 if args.no_dense else args.dense_steps,
                        args.layers, not args.no_graph, with_bulk=True, read_rate=peak_meas)
    shape = inp.shape
    # the other workloads and code widths: graphs of at least 256 steps
    # (200 eager ones for the spread), whatever --steps is
    sub_steps = max(256, args.steps // 8)
    sweep = None
    if not args.no_sweep:
        sweep = {}
        for c in (2, 3, 5, 1):
            if c == args.config:
                continue
            r, _ = measure(c, sub_steps, 16, 0 if args.no_dense else 32, 0,
                           not args.no_graph, with_bulk=False, with_qk=False, read_rate=peak_meas)
            sweep[str(c)] = r

    wsweep = None
    if not args.no_width_sweep:
        wsweep = {}
        for r in (32, 64, 256):
            rr, _ = measure(args.config, sub_steps, 16, 0, 0, not args.no_graph,
                            with_bulk=False, with_qk=False, r=r)
            B_, Hkv_, N_ = shape.B, shape.Hkv, shape.N
            # code rows are stored in r/8 bytes (4 at r = 32): the stored bytes
            # are the formula's
            layout = rr["bytes_per_step"]
            wsweep[str(r)] = {"ms_per_step": rr["ms_per_step"], "steps_per_s": rr["steps_per_s"],
                              "GBs": rr["GBs"], "frac_of_peak": rr["frac_of_peak"],
                              "bytes_per_step": rr["bytes_per_step"], "stored_bytes_per_step": layout}
    pbench = None if args.no_prefill else prefill_bench()
    gbench = None if args.no_paged else paged_bench(args.config)
    msweep = None if args.no_model_sweep else model_sweep()
    tbench = None if args.no_train else train_bench()
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(inp, args.cpu_budget)
        log(f"oracle: {cpu['value']:.2f} steps/s on {cpu['cores']} threads")

    ms_step = head["ms_per_step"]
    res = {
        "metric": "decode steps/s and HBM GB/s (% of peak) for hata_decode_step at 32K\u2013128K ctx",
        "value": 1000.0 / ms_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32+fp32 (bf16 K/V, fp32 W_H)",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}: one decode step of one attention layer",
                   "batch": shape.B, "q_heads": shape.Hq, "kv_heads": shape.Hkv, "head_dim": 128,
                   "context": shape.N, "code_bits": 128, "budget_k": shape.k,
                   "layer_caches_rotated": head["layers"],
                   "timing": "graph of K steps, HIP events" if not args.no_graph else "eager, HIP events"},
        "roofline": {"bound": "hbm", "achieved": head["GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": head["GBs"] / PEAK_HBM_GBS,
                     "traffic": profiled_traffic() if args.config == 4 else None,
                     "kernel": f"decode_step_kernel<{shape.G}, false, 128, false>", "bytes_per_launch": head["bytes_per_step"],
                     "peak_measured": peak_meas, "frac_of_measured": head["GBs"] / peak_meas,
                     "peak_measured_by": "hata_stream_read over 4 GiB, best of 5"},
        "tokens_per_s": head["tokens_per_s"],
        "eager_step_spread": head["eager_step_spread"],
        "separate_key_encoder": head["separate_key_encoder"],
        "code_stream_alone": head["code_stream_alone"],
        "cpu_baseline": cpu,
        "dense_baseline": head["dense"],
        "bulk_encode": head["bulk_encode"],
    }
    if sweep is not None:
        res["sweep"] = sweep
    if msweep is not None:
        res["model_sweep"] = msweep
    if wsweep is not None:
        res["code_widths"] = wsweep
    if tbench is not None:
        res["hash_train"] = tbench
    if pbench is not None:
        res["prefill"] = pbench
    if gbench is not None:
        res["paged_step"] = gbench
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
