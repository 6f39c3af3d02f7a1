#!/usr/bin/env python3
"""Throughput of the paged KV-cache hot path on one MI355X.

A step is one pass of the path over one synthetic batch, all on one stream:
  * the Qwen3-8B-shaped decode layer (the headline workload, default: 1024
    sequences, U[100,2048] tokens, 32 Q / 8 KV heads, head_dim 128, block 256,
    307 sequences sharing a 512-token prefix): each sequence's newest token
    stored and its paged context attended. Both ways of doing that are timed
    per call: pa_store_kv then pa_decode, and pa_store_decode (the two in one
    launch); each way is timed as a whole step and the faster is the step
    (--path fused|separate forces one);
  * the mixed chunked-prefill step (--workload 4): pa_store_kv of 4344 new
    tokens, pa_prefill_varlen of 8 chunks of 512 on cached prefixes, pa_decode
    of 248 sequences.
The step's calls are captured once as a HIP graph and replayed (--eager times
them as separate calls).
Inputs are resident in HBM before the timed region, and the caches are cold:
before every timed step (and every timed launch of a per-call figure) an
elementwise kernel reads 512 MiB and writes 512 MiB, four times the 256 MB
Infinity Cache, so that nothing of the step's working set is served from L2
or the MALL. That flush is timed on its own and subtracted: a graph of
[flush, step] and a graph of [flush] are each replayed K times between HIP
events on the launch stream. `value` is the step's algorithmic bytes (unique KV
bytes read by decode and prefill, q/out, tables, plus the store's reads and
writes) divided by the cold time per step. The `roofline` object is the
dominant kernel (the decode kernel, as pa_decode launches it) timed the same
way on its own; `step_launch` is the pa_store_decode call (the same decode
kernel, then the store) when the step uses it; `prefill_roofline` is
the prefill kernel of the mixed chunked-prefill step against the dense bf16
MFMA peak. `traffic`, `overfetch` and `mfma_util` are read from the committed
rocprofv3 counter summaries in profiles/ while the kernel's sources are
unchanged since they were taken (null otherwise). `ms_per_step_percentiles`
(p10/p50/p90) times each step on its own, less the median flush. --warm adds
the figures of back-to-back launches with warm caches.
`cpu_baseline` times the CPU oracle (numpy float64) on this host: store +
decode on a bounded sample of the headline workload's sequences, and the
mixed step's prefill.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload 3]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_TBS = 8.0              # MI355X HBM3E, TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
MFMA_PROFILE = os.path.join(ROOT, "profiles", "prefill_mfma_counters.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work
def decode_bytes(w, seqs=None):
    """Algorithmic bytes of one pa_decode: K and V of every valid token of every
    *unique* (physical block, KV head) read, plus q, out, the table entries read
    and the context lengths (plus fp8 scales). Also returns the logical KV bytes
    (shared blocks counted once per sequence that reads them)."""
    es = 1 if w.kv_dtype == "fp8" else 2
    row = w.num_kv_heads * w.head_dim * es * 2         # K+V bytes of one token, all KV heads
    seqs = range(w.num_seqs) if seqs is None else seqs
    unique = {}
    logical = 0
    entries = 0
    for s in seqs:
        n = int(w.context_lens[s])
        nb = math.ceil(n / w.block_size)
        entries += nb
        logical += n * row
        for j in range(nb):
            b = int(w.block_tables[s, j])
            unique[b] = max(unique.get(b, 0), min(w.block_size, n - j * w.block_size))
    kv_unique = sum(unique.values()) * row
    S = len(list(seqs)) if not isinstance(seqs, range) else len(seqs)
    extra = 2 * S * w.num_q_heads * w.head_dim * 2 + 4 * entries + 4 * S
    if w.kv_dtype == "fp8":
        extra += 2 * 4 * w.num_kv_heads
    return kv_unique + extra, logical + extra, kv_unique


def store_bytes(w):
    """k, v read (bf16) + slots read + pool bytes written."""
    T = w.new_slots.size
    es = 1 if w.kv_dtype == "fp8" else 2
    return T * w.num_kv_heads * w.head_dim * (2 * 2 + 2 * es) + 4 * T


def prefill_work(w):
    """(flops, bytes): 4*D*Hq per unmasked (query, key) pair (QK^T and PV), and the
    K/V of each sequence's Lk keys + q + out + table entries + cu_seqlens."""
    cu_q, cu_k = w.cu_seqlens_q, w.cu_seqlens_k
    pairs = 0
    kv = 0
    entries = 0
    for s in range(len(cu_q) - 1):
        lq = int(cu_q[s + 1] - cu_q[s])
        lk = int(cu_k[s + 1] - cu_k[s])
        pairs += sum(lk - lq + i + 1 for i in range(lq))
        kv += lk * w.num_kv_heads * w.head_dim * 2 * 2
        entries += math.ceil(lk / w.block_size)
    tq = int(cu_q[-1])
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    byts = kv + 2 * tq * w.num_q_heads * w.head_dim * 2 + 4 * entries + 8 * (len(cu_q))
    return flops, byts


# The kernel sources each call's counter figures depend on.
# the sources of each call's kernels (pa_store_decode: the decode kernel, then the store kernel)
CALL_SOURCES = {"decode": ("decode.hip", "pa_device.h"),
                "store_decode": ("decode.hip", "store_kv.hip", "pa_device.h"),
                "prefill": ("prefill.hip", "pa_device.h"), "store": ("store_kv.hip", "pa_device.h")}


def sources_sha256(call):
    import hashlib
    h = hashlib.sha256()
    for f in CALL_SOURCES[call]:
        with open(os.path.join(ROOT, "paged_kv_cache_store_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_figure(path, name, workload, call):
    """A counter figure from a committed rocprofv3 summary: the line
    `<name> w<workload>/<call>: <value>`, used only while the line
    `sources_sha256 <call>: <hash>` of the same file matches the sources the
    call's kernel is built from (else None: the kernel changed since)."""
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        key, sep, val = line.partition(": ")
        if sep and (key.startswith(name + " ") or key.startswith("sources_sha256 ")):
            fields[key.strip()] = val.strip()
    if fields.get(f"sources_sha256 {call}") != sources_sha256(call):
        return None
    val = fields.get(f"{name} w{workload}/{call}")
    return None if val is None else float(val)


# ---------------------------------------------------------------- GPU set-up
class Setup:
    def __init__(self, w):
        import torch

        import paged_kv_cache_store_amd as pa
        import workloads as W
        self.w, self.pa, self.torch = w, pa, torch

        def dev_bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

        def dev_i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

        self.kc, self.vc = pa.empty_pools(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim,
                                          w.kv_dtype)
        self.ks = self.vs = None
        if w.kv_dtype == "fp8":
            self.kc.fill_(int(W.FP8_NAN))
            self.vc.fill_(int(W.FP8_NAN))
            self.ks = torch.from_numpy(w.k_scale).cuda()
            self.vs = torch.from_numpy(w.v_scale).cuda()
        else:
            self.kc.view(torch.int16).fill_(int(W.BF16_NAN))
            self.vc.view(torch.int16).fill_(int(W.BF16_NAN))
        # cached context, written once before timing (in slices to bound host memory)
        step = 1 << 18
        for lo in range(0, w.fill_slots.size, step):
            hi = min(w.fill_slots.size, lo + step)
            pa.store_kv(dev_bf16(w.fill_k[lo:hi]), dev_bf16(w.fill_v[lo:hi]),
                        dev_i32(w.fill_slots[lo:hi]), self.kc, self.vc, self.ks, self.vs)
        self.new_k, self.new_v = dev_bf16(w.new_k), dev_bf16(w.new_v)
        self.new_slots = dev_i32(w.new_slots)
        # a decode-only step may store each sequence's newest token inside the
        # decode launch (pa_store_decode): one token per sequence, slot -1 where empty
        self.decode_only = not w.has_prefill
        if self.decode_only:
            live = np.flatnonzero(w.context_lens > 0)
            assert live.size == w.new_slots.size
            k1 = np.zeros((w.num_seqs,) + w.new_k.shape[1:], np.uint16)
            v1 = np.zeros_like(k1)
            s1 = np.full(w.num_seqs, -1, np.int32)
            k1[live], v1[live], s1[live] = w.new_k, w.new_v, w.new_slots
            self.seq_k, self.seq_v, self.seq_slots = dev_bf16(k1), dev_bf16(v1), dev_i32(s1)
        self.q = dev_bf16(w.q)
        self.bt = dev_i32(w.block_tables)
        self.lens = dev_i32(w.context_lens)
        self.out = torch.empty_like(self.q)
        self.P = pa.decode_partition_size(w.num_seqs, w.num_q_heads, w.max_context_len, w.partition_size)
        need = pa.decode_workspace_size(w.num_seqs, w.num_q_heads, w.head_dim, w.max_context_len, self.P)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        if w.has_prefill:
            self.pq = dev_bf16(w.pq)
            self.cu_q, self.cu_k = dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k)
            self.pbt = dev_i32(w.p_block_tables)
            self.pout = torch.empty_like(self.pq)
        torch.cuda.synchronize()

    def store(self):
        self.pa.store_kv(self.new_k, self.new_v, self.new_slots, self.kc, self.vc, self.ks, self.vs)

    def decode(self):
        w = self.w
        self.pa.decode(self.q, self.kc, self.vc, self.bt, self.lens, float(w.scale), w.max_context_len,
                       out=self.out, k_scale=self.ks, v_scale=self.vs, partition_size=self.P,
                       workspace=self.ws)

    def store_decode(self):
        w = self.w
        self.pa.decode(self.q, self.kc, self.vc, self.bt, self.lens, float(w.scale), w.max_context_len,
                       out=self.out, k_scale=self.ks, v_scale=self.vs, partition_size=self.P,
                       workspace=self.ws, new_k=self.seq_k, new_v=self.seq_v, slot_mapping=self.seq_slots)

    def prefill(self):
        w = self.w
        self.pa.prefill_varlen(self.pq, self.kc, self.vc, self.cu_q, self.cu_k, self.pbt, float(w.scale),
                               w.max_seqlen_q, w.max_seqlen_k, out=self.pout, k_scale=self.ks,
                               v_scale=self.vs)


def time_launches(pa, torch, fn, reps, iters):
    """GPU time of one call of fn: a HIP graph of `reps` back-to-back calls,
    replayed `iters` times between two HIP events on the launch stream (so no
    host-side gap between launches is counted). Returns ms per call."""
    g = pa.capture_step(lambda: [fn() for _ in range(reps)])
    g.replay()
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(iters):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / (reps * iters)


class Flush:
    """Evicts L2 and the Infinity Cache (MALL, 256 MB) between timed launches: one
    elementwise kernel (no memset, capturable) reading 512 MiB and writing 512 MiB."""

    def __init__(self, torch):
        self.torch = torch
        self.src = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
        self.dst = torch.empty_like(self.src)

    def __call__(self):
        self.torch.add(self.src, 1.0, out=self.dst)


def _replay_ms(torch, g, n):
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def cold_launches(pa, torch, fn, flush, reps, iters):
    """GPU time of one call of fn with cold caches: a HIP graph of `reps` times
    [flush, fn] and a graph of `reps` flushes, replayed alternately `iters` times
    each between HIP events on the launch stream; the difference per call."""
    g1 = pa.capture_step(lambda: [(flush(), fn()) for _ in range(reps)])
    g0 = pa.capture_step(lambda: [flush() for _ in range(reps)])
    g1.replay()
    g0.replay()
    t1 = t0 = 0.0
    for _ in range(iters):
        t1 += _replay_ms(torch, g1, 1)
        t0 += _replay_ms(torch, g0, 1)
    del g1, g0
    return (t1 - t0) / (reps * iters)


def run_steps(st, steps, warmup, path="auto", graph=True, warm=False):
    """Warm up; time each call on its own with cold caches (cold_launches); pick
    the step's calls; then time `steps` whole steps with cold caches: with
    graph=True one captured HIP graph of [flush, step] replayed `steps` times
    between HIP events (bracketed by synchronisations), minus the same number of
    replays of [flush]; with graph=False the calls are issued eagerly, events
    around each step after its flush. A decode-only step is pa_store_kv +
    pa_decode ("separate") or pa_store_decode ("fused"); path="auto" takes the
    one whose whole step is faster with cold caches. warm=True adds back-to-back
    (warm-cache) figures. Returns a dict."""
    torch = st.torch
    flush = Flush(torch)
    if st.decode_only:
        candidates = [("store", st.store), ("decode", st.decode), ("store_decode", st.store_decode)]
    else:
        candidates = [("store", st.store)]
        if st.w.has_prefill:
            candidates.append(("prefill", st.prefill))
        candidates.append(("decode", st.decode))
    for _ in range(warmup):
        for _, f in candidates:
            f()
    torch.cuda.synchronize()
    out = {"ms": {name: cold_launches(st.pa, torch, f, flush, 10, max(3, steps // 4))
                  for name, f in candidates}}
    if st.decode_only:
        # the two ways of doing the step, each timed as a whole (the separate
        # store changes what the decode after it reads, so the per-call
        # figures do not add up to the step)
        ways = {"fused": [("store_decode", st.store_decode)],
                "separate": [("store", st.store), ("decode", st.decode)]}
        out["ms_step_ways"] = {k: cold_launches(st.pa, torch, lambda fs=fs: [f() for _, f in fs], flush, 10,
                                                max(3, steps // 4)) for k, fs in ways.items()}
        if path == "auto":
            path = min(ways, key=lambda k: out["ms_step_ways"][k])
        calls = ways[path]
    else:
        path = "separate"
        calls = candidates
    out["path"] = path

    def step():
        for _, f in calls:
            f()

    if graph:
        g1 = st.pa.capture_step(lambda: (flush(), step()))
        g0 = st.pa.capture_step(flush)
        for _ in range(warmup):
            g1.replay()
        t1 = _replay_ms(torch, g1, steps)      # exactly `steps` steps, each after a flush
        t0 = _replay_ms(torch, g0, steps)
        out["ms_step"] = (t1 - t0) / steps
        # spread: each replay timed on its own, less the median flush
        flush_ms = float(np.median([_replay_ms(torch, g0, 1) for _ in range(steps)]))
        per = np.array([_replay_ms(torch, g1, 1) for _ in range(steps)]) - flush_ms
        out["step_ms_pct"] = {k: round(float(np.percentile(per, q)), 5)
                              for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}
        del g1, g0
    else:
        stream = torch.cuda.current_stream()
        per = []
        for _ in range(steps):
            flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b))
        out["ms_step"] = sum(per) / steps
        out["step_ms_pct"] = {k: round(float(np.percentile(per, q)), 5)
                              for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}
    if warm:
        out["ms_warm"] = {name: time_launches(st.pa, torch, f, 10, max(2, steps // 4))
                          for name, f in candidates}
        g = st.pa.capture_step(step)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        out["ms_step_warm"] = (time.perf_counter() - t0) * 1e3 / steps
        del g
    del flush
    return out


def norm_bench(torch, T, H, steps, warmup):
    """Time pa_add_rmsnorm (with residual) on [T, H] bf16 rows with cold caches
    (cold_launches: 20 launches per graph, each after a flush). Algorithmic
    bytes: x and r read, y and the new residual written (4·T·H·2) plus the
    weight once (H·2)."""
    import paged_kv_cache_store_amd as pa
    import workloads as W
    x, r, w = W.norm_inputs(7, T, H)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    xd, rd, wd = dev(x), dev(r), dev(w)
    out, hres = torch.empty_like(xd), torch.empty_like(xd)

    def launch():
        pa.add_rmsnorm(xd, wd, 1e-6, residual=rd, out=out, residual_out=hres)

    for _ in range(warmup):
        launch()
    flush = Flush(torch)
    ms = cold_launches(pa, torch, launch, flush, 20, max(2, steps // 2))
    del flush
    nbytes = 4 * T * H * 2 + H * 2
    return {"TBps": round(nbytes / (ms * 1e-3) / 1e12, 4), "ms": round(ms, 5), "bytes": nbytes,
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e12 / HBM_PEAK_TBS, 4)}




# ---------------------------------------------------------------- CPU oracle baseline
def host_info():
    """The host the CPU figures come from: usable cores, all cores, CPU model,
    BLAS threads (numpy's matrix products are the oracle's only threaded part)."""
    model = "unknown"
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
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        pass
    return {"cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(), "cpu_model": model,
            "blas_threads": blas}


def _oracle_pools(w):
    import oracle
    ks, vs = oracle.cache.pool_shapes(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.kv_dtype)
    dt = np.uint8 if w.kv_dtype == "fp8" else np.uint16
    kc, vc = np.zeros(ks, dt), np.zeros(vs, dt)
    oracle.cache.store(w.fill_k, w.fill_v, w.fill_slots, kc, vc, w.block_size, w.k_scale, w.v_scale)
    return kc, vc


def oracle_decode_baseline(w, budget_s=12.0):
    """The oracle's store + decode of a decode workload, 16 sequences at a time
    (each sequence's newest token stored, then its context attended), until
    about budget_s seconds of work; TB/s over the same algorithmic bytes as the
    GPU figure. The cached context is stored before timing."""
    import oracle
    kc, vc = _oracle_pools(w)
    done = passes = nbytes = 0
    t_total = 0.0
    while t_total < budget_s and passes < 50:
        chunk = np.arange(done % w.num_seqs, min(w.num_seqs, done % w.num_seqs + 16))
        last = [int(w.block_tables[s, (int(w.context_lens[s]) - 1) // w.block_size]) * w.block_size
                + (int(w.context_lens[s]) - 1) % w.block_size for s in chunk]
        sel = np.isin(w.new_slots, last)
        t0 = time.perf_counter()
        oracle.cache.store(w.new_k[sel], w.new_v[sel], w.new_slots[sel], kc, vc, w.block_size,
                           w.k_scale, w.v_scale)
        oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size,
                                w.k_scale, w.v_scale, seqs=chunk)
        t_total += time.perf_counter() - t0
        nbytes += decode_bytes(w, chunk)[0] + store_bytes_of(w, int(sel.sum()))
        done += len(chunk)
        if done % w.num_seqs == 0:
            passes += 1
    return {"value": round(nbytes / t_total / 1e12, 6), "unit": "TB/s", "kind": "oracle",
            "sample": f"{done} sequence decodes of the {w.name} workload ({done / w.num_seqs:.2f} passes "
                      f"over its {w.num_seqs} sequences; store of each newest token + decode, float64), "
                      f"{t_total:.1f} s of work",
            "seconds": round(t_total, 2), "sequences": done}


def store_bytes_of(w, tokens):
    es = 1 if w.kv_dtype == "fp8" else 2
    return tokens * w.num_kv_heads * w.head_dim * (2 * 2 + 2 * es) + 4 * tokens


def oracle_prefill_baseline(w, budget_s=20.0):
    """The oracle's prefill of the mixed step's chunks, one sequence at a time
    until every chunk is done or about budget_s seconds have passed; GFLOP/s
    over the same algorithmic flops as the GPU figure."""
    import oracle
    kc, vc = _oracle_pools(w)
    oracle.cache.store(w.new_k, w.new_v, w.new_slots, kc, vc, w.block_size, w.k_scale, w.v_scale)
    t_total = 0.0
    flops = 0
    done = 0
    for s in range(len(w.cu_seqlens_q) - 1):
        if t_total >= budget_s:
            break
        t0 = time.perf_counter()
        oracle.attention.prefill(w.pq, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k, w.p_block_tables, w.scale,
                                 w.block_size, w.k_scale, w.v_scale, seqs=[s])
        t_total += time.perf_counter() - t0
        lq = int(w.cu_seqlens_q[s + 1] - w.cu_seqlens_q[s])
        lk = int(w.cu_seqlens_k[s + 1] - w.cu_seqlens_k[s])
        flops += 4 * w.head_dim * w.num_q_heads * sum(lk - lq + i + 1 for i in range(lq))
        done += 1
    return {"value": round(flops / t_total / 1e9, 3), "unit": "GFLOP/s", "kind": "oracle",
            "sample": f"prefill of {done} of the {len(w.cu_seqlens_q) - 1} chunks of the {w.name} step "
                      f"(float64), {t_total:.1f} s of work",
            "seconds": round(t_total, 2)}


def copy_calibration(torch, reps):
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 4),
                      "read_plus_write_TBps": round(2 * n / (ms * 1e-3) / 1e12, 4)}), flush=True)


# ---------------------------------------------------------------- main
def device_info(torch):
    """The GPU the figures come from (name, architecture, compute units, memory)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2 ** 30, 1)}


def tbps(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e12


def decode_entry(r):
    """Per-call figures of a decode workload: pa_decode alone, pa_store_kv, and
    (decode-only steps) pa_store_decode against the two separate calls."""
    ms = r["ms"]
    ent = {"decode_TBps": round(tbps(r["decode_bytes"], ms["decode"]), 4),
           "decode_ms": round(ms["decode"], 5), "decode_unique_bytes": r["decode_bytes"],
           "decode_logical_TBps": round(tbps(r["decode_logical"], ms["decode"]), 4),
           "store_ms": round(ms["store"], 5), "partition_size": r["P"], "step_path": r["path"],
           "step_ms": round(r["ms_step"], 5)}
    if "store_decode" in ms:
        both = r["decode_bytes"] + r["store_bytes"]
        ent.update({"store_decode_ms": round(ms["store_decode"], 5),
                    "store_decode_TBps": round(tbps(both, ms["store_decode"]), 4)})
    if r.get("ms_step_ways"):
        # each way of doing the decode step timed whole (cold caches)
        ent["step_ways_ms"] = {k: round(v, 5) for k, v in r["ms_step_ways"].items()}
    if "prefill" in ms:
        tf = r["prefill_flops"] / (ms["prefill"] * 1e-3) / 1e12
        ent.update({"prefill_TFLOPs": round(tf, 2), "prefill_ms": round(ms["prefill"], 5),
                    "prefill_frac_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                    "prefill_flops": r["prefill_flops"]})
    return ent


def prefill_roofline(r):
    """Roofline object of the prefill kernel of a mixed step (dense bf16 MFMA peak)."""
    w = r["w"]
    ms = r["ms"]["prefill"]
    tf = r["prefill_flops"] / (ms * 1e-3) / 1e12
    mfma = profile_figure(MFMA_PROFILE, "mfma_util", w.number, "prefill")
    traffic = profile_figure(TRAFFIC_PROFILE, "traffic_bytes_per_launch", w.number, "prefill")
    return {"bound": "mfma", "workload": w.name, "kernel": "prefill_persist_kernel (pa_prefill_varlen)",
            "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "flops_per_launch": r["prefill_flops"],
            "ms_per_launch": round(ms, 5), "mfma_util": mfma,
            "traffic": None if traffic is None else int(traffic),
            "bytes_per_launch": r["prefill_bytes"],
            "overfetch": None if traffic is None else round(traffic / r["prefill_bytes"], 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--partition-size", type=int, default=None,
                    help="decode partition size (default: the workload's, else automatic)")
    ap.add_argument("--path", choices=["auto", "fused", "separate"], default="auto",
                    help="decode-only steps: pa_store_decode (fused), pa_store_kv + pa_decode "
                         "(separate), or the faster of the two, each timed as a whole step (auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the figures of the other workloads")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as individual calls instead of one HIP-graph replay")
    ap.add_argument("--warm", action="store_true",
                    help="also time back-to-back launches with warm caches (context figures)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="time a plain 1 GiB device copy (counter calibration / HBM ceiling) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: --gpus must be 1 (no multi-GPU path exists)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calib:
        copy_calibration(torch, args.steps)
        return

    def measure(number, steps, warmup, path):
        w = W.make(number)
        if args.partition_size is not None:
            w.partition_size = args.partition_size
        st = Setup(w)
        t = run_steps(st, steps, warmup, path=path, graph=not args.eager, warm=args.warm)
        dec_b, dec_logical, dec_kv = decode_bytes(w)
        res = {"w": w, "ms_step": t["ms_step"], "step_ms_pct": t.get("step_ms_pct"), "ms": t["ms"],
               "ms_warm": t.get("ms_warm"), "path": t["path"], "ms_step_ways": t.get("ms_step_ways"),
               "ms_step_warm": t.get("ms_step_warm"), "decode_bytes": dec_b,
               "decode_logical": dec_logical, "store_bytes": store_bytes(w), "P": st.P}
        if w.has_prefill:
            res["prefill_flops"], res["prefill_bytes"] = prefill_work(w)
        del st
        torch.cuda.empty_cache()
        return res

    log(f"[bench] workload {args.workload}: generating + set-up")
    r = measure(args.workload, args.steps, args.warmup, args.path)
    w = r["w"]
    step_bytes = r["decode_bytes"] + r["store_bytes"] + r.get("prefill_bytes", 0)
    value = step_bytes / (r["ms_step"] * 1e-3) / 1e12
    # the dominant kernel: the decode (decode_kernel), timed on its own as
    # pa_decode launches it; pa_store_decode runs the same kernel with the
    # newest tokens read from its arguments, then the store of those tokens
    whole = r["P"] >= w.max_context_len
    dom_name, dom_bytes = "decode", r["decode_bytes"]
    dom_kernel = ("decode_kernel (as pa_decode launches it; contexts whole, no reduce)" if whole
                  else "decode_kernel + decode_reduce_kernel (as pa_decode launches them)")
    dec_tbs = tbps(dom_bytes, r["ms"][dom_name])
    traffic = None
    if args.partition_size is None:
        traffic = profile_figure(TRAFFIC_PROFILE, "traffic_bytes_per_launch", w.number, dom_name)
    line = {
        "metric": "paged-attn decode KV TB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak)",
        "value": round(value, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 5),
        # per-step spread (each step timed alone, the median flush subtracted)
        "ms_per_step_percentiles": r["step_ms_pct"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8-e4m3 KV, bf16 q/out",
        "data": "synthetic (seeded; bf16 N(0,1) q/k/v, random block permutation)",
        "device": device_info(torch),
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "context_lens": f"U[{int(w.context_lens.min())},{int(w.context_lens.max())}] "
                                   f"mean {float(w.context_lens.mean()):.1f}",
                   "kv_dtype": w.kv_dtype, "partition_size": r["P"], "parallelism": "single GPU",
                   "step_path": ("pa_store_decode (the decode, taking the newest tokens from its arguments, "
                                 "then their store)" if r["path"] == "fused"
                                 else "pa_store_kv then pa_decode" + (" (+ pa_prefill_varlen)"
                                                                      if w.has_prefill else "")),
                   "launch": "eager calls" if args.eager else "one HIP-graph replay per step",
                   "caches": "cold (512 MiB read + 512 MiB written before every timed step or launch, "
                             "timed separately and subtracted)"},
        "roofline": {"bound": "hbm", "kernel": dom_kernel,
                     "achieved": round(dec_tbs * 1e3, 2), "peak": HBM_PEAK_TBS * 1e3, "unit": "GB/s",
                     "frac": round(dec_tbs / HBM_PEAK_TBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "overfetch": None if traffic is None else round(traffic / dom_bytes, 4),
                     "bytes_per_launch": dom_bytes, "ms_per_launch": round(r["ms"][dom_name], 5)},
        "per_call_ms": {k: round(v, 5) for k, v in r["ms"].items()},
        "this_workload": decode_entry(r),
    }
    if w.number == 3:
        line["roofline"]["logical_GBps"] = round(tbps(r["decode_logical"], r["ms"]["decode"]) * 1e3, 2)
    if r["path"] == "fused":
        # the step's decode launch as the step makes it (pa_store_decode: the
        # decode kernel, then the store of the newest tokens), over its bytes
        both = r["decode_bytes"] + r["store_bytes"]
        line["step_launch"] = {"call": "pa_store_decode", "bytes_per_call": both,
                               "ms_per_call": round(r["ms"]["store_decode"], 5),
                               "achieved_GBps": round(tbps(both, r["ms"]["store_decode"]) * 1e3, 2),
                               "frac": round(tbps(both, r["ms"]["store_decode"]) / HBM_PEAK_TBS, 4)}
    if w.has_prefill:
        line["prefill_roofline"] = prefill_roofline(r)
    if args.warm:
        wdom = r["ms_warm"][dom_name]
        line["warm"] = {"ms_per_step": round(r["ms_step_warm"], 5),
                        "value": round(step_bytes / (r["ms_step_warm"] * 1e-3) / 1e12, 4),
                        "dominant_achieved_GBps": round(dom_bytes / (wdom * 1e-3) / 1e9, 2),
                        "per_call_ms": {k: round(v, 5) for k, v in r["ms_warm"].items()},
                        "note": "back-to-back launches, caches warm (context only)"}
    w_prefill = w if w.has_prefill else None
    if not args.no_extra:
        extra = {}
        for number in [n for n in (2, 3, 4, 5, 6) if n != args.workload]:
            log(f"[bench] workload {number}")
            e = measure(number, max(5, args.steps // 2), 2, "auto")
            extra[e["w"].name] = decode_entry(e)
            if number == 4 and "prefill_roofline" not in line:
                line["prefill_roofline"] = prefill_roofline(e)
                w_prefill = e["w"]
            del e
        for name, (T, H) in W.NORM_WORKLOADS.items():
            log(f"[bench] add_rmsnorm {name}")
            extra["add_rmsnorm: " + name] = norm_bench(torch, T, H, 10, 2)
        line["other_workloads"] = extra
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        base = oracle_decode_baseline(w)
        base.update(host_info())
        base["threads_note"] = ("one Python thread; numpy's matrix products may use up to "
                                "blas_threads threads")
        if w_prefill is not None:
            log("[bench] CPU oracle prefill baseline")
            base["prefill"] = oracle_prefill_baseline(w_prefill)
        line["cpu_baseline"] = base
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
