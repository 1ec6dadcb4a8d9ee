#!/usr/bin/env python3
"""Benchmark of the ring-attention rank share on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the forward (every active ring step of the flash forward with its fused LSE
merge and finalisation) followed by the backward (Delta preprocess, every
active ring step of the backward with fp32 dQ/dK/dV accumulation), through the
C ABI.  Default workload: basic causal ring, rank 7 of D = 8, global sequence
65536 (8192 rows per block), 32 heads, head_dim 128, bf16, batch 1.

Prints ONE JSON line.  Throughput counts algorithmic work only (visible
(query, key) pairs): forward 4*d*Hq*B*pairs flops, backward 10*d*Hq*B*pairs.
`--calibrate-copy` runs only a plain copy kernel of known size, the reference
for scaling the FETCH_SIZE / WRITE_SIZE counters.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

METRIC = "causal attn fwd/bwd TFLOP/s per rank share (bf16) + % of MFMA peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_inputs(ca, w, torch):
    from context_attention_flash_amd import synth
    t0 = time.time()
    g = synth.draw_global(w)
    desc = ca.desc_from_workload(w)
    pos_q = ca.ring_attn_positions(desc, w.cu_seqlens)
    _, _, nb = ca.shard_sizes(desc)
    blocks = [ca.ring_attn_kv_positions(desc, w.cu_seqlens, j) for j in range(nb)]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()

    t = {"q": dev(g["q"][:, pos_q]),
         "k": dev(np.stack([g["k"][:, p] for p in blocks])),
         "v": dev(np.stack([g["v"][:, p] for p in blocks]))}
    if w.with_grad:
        t["dout"] = dev(g["dout"][:, pos_q])
    log(f"inputs ready in {time.time() - t0:.1f}s")
    return g, desc, t


def _oracle_worker(args):
    """One host process of the CPU baseline: the fp64 oracle's forward (and
    backward) of one q head's rows, heaviest first, 128 rows at a time, until
    its share of the time budget is spent.  BLAS runs single-threaded here
    (the pool sets the thread variables before the workers start)."""
    (w, h, q1, k1, v1, dout1, budget_s) = args
    import oracle
    S = w.seqlen // w.world
    cu = list(w.cu_seqlens) if w.cu_seqlens else None
    pos_q = oracle.positions(w.layout, w.seqlen, w.world, w.rank, cu)
    chunk, done_rows, flops = 128, 0, 0.0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done_rows < S:
        hi = S - done_rows   # the heaviest rows of a causal shard first
        rows = np.arange(max(0, hi - chunk), hi)
        oracle.rank_share_forward(q1, k1, v1, w.layout, w.world, w.rank, w.causal, cu,
                                  rows=rows, heads=[0])
        m = oracle.allowed(pos_q[rows], np.arange(w.seqlen), w.causal,
                           cu if w.layout in oracle.PACKED else None)
        pairs = float(m.sum())
        flops += 4.0 * w.head_dim * pairs
        if dout1 is not None:
            oracle.rank_share_backward(q1, k1, v1, dout1, w.layout, w.world, w.rank, w.causal,
                                       cu, rows=rows, heads=[0])
            flops += 10.0 * w.head_dim * pairs
        done_rows += len(rows)
    return h, done_rows, flops, time.perf_counter() - t0


# Host cores the baseline may use: the CPU share of one GPU on the boxes this
# runs on (what os.cpu_count() reports there can be the whole machine).
HOST_CORE_SHARE = 16


def start_host_pool(w):
    """The worker processes of the CPU baseline, one per host core of the share
    (at most one per q head), each with one BLAS thread.  They are started
    before this process touches the GPU, so no child is ever started from a
    process that holds a GPU context."""
    import multiprocessing as mp
    workers = max(1, min(os.cpu_count() or 1, HOST_CORE_SHARE, w.batch * w.heads_q))
    saved = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    for var in saved:
        os.environ[var] = "1"   # inherited by the spawned workers
    pool = mp.get_context("spawn").Pool(workers)
    for var, val in saved.items():
        if val is None:
            os.environ.pop(var, None)
        else:
            os.environ[var] = val
    return pool, workers


def cpu_baseline(w, g, budget_s: float, pool, workers: int):
    """The fp64 oracle timed on the host cores, on a bounded sample of the same
    workload: a process pool over (batch, q head) with one BLAS thread per
    worker, each worker taking the rows of one head, heaviest first, for about
    budget_s seconds."""
    n_cpu = os.cpu_count() or 1
    group = w.heads_q // w.heads_kv
    pos_q = None
    if w.with_grad:
        import oracle
        cu = list(w.cu_seqlens) if w.cu_seqlens else None
        pos_q = oracle.positions(w.layout, w.seqlen, w.world, w.rank, cu)
    tasks = []
    for i in range(workers):   # (batch 0, q head i): one head's slices per worker
        h, hk = i % w.heads_q, (i % w.heads_q) // group
        sl = lambda x, hh: np.ascontiguousarray(x[:1, :, hh:hh + 1])
        d1 = np.ascontiguousarray(g["dout"][:1, pos_q, h:h + 1]) if w.with_grad else None
        tasks.append((w.replace(batch=1, heads_q=1, heads_kv=1), h, sl(g["q"], h), sl(g["k"], hk),
                      sl(g["v"], hk), d1, budget_s))
    t0 = time.perf_counter()
    res = pool.map(_oracle_worker, tasks, chunksize=1)
    wall = time.perf_counter() - t0
    busy = max(r[3] for r in res)
    rows = sum(r[1] for r in res)
    flops = sum(r[2] for r in res)
    return {"value": flops / busy / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "host_cpu_count": n_cpu,
            "sample": f"fp64 numpy oracle, {'fwd+bwd' if w.with_grad else 'fwd'} of {rows} query "
                      f"rows in all ({workers} worker processes, one q head each, 1 BLAS thread "
                      f"each, the heaviest rows of the rank share first; {flops / 1e9:.1f} GFLOP "
                      f"algorithmic in {busy:.1f} s of compute, {wall:.1f} s with start-up)"}


def merge_bandwidth(ca, torch, rows=524288, d=128, reps=20):
    """Standalone LSE merge at 524288 rows x 128 (the zigzag rank share's
    per-step partial, 774 MiB per call, larger than the 256 MB MALL)."""
    B, H = 1, 32
    S = rows // H
    o = torch.randn(B, S, H, d, device="cuda")
    oj = torch.randn(B, S, H, d, device="cuda")
    l = torch.randn(B, H, S, device="cuda")
    lj = torch.randn(B, H, S, device="cuda")
    for _ in range(3):
        ca.ring_attn_lse_merge(o, l, oj, lj)
    torch.cuda.synchronize()
    ca.ring_attn_timing_enable(False)
    ca.ring_attn_timing_enable(True)
    for _ in range(reps):
        ca.ring_attn_lse_merge(o, l, oj, lj)
    n, ms = ca.ring_attn_timing_read("lse_merge")
    ca.ring_attn_timing_enable(False)
    nbytes = (12 * d + 12) * rows
    gbs = nbytes / (ms / n * 1e-3) / 1e9
    from context_attention_flash_amd import profsum
    # HBM bytes per launch counted by FETCH_SIZE + WRITE_SIZE (scaled by the
    # copy calibration), while the summary matches the kernel's sources
    traffic = profsum.read_traffic(os.path.join(ROOT, "profiles", MERGE_TRAFFIC_MD), "lse_merge_kernel")
    return {"kernel": "lse_merge", "rows": rows, "head_dim": d, "bytes_per_launch": nbytes,
            "avg_ms": ms / n, "GB/s": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS,
            "traffic": traffic,
            "traffic_GB/s": None if traffic is None else traffic / (ms / n * 1e-3) / 1e9}


MERGE_TRAFFIC_MD = "traffic_lse_merge_kernel_rows524288_d128.md"


def merge_rotating(ca, torch, rows=131072, d=128, sets=3, reps=30):
    """The merge at basic_s4096's per-step shape (131072 rows x 128, 193.5 MiB
    per call, which alone would fit in the 256 MB MALL), cycling through three
    buffer sets so that a call does not find its operands cached by the last."""
    B, H = 1, 32
    S = rows // H
    bufs = [(torch.randn(B, S, H, d, device="cuda"), torch.randn(B, H, S, device="cuda"),
             torch.randn(B, S, H, d, device="cuda"), torch.randn(B, H, S, device="cuda"))
            for _ in range(sets)]
    for i in range(sets):
        ca.ring_attn_lse_merge(bufs[i][0], bufs[i][1], bufs[i][2], bufs[i][3])
    torch.cuda.synchronize()
    ca.ring_attn_timing_enable(False)
    ca.ring_attn_timing_enable(True)
    for i in range(reps):
        o, l, oj, lj = bufs[i % sets]
        ca.ring_attn_lse_merge(o, l, oj, lj)
    n, ms = ca.ring_attn_timing_read("lse_merge")
    ca.ring_attn_timing_enable(False)
    nbytes = (12 * d + 12) * rows
    gbs = nbytes / (ms / n * 1e-3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return {"rows": rows, "head_dim": d, "buffer_sets": sets, "bytes_per_launch": nbytes,
            "avg_ms": ms / n, "GB/s": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS}


class MfmaProbe:
    """libraprobe.so's MFMA-only kernels (two work-groups of four waves per
    CU, 4.4 bf16 TFLOP per launch), on nearly constant operands or (random)
    on operands with the bit statistics of N(0,1) data."""

    def __init__(self, torch, random_operands):
        import ctypes
        path = os.path.join(ROOT, "context_attention_flash_amd", "libraprobe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with python -c 'import __graft_entry__ as g; g.build()'")
        probe = ctypes.CDLL(path)
        probe.ra_probe_mfma_flops.restype = ctypes.c_double
        probe.ra_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
        self.fn = probe.ra_probe_mfma_random if random_operands else probe.ra_probe_mfma
        self.fn.restype = ctypes.c_int
        self.fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        self.torch, self.ctypes = torch, ctypes
        self.blocks, self.iters = 512, 16384
        self.flops = probe.ra_probe_mfma_flops(self.blocks, self.iters)
        self.out = torch.empty(self.blocks * 256, device="cuda")
        self.stream = torch.cuda.current_stream()

    def launch(self, n=1):
        for _ in range(n):
            rc = self.fn(self.out.data_ptr(), self.blocks, self.iters,
                         self.ctypes.c_void_p(self.stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"MFMA probe failed ({rc})")

    def timed(self, n):
        ev0, ev1 = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
        ev0.record(self.stream)
        self.launch(n)
        ev1.record(self.stream)
        self.torch.cuda.synchronize()
        assert self.torch.isfinite(self.out).all().item()
        return self.flops * n / (ev0.elapsed_time(ev1) * 1e-3) / 1e12

    def sustained(self, seconds=2.0):
        """Launches queued back to back for `seconds`, the rate of the last
        half: the steady state at the clock the chip holds under this load, as
        the attention kernels run in the timed steps (a 10-launch burst
        measures the same)."""
        rates, t0 = [], time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            rates.append(self.timed(25))
        return statistics.mean(rates[len(rates) // 2:])


def measured_peaks(torch):
    """What this GPU delivers in isolation, beside the spec peaks: bf16 MFMAs
    alone (MfmaProbe), on nearly constant operands and on operands with the
    bit statistics of N(0,1) data (on which the chip holds a lower clock),
    queued back to back for two seconds as the attention kernels run in the
    timed steps; and streaming over 1 GiB per operand, bytes read + written:
    torch's copy kernel, and libraprobe.so's streaming copy (one byte read per
    byte written), streaming add (two read per byte written, the LSE merge's
    ratio) and read-only fold, each the best over grid sizes and cache
    policies."""
    import ctypes
    path = os.path.join(ROOT, "context_attention_flash_amd", "libraprobe.so")
    probe = ctypes.CDLL(path)
    mfma = {}
    for random_operands in (False, True):
        pr = MfmaProbe(torch, random_operands)
        mfma[random_operands] = pr.sustained()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    x = torch.empty(1 << 28, device="cuda")   # 1 GiB of fp32
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    ev0.record(stream)
    for _ in range(reps):
        y.copy_(x)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * x.numel() * 4 * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    probe.ra_probe_stream.restype = ctypes.c_int
    probe.ra_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    nbytes = x.numel() * 4
    z = torch.empty_like(x)
    best = {}
    for kind, b_ptr, moved in (("copy", None, 2 * nbytes), ("add", z.data_ptr(), 3 * nbytes)):
        best[kind] = (0.0, 0, 0)
        for flags in range(4):
            for blocks in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
                def run():
                    rc = probe.ra_probe_stream(x.data_ptr(), b_ptr, y.data_ptr(), nbytes, blocks, flags,
                                               ctypes.c_void_p(stream.cuda_stream))
                    if rc != 0:
                        raise RuntimeError(f"ra_probe_stream failed ({rc})")
                for _ in range(3):
                    run()
                ev0.record(stream)
                for _ in range(reps):
                    run()
                ev1.record(stream)
                torch.cuda.synchronize()
                gbs = moved * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
                best[kind] = max(best[kind], (gbs, blocks, flags))
    probe.ra_probe_stream_read.restype = ctypes.c_int
    probe.ra_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    sink = torch.empty(32768 * 256, dtype=torch.int32, device="cuda")
    best["read"] = (0.0, 0, 0)
    for flags in range(2):
        for blocks in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
            def run():
                rc = probe.ra_probe_stream_read(x.data_ptr(), sink.data_ptr(), nbytes, blocks, flags,
                                                ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"ra_probe_stream_read failed ({rc})")
            for _ in range(3):
                run()
            ev0.record(stream)
            for _ in range(reps):
                run()
            ev1.record(stream)
            torch.cuda.synchronize()
            gbs = nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
            best["read"] = max(best["read"], (gbs, blocks, flags))
    del z, sink
    del x, y
    torch.cuda.empty_cache()
    return {"mfma_only_bf16_TFLOP/s": mfma[False], "mfma_only_frac_of_spec": mfma[False] / PEAK_BF16_TFLOPS,
            "mfma_only_bf16_random_operands_TFLOP/s": mfma[True],
            "mfma_only_random_operands_frac_of_spec": mfma[True] / PEAK_BF16_TFLOPS,
            "copy_GB/s": copy_gbs, "copy_frac_of_spec": copy_gbs / PEAK_HBM_GBS,
            "stream_copy_GB/s": best["copy"][0], "stream_copy_frac_of_spec": best["copy"][0] / PEAK_HBM_GBS,
            "stream_add_GB/s": best["add"][0], "stream_add_frac_of_spec": best["add"][0] / PEAK_HBM_GBS,
            "stream_read_GB/s": best["read"][0], "stream_read_frac_of_spec": best["read"][0] / PEAK_HBM_GBS,
            "stream_best_config": {k: {"blocks": v[1], "nt_loads": bool(v[2] & 1),
                                       "nt_stores": bool(v[2] & 2)} for k, v in best.items()},
            "spec": {"bf16_TFLOP/s": PEAK_BF16_TFLOPS, "hbm_GB/s": PEAK_HBM_GBS}}


def plan_cost(ca, torch, desc, w, call):
    """Time of the first call for a shape (plan built on the host and uploaded,
    then the kernels) against the same call once the plan is cached."""
    ca.ring_attn_clear_cache()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call()
    torch.cuda.synchronize()
    first = time.perf_counter() - t0
    t0 = time.perf_counter()
    call()
    torch.cuda.synchronize()
    cached = time.perf_counter() - t0
    return {"first_call_ms": first * 1e3, "cached_call_ms": cached * 1e3,
            "plan_ms": (first - cached) * 1e3}


# Forward-only configurations timed in the same run as the headline step (their
# parity is covered by the tests; here they are timed on seeded N(0,1) inputs
# drawn on the device, which have the same distribution as the tests' inputs).
OTHER_FWD = ("basic_s4096", "zigzag", "llama3")


def time_forward(ca, torch, synth, name, steps, warmup):
    w = synth.WORKLOADS[name]
    desc = ca.desc_from_workload(w)
    S, Skv, nb = ca.shard_sizes(desc)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    dt = torch.bfloat16
    q = torch.randn(w.batch, S, w.heads_q, w.head_dim, device="cuda", generator=gen).to(dt)
    k = torch.randn(nb, w.batch, Skv, w.heads_kv, w.head_dim, device="cuda", generator=gen).to(dt)
    v = torch.randn(nb, w.batch, Skv, w.heads_kv, w.head_dim, device="cuda", generator=gen).to(dt)
    out = torch.empty_like(q)
    lse = torch.empty(w.batch, w.heads_q, S, device="cuda")
    ws = ca.alloc_workspace(desc, False)
    pairs = sum(p for _, _, p in ca.ring_attn_schedule(desc, w.cu_seqlens))
    flops = 4.0 * w.head_dim * w.heads_q * w.batch * pairs
    plan = plan_cost(ca, torch, desc, w, lambda: ca.ring_attn_fwd(desc, q, k, v, w.cu_seqlens, out, lse, ws))
    for _ in range(warmup):
        ca.ring_attn_fwd(desc, q, k, v, w.cu_seqlens, out, lse, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ca.ring_attn_fwd(desc, q, k, v, w.cu_seqlens, out, lse, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    assert torch.isfinite(out.float()).all().item(), f"{name}: non-finite output"
    tf = flops / (ms * 1e-3) / 1e12
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    return {"workload": f"{name}: {synth.LAYOUT_NAMES[w.layout]} causal fwd rank share, "
                        f"N {w.seqlen}, D {w.world}, rank {w.rank}, {w.heads_q}/{w.heads_kv} heads, "
                        f"d {w.head_dim}", "fwd_tflop": flops / 1e12, "ms": ms, "TFLOP/s": tf,
            "frac_peak": tf / PEAK_BF16_TFLOPS, "steps": steps,
            "plan": plan}


# Algorithmic flops per visible (query, key) pair and query head, per kernel.
# The backward's 10*d splits into S, dP, dV, dK (the dK/dV kernel, 8*d) and dQ
# (2*d); the dQ kernel also recomputes S and dP, which count as issued work
# only.
ALGO_FLOPS_PER_PAIR = {"fwd_step": 4, "bwd_step": 8, "bwd_dq": 2, "bwd_dq_ds": 2}
ISSUED_FLOPS_PER_PAIR = {"fwd_step": 4, "bwd_step": 8, "bwd_dq": 6, "bwd_dq_ds": 2}
ROCPROF_NAME = {"fwd_step": "fwd_step_bf16_kernel", "bwd_step": "bwd_dkdv_bf16_kernel",
                "bwd_dq": "bwd_dq_bf16_kernel", "bwd_dq_ds": "bwd_dq_ds_bf16_kernel"}


def dkdv_bytes_per_launch(ca, desc, w, sched, ds_store: bool) -> float:
    """HBM bytes one dK/dV launch must move, averaged over the step's launches:
    Q and dO read (bf16), K_j and V_j read (bf16), dK_j and dV_j read and
    written (fp32), and with the dS store its 16 KiB bf16 tiles (one per
    non-empty 64-row x 128-key tile and q head)."""
    S, Skv = w.seqlen // w.world, ca.shard_sizes(desc)[1]
    active = [(s, p) for s, _, p in sched if p > 0]
    per = (2 * 2 * w.batch * S * w.heads_q * w.head_dim
           + 2 * 2 * w.batch * Skv * w.heads_kv * w.head_dim
           + 2 * 2 * 4 * w.batch * Skv * w.heads_kv * w.head_dim)
    ds = 0.0
    if ds_store:
        for s, _ in active:
            tiles = int((ca.ring_attn_tile_kinds(desc, w.cu_seqlens, s, 64, 128) > 0).sum())
            ds += w.batch * w.heads_q * tiles * 64 * 128 * 2
    return per + ds / max(1, len(active))


def calibrate_copy(torch, nbytes=256 << 20, reps=5):
    """A plain copy kernel of known size for scaling the FETCH_SIZE / WRITE_SIZE
    counters: each dispatch reads nbytes and writes nbytes."""
    x = torch.randn(nbytes // 4, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "elementwise mul by 1.0", "bytes_read_per_dispatch": nbytes,
                      "bytes_written_per_dispatch": nbytes, "dispatches": reps}), flush=True)


def sustain(ca, torch, args, desc, w, t, out, lse, ws_f, ws_b, grads):
    """Run one pass of the workload back to back for args.seconds, so that the
    GPU's power draw and clocks can be read while it holds a steady load."""
    def one():
        if args.sustain in ("fwd", "step"):
            ca.ring_attn_fwd(desc, t["q"], t["k"], t["v"], w.cu_seqlens, out, lse, ws_f)
        if args.sustain in ("bwd", "step"):
            ca.ring_attn_bwd(desc, t["dout"], t["q"], t["k"], t["v"], out, lse, w.cu_seqlens,
                             *grads, ws_b)
    ca.ring_attn_fwd(desc, t["q"], t["k"], t["v"], w.cu_seqlens, out, lse, ws_f)
    torch.cuda.synchronize()
    log(f"sustain {args.sustain} for {args.seconds} s")
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.seconds:
        for _ in range(4):
            one()
        n += 4
        torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(json.dumps({"sustain": args.sustain, "workload": w.name, "calls": n,
                      "ms_per_call": elapsed / n * 1e3, "seconds": elapsed}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="basic_s8192")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-merge", action="store_true")
    ap.add_argument("--with-grad", action="store_true",
                    help="also time the backward on a workload defined forward-only")
    ap.add_argument("--no-ds-store", action="store_true",
                    help="give the backward no room for the dS tile store (dQ recomputes S, dP)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the copy kernel used to scale the traffic counters")
    ap.add_argument("--merge-only", action="store_true",
                    help="only run the standalone LSE merge measurement")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the forward timing of the other bf16 configurations")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the forward alone (drop the backward of the workload)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the MFMA-only and copy-bandwidth measurements")
    ap.add_argument("--peaks-only", action="store_true",
                    help="only run the MFMA-only and copy-bandwidth measurements")
    ap.add_argument("--sustain", choices=("fwd", "bwd", "step", "mfma", "mfma_random"),
                    help="only run that pass of the workload (or the MFMA-only kernel, on "
                         "nearly constant or on N(0,1)-like operands) back to back for "
                         "--seconds (a steady load for reading power and clocks from outside)")
    ap.add_argument("--seconds", type=float, default=20.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one rank's share on ONE GPU; this library has no multi-GPU "
              "path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    from context_attention_flash_amd import synth
    w = synth.WORKLOADS[args.workload]
    if args.with_grad:
        w = w.replace(with_grad=True)
    if args.fwd_only:
        w = w.replace(with_grad=False)
    if args.sustain in ("fwd", "bwd", "step"):
        w = w.replace(with_grad=args.sustain != "fwd")
    pool = None
    if not (args.no_cpu_baseline or args.calibrate_copy or args.merge_only or args.sustain
            or args.peaks_only):
        pool, workers = start_host_pool(w)   # before any GPU call

    import torch
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    import context_attention_flash_amd as ca
    from context_attention_flash_amd import profsum
    if args.merge_only:
        torch.cuda.set_device(0)
        print(json.dumps({"merge": merge_bandwidth(ca, torch)}), flush=True)
        return
    if args.sustain in ("mfma", "mfma_random"):
        torch.cuda.set_device(0)
        pr = MfmaProbe(torch, args.sustain == "mfma_random")
        log(f"sustain {args.sustain} for {args.seconds} s")
        rates, t0 = [], time.perf_counter()
        while time.perf_counter() - t0 < args.seconds:
            rates.append(pr.timed(25))
        print(json.dumps({"sustain": args.sustain, "launches": 25 * len(rates),
                          "TFLOP/s": statistics.mean(rates[len(rates) // 2:]),
                          "seconds": time.perf_counter() - t0}), flush=True)
        return
    if args.peaks_only:
        torch.cuda.set_device(0)
        print(json.dumps({"measured_peaks": measured_peaks(torch)}), flush=True)
        return

    torch.cuda.set_device(0)
    g, desc, t = build_inputs(ca, w, torch)
    sched = ca.ring_attn_schedule(desc, w.cu_seqlens)
    pairs = sum(p for _, _, p in sched)
    heads_b = w.heads_q * w.batch
    fwd_flops = 4.0 * w.head_dim * heads_b * pairs
    bwd_flops = 10.0 * w.head_dim * heads_b * pairs if w.with_grad else 0.0

    ws_f = ca.alloc_workspace(desc, False)
    out = torch.empty_like(t["q"])
    lse = torch.empty(w.batch, w.heads_q, w.seqlen // w.world, device="cuda")
    if w.with_grad:
        ws_b = ca.alloc_workspace(desc, True, cu_seqlens=w.cu_seqlens, ds_store=not args.no_ds_store)
        dq = torch.empty(t["q"].shape, dtype=torch.float32, device="cuda")
        dk = torch.zeros(t["k"].shape, dtype=torch.float32, device="cuda")
        dv = torch.zeros(t["v"].shape, dtype=torch.float32, device="cuda")

    def step():
        ca.ring_attn_fwd(desc, t["q"], t["k"], t["v"], w.cu_seqlens, out, lse, ws_f)
        if w.with_grad:
            ca.ring_attn_bwd(desc, t["dout"], t["q"], t["k"], t["v"], out, lse, w.cu_seqlens,
                             dq, dk, dv, ws_b)

    if args.sustain:
        sustain(ca, torch, args, desc, w, t, out, lse, ws_f, ws_b if w.with_grad else None,
                (dq, dk, dv) if w.with_grad else None)
        return

    plan = plan_cost(ca, torch, desc, w, step)
    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # timed region: K steps; per-kernel HIP events on the launching stream
    ca.ring_attn_timing_enable(False)
    ca.ring_attn_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern = {}
    for name in ("fwd_step", "bwd_pre", "bwd_step", "bwd_dq", "bwd_dq_ds", "bwd_post", "lse_merge",
                 "finalize"):
        n, ms = ca.ring_attn_timing_read(name)
        if n:
            kern[name] = {"launches": n // args.steps, "ms_per_step": ms / args.steps,
                          "avg_launch_ms": ms / n}
    ca.ring_attn_timing_enable(False)
    log(f"timed {args.steps} steps in {elapsed:.3f}s")
    assert torch.isfinite(out.float()).all().item(), "non-finite output"

    ms_step = elapsed / args.steps * 1e3
    total_flops = fwd_flops + bwd_flops
    value = total_flops / (ms_step * 1e-3) / 1e12
    flops_unit = w.head_dim * heads_b * pairs   # d * Hq * B * pairs
    issued_md = os.path.join(ROOT, "profiles", f"mfma_issued_{w.name}.md")
    for name, k in kern.items():
        if name in ALGO_FLOPS_PER_PAIR:
            k["algorithmic_TFLOP/s"] = ALGO_FLOPS_PER_PAIR[name] * flops_unit / (k["ms_per_step"] * 1e-3) / 1e12
            # issued: the bf16 MFMA flops the hardware counted per launch (whole
            # tiles, masked elements included) when a summary for the current
            # sources exists, else the per-pair count of the kernel's products
            issued = profsum.read_issued(issued_md, ROCPROF_NAME[name])
            if issued is not None:
                k["issued_TFLOP/s"] = issued / (k["avg_launch_ms"] * 1e-3) / 1e12
                k["issued_from"] = "SQ_INSTS_VALU_MFMA_MOPS_BF16"
            else:
                k["issued_TFLOP/s"] = ISSUED_FLOPS_PER_PAIR[name] * flops_unit / (k["ms_per_step"] * 1e-3) / 1e12
                k["issued_from"] = "products per visible pair"

    # roofline of the dominant kernel (most time per step): algorithmic flops
    # per launch (per-pair figure x the visible pairs of one launch, averaged
    # over the step's launches) over its average launch duration
    dom = max((n for n in kern if n in ALGO_FLOPS_PER_PAIR), key=lambda n: kern[n]["ms_per_step"])
    n_launch = kern[dom]["launches"]
    flops_per_launch = ALGO_FLOPS_PER_PAIR[dom] * flops_unit / n_launch
    achieved = flops_per_launch / (kern[dom]["avg_launch_ms"] * 1e-3) / 1e12
    traffic = profsum.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{ROCPROF_NAME[dom]}_{w.name}.md"),
                                   ROCPROF_NAME[dom])
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": ROCPROF_NAME[dom],
                "flops_per_launch": flops_per_launch, "avg_launch_ms": kern[dom]["avg_launch_ms"],
                "launches_per_step": n_launch}
    if dom == "bwd_step":
        roofline["algorithmic_bytes_per_launch"] = dkdv_bytes_per_launch(ca, desc, w, sched,
                                                                         "bwd_dq_ds" in kern)

    res = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1), bf16-rounded)",
        "config": {"workload": f"{w.name}: {synth.LAYOUT_NAMES[w.layout]} "
                               f"{'causal' if w.causal else 'non-causal'} "
                               f"{'fwd+bwd' if w.with_grad else 'fwd'} rank share",
                   "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "head_dim": w.head_dim, "global_seqlen": w.seqlen, "world": w.world,
                   "rank": w.rank, "shard_rows": w.seqlen // w.world,
                   "visible_pairs_per_head": pairs, "fwd_tflop": fwd_flops / 1e12,
                   "bwd_tflop": bwd_flops / 1e12},
        "roofline": roofline,
        "kernels": kern,
        "plan": plan,
        "mfma_frac_whole_step": value / PEAK_BF16_TFLOPS,
    }
    if not args.no_merge:
        res["merge"] = merge_bandwidth(ca, torch)
        res["merge"]["rotating_basic_s4096_shape"] = merge_rotating(ca, torch)
    if not args.no_other and args.workload == "basic_s8192":
        del t, out, lse
        if w.with_grad:
            del ws_b, dq, dk, dv
        torch.cuda.empty_cache()
        res["other_workloads"] = {}
        for name in OTHER_FWD:
            log(f"forward of {name} ...")
            res["other_workloads"][name] = time_forward(ca, torch, synth, name, 10, 3)
    if not args.no_peaks:
        log("measuring the MFMA-only and copy peaks ...")
        res["measured_peaks"] = measured_peaks(torch)
    if pool is not None:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(w, g, args.cpu_budget, pool, workers)
        pool.close()
        pool.join()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
