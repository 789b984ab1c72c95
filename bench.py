#!/usr/bin/env python3
"""Benchmark: batch-1 rotated W4A16 dequant GEMV on one MI355X.

One step = one pass of the hot path over one batch: the seven projections
of a 4B-class decoder block (q 2560->4096, k/v 2560->1024, o 4096->2560,
gate/up 2560->9728, down 9728->2560), int4 codes with fp16 scale and zero
per group of 128 along K, block-128 random Hadamard rotation of the
activations fused into the product, M = 1, fp16 outputs.  The seven
linears have independent inputs, so one step is a single grouped launch.

Weights are cold: a rotating pool of distinct weight copies (>= 1 GB, well
above the 256 MB Infinity Cache) is cycled, one copy per step.  The timed
region is K steps replayed from a HIP graph (so the host launch path stays
out of it) on one stream, bracketed by HIP events on that stream with a
synchronisation on both sides; after untimed replays for at least
WARMUP_MS of GPU time, whatever K is (graph upload, and the clocks
settling: the first replays after idle run up to ~15% slower), it is
replayed TIMED_REPLAYS times and the median taken.  At M = 1 a step is
exactly one launch of the GEMV, so the region gives its duration per
launch, and the roofline figure is algorithmic bytes per launch over it.
The same K steps launched eagerly (with the host's time to issue one) are
printed beside it.

The read ceiling of the same run: a plain streaming read of the step's
algorithmic bytes (wq_stream_read, cold: a 1 GB pool cycled), K reads in a
graph timed the same way, so that the line separates a slower host from a
slower kernel (frac_of_read_ceiling = ceiling time / step time).

Prints one JSON line on stdout; details go to stderr.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload block_int4] [--m 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "batch-1 RHT+W4A16 dequant GEMV: µs/linear and achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
POOL_BYTES = 1 << 30
WARMUP_MS = 50.0      # untimed GPU work before any timed replay
TIMED_REPLAYS = 7
COUNTERS = os.path.join(ROOT, "profiles", "gemv_traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_per_weight(bits: int) -> float:
    # packed codes plus one fp16 scale and one fp16 zero per 128 weights
    return bits / 8.0 + 4.0 / 128.0


def algorithmic_bytes(lins, m: int) -> int:
    """What the method itself must move for one pass: codes + scales + zeros,
    activations in, outputs out, rotation signs."""
    total = 0
    for lin in lins:
        total += int(lin.n * lin.k * bytes_per_weight(lin.bits))
        total += 2 * m * lin.k                      # fp16 activations
        total += (4 if lin.out_f32 else 2) * m * lin.n
        total += lin.k // 8 if lin.rht else 0        # sign bits
    return total


def linear_bytes(lin, m: int, sel=None) -> int:
    """Algorithmic bytes of one linear at batch m.  Mixed width (bits 0): the
    64-row blocks' codes at their own widths plus the per-block selectors."""
    if lin.bits:
        w = int(lin.n * lin.k * bytes_per_weight(lin.bits))
    else:
        w = int(sum(64 * lin.k * int(b) // 8 for b in sel)) + lin.n * lin.k // 32 + len(sel)
    w += 2 * m * lin.k + (4 if lin.out_f32 else 2) * m * lin.n
    return w + (lin.k // 8 if lin.rht else 0)


def source_digest() -> str:
    """Digest of the sources that decide the measured kernel and its launch."""
    h = hashlib.sha256()
    for f in ("gemv_stream.hip", "gemv.hip", "wq_internal.h", "api.cpp"):
        with open(os.path.join(ROOT, "dequant_gemv_rht_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def calibrate_copy(nbytes: int, reps: int) -> None:
    """A plain device copy of known size (read nbytes, write nbytes), for
    scaling the FETCH_SIZE / WRITE_SIZE counters of a profiled run."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "reps": reps}),
          flush=True)


PEAK_MFMA_F16_TFLOPS = 2500.0


def kernel_name(bits: int, m: int) -> str:
    """The kernel one step launches (the planner's choice for these shapes)."""
    if m >= 17:
        mb, nb = (1, 1) if m <= 32 else (2, 1) if m <= 64 else (4, 2)
        return (f"gemm_kernel<{bits}, {mb}, {nb}> (matrix cores, all linears in one launch), after "
                f"rht_batch_kernel (and gemm_finalize_kernel where K is split)")
    if m == 1:
        return f"gemv_ring_kernel<{bits}, true> (LDS-ring weight stream)"
    tile = 2 if m == 2 else 4 if m <= 4 else 8 if m <= 12 else 16
    return (f"gemv_quad_kernel<{bits}, {tile}> (row quads, register prefetch; batch tiles of up to {tile} rows "
            f"where they fit in LDS in up to 4 chunks of K, else smaller), "
            f"after xprep_kernel<{bits}> (activations rotated and arranged once)")


def cpu_baseline(wl, lins, m, budget_s: float):
    """The fp64 oracle (explicit rotation, scalar dequant, C triple loop) timed on
    this host over whole steps of the same workload, until ~budget_s of work."""
    from oracle import linear as OL
    from oracle import rtn as OR
    prepared = []
    for i, lin in enumerate(lins):
        w, x, signs, _ = W.linear_inputs(0, wl.wid, i, lin, m)
        q, s, z = OR.prepare(w, signs, lin.bits)
        prepared.append((q, s, z, x, signs))
        del w
    threads = OL.default_threads()
    steps = 0
    t0 = time.perf_counter()
    while True:
        for (q, s, z, x, signs) in prepared:
            OL.linear(q, s, z, x, signs, threads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_step = el / steps
    nbytes = algorithmic_bytes(lins, m)
    return {"value": round(nbytes / per_step / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} full step(s) of the same workload ({len(lins)} linears, M={m}); "
                      f"{per_step * 1e3:.1f} ms per step, {per_step * 1e6 / len(lins):.0f} us per linear; "
                      f"rotation + dequant + fp64 triple loop, excluding quantisation"}


def _pool_views(t, copies: int):
    """``copies`` distinct copies of ``t`` in one allocation, each starting on a
    256-byte boundary (views keep the dtype and shape)."""
    import torch
    nbytes = t.numel() * t.element_size()
    stride = (nbytes + 255) // 256 * 256 // t.element_size()
    buf = torch.empty(copies * stride, dtype=t.dtype, device=t.device)
    out = []
    for i in range(copies):
        v = buf[i * stride:i * stride + t.numel()].view(t.shape)
        v.copy_(t)
        out.append(v)
    return out


def _time_launches(fns, stream, min_launches: int = 200, replays: int = 3) -> float:
    """Mean µs per launch over a graph of back-to-back launches cycling through
    ``fns`` (each call launches once on ``stream``); median over replays,
    after untimed replays that let the clocks settle."""
    import torch
    k = max(min_launches, len(fns))
    sptr = stream.cuda_stream
    with torch.cuda.stream(stream):
        for i in range(min(len(fns), 64)):
            fns[i](sptr)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(k):
            fns[i % len(fns)](sptr)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    times = []
    warm_graph(g, stream)
    with torch.cuda.stream(stream):
        for _ in range(replays):
            t0.record(stream)
            g.replay()
            t1.record(stream)
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1) * 1e3 / k)
    del g
    return float(np.median(times))


def warm_graph(g, stream, ms: float = WARMUP_MS) -> int:
    """Untimed replays of ``g`` on ``stream`` until at least ``ms`` of GPU
    time has passed (the first replay, which uploads the graph, included);
    returns the number of replays."""
    import torch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    done, spent = 0, 0.0
    with torch.cuda.stream(stream):
        while spent < ms:
            batch = 1 if done == 0 else max(1, min(1000, math.ceil((ms - spent) / max(spent / done, 1e-3))))
            t0.record(stream)
            for _ in range(batch):
                g.replay()
            t1.record(stream)
            torch.cuda.synchronize()
            spent += t0.elapsed_time(t1)
            done += batch
    return done


class _ReadCeiling:
    """The plain streaming-read kernel over cold data of a given size."""

    def __init__(self, pool_bytes: int):
        import torch
        self.buf = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda").fill_(7)
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def us(self, nbytes: int, stream, launches: int = 200, replays: int = 3) -> float:
        import dequant_gemv_rht_amd as dq
        nb = (nbytes + 15) // 16 * 16
        stride = (nb + 255) // 256 * 256
        copies = self.buf.numel() // stride
        if copies < 2:
            raise ValueError(f"read ceiling: {nbytes} bytes need a pool of at least {2 * stride} bytes")
        copies = min(copies, 4096)   # one graph node per copy: keep the graph small
        lib, base, sink = dq.lib(), self.buf.data_ptr(), self.sink.data_ptr()

        def one(i):
            off = base + (i % copies) * stride
            return lambda sp: dq._check("wq_stream_read", lib.wq_stream_read(off, nb, sink, sp))
        return _time_launches([one(i) for i in range(copies)], stream, launches, replays)


def _oracle_ms(w_rows, x, signs, bits_rows, lin, threads: int) -> float:
    """The oracle's time for the whole linear, from a row sample: the activation
    rotation once, plus dequantise-and-contract of the sampled rows scaled to
    all N rows (rows are independent and cost the same)."""
    from oracle import linear as OL
    from oracle import rtn as OR
    q, s, z = OR.prepare(w_rows, signs, bits_rows)
    t0 = time.perf_counter()
    x64 = np.atleast_2d(x).astype(np.float64)
    xr = OL.rht(x64, signs) if (lin.rht and signs is not None) else x64
    t_rot = time.perf_counter() - t0
    reps, t_rows = 0, 0.0
    while t_rows < 0.2 or reps < 1:
        t1 = time.perf_counter()
        OL.contract(OL.dequant(q, s, z), xr, threads)
        t_rows += time.perf_counter() - t1
        reps += 1
    return (t_rot + t_rows / reps * lin.n / len(w_rows)) * 1e3


def sweep(args) -> None:
    """Per-config, per-linear and per-step table: µs, GB/s, fraction of 8 TB/s,
    fraction of the plain-read ceiling at the same size, TFLOP/s at M >= 64,
    and the oracle's CPU time for the same linear (row-sampled)."""
    import torch
    import dequant_gemv_rht_amd as dq

    stream = torch.cuda.Stream()
    ceiling = _ReadCeiling(args.pool_bytes)
    threads_all = len(os.sched_getaffinity(0))
    rows_out = []
    hdr = ("| config | linear | M | bits | K→N | alg. bytes | µs | GB/s | % of 8 TB/s | read ceiling µs "
           "| % of ceiling | TFLOP/s (% of 2.5 P) | oracle ms, 1 thread | oracle ms, "
           f"{threads_all} threads |")
    print(hdr, flush=True)
    print("|" + "---|" * (hdr.count("|") - 1), flush=True)
    rng = np.random.default_rng(5)

    def emit(cfg, name, m, bits, shape, nbytes, us, ceil_us, flops, o1, oa):
        gbs = nbytes / us / 1e3
        tf = f"{flops / us / 1e6:.1f} ({flops / us / 1e6 / PEAK_MFMA_F16_TFLOPS:.1%})" if flops else "–"
        f1 = f"{o1:.2f}" if o1 is not None else "–"
        fa = f"{oa:.2f}" if oa is not None else "–"
        line = (f"| {cfg} | {name} | {m} | {bits} | {shape} | {nbytes:,} | {us:.2f} | {gbs:.0f} | "
                f"{gbs / PEAK_HBM_GBS:.1%} | {ceil_us:.2f} | {ceil_us / us:.1%} | {tf} | {f1} | {fa} |")
        print(line, flush=True)
        rows_out.append(line)

    for cfg, wname in (("c1", "single_int4"), ("c2", "block_int4"), ("c3", "block_int3"),
                       ("c4", "block_int6_head_int8"), ("c5", "prefill_and_mixed")):
        wl = W.WORKLOADS[wname]
        if args.sweep_only and cfg not in args.sweep_only.split(","):
            continue
        for m in wl.ms:
            lins = [(i, l) for i, l in enumerate(wl.linears)]
            if cfg == "c5":   # part A is the projections at M=512, part B the mixed down_proj at M=1
                lins = [(i, l) for i, l in lins if (l.bits == 0) == (m == 1)]
            log(f"sweep {cfg} {wname} M={m}: {len(lins)} linear(s)")
            qws, xs, ys, hosts = [], [], [], []
            for i, lin in lins:
                w, x, signs, sel = W.linear_inputs(0, wl.wid, i, lin, m)
                sg = torch.from_numpy(signs.view(np.int32)).cuda() if signs is not None else None
                bb = torch.from_numpy(sel).cuda() if sel is not None else None
                qws.append(dq.quantize_weight(torch.from_numpy(w).cuda(), lin.bits, sg, bb))
                xs.append(torch.from_numpy(x).cuda())
                ys.append(torch.empty((m, lin.n), dtype=torch.float32 if lin.out_f32 else torch.float16,
                                      device="cuda"))
                rows = np.sort(rng.choice(lin.n, min(lin.n, args.cpu_rows if m < 64 else args.cpu_rows // 4),
                                          replace=False))
                bits_rows = np.repeat(sel, 64)[rows] if sel is not None else lin.bits
                hosts.append((w[rows].copy(), x, signs, bits_rows, sel))
                del w
            torch.cuda.synchronize()

            def pooled(ws_list, total_bytes):
                copies = max(2, math.ceil(args.pool_bytes / max(1, total_bytes)))
                views = [[] for _ in range(copies)]
                for q in ws_list:
                    cs = _pool_views(q.codes, copies)
                    ss = _pool_views(q.scales, copies)
                    zs = _pool_views(q.zeros, copies)
                    for c in range(copies):
                        views[c].append(dq.QWeight(q.bits, q.n, q.k, cs[c], ss[c], zs[c], q.signs,
                                                   q.block_bits, q.block_off))
                return views

            step_bytes, step_flops = 0, 0
            for j, (i, lin) in enumerate(lins):
                q = qws[j]
                nbytes = linear_bytes(lin, m, hosts[j][4])
                wbytes = q.codes.numel() * 4 + q.scales.numel() * 4
                pool = pooled([q], wbytes)
                wsz = dq.wq_linear_batch_workspace([q], m)
                ws = dq.new_workspace(wsz)
                calls = [dq.BatchCall(p, [xs[j]], [ys[j]], True, ws) for p in pool]
                us = _time_launches(calls, stream)
                del calls, pool
                ceil_us = ceiling.us(nbytes, stream)
                flops = 2 * m * lin.n * lin.k if m >= 64 else 0
                w_rows, x, signs, bits_rows, _ = hosts[j]
                o1 = oa = None
                if not args.no_cpu_baseline:
                    o1 = _oracle_ms(w_rows, x, signs, bits_rows, lin, 1)
                    oa = _oracle_ms(w_rows, x, signs, bits_rows, lin, threads_all)
                emit(cfg, lin.name, m, lin.bits or "6/8", f"{lin.k}→{lin.n}", nbytes, us, ceil_us, flops, o1, oa)
                step_bytes += nbytes
                step_flops += flops
            # the grouped step: all linears of one width in one call
            same = [j for j, (_, l) in enumerate(lins) if l.bits == lins[0][1].bits and l.bits and not l.out_f32]
            if len(same) > 1:
                sb = sum(linear_bytes(lins[j][1], m) for j in same)
                sf = sum(2 * m * lins[j][1].n * lins[j][1].k for j in same) if m >= 64 else 0
                sel_q = [qws[j] for j in same]
                pool = pooled(sel_q, sum(q.codes.numel() * 4 + q.scales.numel() * 4 for q in sel_q))
                ws = dq.new_workspace(dq.wq_linear_batch_workspace(sel_q, m))
                calls = [dq.BatchCall(p, [xs[j] for j in same], [ys[j] for j in same], True, ws) for p in pool]
                us = _time_launches(calls, stream)
                del calls, pool
                emit(cfg, f"**{len(same)} linears, one call**", m, lins[same[0]][1].bits, "all", sb, us,
                     ceiling.us(sb, stream), sf, None, None)
                _sweep_shared(cfg, wl, m, lins, same, qws, xs, pooled, stream, ceiling, emit, sb, sf)
            del qws, xs, ys, hosts
            torch.cuda.empty_cache()
    if not args.sweep_only or "f2" in args.sweep_only.split(","):
        _sweep_embed(stream, ceiling, emit)
    log(f"sweep done: {len(rows_out)} rows; host threads {threads_all}")


def _sweep_shared(cfg, wl, m, lins, same, qws, xs, pooled, stream, ceiling, emit, sb, sf) -> None:
    """The grouped call with the inputs a decoder block shares: k and v on
    q's activations, up on gate's, each quantised with its group's sign
    vector, so the call rotates (and arranges) four inputs instead of seven.
    Above one batch row only (at one row every workgroup rotates its own)."""
    import torch
    import dequant_gemv_rht_amd as dq
    lead = {"k_proj": "q_proj", "v_proj": "q_proj", "up_proj": "gate_proj"}
    names = [lins[j][1].name for j in same]
    if m < 2 or not all(n in names for n in list(lead) + list(lead.values())):
        return
    sq, sx, saved = [], [], 0
    for j in same:
        i, lin = lins[j]
        lj = same[names.index(lead.get(lin.name, lin.name))]
        if lj == j:
            sq.append(qws[j])
            sx.append(xs[j])
            continue
        w, _, _, _ = W.linear_inputs(0, wl.wid, i, lin, m)
        sq.append(dq.quantize_weight(torch.from_numpy(w).cuda(), lin.bits, qws[lj].signs))
        sx.append(xs[lj])
        saved += 2 * m * lin.k + lin.k // 8     # its activations and signs are the leader's
        del w
    pool = pooled(sq, sum(q.codes.numel() * 4 + q.scales.numel() * 4 for q in sq))
    ws = dq.new_workspace(dq.wq_linear_batch_workspace(sq, m))
    ys = [torch.empty((m, lins[j][1].n), dtype=torch.float16, device="cuda") for j in same]
    calls = [dq.BatchCall(p, sx, ys, True, ws) for p in pool]
    us = _time_launches(calls, stream)
    del calls, pool
    emit(cfg, f"**{len(same)} linears, one call, shared inputs**", m, lins[same[0]][1].bits, "all",
         sb - saved, us, ceiling.us(sb - saved, stream), sf, None, None)


def _sweep_embed(stream, ceiling, emit) -> None:
    """The head table of the int6 block config (151936 x 2560 int8, no
    rotation) as the tied token embedding: wq_embed of T token ids to fp16.
    Call c gathers ids perm[c T : (c + 1) T] of one random permutation of the
    table's rows (up to 1024 calls), so a graph replay touches every row at
    most once (T = 1 and 64: 1024 and 65536 rows, 2.6 and 170 MB, which may
    stay in the last-level cache)."""
    import ctypes
    import torch
    import dequant_gemv_rht_amd as dq
    from oracle import embed as OE
    from oracle import rtn as OR
    wl = W.WORKLOADS["block_int6_head_int8"]
    idx = len(wl.linears) - 1
    lin = wl.linears[idx]
    log(f"sweep f2 embedding gather: {lin.n} x {lin.k} int8 table")
    w, _, _, _ = W.linear_inputs(0, wl.wid, idx, lin, 1)
    qw = dq.quantize_weight(torch.from_numpy(w).cuda(), 8, None)
    rng = np.random.default_rng(21)
    sample = np.sort(rng.choice(lin.n, 512, replace=False))
    q, sc, z = OR.rtn(w[sample], 8)
    del w
    perm = torch.from_numpy(rng.permutation(lin.n).astype(np.int32)).cuda()
    st = qw.c_struct()
    lib = dq.lib()
    for T in (1, 64, 512):
        out = torch.empty((T, lin.k), dtype=torch.float16, device="cuda")
        ncalls = min(1024, lin.n // T)

        def one(c, T=T, out=out):
            ids = perm.data_ptr() + 4 * c * T
            return lambda sp: dq._check("wq_embed", lib.wq_embed(ctypes.byref(st), ids, T, out.data_ptr(),
                                                                 dq.WQ_F16, lin.k, sp))
        log(f"f2 T={T}: {ncalls} gathers in a graph")
        us = _time_launches([one(c) for c in range(ncalls)], stream)
        # codes, scales and zeros of T rows, the ids, the fp16 rows out
        nbytes = T * (lin.k + 4 * (lin.k // 128) + 4 + 2 * lin.k)
        log(f"f2 T={T}: read ceiling, oracle")
        ids = rng.integers(0, len(sample), T)
        t0 = time.perf_counter()
        reps = 0
        while reps < 3 or time.perf_counter() - t0 < 0.2:
            OE.embed(q, sc, z, ids)
            reps += 1
        o1 = (time.perf_counter() - t0) / reps * 1e3
        emit("f2", "embed_gather", T, 8, f"{lin.n}x{lin.k} table, {T} ids", nbytes, us,
             ceiling.us(nbytes, stream), 0, o1, None)
    del qw, perm
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="block_int4")
    ap.add_argument("--m", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pool-bytes", type=int, default=POOL_BYTES)
    ap.add_argument("--sweep", action="store_true",
                    help="print the per-config, per-linear table instead of the headline JSON line")
    ap.add_argument("--sweep-only", default="", help="comma-separated configs for --sweep (c1..c5; f2: the embedding gather)")
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="output rows the oracle computes per linear in --sweep (scaled to all rows)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (for counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X and has no "
              "multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import dequant_gemv_rht_amd as dq

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return
    dq.lib()  # fail loudly if the library is missing
    if args.sweep:
        sweep(args)
        return

    wl = W.WORKLOADS[args.workload]
    m = args.m
    lins = [l for l in wl.linears if l.bits != 0 and not l.out_f32]
    bits = lins[0].bits
    nbytes = algorithmic_bytes(lins, m)
    log(f"workload {wl.name}: {len(lins)} linears, M={m}, {nbytes / 1e6:.3f} MB algorithmic per step")

    # ---- weights: generated on the host, prepared on the GPU (untimed)
    base, xs = [], []
    for i, lin in enumerate(lins):
        w, x, signs, _ = W.linear_inputs(0, wl.wid, i, lin, m)
        sg = torch.from_numpy(signs.view(np.int32)).cuda()
        base.append(dq.quantize_weight(torch.from_numpy(w).cuda(), lin.bits, sg))
        xs.append(torch.from_numpy(x).cuda())
        del w
    torch.cuda.synchronize()
    weight_bytes = sum(q.codes.numel() * 4 + q.scales.numel() * 4 for q in base)
    copies = max(2, math.ceil(args.pool_bytes / weight_bytes))
    pool = [base]
    for _ in range(copies - 1):
        pool.append([dq.QWeight(q.bits, q.n, q.k, q.codes.clone(), q.scales.clone(), q.zeros.clone(),
                                q.signs) for q in base])
    ys = [torch.empty((m, lin.n), dtype=torch.float16, device="cuda") for lin in lins]
    ws = dq.new_workspace(dq.wq_linear_batch_workspace(base, m))
    calls = [dq.BatchCall(p, xs, ys, True, ws) for p in pool]
    torch.cuda.synchronize()
    log(f"pool: {copies} copies x {weight_bytes / 1e6:.1f} MB = {copies * weight_bytes / 1e9:.2f} GB")

    stream = torch.cuda.Stream()
    sptr = stream.cuda_stream

    # ---- warmup, then the timed region: exactly K steps, eager and as a graph
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            calls[i % copies](sptr)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(args.steps):
            calls[i % copies](sptr)
    n_warm = warm_graph(graph, stream)   # graph upload, then the clocks settle

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        t0.record(stream)
        h0 = time.perf_counter()
        for i in range(args.steps):
            calls[i % copies](sptr)
        h1 = time.perf_counter()
        t1.record(stream)
    torch.cuda.synchronize()
    eager_ms_per_step = t0.elapsed_time(t1) / args.steps
    host_ms_per_step = (h1 - h0) * 1e3 / args.steps

    replays = []
    for _ in range(TIMED_REPLAYS):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            t0.record(stream)
            graph.replay()
            t1.record(stream)
        torch.cuda.synchronize()
        replays.append(t0.elapsed_time(t1) / args.steps)
    graph_ms_per_step = float(np.median(replays))
    ms_per_step = graph_ms_per_step
    timing = (f"HIP graph of the K steps, median of {TIMED_REPLAYS} replays after {n_warm} untimed replays "
              f"(>= {WARMUP_MS:.0f} ms of GPU time)")

    # ---- per-launch duration of the dominant kernel: at M = 1 a step is
    # exactly one launch of it, so the timed region gives it directly (events
    # recorded on the launch stream).  Single launches bracketed by events
    # are reported beside it for context.
    launch_ms = ms_per_step
    n_single = max(50, copies * 3)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_single)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_single)]
    with torch.cuda.stream(stream):
        for i in range(n_single):
            starts[i].record(stream)
            calls[i % copies](sptr)
            ends[i].record(stream)
    torch.cuda.synchronize()
    durs = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))

    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    flops = sum(2 * m * lin.n * lin.k for lin in lins)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    log(f"timed ({timing}): {ms_per_step * 1e3:.2f} us/step = {gbs:.0f} GB/s (replays "
        f"{', '.join(f'{r * 1e3:.2f}' for r in replays)}); eager {eager_ms_per_step * 1e3:.2f} "
        f"us/step (host {host_ms_per_step * 1e3:.2f} us to issue one); "
        f"single launch (events) mean {np.mean(durs) * 1e3:.2f} us, p10 {durs[len(durs) // 10] * 1e3:.2f}, "
        f"p90 {durs[9 * len(durs) // 10] * 1e3:.2f}")

    # the same run's read ceiling: a plain read of the step's bytes, timed the same way
    ceiling_us = _ReadCeiling(args.pool_bytes).us(nbytes, stream, launches=args.steps, replays=TIMED_REPLAYS)
    log(f"read ceiling (plain streaming read of {nbytes} bytes, cold, same protocol): {ceiling_us:.2f} us "
        f"= {nbytes / ceiling_us / 1e3:.0f} GB/s; the step runs at {ceiling_us / (ms_per_step * 1e3):.1%} of it")

    traffic = None
    digest = source_digest()
    if os.path.exists(COUNTERS):
        try:
            rec = json.load(open(COUNTERS))
            key = f"{wl.name}/m{m}"
            if rec.get("source_digest") == digest and key in rec.get("per_launch_bytes", {}):
                traffic = rec["per_launch_bytes"][key]["total"]
        except (OSError, ValueError):
            traffic = None

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": wl.title + f", M={m}",
            "m": m, "bits": bits, "group": 128, "linears": len(lins),
            "algorithmic_bytes_per_step": nbytes,
            "launch": "one grouped launch per step (7 independent linears), back to back on one stream from a HIP graph",
            "timing": timing,
            "weight_pool": f"{copies} copies, {copies * weight_bytes / 1e9:.2f} GB (cold weights)",
        },
        "us_per_linear": round(ms_per_step * 1e3 / len(lins), 4),
        "eager_us_per_step": round(eager_ms_per_step * 1e3, 3),
        "graph_us_per_step": round(graph_ms_per_step * 1e3, 3),
        "host_us_per_step": round(host_ms_per_step * 1e3, 3),
        "frac_of_peak_hbm": round(gbs / PEAK_HBM_GBS, 4),
        "read_ceiling_us_per_step": round(ceiling_us, 3),
        "read_ceiling_gbs": round(nbytes / ceiling_us / 1e3, 2),
        "frac_of_read_ceiling": round(ceiling_us / (ms_per_step * 1e3), 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        } if m < 64 else {
            # batch >= 64: a dense contraction on the matrix cores; one step is
            # the seven rotations and GEMMs, so this is per step, not per kernel
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
            "traffic": None,
            "flops_per_step": flops,
        },
        "kernel": {
            "name": kernel_name(bits, m),
            "us_per_step": round(launch_ms * 1e3, 3),
            "single_launch_us_mean": round(float(np.mean(durs)) * 1e3, 3),
            "bytes_per_step": nbytes,
            "source_digest": digest,
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle ...")
        result["cpu_baseline"] = cpu_baseline(wl, lins, m, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
