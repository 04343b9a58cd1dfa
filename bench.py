#!/usr/bin/env python3
"""Benchmark of the pooled-embedding training step on one MI355X.

A step is one pass of the whole path over one batch: pooled forward
(emb_forward_pooled), key dedup + segmented reduction (emb_backward_dedup /
emb_backward_unique_reduce) and the fused sparse Adagrad/SGD update
(emb_sparse_update). Inputs (tables, indices, offsets, upstream gradient) are
resident in HBM before timing starts. By default the steps are software-
pipelined: the next batch's dedup (which needs only its indices) runs on a
second stream, into a second workspace, while the current step's forward and
update run; K timed steps do exactly K dedups, forwards and updates.

Default workload: 26 fp32 tables x 4,000,000 rows x 128 (53 GB of weights +
53 GB of Adagrad state), batch 65536, one lookup per bag, Zipf(1.05) keys, sum
pooling, Adagrad lr 0.01 eps 1e-8. Seeded synthetic data; 4 different batches
are cycled so consecutive steps see different keys.

Prints ONE JSON line. `value` is lookups/s of the whole step; the forward and
backward+update phases are also reported with their algorithmic GB/s, the
dominant kernel against the 8 TB/s HBM roofline (per-kernel HIP events on the
launch stream, recorded by the library), and the CPU oracle on a bounded
sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "pooled lookups/sec + achieved HBM GB/s (fwd, bwd+update) on 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = the headline)")
    ap.add_argument("--batches", type=int, default=4)
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="samples per batch the oracle runs on (0 = the whole batch)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the oracle runs on successive cycled batches until this much CPU time is spent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--uniform-keys", action="store_true", help="control run: uniform keys instead of Zipf")
    ap.add_argument("--schedule", choices=["overlap", "serial", "pipeline"], default="pipeline",
                    help="overlap: the key dedup (emb_backward_dedup) runs on a second stream "
                         "concurrently with the forward; serial: one stream, dedup inside the backward; "
                         "pipeline: the dedup of the next batch runs on a second stream (with its own "
                         "workspace) alongside the current step's forward and update")
    ap.add_argument("--reduce", choices=["fused", "atomic"], default="fused",
                    help="fused: sorted-segment reduction fused with the optimizer (the path); atomic: the "
                         "evidence variant, fp32 atomics into a materialised gradient, then the update")
    ap.add_argument("--master", action="store_true",
                    help="bf16/fp16 tables trained from fp32 master weights (the update steps the master "
                         "and writes the master and its RNE copy in one pass)")
    ap.add_argument("--pack", type=int, default=0, metavar="S",
                    help="RB step for an S-shard layout instead of the local update: after the dedup, "
                         "emb_pack_by_shard routes the unique keys to their owners (cyclic rows) and "
                         "reduces their gradients straight into the send slots")
    ap.add_argument("--unique-forward", action="store_true",
                    help="unique-first forward: dedup first, gather each unique row once, pool from the "
                         "compact rows (emb_forward_pooled_unique); implies the serial schedule")
    ap.add_argument("--hashed", action="store_true",
                    help="lookups carry 64-bit ids: every step first translates them to rows through the "
                         "tables' hash maps (emb_hash_translate with insertion), then runs the step on the rows")
    ap.add_argument("--rows", type=int, default=0,
                    help="cap the rows of every table (0 = the workload's own sizes)")
    ap.add_argument("--single-schedule", action="store_true",
                    help="time only --schedule (no comparison schedule, no isolated-kernel pass), so a "
                         "profiler trace of the run holds that schedule's launches alone")
    ap.add_argument("--ceiling", action="store_true",
                    help="only time plain library kernels (copy, read-only sum, fill) over 4 GiB, and "
                         "random 512-byte row reads served by L2, MALL and HBM, and the fused update's "
                         "random row read/write mix: the practical ceilings "
                         "the path's kernels are compared with")
    ap.add_argument("--ahead", type=int, default=2, choices=[1, 2],
                    help="pipeline schedule: how many batches ahead the dedup runs (1: the next batch's "
                         "dedup runs beside the current forward and update; 2 (default): two batches "
                         "ahead, with a third workspace, so a dedup slowed by the main stream's kernels "
                         "has a second step to finish before its update needs it)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-configuration block (configs 1, 2, 4, 5 after the headline)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times) and exit: the reference "
                         "point for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def kernel_source_sha(name: str) -> str:
    p = os.path.join(ROOT, "dlrm_sparse_embedding_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_counters(kernel: str, workload_tag: str):
    """(HBM bytes per launch, L2 hit rate) from the committed rocprofv3
    counter summary of the kernel on this workload; None for either if there
    is no summary, it lacks the figure, or the kernel source changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_tag}_counters.md")
    if not os.path.exists(path):
        return None, None
    txt = open(path).read()
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    m_h = re.search(r"l2_hit_rate:\s*([0-9.]+)", txt)
    m_s = re.search(r"source_sha256_16:\s*([0-9a-f]+)", txt)
    m_f = re.search(r"source_file:\s*(\S+)", txt)
    if not (m_s and m_f) or kernel_source_sha(m_f.group(1)) != m_s.group(1):
        return None, None
    return (float(m_b.group(1)) if m_b else None), (float(m_h.group(1)) if m_h else None)


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this implementation is the single-GPU "
              "embedding path (one GPU's share of the tables); it runs on exactly one GPU and has no "
              "multi-GPU mode.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from dataclasses import replace

    if args.ceiling:
        n = (4 << 30) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        acc = torch.empty((), dtype=torch.float32, device="cuda")
        res = {}
        for name, nbytes, fn in (("copy", 2 * n * 4, lambda: dst.copy_(src)),
                                 ("read_sum", n * 4, lambda: torch.sum(src, dim=0, out=acc)),
                                 ("fill", n * 4, lambda: dst.fill_(1.0))):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[name + "_GBps"] = round(nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del src, dst
        # random 512-byte row reads (the library's probe kernel), the way the
        # multi-hot reduce reads dY rows: rows 51200 bytes apart (a 100-table,
        # 128-column fp32 dY), every XCD reading only its own eighth (an L2-
        # resident 2 MB each), or all XCDs the whole 16 MB (MALL-resident);
        # and rows packed over 2 GiB (HBM)
        from dlrm_sparse_embedding_amd import emb as E
        probe = torch.zeros(1 << 29, dtype=torch.float32, device="cuda")   # 2 GiB
        sink = torch.empty(E.emb_probe_blocks(), dtype=torch.float32, device="cuda")
        reads = 240
        logical = E.emb_probe_blocks() * 8 * reads * 512
        # and the same with 256-byte rows (a 128-column bf16 row, as the
        # 100-table forward reads them): 65536 packed rows (2 MB per eighth)
        for name, nrows, stride, local, rb in (("l2_xcd_local_rows", 32768, 51200, True, 512),
                                               ("mall_shared_rows", 32768, 51200, False, 512),
                                               ("hbm_random_rows", (1 << 31) // 512, 512, False, 512),
                                               ("l2_xcd_local_rows256", 65536, 256, True, 256),
                                               ("mall_shared_rows256", 65536, 256, False, 256),
                                               ("hbm_random_rows256", (1 << 31) // 256, 256, False, 256)):
            E.emb_probe_reads(probe, nrows, stride, local, reads, sink, row_bytes=rb)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                E.emb_probe_reads(probe, nrows, stride, local, reads, sink, row_bytes=rb)
            e1.record()
            torch.cuda.synchronize()
            res[name + "_GBps"] = round(logical * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del probe
        # the fused Adagrad update's mix at the 26 x 4M x 128 fp32 workload's
        # sizes: per item 2-3 random rows of a 65536 x 26-row dY, then one
        # random weight row and state row read and written (two 53 GB arrays),
        # 636 k items (the workload's unique rows per step)
        nsrc, nrows, items = 65536 * 26, 26 * 4_000_000, 636_000
        usrc = torch.zeros(nsrc * 128, dtype=torch.float32, device="cuda")
        ua = torch.zeros(nrows * 128, dtype=torch.float32, device="cuda")
        ub = torch.zeros(nrows * 128, dtype=torch.float32, device="cuda")
        E.emb_probe_update(usrc, nsrc, ua, ub, nrows, items)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            E.emb_probe_update(usrc, nsrc, ua, ub, nrows, items)
        e1.record()
        torch.cuda.synchronize()
        ub_ms = e0.elapsed_time(e1) / 20
        ubytes = E.emb_probe_update_bytes(items)
        res["update_rows_GBps"] = round(ubytes / (ub_ms * 1e-3) / 1e9, 1)
        res["update_rows_us"] = round(ub_ms * 1e3, 1)
        del usrc, ua, ub
        print(json.dumps({"ceiling": res, "bytes_per_buffer": n * 4, "probe_bytes_per_launch": logical,
                          "update_probe_bytes_per_launch": ubytes}), flush=True)
        return 0

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 5}), flush=True)
        return 0

    out = run_workload(args)
    if isinstance(out, int):
        return out
    per_config_ok = (args.config == 3 and not args.no_per_config and not args.single_schedule and
                     not (args.pack or args.hashed or args.unique_forward or args.master or args.uniform_keys or
                          args.rows or args.reduce != "fused"))
    if per_config_ok:
        # the other workloads, each alone on the GPU after the headline (tables
        # freed in between); fewer steps and a shorter oracle sample each
        import gc
        per = {}
        for c in (1, 2, 4, 5):
            sub = argparse.Namespace(**vars(args))
            sub.config = c
            sub.steps = min(args.steps, 10)
            sub.warmup = min(args.warmup, 3)
            sub.batches = 2 if c == 4 else min(args.batches, 4)
            sub.cpu_seconds = min(args.cpu_seconds, 3.0)
            sub.single_schedule = True          # the timed schedule only: no comparison or isolated pass
            gc.collect()
            torch.cuda.empty_cache()
            print(f"[bench] per-config: config {c}", file=sys.stderr, flush=True)
            per[f"cfg{c}"] = run_workload(sub, compact=True)
        out["per_config"] = per
    print(json.dumps(out), flush=True)
    return 0


def run_workload(args, compact=False):
    """Times one workload (args.config) and returns its JSON record (the
    headline's full record, or a compact one for the per-configuration
    block). The tables and buffers are freed before it returns."""
    import numpy as np
    import torch
    from dataclasses import replace

    from dlrm_sparse_embedding_amd import emb as E
    from dlrm_sparse_embedding_amd import workloads as W

    if args.schedule == "pipeline" and (args.pack or args.reduce != "fused" or args.hashed or args.unique_forward):
        # the variants run with the schedule given explicitly, else serial
        if "--schedule" in sys.argv:
            print("bench.py: --schedule pipeline runs the plain training step only", file=sys.stderr)
            return 2
        args.schedule = "serial"
    cfg = W.make_config(args.config, rows=args.rows or None)
    if args.master and cfg.dtype == "f32":
        print("bench.py: --master needs a bf16/fp16 workload (configs 4, 5)", file=sys.stderr)
        return 2
    if args.uniform_keys:
        cfg = replace(cfg, zipf_s=None)
    T, B, D = cfg.T, cfg.batch, cfg.dim
    elt = W.DTYPE_BYTES[cfg.dtype]
    rowbytes = D * elt

    torch.cuda.set_device(0)
    specs = [E.TableSpec(t.rows, t.dim, t.dtype, t.col_slices) for t in cfg.tables]
    tabs = E.EmbeddingTables(specs, with_state=cfg.opt == "adagrad", with_master=args.master)
    tabs.init_uniform(cfg.init_seed)
    print(f"[bench] tables ready: {T} x {cfg.tables[0].rows} x {D} {cfg.dtype}", file=sys.stderr, flush=True)

    host_batches = [W.make_batch(cfg, k=k) for k in range(args.batches)]
    dev = []
    for b in host_batches:
        dev.append((torch.from_numpy(b.indices).cuda(), torch.from_numpy(b.offsets).cuda(), b.N))
    if args.hashed:
        # ids: a fixed scramble of (table, row) over the whole int64 range; the
        # maps hand rows out by first appearance, so rows differ from the ids'
        # source rows but the step's work is the same
        ids_dev, rows_dev = [], []
        for b in host_batches:
            t_of = np.repeat(np.arange(T), np.diff(b.offsets[::B].astype(np.int64)))
            x = (b.indices.astype(np.uint64) * np.uint64(0x9E3779B97F4A7C15)) ^ (
                t_of.astype(np.uint64) * np.uint64(0xD1B54A32D192ED03))
            ids_dev.append(torch.from_numpy(x.view(np.int64)).cuda())
        tabs.hash_attach()
        hws = torch.empty(E.emb_hash_workspace_bytes(tabs.ctx, max(b.N for b in host_batches)),
                          dtype=torch.uint8, device="cuda")
        for k, b in enumerate(host_batches):
            rows_dev.append(torch.empty(b.N, dtype=dev[k][1].dtype, device="cuda"))
            E.emb_hash_translate(tabs.ctx, ids_dev[k], dev[k][1], B, True, hws, rows_dev[k])
        dev = [(rows_dev[k], dev[k][1], dev[k][2]) for k in range(len(dev))]
        torch.cuda.synchronize()
        tabs.check_device_error()
    dY_host = W.make_dy(cfg)
    dy = torch.from_numpy(dY_host).cuda()
    Y = torch.empty((B, T * D), dtype=torch.float32, device="cuda")
    nmax = max(b.N for b in host_batches)
    bufs = tabs.backward_buffers(nmax, B, with_grad=args.reduce == "atomic")
    rows_buf = tabs.unique_rows_buffer(nmax) if args.unique_forward else None
    pbufs = None
    if args.pack:
        tabs.set_shard_map([("row_cyclic", t % args.pack) for t in range(T)], args.pack)
        pbufs = tabs.pack_buffers(nmax, args.pack, with_grad=True)
    torch.cuda.synchronize()
    print(f"[bench] {len(dev)} batches on device, N = {[b.N for b in host_batches]}", file=sys.stderr, flush=True)

    # unique keys per batch (for the byte counts), read outside any timed region
    U_of = []
    for idx, off, n in dev:
        E.emb_backward_unique_reduce(tabs.ctx, idx, off, B, cfg.pool, dy, bufs["ws"], bufs["unique_keys"],
                                     bufs["counts"], bufs["inverse"], bufs["num_unique"], None)
        torch.cuda.synchronize()
        U_of.append(int(bufs["num_unique"].item()))

    # the pipeline schedule cycles ahead + 1 workspaces / dedup outputs: the
    # dedup of batch i goes to set i % nsets
    ahead = args.ahead if args.schedule == "pipeline" else 1
    nsets = ahead + 1
    bufs2 = [bufs] + [tabs.backward_buffers(nmax, B, with_grad=args.reduce == "atomic") for _ in range(nsets - 1)]
    ev_free2 = [torch.cuda.Event() for _ in range(nsets)]   # buffer set j free (its update done)
    ev_dd2 = [torch.cuda.Event() for _ in range(nsets)]     # dedup into buffer set j done

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()          # default priority
    ev_free = torch.cuda.Event()        # ws / dedup outputs free again (previous update done)
    ev_dd = torch.cuda.Event()          # dedup done
    ev_tr = torch.cuda.Event()          # id translation done (hashed ids)
    ev_free.record(main)

    def issue_dedup(i):
        """Pipeline schedule: the dedup of batch i on the side stream into
        buffer set i % nsets, once that set's previous update is done."""
        j = i % nsets
        idx, off, _ = dev[i % len(dev)]
        side.wait_event(ev_free2[j])
        with torch.cuda.stream(side):
            tabs.dedup(idx, off, B, cfg.pool, bufs2[j])
        ev_dd2[j].record(side)

    def step(i, sched, evs=None, last=False):
        """One training step; evs = three timing events (start, after forward
        [+ dedup], end) recorded on the main stream. Under the pipeline
        schedule the step's dedup was issued `ahead` steps earlier (or by the
        prologue) and this step issues batch i + ahead's unless that is past
        the last step."""
        idx, off, n = dev[i % len(dev)]
        if evs:
            evs[0].record(main)
        if sched == "pipeline":
            j = i % nsets
            tabs.forward(idx, off, B, cfg.pool, out=Y)
            if evs:
                evs[1].record(main)
            main.wait_event(ev_dd2[j])
            tabs.backward(idx, off, B, cfg.pool, dy, bufs2[j])   # skips the dedup done ahead
            tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs2[j], dY=dy)
            ev_free2[j].record(main)
            if i + ahead < nsteps[0]:
                issue_dedup(i + ahead)
            if evs:
                evs[2].record(main)
            return
        if args.hashed:
            E.emb_hash_translate(tabs.ctx, ids_dev[i % len(dev)], off, B, True, hws, idx)
            ev_tr.record(main)
        if args.unique_forward:
            tabs.dedup(idx, off, B, cfg.pool, bufs)
            tabs.forward_unique(idx, off, B, cfg.pool, bufs, rows_buf, out=Y)
        elif sched == "overlap":
            side.wait_event(ev_free)
            if args.hashed:
                side.wait_event(ev_tr)
            with torch.cuda.stream(side):
                tabs.dedup(idx, off, B, cfg.pool, bufs)
            ev_dd.record(side)
            tabs.forward(idx, off, B, cfg.pool, out=Y)
            main.wait_event(ev_dd)
        else:
            tabs.forward(idx, off, B, cfg.pool, out=Y)
        if evs:
            evs[1].record(main)
        if args.pack:
            tabs.backward(idx, off, B, cfg.pool, dy, bufs)   # skips the dedup done ahead
            tabs.pack(bufs, pbufs, dY=dy)
        elif args.reduce == "fused":
            tabs.backward(idx, off, B, cfg.pool, dy, bufs)   # skips the dedup done ahead
            tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs, dY=dy)
        else:
            E.emb_backward_unique_reduce(tabs.ctx, idx, off, B, cfg.pool, dy, bufs["ws"], bufs["unique_keys"],
                                         bufs["counts"], bufs["inverse"], bufs["num_unique"], None)
            tabs.atomic_reduce(off, n, B, cfg.pool, dy, bufs)
            tabs.update(cfg.opt, cfg.lr, cfg.eps, bufs)
        ev_free.record(main)
        if evs:
            evs[2].record(main)

    nsteps = [0]

    def run(sched, K, ev=None):
        nsteps[0] = K
        if sched == "pipeline":
            # the prologue dedups start after everything before them on main
            for e in ev_free2:
                e.record(main)
            for i in range(min(ahead, K)):
                issue_dedup(i)
        for i in range(K):
            step(i, sched, ev[i] if ev else None, last=i == K - 1)

    def timed(sched, K, phases=False):
        """K steps after the warmup steps, timed by one event pair around them.
        With phases, every step also records three events on the main stream
        (start, forward done, end) for the per-phase split; those records
        cost ≈ 15 µs per step, so the headline is timed without them."""
        run(sched, args.warmup)
        torch.cuda.synchronize()
        tabs.check_device_error()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)] if phases else None
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record(main)
        run(sched, K, ev)
        t1.record(main)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total = t0.elapsed_time(t1)
        print(f"[bench] {sched}{' (phase events)' if phases else ''}: {K} steps {total:.3f} ms "
              f"(wall {wall * 1e3:.1f} ms)", file=sys.stderr, flush=True)
        if not phases:
            return total, None, None, None
        fwd = sum(e[0].elapsed_time(e[1]) for e in ev)
        bwd = sum(e[1].elapsed_time(e[2]) for e in ev)
        per_step = sorted(e[0].elapsed_time(e[2]) for e in ev)
        return total, fwd, bwd, per_step

    K = args.steps
    other = "serial" if args.schedule != "serial" else "overlap"
    # the headline: K steps with nothing recorded between them; then K more
    # with the per-step phase events, for the forward / backward split
    total_ms = timed(args.schedule, K)[0]
    phase_total_ms, fwd_ms, bwd_ms, per_step = timed(args.schedule, K, phases=True)
    other_ms = None if args.single_schedule else timed(other, K)[0]

    def pct(q):
        return round(float(np.percentile(np.asarray(per_step), q)), 4)

    # algorithmic bytes per step (what the method must move, from the actual N and U)
    ib = 4 if host_batches[0].indices.dtype == np.int32 else 8
    state_b = D * 4 if cfg.opt == "adagrad" else 0
    # weight bytes per unique row: stored row read + written, or with a master
    # the fp32 master read + written and the low-precision copy written
    wrow_b = 2 * D * 4 + rowbytes if args.master else 2 * rowbytes
    steps_N = [dev[i % len(dev)][2] for i in range(K)]
    steps_U = [U_of[i % len(dev)] for i in range(K)]
    fwd_bytes = sum(n * rowbytes + n * ib + (T * B + 1) * ib + B * T * D * 4 for n in steps_N)
    # per unique row: the update's weight (+ state) traffic, or in the RB step
    # its reduced gradient row written to the send buffer (+ key and slot)
    urow_b = D * 4 + 8 if args.pack else wrow_b + 2 * state_b
    bwd_bytes = sum(B * T * D * 4 + n * ib + (T * B + 1) * ib + u * urow_b + u * 8 + n * 4
                    for n, u in zip(steps_N, steps_U))
    lookups = sum(steps_N)
    if args.schedule in ("overlap", "pipeline") or args.unique_forward:
        # the dedup's own I/O (indices, offsets, unique keys + counts, inverse)
        # runs in the forward phase under this schedule
        dd = sum(n * ib + (T * B + 1) * ib + u * 8 + n * 4 for n, u in zip(steps_N, steps_U))
        fwd_bytes += dd
        bwd_bytes -= dd

    # hashed ids: the fused lookup-only forward (hash probe + gather + pooling
    # in one kernel) against the plain forward on translated rows
    hashed_fwd = None
    if args.hashed:
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(main)
        for i in range(K):
            tabs.forward_hashed(ids_dev[i % len(dev)], dev[i % len(dev)][1], B, cfg.pool, out=Y)
        e1.record(main)
        for i in range(K):
            tabs.forward(dev[i % len(dev)][0], dev[i % len(dev)][1], B, cfg.pool, out=Y)
        e2.record(main)
        torch.cuda.synchronize()
        hashed_fwd = {"fused_hashed_forward_ms": round(e0.elapsed_time(e1) / K, 4),
                      "forward_on_rows_ms": round(e1.elapsed_time(e2) / K, 4)}

    # per-kernel times (HIP events around each launch, on the launch stream)
    def kernel_times(sched):
        E.emb_set_kernel_timing(tabs.ctx, True)
        run(sched, K)
        torch.cuda.synchronize()
        kt = E.emb_kernel_times(tabs.ctx)
        E.emb_set_kernel_timing(tabs.ctx, False)
        return ({k: (ms / n * 1e3 if n else 0.0) for k, (ms, n) in kt.items()},
                {k: ms for k, (ms, n) in kt.items()})

    kavg_us, ktot = kernel_times(args.schedule)

    # algorithmic bytes of one launch of the dominant kernel
    Navg = lookups / K
    Uavg = sum(steps_U) / K
    per_launch = {
        "forward": Navg * rowbytes + Navg * ib + (T * B + 1) * ib + B * T * D * 4,
        # fused reduce + update: every bag's dY row once, each unique row's
        # weight (+ state) read and written once, the sorted bag ids
        "reduce": B * T * D * 4 + Uavg * (D * 4 if args.pack else wrow_b + 2 * state_b) + Navg * 4,
        "sort_scatter": Navg * 8 * 2,
        "sort_hist": Navg * 8,
        "keys": Navg * ib * 2 + Navg * (8 + 4),
        # atomic reduction: every bag's dY row once, every lookup's atomic
        # read-modify-write of its unique row (D*4 each way), inverse reads
        "atomic": B * T * D * 4 + Navg * D * 4 * 2 + Navg * 4,
    }
    # the kernel family with the most time per step among those the roofline
    # has a byte count for (on the real workloads: the fused update). When the
    # dedup runs on the second stream (pipeline, overlap) only the main
    # stream's kernels are ranked: a side-stream launch's duration includes
    # the time it waits for wave slots beside the main stream's kernels.
    side = {"keys", "sort_hist", "sort_scan", "sort_scatter", "rle"} if args.schedule != "serial" else set()
    dominant = max((k for k in ktot if k in per_launch and ktot[k] > 0 and k not in side), key=lambda k: ktot[k])
    alg = per_launch.get(dominant)

    def roofline_of(avg_us):
        if alg is None or avg_us <= 0:
            return None
        achieved = alg / (avg_us * 1e-6) / 1e9
        wtag = f"cfg{args.config}" + ("_uniform" if args.uniform_keys else "")
        src = {"forward": "k_forward.hip", "reduce": "k_reduce.hip", "sort_scatter": "k_keys_sort.hip",
               "sort_hist": "k_keys_sort.hip", "keys": "k_keys_sort.hip", "atomic": "k_atomic.hip"}[dominant]
        traffic, l2_hit = measured_counters(dominant, wtag)
        return {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "l2_hit_rate": l2_hit, "alg_bytes_per_launch": int(alg),
                "avg_launch_us": round(avg_us, 2), "source": src}

    # live: launch durations under the timed schedule (with the pipeline the
    # dominant kernel shares the GPU with the next batch's dedup)
    roofline = roofline_of(kavg_us[dominant])
    roofline_alone = None
    if args.schedule != "serial" and not args.single_schedule:
        kavg_serial, _ = kernel_times("serial")
        roofline_alone = roofline_of(kavg_serial.get(dominant, 0.0))
        if roofline_alone:
            roofline_alone["schedule"] = "serial (the kernel alone on the GPU)"

    # CPU oracle on a bounded sample of batch 0
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, host_batches, dY_host, args.cpu_sample, args.cpu_seconds, ib, args.master)

    ms_step = total_ms / K
    out = {
        "metric": METRIC,
        "value": round(lookups / (total_ms * 1e-3), 1),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_p50_p90": [pct(10), pct(50), pct(90)],
        "ms_per_step_phase_pass": round(phase_total_ms / K, 4),
        "schedule": args.schedule,
        "dedup_ahead": ahead if args.schedule == "pipeline" else None,
        "reduce": args.reduce if not args.pack else f"pack to {args.pack} shards (RB)",
        f"ms_per_step_{other}": round(other_ms / K, 4) if other_ms is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else f"{cfg.dtype}-storage/f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{T} {cfg.dtype} tables x {rows_desc(cfg)} rows x {D}"
                         f"{f' ({cfg.tables[0].col_slices} column slices)' if cfg.tables[0].col_slices > 1 else ''}"
                         f"{' + fp32 masters' if args.master else ''}, batch {B}, "
                         f"{'uniform' if cfg.zipf_s is None else f'Zipf({cfg.zipf_s})'} keys, "
                         f"{hot_desc(cfg)}, {cfg.pool} pooling, {cfg.opt}"),
            "config_id": args.config,
            "global_batch": B,
            "lookups_per_step": int(round(Navg)),
            "unique_per_step": int(round(Uavg)),
            "batches_cycled": len(dev),
        },
        "phases": ("fwd includes the id -> row translation; " if args.hashed else "") + (
                   "fwd = dedup, then the unique-first forward (unique rows gathered once); bwd_update = "
                   if args.unique_forward else
                   f"fwd = forward (the dedup of the batch {ahead} step(s) ahead runs on a second stream "
                   "alongside the forward and the update); bwd_update = " if args.schedule == "pipeline" else
                   "fwd = forward with the dedup on a second stream alongside it; bwd_update = " if args.schedule == "overlap"
                   else "fwd = forward; bwd_update = dedup + ") + (
                   f"routing to {args.pack} shards + reduce into the send slots (RB)" if args.pack
                   else "segmented reduce + fused optimizer") + (
                   "; the phases and the per-step percentiles come from a second pass of the same K steps "
                   "with three events recorded per step (ms_per_step_phase_pass), the headline from a "
                   "pass with none"),
        "fwd": {"ms": round(fwd_ms / K, 4), "lookups_per_s": round(lookups / (fwd_ms * 1e-3), 1),
                "alg_GBps": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1),
                "alg_bytes_per_step": int(fwd_bytes / K)},
        "bwd_update": {"ms": round(bwd_ms / K, 4), "lookups_per_s": round(lookups / (bwd_ms * 1e-3), 1),
                       "alg_GBps": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9, 1),
                       "alg_bytes_per_step": int(bwd_bytes / K)},
        "kernels_avg_us": {k: round(v, 2) for k, v in kavg_us.items() if v > 0},
        "kernels_ms_per_step": {k: round(v / K, 4) for k, v in ktot.items() if v > 0},
        "roofline": roofline,
        "roofline_alone": roofline_alone,
        "cpu_baseline": cpu,
    }
    if hashed_fwd:
        out["hashed"] = hashed_fwd
    if compact:
        out = {k: out[k] for k in ("value", "unit", "ms_per_step", "ms_per_step_p10_p50_p90", "schedule", "dtype",
                                   "config", "fwd", "bwd_update", "kernels_avg_us", "roofline", "cpu_baseline")}
    tabs.close()
    del tabs, dev, bufs, bufs2, dy, Y
    return out


def rows_desc(cfg) -> str:
    rr = [t.rows for t in cfg.tables]
    if min(rr) == max(rr):
        return str(rr[0])
    return f"{min(rr)}..{max(rr)} ({sum(rr)} in total)"


def hot_desc(cfg) -> str:
    h = cfg.hotness
    if all(x == 1 for x in h):
        return "one lookup per bag"
    if all(isinstance(x, int) for x in h):
        if min(h) == max(h):
            return f"{h[0]} lookups per bag"
        return f"{min(h)}..{max(h)} lookups per bag by table (log-uniform)"
    return "variable lookups per bag"


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, batches, dY, n_samples, seconds, ib, master=False):
    """The oracle, as it stands, on the cycled batches of the workload (the
    first n_samples samples of each, every table; 0 = whole batches, or as
    many samples as hold about 2 M lookups when a batch holds more): the
    forward, then dedup + reduced gradient + optimizer step, each phase timed
    on its own. Batches are taken in turn until `seconds` of CPU time have
    been spent. numpy's thread pools are held to one thread, so `cores` is
    what it used. Algorithmic bytes per phase use the GPU's formula on the
    sample's own N and U."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    from dlrm_sparse_embedding_amd import workloads as W

    B = cfg.batch
    if n_samples > 0:
        ns = min(n_samples, B)
    else:
        nb = batches[0].N
        ns = B if nb <= 2_000_000 else max(1, int(B * 2_000_000 / nb))
    ro = cfg.row_offset()
    D = cfg.dim
    rowbytes = D * W.DTYPE_BYTES[cfg.dtype]
    state_b = D * 4 if cfg.opt == "adagrad" else 0
    wrow_b = 2 * D * 4 + rowbytes if master else 2 * rowbytes
    total_n = total_u = 0
    t_fwd = t_bwd = 0.0
    by_fwd = by_bwd = 0
    used = 0
    with threadpool_limits(limits=1):
        for batch in batches:
            lens, keys = [], []
            for t in range(cfg.T):
                a, b = int(batch.offsets[t * B]), int(batch.offsets[t * B + ns])
                lens.append(np.diff(batch.offsets[t * B:t * B + ns + 1].astype(np.int64)))
                keys.append(batch.indices[a:b])
            sub = W.make_batch_from_lengths(lens, keys, ns)
            dYs = np.ascontiguousarray(dY[:ns])
            # untimed preparation: the stored contents of the touched rows
            otabs = [O.TouchedRows(cfg.init_seed, t, cfg.dim, cfg.dtype,
                                   sub.indices[int(sub.offsets[t * ns]):int(sub.offsets[(t + 1) * ns])])
                     for t in range(cfg.T)]
            t0 = time.perf_counter()
            O.pooled_forward(otabs, sub.indices, sub.offsets, cfg.T, ns, cfg.dim, cfg.pool)
            t1 = time.perf_counter()
            g = O.global_keys(sub.indices, sub.offsets, ro, cfg.T, ns)
            u, c, inv = O.dedup(g)
            gU = O.reduced_grad(dYs, sub.offsets, cfg.T, ns, cfg.dim, cfg.pool, inv, len(u))
            t_of = np.searchsorted(ro, u, side="right") - 1
            w_old = np.concatenate([otabs[t][u[t_of == t] - ro[t]] for t in range(cfg.T)])
            G_old = np.zeros_like(w_old) if cfg.opt == "adagrad" else None
            O.update_rows(w_old, G_old, gU, cfg.opt, cfg.lr, cfg.eps, cfg.dtype)
            t2 = time.perf_counter()
            n, U = sub.N, len(u)
            t_fwd += t1 - t0
            t_bwd += t2 - t1
            by_fwd += n * rowbytes + n * ib + (cfg.T * ns + 1) * ib + ns * cfg.T * D * 4
            by_bwd += (ns * cfg.T * D * 4 + n * ib + (cfg.T * ns + 1) * ib + U * (wrow_b + 2 * state_b)
                       + U * 8 + n * 4)
            total_n += n
            total_u += U
            used += 1
            if t_fwd + t_bwd >= seconds:
                break
    try:
        avail = len(os.sched_getaffinity(0))
    except Exception:
        avail = os.cpu_count()
    el = t_fwd + t_bwd
    return {"value": round(total_n / el, 1), "unit": "lookups/s", "cores": 1, "kind": "oracle",
            "fwd": {"s": round(t_fwd, 3), "lookups_per_s": round(total_n / t_fwd, 1),
                    "alg_GBps": round(by_fwd / t_fwd / 1e9, 3)},
            "bwd_update": {"s": round(t_bwd, 3), "lookups_per_s": round(total_n / t_bwd, 1),
                           "alg_GBps": round(by_bwd / t_bwd / 1e9, 3)},
            "sample": (f"{used} batch(es) x first {ns} samples, all {cfg.T} tables ({total_n} lookups, "
                       f"{total_u} unique keys in total): forward, then dedup + reduce + optimizer, "
                       f"{el:.2f} s, single-threaded numpy on {cpu_model()}; {avail} host cores available")}


if __name__ == "__main__":
    sys.exit(main())
