"""Throughput of the speculative-sampling verifier on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c5]

One step is one spec_verify_sample call (or spec_verify_greedy for the greedy
workload) over the whole batch: ban-list preparation, row statistics of every
target and draft row, the acceptance walk and the final draw. Inputs are
synthetic (lossless_draft_verification_sample_amd.synth) and already resident
in HBM; the timed loop rotates four device copies of them so the 256 MB
Infinity Cache cannot serve repeated reads. Draft tokens are the stored,
oracle-drawn proposals of tests/golden/proposals.json.

Prints one JSON line. `value` is verified logit rows per second
(B*(2*gamma+1) rows per sampling call). `roofline` rates the dominant kernel
(row_stats, or greedy_argmax) on algorithmic bytes (every logit read once)
divided by its average duration, measured with HIP events that the benchmark
build of the library (libspecverify_bench.so: same kernels, plus event pairs
around each launch on the launch stream) records in a second loop. The line
also carries the accepted-prefix histogram of the last timed call and the
conditional acceptance rate by position derived from it. `cpu_baseline` times
the float64 oracle on a bounded sample of the same workload on one host core;
`cpu_baseline_pool` runs it over the whole batch split across up to 16 host
processes. `parity` compares the last timed call's tokens, accepted counts
and flags with the one-core oracle run's, request by request.

Before the W warm-up steps the GPU is brought to steady clocks by untimed
calls for about --ramp-ms milliseconds (reported as `clock_ramp`); from a cold
start the first ~150 calls run at lower clocks.

With --diagnostics every step also asks for the per-position overlaps; the
line then carries a `diagnostics` object that
rates the overlap kernel the same way (algorithmic bytes: the row of each pair
that is read in full, both rows when neither is truncated).

With --mixed the batch carries per-request settings (sv_requests): every
fourth request is greedy, draft lengths are gamma, gamma-1, gamma-2 in turn,
and temperature, top-k and top-p vary per request; `value` then counts the
rows the requests use (2 g_b + 1 per sampled request, g_b + 1 per greedy one).

With --penalty every request also carries a 64-token history (its first
target row's 32 largest logits and 32 random ids) and repetition penalties
1.2 (target) and 1.1 (draft).

With --graph the line also carries `graph`: the step time when the calls are
replayed from a captured HIP graph (launch overhead removed), next to the
eager `value`.

With --commit every step is followed by spec_verify_commit (chain KV-commit
metadata from the step's outputs, with synthetic KV lengths and slots); the
line then carries a `commit` object with that kernel's time and bytes.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COPIES = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_label(cfg):
    trunc = []
    if cfg.top_k:
        trunc.append(f"top-k {cfg.top_k}")
    if cfg.top_p < 1:
        trunc.append(f"top-p {cfg.top_p}")
    if cfg.n_banned:
        trunc.append(f"{cfg.n_banned} banned ids")
    t = ", ".join(trunc) or "no truncation"
    if cfg.mode == "greedy":
        return f"{cfg.name}: greedy B={cfg.B} gamma={cfg.gamma} V={cfg.V} {cfg.dtype}"
    return (f"{cfg.name}: B={cfg.B} gamma={cfg.gamma} V={cfg.V} {cfg.dtype} "
            f"T={cfg.temperature} {t}")


def traffic_record(kernel, workload):
    """Counter-measured HBM bytes per launch, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(f"{kernel}/{workload}")
    from lossless_draft_verification_sample_amd.rocprof_summary import source_digest
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("bytes_per_launch")


def read_ceiling(dev, nbytes, chunk_bytes, iters=50):
    """Plain read bandwidth of this GPU on `nbytes` of device memory (two
    buffers alternate, so the last-level cache serves no repeat): a
    grid-stride sweep, and one `chunk_bytes` chunk per workgroup, the access
    shape of the row kernels. GB/s from events around `iters` launches."""
    import ctypes
    import torch
    from lossless_draft_verification_sample_amd import build as b
    lib = ctypes.CDLL(os.path.join(b.PKG_DIR, b.CALIB_LIB_NAME))
    lib.sv_calib_read_blocks.restype = ctypes.c_int64
    lib.sv_calib_read_blocks.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    lib.sv_calib_read.restype = ctypes.c_int
    lib.sv_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = nbytes // 16 * 16
    bufs = [torch.randint(0, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream().cuda_stream
    out = {"bytes": nbytes, "chunk_bytes": chunk_bytes}
    for name, mode, grid in (("grid_stride", 0, 256 * 8), ("chunk_per_workgroup", 1, 0)):
        nblk = lib.sv_calib_read_blocks(nbytes, mode, chunk_bytes, grid)
        sink = torch.empty(nblk, dtype=torch.int32, device=dev)

        def call(k):
            rc = lib.sv_calib_read(bufs[k % 2].data_ptr(), nbytes, mode, chunk_bytes, grid,
                                   sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"sv_calib_read failed ({rc})")
        for k in range(20):
            call(k)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for k in range(iters):
            call(k)
        e.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(e) / iters * 1e3
        out[name] = {"us": us, "gbps": nbytes / (us / 1e6) / 1e9, "workgroups": nblk}
    log(f"[bench] read ceiling {out}")
    return out


def host_cpu():
    """CPU model and the core counts this process sees (for the baseline lines)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(wl, xs, budget_s, results=None):
    """The float64 oracle, as it stands, on the first requests of the workload.
    When `results` is a list, the oracle's outputs of each timed slice are
    appended to it (untimed)."""
    import oracle
    cfg = wl.cfg
    n = 1
    rows_per_req = (2 * cfg.gamma + 1) if cfg.mode == "sample" else (cfg.gamma + 1)
    t_total, done = 0.0, 0
    u_all = (np.array(oracle.uniforms(cfg.philox_seed, cfg.philox_offset, cfg.B, cfg.gamma))
             if cfg.mode == "sample" else None)
    while t_total < budget_s and done < cfg.B:
        take = min(n, cfg.B - done)
        sl = slice(done, done + take)
        tgt = wl.target[sl].astype(np.float64)
        if cfg.mode == "sample":
            dft = wl.draft[sl].astype(np.float64)
            u = u_all[sl]
            s = oracle.Sampler(cfg.temperature, cfg.top_k, cfg.top_p)
            t0 = time.perf_counter()
            ref = oracle.verify_sample(tgt, dft, xs[sl], u, s, s,
                                       None if wl.banned is None else wl.banned[sl])
        else:
            t0 = time.perf_counter()
            ref = oracle.verify_greedy(tgt, xs[sl])
        t_total += time.perf_counter() - t0
        if results is not None:
            results.append(ref)
        done += take
        n = min(2 * n, 8)
    rows = done * rows_per_req
    return {"value": rows / t_total, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {cfg.B} requests ({rows} rows), float64 NumPy on one "
                      f"host core, {t_total:.1f} s; bf16->f64 upcast not timed",
            **host_cpu()}


def parity_summary(cfg, out, refs, band=1e-10):
    """The last timed call's outputs against the oracle's on the requests the
    one-core oracle run covered: tokens, accepted counts and flags must be
    identical except for requests with a decision within `band` of its edge
    (sampling only; greedy compares every request)."""
    n = sum(len(r.num_accepted) for r in refs)
    tok = out.tokens.cpu().numpy()[:n]
    nacc = out.num_accepted.cpu().numpy()[:n]
    flg = out.flags.cpu().numpy().astype(np.uint32)[:n]
    rtok = np.concatenate([r.tokens for r in refs])
    rnacc = np.concatenate([r.num_accepted for r in refs])
    rflg = np.concatenate([r.flags for r in refs]).astype(np.uint32)
    same = (tok == rtok).all(axis=1) & (nacc == rnacc) & (flg == rflg)
    if cfg.mode == "sample":
        margin = np.concatenate([r.margin for r in refs])
        keep = margin > band
        within_1e6 = int(np.concatenate([r.boundary for r in refs]).sum())
    else:
        keep = np.ones(n, bool)
        within_1e6 = 0
    return {"requests": int(n), "compared": int(keep.sum()),
            "mismatched": int((~same & keep).sum()), "excluded_band": band,
            "excluded": int((~keep).sum()), "decisions_within_1e-6": within_1e6}


def _oracle_worker(conn):
    """One host process of the pooled oracle run (module level, so that spawned
    processes can import it): receives its requests, upcasts them, reports
    ready, and on "go" runs the oracle and sends back its own seconds."""
    import oracle
    mode, tgt, dft, xs, u, banned, samp = conn.recv()
    tgt = tgt.astype(np.float64)
    dft = None if dft is None else dft.astype(np.float64)
    conn.send("ready")
    conn.recv()
    t0 = time.perf_counter()
    if mode == "sample":
        s = oracle.Sampler(*samp)
        oracle.verify_sample(tgt, dft, xs, u, s, s, banned)
    else:
        oracle.verify_greedy(tgt, xs)
    conn.send(time.perf_counter() - t0)


def cpu_baseline_pool(wl, xs, max_workers=16, timeout_s=300.0):
    """The same float64 oracle over the whole batch, its requests split across up
    to 16 host processes. Each process gets and upcasts its share before the
    clock starts (as the one-core figure leaves out the upcast); the wall clock
    runs from the common start signal until the last process is done."""
    import multiprocessing as mp
    import oracle
    cfg = wl.cfg
    n = max(1, min(max_workers, os.cpu_count() or 1, cfg.B))
    rows_per_req = (2 * cfg.gamma + 1) if cfg.mode == "sample" else (cfg.gamma + 1)
    u_all = (np.array(oracle.uniforms(cfg.philox_seed, cfg.philox_offset, cfg.B, cfg.gamma))
             if cfg.mode == "sample" else None)
    bounds = np.linspace(0, cfg.B, n + 1).astype(int)
    ctx = mp.get_context("spawn")
    procs, conns = [], []
    try:
        for k in range(n):
            sl = slice(bounds[k], bounds[k + 1])
            mine, theirs = ctx.Pipe()
            p = ctx.Process(target=_oracle_worker, args=(theirs,), daemon=True)
            p.start()
            mine.send((cfg.mode, wl.target[sl], wl.draft[sl] if cfg.mode == "sample" else None,
                       xs[sl], None if u_all is None else u_all[sl],
                       None if wl.banned is None else wl.banned[sl],
                       (cfg.temperature, cfg.top_k, cfg.top_p)))
            procs.append(p)
            conns.append(mine)

        def recv(c):
            if not c.poll(timeout_s):
                raise RuntimeError("oracle worker timed out")
            return c.recv()
        for c in conns:
            assert recv(c) == "ready"
        t0 = time.perf_counter()
        for c in conns:
            c.send("go")
        inner = [recv(c) for c in conns]
        wall = time.perf_counter() - t0
    finally:
        for p in procs:
            p.join(timeout=10)
            if p.is_alive():
                p.terminate()
    rows = cfg.B * rows_per_req
    return {"value": rows / wall, "unit": "rows/s", "cores": n, "kind": "oracle",
            "sample": f"all {cfg.B} requests ({rows} rows) split over {n} host processes, "
                      f"float64 NumPy, {wall:.2f} s wall clock from a common start (longest "
                      f"process {max(inner):.2f} s); bf16->f64 upcast not timed",
            **host_cpu()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # the GPU reaches its steady clocks after about 150 calls (~30 ms)
    ap.add_argument("--ramp-ms", type=float, default=100.0,
                    help="untimed calls for about this long before the warm-up steps")
    ap.add_argument("--config", default="c5")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--diagnostics", action="store_true",
                    help="also compute per-position overlaps and the accepted-prefix histogram")
    ap.add_argument("--mixed", action="store_true",
                    help="per-request draft lengths and samplers, a quarter of the requests greedy")
    ap.add_argument("--penalty", action="store_true",
                    help="repetition penalties over a 64-token history per request")
    ap.add_argument("--commit", action="store_true",
                    help="follow every step with the chain KV-commit metadata kernel")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="also time the read-only calibration kernels (libsvcalib.so): "
                         "a grid-stride sweep and one row-sized chunk per workgroup over "
                         "the step's logit bytes")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only (use --gpus 1): the verifier shards over "
              "requests with no communication, so N GPUs each run this measurement on "
              "their own B/N requests.", file=sys.stderr)
        sys.exit(2)

    import torch
    import lossless_draft_verification_sample_amd as sv
    from lossless_draft_verification_sample_amd import synth

    sv._lib.load()
    dev = torch.device("cuda:0")
    cfg = synth.config(args.config)
    log(f"[bench] generating {workload_label(cfg)}")
    t0 = time.perf_counter()
    wl = synth.make_workload(cfg)
    with open(os.path.join(ROOT, "tests", "golden", "proposals.json")) as f:
        xs = np.array(json.load(f)[cfg.name]["tokens"], dtype=np.int32)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")

    def to_dev(bits, vals):
        if cfg.dtype == "bf16":
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(vals).to(dev)

    tgt0 = to_dev(wl.target_bits, wl.target)
    copies = [tgt0] + [tgt0.clone() for _ in range(COPIES - 1)]
    if cfg.mode == "sample":
        dft0 = to_dev(wl.draft_bits, wl.draft)
        dcopies = [dft0] + [dft0.clone() for _ in range(COPIES - 1)]
        rows = cfg.B * (2 * cfg.gamma + 1)
    else:
        dcopies = [None] * COPIES
        rows = cfg.B * (cfg.gamma + 1)
    toks = torch.from_numpy(xs).to(dev)
    bans = None if wl.banned is None else torch.from_numpy(wl.banned).to(dev)
    samp = (cfg.temperature, cfg.top_k, cfg.top_p)
    if cfg.mode == "sample":
        ws = torch.empty(sv.spec_verify_workspace_bytes(cfg.B, cfg.gamma, cfg.V),
                         dtype=torch.uint8, device=dev)
        out = sv.SampleOut(torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev),
                           torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                           torch.empty((cfg.B,), dtype=torch.int32, device=dev), None, None,
                           torch.empty((cfg.B, cfg.gamma), dtype=torch.float64, device=dev)
                           if args.diagnostics else None,
                           torch.empty((cfg.gamma + 1,), dtype=torch.int32, device=dev))
    else:
        out = sv.GreedyOut(torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev),
                           torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                           torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                           torch.empty((cfg.gamma + 1,), dtype=torch.int32, device=dev))

    if args.commit:
        G1 = cfg.gamma + 1
        kv_len = torch.arange(cfg.B, dtype=torch.int32, device=dev) * 4096
        slots = (torch.arange(cfg.B * G1, dtype=torch.int32, device=dev).reshape(cfg.B, G1)
                 + 1_000_000)
        cout = sv.CommitOut(torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B, cfg.gamma), dtype=torch.int32, device=dev))

    requests = None
    if args.mixed:
        if cfg.mode != "sample":
            raise SystemExit("--mixed needs a sampling workload")
        temps, topps, topks = (0.6, 0.8, 1.0, 1.2), (0.9, 0.95, 1.0), (0, 50)
        per = [(temps[b % 4], topks[b % 2], topps[b % 3]) for b in range(cfg.B)]
        for b in range(0, cfg.B, 4):
            per[b] = (0.0, 0, 1.0)
        gam = np.array([cfg.gamma - (b % 3) for b in range(cfg.B)], dtype=np.int32).clip(0)
        requests = sv.Requests(gamma=torch.from_numpy(gam).to(dev),
                               target=sv.sampler_array(per, dev), draft=sv.sampler_array(per, dev))
        greedy = np.array([t[0] == 0.0 for t in per])
        rows = int(np.where(greedy, gam + 1, 2 * gam + 1).sum())
    if args.penalty:
        if cfg.mode != "sample":
            raise SystemExit("--penalty needs a sampling workload")
        prng = np.random.default_rng(cfg.seed + 7)
        hist = np.concatenate([np.argsort(-wl.target[:, 0], axis=1)[:, :32],
                               prng.integers(0, cfg.V, (cfg.B, 32))], axis=1).astype(np.int32)
        base = requests if requests is not None else sv.Requests()
        requests = base._replace(
            history=torch.from_numpy(hist).to(dev),
            penalty=torch.full((cfg.B,), 1.2, dtype=torch.float32, device=dev),
            penalty_draft=torch.full((cfg.B,), 1.1, dtype=torch.float32, device=dev))

    def step(k, lib=None):
        c = k % COPIES
        if cfg.mode == "sample":
            sv.spec_verify_sample(copies[c], dcopies[c], toks, samp, samp, bans,
                                  seed=cfg.philox_seed, offset=cfg.philox_offset,
                                  requests=requests, workspace=ws, out=out, lib=lib)
        else:
            sv.spec_verify_greedy(copies[c], toks, out=out, lib=lib)
        if args.commit:
            sv.spec_verify_commit(out.tokens, out.num_accepted, kv_len, slots, out=cout, lib=lib)

    # clock ramp: untimed calls until about ramp_ms have passed on the GPU
    ramp_calls, t_ramp = 0, time.perf_counter()
    while (time.perf_counter() - t_ramp) * 1e3 < args.ramp_ms:
        for _ in range(10):
            step(ramp_calls)
            ramp_calls += 1
        torch.cuda.synchronize()
    ramp_ms = (time.perf_counter() - t_ramp) * 1e3
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    log(f"[bench] clock ramp {ramp_calls} calls in {ramp_ms:.0f} ms; warmup {args.warmup} done; "
        f"timing {args.steps} steps")

    # step time: a plain loop, bracketed by events on the launch stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(k)
    stop.record()
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(stop)
    log(f"[bench] timed loop {elapsed_ms:.2f} ms")
    # keep the timed loop's outputs for the parity and histogram lines (the
    # loops below overwrite `out`)
    timed_out = type(out)(*[None if t is None else t.clone() for t in out])
    # per-kernel durations: a second loop through the benchmark build, which
    # records event pairs around each of its launches (those records add gaps,
    # so this loop is not the step time)
    blib = sv._lib.load_bench()
    for k in range(5):
        step(k, blib)
    torch.cuda.synchronize()
    sv.bench_profile_start(args.steps)
    for k in range(args.steps):
        step(k, blib)
    torch.cuda.synchronize()
    prof = sv.bench_profile_stop()
    # per-call device time and its spread: events around every step of a
    # third loop (the records between calls add gaps, not call time)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for k in range(args.steps):
        evs[k][0].record()
        step(k)
        evs[k][1].record()
    torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    ms_step = elapsed_ms / args.steps
    value = rows * args.steps / (elapsed_ms / 1e3)
    s = 2 if cfg.dtype == "bf16" else 4
    algo_bytes = rows * cfg.V * s
    dom = "row_stats" if cfg.mode == "sample" else "greedy_argmax"
    dom_ms, dom_n = prof[dom]
    dom_avg_ms = dom_ms / max(dom_n, 1)
    # every used row is read once by the dominant kernel (in a mixed batch the
    # target rows of greedy requests too, for their argmax)
    dom_bytes = rows * cfg.V * s
    achieved = dom_bytes / (dom_avg_ms / 1e3) / 1e9
    # counter traffic is recorded for the plain call of each workload only
    traffic = None if (args.mixed or args.penalty) else traffic_record(dom, cfg.name)

    graph = None
    if args.graph:
        # one graph holds COPIES steps (one per input copy); replays are timed
        # with events on the current stream
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(COPIES):
                step(k)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(COPIES):
                step(k)
        reps = max(1, args.steps // COPIES)
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            g.replay()
        stop.record()
        torch.cuda.synchronize()
        g_ms = start.elapsed_time(stop) / (reps * COPIES)
        graph = {"ms_per_step": g_ms, "value": rows / (g_ms / 1e3), "unit": "rows/s",
                 "steps": reps * COPIES}
        log(f"[bench] graph replays: {g_ms * 1e3:.1f} us per step")

    out = timed_out
    n_acc = out.num_accepted.cpu().numpy()
    flags = out.flags.cpu().numpy()
    hist = out.accept_hist.cpu().numpy().astype(np.int64)
    # position i was reached by sum_{n >= i} h_n requests and accepted by sum_{n > i} h_n
    reached = np.cumsum(hist[::-1])[::-1]
    cond_acc = [float(reached[i + 1] / reached[i]) if reached[i] else None
                for i in range(cfg.gamma)]
    res = {
        "metric": "verified logit rows/sec",
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": workload_label(cfg), "B": cfg.B, "gamma": cfg.gamma, "V": cfg.V,
                   "rows_per_step": rows, "algorithmic_bytes_per_step": algo_bytes,
                   "parallelism": "single GPU"},
        "hbm_gbps_step": algo_bytes / (ms_step / 1e3) / 1e9,
        "hbm_frac_step": algo_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "avg_kernel_ms": dom_avg_ms, "launches": dom_n, "traffic": traffic},
        "kernel_ms_per_step": {k: v[0] / v[1] for k, v in prof.items() if v[1]},
        "call_us": {"p10": float(np.percentile(call_us, 10)),
                    "p50": float(np.median(call_us)),
                    "p90": float(np.percentile(call_us, 90))},
        "mean_accepted": float(n_acc.mean()),
        "mean_emitted_per_request": float(n_acc.mean() + 1),
        "accept_hist": hist.tolist(),
        "conditional_acceptance_by_position": cond_acc,
        "flags_nonzero": int((flags != 0).sum()),
        "clock_ramp": {"calls": ramp_calls, "ms": ramp_ms},
    }
    if graph is not None:
        res["graph"] = graph
    if args.penalty:
        res["config"]["repetition_penalty"] = "64-token history, 1.2 target, 1.1 draft"
    if args.mixed:
        res["config"]["mixed"] = ("a quarter greedy; draft lengths gamma, gamma-1, gamma-2; "
                                  "T in {0.6, 0.8, 1.0, 1.2}, top-k in {0, 50}, top-p in "
                                  "{0.9, 0.95, 1.0} per request")
        res["roofline"]["algorithmic_bytes"] = dom_bytes
    if args.diagnostics:
        res["config"]["diagnostics"] = True
        diag = {}
        if cfg.mode == "sample":
            ov_ms, ov_n = prof["overlap"]
            ov_avg = ov_ms / max(ov_n, 1)
            truncated = cfg.top_k > 0 or cfg.top_p < 1.0
            ov_bytes = cfg.B * cfg.gamma * cfg.V * s * (1 if truncated else 2)
            ov_gbps = ov_bytes / (ov_avg / 1e3) / 1e9
            diag.update({
                "mean_overlap": float(out.overlap.mean().item()),
                "roofline": {"kernel": "overlap", "bound": "hbm", "achieved": ov_gbps,
                             "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": ov_gbps / HBM_PEAK_GBPS, "avg_kernel_ms": ov_avg,
                             "launches": ov_n, "algorithmic_bytes": ov_bytes,
                             "traffic": traffic_record("overlap", cfg.name)}})
        res["diagnostics"] = diag
    if args.commit:
        res["config"]["commit"] = True
        cm_ms, cm_n = prof["commit"]
        cm_avg = cm_ms / max(cm_n, 1)
        G1 = cfg.gamma + 1
        # tokens, slots, accepted counts and KV lengths in; lengths, anchors,
        # free counts and free slots out
        cm_bytes = 4 * (2 * cfg.B * G1 + 2 * cfg.B + 3 * cfg.B + cfg.B * cfg.gamma)
        res["commit"] = {"kernel": "commit", "avg_kernel_ms": cm_avg, "launches": cm_n,
                         "bytes_per_launch": cm_bytes,
                         "achieved_gbps": cm_bytes / (cm_avg / 1e3) / 1e9,
                         "bound": "launch latency (one wave per request)"}
    if args.read_ceiling:
        res["read_ceiling"] = read_ceiling(dev, algo_bytes, cfg.V * s)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 2**20 // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = {"read": n * 4, "write": n * 4}
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        refs = []
        res["cpu_baseline"] = cpu_baseline(wl, xs, args.cpu_budget, refs)
        if not (args.mixed or args.penalty):
            res["parity"] = parity_summary(cfg, out, refs)
        log("[bench] timing the oracle on a pool of host processes")
        res["cpu_baseline_pool"] = cpu_baseline_pool(wl, xs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
