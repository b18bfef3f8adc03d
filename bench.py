"""Benchmark: fused stable softmax cross-entropy forward + backward on one
MI355X, page-scale workload (T = 16384 tokens, V = 128256, bf16 logits and
bf16 gradient, mean over non-ignored rows; the shapes of the H100 table in
torchtitan PR "[loss] fix softmax collapse with improved ce perf").

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one ce_fused_fwd_bwd call over the resident batch: the count
pre-pass, the row-resident fused kernel (max, non-target sum, finalize,
gradient) and the loss reduction.  Inputs are generated on the GPU from a
fixed seed before timing and stay in HBM.  Prints one JSON line.

Every timed section runs W untimed calls first (default 10): after the GPU
has been idle, the first steps of an HBM-bound loop run slow while the clocks
come back up (split-V steps right after a synchronize: 2.46, 2.37, 2.32,
2.31, 2.29 ms, then 2.24-2.26 from about the eighth step on).

Algorithmic bytes of a fused step: the logits of every non-ignored row read
once (an ignored row's logits are not needed), every gradient row written
once (zeros for ignored rows), and per row the int64 target read and the
fp32 loss written.

Objects in the line besides the contract's keys:
  timing        median / min / max of the K steps (HIP events between
                consecutive steps on the launch stream).
  roofline      HBM roofline of the fused kernel: its algorithmic bytes /
                its average duration, from HIP events the library records
                around it (ce_fused_fwd_bwd_timed; the step also holds the
                target count and the loss reduction); peak 8 TB/s.  traffic
                is the HBM byte count the rocprofv3 FETCH_SIZE / WRITE_SIZE
                counters gave for this kernel source
                (profiles/fused_page_counters.md), null if the source changed.
  inputs        SHA-256 of the logits and target bytes of each workload.
  host          CPU model, logical CPUs and affinity of this host.
  cpu_baseline  the fp64 oracle timed on this host (all its OpenMP threads) on
                a bounded sample of the same workload, in GB/s of the same
                algorithmic bytes; per_core: one thread on the mid workload.
  configs       the small workloads, each call timed alone after a 512 MiB
                write that evicts the caches: tiny (64 x 1000 fp32, us) and
                mid (4096 x 32000 bf16).
  split_v       the vocabulary split in two 64128-column shards with label
                smoothing 0.1: ce_forward per shard, ce_merge_shard_stats,
                ce_backward per shard.
  in_place      the fused call with the gradient written over the logits
                (the logits restored between steps, outside the timing).
  unfused       ce_forward (whole vocabulary: row statistics, finalize, loss)
                then ce_backward, no smoothing.
  linear_ce     cross-entropy of a linear classifier without stored logits
                (ce_linear_fwd_bwd): E [8192, 2048] and C [128256, 2048] bf16,
                loss + dE + dC; MFMA roofline: 4 products of 2 N V D flops
                against the 2.5 PFLOP/s dense bf16 peak; "filtered": the same
                call with gradient filtering at 2^-8 and the time it saves.
  memory        peak device memory (torch allocator) of one call of each
                path, inputs included.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFS = 2500.0
T, V = 16384, 128256
COUNTERS = os.path.join(ROOT, "profiles", "fused_page_counters.md")
# the sources the fused kernels are built from (their launch arguments and the
# device helpers); counter figures are reported only while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "vocab_softmax_cross_row_amd", "csrc", f)
                  for f in ("ce_fused.hip", "ce_device.h")]
GIB = float(1 << 30)


def fused_bytes(T, V, T_read=None, in_size=2, out_size=2):
    """Algorithmic bytes of one fused launch: the logits of the T_read rows
    that need them (default all) read once, every gradient written once,
    plus per row the int64 target and the fp32 loss."""
    T_read = T if T_read is None else T_read
    return T_read * V * in_size + T * V * out_size + T * (8 + 4)


def split_bytes(T, V, T_read=None, in_size=2, out_size=2):
    """Split-vocabulary path: the forward reads the needed logits, the
    backward reads them again and writes every gradient (the per-row
    targets, 32-byte stats and 24-byte row constants are under 1 MB)."""
    T_read = T if T_read is None else T_read
    return 2 * T_read * V * in_size + T * V * out_size


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per fused launch from the committed counter summary, if it
    was taken on the current kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    fields = {}
    with open(COUNTERS) as f:
        for line in f:
            if ":" in line and line.strip().startswith("-"):
                k, _, v = line.strip()[1:].partition(":")
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256_16") != source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def sha256_of(t, block=1 << 28):
    import torch
    h = hashlib.sha256()
    flat = t.detach().contiguous().view(torch.uint8).reshape(-1)
    for i in range(0, flat.numel(), block):
        h.update(flat[i:i + block].cpu().numpy())
    return h.hexdigest()


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def stats_ms(times):
    return {"mean_ms": round(statistics.fmean(times), 4),
            "median_ms": round(statistics.median(times), 4),
            "min_ms": round(min(times), 4), "max_ms": round(max(times), 4), "n": len(times)}


def time_steps(fn, steps, warmup, stream):
    """W untimed calls, then K back-to-back calls with an event between
    consecutive ones: per-step times and the whole span (ms)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[steps]), wall


def time_each(fn, steps, warmup, stream, before=None):
    """Each call timed alone between its own pair of events; `before` runs
    untimed ahead of every call (a cache flush, an input restore)."""
    import torch
    for _ in range(warmup):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(steps):
        if before:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def cpu_baseline(logits, target, budget_s, mid):
    """The oracle (as it stands) on the first rows of the batch, chunk by
    chunk until about budget_s seconds of wall time have been spent, on all
    its OpenMP threads; then one thread on the first rows of the mid
    workload for a fifth of that budget."""
    import numpy as np
    from oracle import ce_oracle as O
    from synth.ce_inputs import to_numpy_logits

    def run(z_dev, t_dev, budget, chunk):
        n_valid = int((t_dev != -100).sum().item())
        t_host = t_dev.cpu().numpy()
        rows = read_rows = 0
        secs = 0.0
        while secs < budget and rows < z_dev.shape[0]:
            z = to_numpy_logits(z_dev[rows:rows + chunk])
            t = np.ascontiguousarray(t_host[rows:rows + chunk])
            t0 = time.perf_counter()
            O.fwd_bwd(z, t, reduction="mean", n_valid=n_valid)
            secs += time.perf_counter() - t0
            rows += z.shape[0]
            read_rows += int((t != -100).sum())
        Vz = z_dev.shape[1]
        es = z_dev.element_size()
        return rows, secs, fused_bytes(rows, Vz, read_rows, es, es) / secs / 1e9

    threads = O.threads()
    rows, secs, gbs = run(logits, target, budget_s, 256)
    O.set_threads(1)
    try:
        mrows, msecs, mgbs = run(mid[0], mid[1], budget_s / 5, 32)
    finally:
        O.set_threads(threads)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {logits.shape[0]} rows (V={logits.shape[1]} bf16), "
                      f"fp64 forward + gradient, {secs:.1f} s on {threads} threads",
            "per_core": {"value": round(mgbs, 4), "unit": "GB/s", "cores": 1,
                         "sample": f"first {mrows} of {mid[0].shape[0]} rows of the mid "
                                   f"workload (V={mid[0].shape[1]} bf16), {msecs:.1f} s"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-split", action="store_true", help="skip the split-V measurement")
    ap.add_argument("--no-linear", action="store_true", help="skip the linear-classifier run")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the separate forward / backward measurement")
    ap.add_argument("--no-small", action="store_true", help="skip the tiny and mid workloads")
    ap.add_argument("--no-inplace", action="store_true", help="skip the in-place measurement")
    ap.add_argument("--no-memory", action="store_true", help="skip the peak-memory calls")
    ap.add_argument("--no-hash", action="store_true", help="skip the input SHA-256")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy of known size (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no "
              "collectives; the split-vocabulary measurement shows one GPU's shard of a "
              "vocabulary-parallel step", file=sys.stderr)
        sys.exit(2)

    import torch
    from vocab_softmax_cross_row_amd import _binding as B
    from synth import ce_inputs as S

    def say(msg):
        print(msg, file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    case = S.PAGE
    logits, target = S.generate(case, device=dev, block_rows=2048)
    n_read = T - case.n_ignored
    grad = torch.empty_like(logits)
    prob = B.make_problem(T, V, ignore_index=case.ignore_index, reduction="mean")
    nws = B.ce_workspace_bytes(prob, B.CE_OP_FUSED)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    loss_rows = torch.empty(T, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev)
    err = torch.empty(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step():
        B.ce_fused_fwd_bwd(prob, logits, B.CE_BF16, target, None, loss_rows, loss, n_valid, err,
                           grad, B.CE_BF16, V, ws, nws, stream)

    per, span, wall = time_steps(step, args.steps, args.warmup, stream)
    ms = span / args.steps
    nbytes = fused_bytes(T, V, n_read)
    gbs = nbytes / (ms * 1e-3) / 1e9
    timing = stats_ms(per)
    say(f"# fused: {ms:.4f} ms/step (events), {wall / args.steps * 1e3:.4f} ms/step (wall), "
        f"median {timing['median_ms']:.4f}, min {timing['min_ms']:.4f}, max "
        f"{timing['max_ms']:.4f}; loss {loss.item():.6f}, n_valid {n_valid.item()}")

    # the fused kernel alone: events the library records around the step's
    # main kernel on the launch stream (ce_fused_fwd_bwd_timed), per step
    pairs = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)  # torch times only events it has seen recorded; the
        b.record(stream)  # library records them again around the kernel
        pairs.append((a, b))
    torch.cuda.synchronize()
    for a, b in pairs:
        B.ce_fused_fwd_bwd_timed(prob, logits, B.CE_BF16, target, None, loss_rows, loss, n_valid,
                                 err, grad, B.CE_BF16, V, ws, nws, stream, a.cuda_event,
                                 b.cuda_event)
    torch.cuda.synchronize()
    kms = statistics.fmean(a.elapsed_time(b) for a, b in pairs)
    kgbs = nbytes / (kms * 1e-3) / 1e9
    say(f"# fused kernel alone: {kms * 1e3:.1f} us per launch (events around it)")

    inputs = {}
    if not args.no_hash:
        inputs["page"] = {"logits_sha256": sha256_of(logits), "target_sha256": sha256_of(target),
                          "seed": case.seed}

    small = None
    mid_inputs = None
    if not args.no_small or not args.no_cpu:
        mid_inputs = S.generate(S.MID, device=dev)
    if not args.no_small:
        # each call alone after a 512 MiB write that evicts L2 and the MALL
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        small = {}
        for c, (lg, tg) in ((S.TINY, S.generate(S.TINY, device=dev)), (S.MID, mid_inputs)):
            Tc, Vc = lg.shape
            pc = B.make_problem(Tc, Vc, ignore_index=c.ignore_index, reduction=c.reduction)
            nwc = B.ce_workspace_bytes(pc, B.CE_OP_FUSED)
            wsc = torch.empty(max(nwc, 1), dtype=torch.uint8, device=dev)
            gc = torch.empty_like(lg)
            dt = B.dtype_code(lg.dtype)
            lc = torch.empty(1, dtype=torch.float32, device=dev)
            lrc = torch.empty(Tc, dtype=torch.float32, device=dev)
            nvc = torch.empty(1, dtype=torch.int32, device=dev)
            ec = torch.empty(1, dtype=torch.int32, device=dev)

            def call():
                B.ce_fused_fwd_bwd(pc, lg, dt, tg, None, lrc, lc, nvc, ec, gc, dt, Vc, wsc, nwc,
                                   stream)

            times = time_each(call, args.steps, args.warmup, stream, before=flush.zero_)
            st = stats_ms(times)
            nr = int((tg != c.ignore_index).sum().item())
            b = fused_bytes(Tc, Vc, nr, lg.element_size(), gc.element_size())
            ent = {"workload": f"{c.name}: {Tc} x {Vc} {str(lg.dtype).split('.')[-1]}, fused, "
                               "caches flushed before each call",
                   "median_us": round(st["median_ms"] * 1e3, 2),
                   "min_us": round(st["min_ms"] * 1e3, 2), "max_us": round(st["max_ms"] * 1e3, 2),
                   "steps": st["n"], "algorithmic_bytes": b,
                   "GB/s_median": round(b / (st["median_ms"] * 1e-3) / 1e9, 1),
                   "frac_of_peak_median": round(b / (st["median_ms"] * 1e-3) / 1e9
                                                / PEAK_HBM_GBS, 4)}
            if not args.no_hash:
                inputs[c.name] = {"logits_sha256": sha256_of(lg), "target_sha256": sha256_of(tg),
                                  "seed": c.seed}
            small[c.name] = ent
            say(f"# {c.name}: median {ent['median_us']} us (min {ent['min_us']}, "
                f"max {ent['max_us']})")
            del wsc, gc
        del flush

    split = None
    if not args.no_split:
        half = V // 2
        eps = 0.1
        p1 = B.make_problem(T, half, V, vocab_start=0, V_total=V, label_smoothing=eps)
        p2 = B.make_problem(T, V - half, V, vocab_start=half, V_total=V, label_smoothing=eps)
        pm = B.make_problem(T, 1, 1, V_total=V, label_smoothing=eps)
        nfw = max(B.ce_workspace_bytes(p1, B.CE_OP_FORWARD),
                  B.ce_workspace_bytes(p2, B.CE_OP_FORWARD))
        nmw = B.ce_workspace_bytes(pm, B.CE_OP_MERGE)
        wsf = torch.empty(max(nfw, 1), dtype=torch.uint8, device=dev)
        wsm = torch.empty(max(nmw, 1), dtype=torch.uint8, device=dev)
        stats = torch.empty((2, T, B.ROW_STATS_BYTES), dtype=torch.uint8, device=dev)
        fin = torch.empty((T, B.ROW_FINAL_BYTES), dtype=torch.uint8, device=dev)
        l2 = logits[:, half:]
        g2 = grad[:, half:]

        def split_step():
            B.ce_forward(p1, logits, B.CE_BF16, target, stats[0], None, None, None, None, None,
                         wsf, nfw, stream)
            B.ce_forward(p2, l2, B.CE_BF16, target, stats[1], None, None, None, None, None,
                         wsf, nfw, stream)
            B.ce_merge_shard_stats(pm, 2, stats, target, fin, loss_rows, loss, n_valid, err,
                                   wsm, nmw, stream)
            B.ce_backward(p1, logits, B.CE_BF16, target, fin, n_valid, None, grad, B.CE_BF16, V,
                          stream)
            B.ce_backward(p2, l2, B.CE_BF16, target, fin, n_valid, None, g2, B.CE_BF16, V,
                          stream)

        sper, sspan, _ = time_steps(split_step, args.steps, args.warmup, stream)
        sms = sspan / args.steps
        sb = split_bytes(T, V, n_read)
        split = {"workload": "2 shards x 64128 columns, label_smoothing 0.1", "steps": args.steps,
                 "ms_per_step": round(sms, 4), "timing": stats_ms(sper),
                 "GB/s": round(sb / (sms * 1e-3) / 1e9, 1), "algorithmic_bytes": sb,
                 "frac_of_peak": round(sb / (sms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        say(f"# split-V: {sms:.4f} ms/step")
        del wsf, wsm, stats, fin

    in_place = None
    if not args.no_inplace:
        # the gradient written over the logits: a working copy is restored
        # from the batch before every call, outside the timed events
        work = torch.empty_like(logits)

        def restore():
            work.copy_(logits)

        def ip_call():
            B.ce_fused_fwd_bwd(prob, work, B.CE_BF16, target, None, loss_rows, loss, n_valid, err,
                               work, B.CE_BF16, V, ws, nws, stream)

        times = time_each(ip_call, args.steps, args.warmup, stream, before=restore)
        st = stats_ms(times)
        in_place = {"workload": "fused, gradient written over the logits", "timing": st,
                    "GB/s_mean": round(nbytes / (st["mean_ms"] * 1e-3) / 1e9, 1),
                    "frac_of_peak_mean": round(nbytes / (st["mean_ms"] * 1e-3) / 1e9
                                               / PEAK_HBM_GBS, 4)}
        say(f"# in place: {st['mean_ms']:.4f} ms/call")
        del work

    unfused = None
    if not args.no_unfused:
        pu = B.make_problem(T, V, ignore_index=case.ignore_index, reduction="mean")
        nuw = B.ce_workspace_bytes(pu, B.CE_OP_FORWARD)
        wsu = torch.empty(max(nuw, 1), dtype=torch.uint8, device=dev)
        ustats = torch.empty((T, B.ROW_STATS_BYTES), dtype=torch.uint8, device=dev)
        ufin = torch.empty((T, B.ROW_FINAL_BYTES), dtype=torch.uint8, device=dev)

        def fwd_only():
            B.ce_forward(pu, logits, B.CE_BF16, target, ustats, ufin, loss_rows, loss, n_valid,
                         err, wsu, nuw, stream)

        def bwd_only():
            B.ce_backward(pu, logits, B.CE_BF16, target, ufin, n_valid, None, grad, B.CE_BF16, V,
                          stream)

        res = {}
        for name, fn in (("forward", fwd_only), ("backward", bwd_only)):
            p, span_, _ = time_steps(fn, args.steps, args.warmup, stream)
            res[name] = (span_ / args.steps, stats_ms(p))
        fb = n_read * V * 2
        bb = n_read * V * 2 + T * V * 2
        fms, bms = res["forward"][0], res["backward"][0]
        unfused = {"workload": "ce_forward (whole vocabulary) then ce_backward, no smoothing",
                   "steps": args.steps,
                   "forward_ms": round(fms, 4), "forward_timing": res["forward"][1],
                   "forward_GB/s": round(fb / (fms * 1e-3) / 1e9, 1),
                   "forward_frac_of_peak": round(fb / (fms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "backward_ms": round(bms, 4), "backward_timing": res["backward"][1],
                   "backward_GB/s": round(bb / (bms * 1e-3) / 1e9, 1),
                   "backward_frac_of_peak": round(bb / (bms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "forward_bytes": fb, "backward_bytes": bb}
        say(f"# unfused: forward {fms:.4f} ms, backward {bms:.4f} ms")
        del wsu, ustats, ufin

    linear = None
    if not args.no_linear:
        lc = S.LINEAR
        E, Cw, tl = S.generate_linear(lc, device=dev)
        lp = B.make_linear_problem(lc.N, lc.D, lc.V, ignore_index=lc.ignore_index)
        nlw = B.ce_linear_workspace_bytes(lp, 1)
        lws = torch.empty(nlw, dtype=torch.uint8, device=dev)
        lrows = torch.empty(lc.N, dtype=torch.float32, device=dev)
        dE = torch.empty((lc.N, lc.D), dtype=torch.float32, device=dev)
        dC = torch.empty((lc.V, lc.D), dtype=torch.float32, device=dev)

        def linear_step():
            B.ce_linear_fwd_bwd(lp, E, Cw, tl, None, lrows, loss, n_valid, err, dE, dC, lws,
                                nlw, stream)

        klin = max(2, args.steps // 4)
        lper, lspan, _ = time_steps(linear_step, klin, 2, stream)
        lms = lspan / klin
        flops = 4 * 2 * lc.N * lc.V * lc.D
        tfs = flops / (lms * 1e-3) / 1e12
        linear = {"workload": f"E [{lc.N}, {lc.D}] x C [{lc.V}, {lc.D}] bf16, loss + dE + dC "
                              "(fp32), logits never stored",
                  "steps": klin, "ms_per_step": round(lms, 3), "timing": stats_ms(lper),
                  "TFLOP/s": round(tfs, 1), "algorithmic_flops": flops,
                  "peak_TFLOP/s": PEAK_BF16_TFS, "frac_of_peak": round(tfs / PEAK_BF16_TFS, 4),
                  "workspace_bytes": nlw, "loss": round(loss.item(), 6)}
        if not args.no_hash:
            inputs["linear"] = {"E_sha256": sha256_of(E), "C_sha256": sha256_of(Cw),
                                "target_sha256": sha256_of(tl), "seed": lc.seed}
        say(f"# linear CE: {lms:.3f} ms/step, {tfs:.1f} TFLOP/s, workspace {nlw / GIB:.3f} GiB")

        # the same call with gradient filtering at 2^-8 (256 x 256 blocks of
        # softmax - q whose entries are all below it skipped in the backward)
        tau = 2.0 ** -8
        fp = B.make_linear_problem(lc.N, lc.D, lc.V, ignore_index=lc.ignore_index,
                                   filter_eps=tau)
        nfw_ = B.ce_linear_workspace_bytes(fp, 1)
        fws = torch.empty(nfw_, dtype=torch.uint8, device=dev)

        def filtered_step():
            B.ce_linear_fwd_bwd(fp, E, Cw, tl, None, lrows, loss, n_valid, err, dE, dC, fws,
                                nfw_, stream)

        fper, fspan, _ = time_steps(filtered_step, klin, 2, stream)
        fms = fspan / klin
        linear["filtered"] = {
            "filter_eps": tau, "ms_per_step": round(fms, 3), "timing": stats_ms(fper),
            "saved_ms": round(lms - fms, 3), "speedup": round(lms / fms, 3),
            "TFLOP/s_of_exact_flops": round(flops / (fms * 1e-3) / 1e12, 1),
            "workspace_bytes": nfw_}
        say(f"# linear CE filtered at 2^-8: {fms:.3f} ms/step ({lms / fms:.3f}x)")
        del lws, fws, dE, dC

    memory = None
    if not args.no_memory:
        # peak of one call of each path: what it allocates plus its inputs
        import vocab_softmax_cross_row_amd as vce
        del grad
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

        def peak(fn, input_bytes):
            torch.cuda.synchronize()
            base = torch.cuda.memory_allocated() - input_bytes
            torch.cuda.reset_peak_memory_stats()
            fn()
            torch.cuda.synchronize()
            return round((torch.cuda.max_memory_allocated() - base) / GIB, 3)

        page_in = logits.numel() * 2 + target.numel() * 8
        memory = {"unit": "GiB",
                  "fused": peak(lambda: vce.fused_fwd_bwd(logits, target), page_in),
                  "in_place": peak(lambda: vce.fused_fwd_bwd(logits, target, grad=logits),
                                   page_in),
                  "note": "one call, inputs included"}
        # the batch now holds gradients: draw it again for the split path
        logits, target = S.generate(case, device=dev, block_rows=2048)
        torch.cuda.synchronize()

        def split_call():
            half = V // 2
            st = [vce.forward(logits[:, a:b], target, vocab_start=a, V_total=V,
                              label_smoothing=0.1)["stats"] for a, b in ((0, half), (half, V))]
            m = vce.merge_shard_stats(st, target, V, label_smoothing=0.1)
            g = torch.empty_like(logits)
            for a, b in ((0, half), (half, V)):
                vce.backward(logits[:, a:b], target, m["fin"], m["n_valid"], vocab_start=a,
                             V_total=V, label_smoothing=0.1, grad=g[:, a:b])

        memory["split_v"] = peak(split_call, page_in)
        if linear is not None:
            lin_in = E.numel() * 2 + Cw.numel() * 2 + tl.numel() * 8
            memory["linear_ce"] = peak(lambda: vce.linear_cross_entropy(E, Cw, tl), lin_in)
        say(f"# memory: {memory}")

    if args.copy_calibration:
        # a plain device copy of known size for scaling the HBM counters
        buf = torch.empty_like(logits)
        src = logits.view(torch.uint8).reshape(-1)[: 1 << 31]
        dst = buf.view(torch.uint8).reshape(-1)[: 1 << 31]
        dst.copy_(src)
        torch.cuda.synchronize()
        say(f"# copy calibration: {src.numel()} bytes read, {dst.numel()} written")
        del buf

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(logits, target, args.cpu_seconds, mid_inputs)

    out = {
        "metric": "CE fwd+bwd ms and HBM GB/s (% roofline), T=16384 V=128256 bf16, 1 GPU",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "page-scale CE, fused forward+backward (ce_fused_fwd_bwd)",
                   "T": T, "V": V, "logits_dtype": "bf16", "grad_dtype": "bf16",
                   "math": "fp32 (fp64 per-row finalize)",
                   "reduction": "mean", "ignored_rows": case.n_ignored,
                   "confident_rows": case.n_margin, "logits": "N(0, 3^2), seed 1003"},
        "timing": timing,
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic(), "algorithmic_bytes": nbytes,
                     "algorithmic_bytes_all_rows_read": fused_bytes(T, V),
                     "kernel": "k_fused_lds", "kernel_us": round(kms * 1e3, 1),
                     "step_frac": round(gbs / PEAK_HBM_GBS, 4)},
        "inputs": inputs,
        "host": host_info(),
        "cpu_baseline": cpu,
        "configs": small,
        "split_v": split,
        "in_place": in_place,
        "unfused": unfused,
        "linear_ce": linear,
        "memory": memory,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
