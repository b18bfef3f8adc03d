"""Benchmark: fused stable softmax cross-entropy forward + backward on one
MI355X, page-scale workload (T = 16384 tokens, V = 128256, bf16 logits and
bf16 gradient, mean over non-ignored rows; the shapes of the H100 table in
torchtitan PR "[loss] fix softmax collapse with improved ce perf").

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one ce_fused_fwd_bwd call over the resident batch: the count
pre-pass, the row-resident fused kernel (max, non-target sum, finalize,
gradient) and the loss reduction.  Inputs are generated on the GPU from a
fixed seed before timing and stay in HBM.  Prints one JSON line.

Extra objects in the line:
  roofline      HBM roofline of the fused kernel: algorithmic bytes of one
                launch / its average duration, from HIP events the library
                records around it on the launch stream (ce_set_fused_events;
                the step also holds the target count and the loss reduction,
                about 12 us); peak 8 TB/s.  traffic is the HBM byte count the
                rocprofv3 FETCH_SIZE / WRITE_SIZE counters gave for this
                kernel source (profiles/fused_page_counters.md), or null if
                the kernel source changed since.
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of the
                same workload (the first rows of the batch), in GB/s of the
                same algorithmic bytes.
  split_v       the vocabulary split in two 64128-column shards with label
                smoothing 0.1: ce_forward per shard, ce_merge_shard_stats,
                ce_backward per shard, timed the same way.
  unfused       the same batch through ce_forward (whole vocabulary: row
                statistics, finalize, loss) and then ce_backward, no
                smoothing; bytes: one read for the forward, a read and a
                write for the backward.
  linear_ce     cross-entropy of a linear classifier without stored logits
                (ce_linear_fwd_bwd): E [8192, 2048] and C [128256, 2048] bf16,
                loss + dE + dC; MFMA roofline: 4 products of 2 N V D flops
                (forward logits, recomputed logits, dE, dC) against the
                2.5 PFLOP/s dense bf16 peak.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
T, V = 16384, 128256
COUNTERS = os.path.join(ROOT, "profiles", "fused_page_counters.md")
# the sources the fused kernels are built from (their launch arguments and the
# device helpers); counter figures are reported only while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "vocab_softmax_cross_row_amd", "csrc", f)
                  for f in ("ce_fused.hip", "ce_device.h")]


def fused_bytes(T, V, in_size=2, out_size=2):
    """Algorithmic bytes of one fused launch: every logit read once, every
    gradient written once, plus per row the int64 target and the fp32 loss."""
    return T * V * (in_size + out_size) + T * (8 + 4)


def split_bytes(T, V, in_size=2, out_size=2):
    """Split-vocabulary path: forward reads the logits, backward reads them
    again and writes the gradient (per row: target twice, 32-byte stats per
    shard, 24-byte row constants; negligible)."""
    return T * V * (2 * in_size + out_size)


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


def cpu_baseline(logits, target, budget_s):
    """The oracle (as it stands) on the first rows of the batch, chunk by
    chunk until about budget_s seconds of wall time have been spent."""
    import numpy as np
    from oracle import ce_oracle as O
    from synth.ce_inputs import to_numpy_logits
    n_valid = int((target != -100).sum().item())
    rows, secs = 0, 0.0
    chunk = 256
    t_host = target.cpu().numpy()
    while secs < budget_s and rows < logits.shape[0]:
        z = to_numpy_logits(logits[rows:rows + chunk])
        t = np.ascontiguousarray(t_host[rows:rows + chunk])
        t0 = time.perf_counter()
        O.fwd_bwd(z, t, reduction="mean", n_valid=n_valid)
        secs += time.perf_counter() - t0
        rows += z.shape[0]
    gbs = fused_bytes(rows, logits.shape[1]) / secs / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": O.threads(), "kind": "oracle",
            "sample": f"first {rows} of {logits.shape[0]} rows (V={logits.shape[1]} bf16), "
                      f"fp64 forward + gradient, {secs:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-split", action="store_true", help="skip the split-V measurement")
    ap.add_argument("--no-linear", action="store_true", help="skip the linear-classifier run")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the separate forward / backward measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy of known size (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no "
              "collectives; the split-vocabulary measurement shows one GPU's shard of a "
              "vocabulary-parallel step", file=sys.stderr)
        sys.exit(2)

    import torch
    import vocab_softmax_cross_row_amd as vce
    from vocab_softmax_cross_row_amd import _binding as B
    from synth import ce_inputs as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    case = S.PAGE
    logits, target = S.generate(case, device=dev, block_rows=2048)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = fused_bytes(T, V)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"# fused: {ms:.4f} ms/step (events), {wall / args.steps * 1e3:.4f} ms/step (wall), "
          f"loss {loss.item():.6f}, n_valid {n_valid.item()}", file=sys.stderr, flush=True)

    # the fused kernel alone: the library records a pair of HIP events on the
    # launch stream around the step's main kernel (ce_set_fused_events), one
    # pair per step, over another K steps
    pairs = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    for a, b in pairs:
        B.ce_set_fused_events(a.cuda_event, b.cuda_event)
        step()
    B.ce_set_fused_events(None, None)
    torch.cuda.synchronize()
    kms = sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
    kgbs = fused_bytes(T, V) / (kms * 1e-3) / 1e9
    print(f"# fused kernel alone: {kms * 1e3:.1f} us per launch (events around it)",
          file=sys.stderr, flush=True)

    split = None
    if not args.no_split:
        half = V // 2
        eps = 0.1
        p1 = B.make_problem(T, half, V, vocab_start=0, V_total=V, label_smoothing=eps)
        p2 = B.make_problem(T, V - half, V, vocab_start=half, V_total=V, label_smoothing=eps)
        pm = B.make_problem(T, 1, 1, V_total=V, label_smoothing=eps)
        nfw = max(B.ce_workspace_bytes(p1, B.CE_OP_FORWARD), B.ce_workspace_bytes(p2, B.CE_OP_FORWARD))
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

        ksplit = max(1, args.steps // 5)
        for _ in range(max(1, args.warmup // 2)):
            split_step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(ksplit):
            split_step()
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / ksplit
        sb = split_bytes(T, V)
        split = {"workload": "2 shards x 64128 columns, label_smoothing 0.1", "steps": ksplit,
                 "ms_per_step": round(sms, 4), "GB/s": round(sb / (sms * 1e-3) / 1e9, 1),
                 "algorithmic_bytes": sb, "frac_of_peak": round(sb / (sms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        print(f"# split-V: {sms:.4f} ms/step", file=sys.stderr, flush=True)

    unfused = None
    if not args.no_unfused:
        # the same batch through the separate calls: ce_forward over the whole
        # vocabulary (statistics, finalize, loss), then ce_backward
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

        ku = max(1, args.steps // 5)
        times = {}
        for name, fn in (("forward", fwd_only), ("backward", bwd_only)):
            for _ in range(max(1, args.warmup // 2)):
                fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(ku):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times[name] = e0.elapsed_time(e1) / ku
        fb, bb = T * V * 2, T * V * 4
        unfused = {"workload": "ce_forward (whole vocabulary) then ce_backward, no smoothing",
                   "steps": ku,
                   "forward_ms": round(times["forward"], 4),
                   "forward_GB/s": round(fb / (times["forward"] * 1e-3) / 1e9, 1),
                   "forward_frac_of_peak": round(fb / (times["forward"] * 1e-3) / 1e9
                                                 / PEAK_HBM_GBS, 4),
                   "backward_ms": round(times["backward"], 4),
                   "backward_GB/s": round(bb / (times["backward"] * 1e-3) / 1e9, 1),
                   "backward_frac_of_peak": round(bb / (times["backward"] * 1e-3) / 1e9
                                                  / PEAK_HBM_GBS, 4),
                   "forward_bytes": fb, "backward_bytes": bb}
        print(f"# unfused: forward {times['forward']:.4f} ms, backward {times['backward']:.4f} ms",
              file=sys.stderr, flush=True)

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

        klin = max(1, args.steps // 10)
        for _ in range(2):
            linear_step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(klin):
            linear_step()
        e1.record(stream)
        torch.cuda.synchronize()
        lms = e0.elapsed_time(e1) / klin
        flops = 4 * 2 * lc.N * lc.V * lc.D
        tfs = flops / (lms * 1e-3) / 1e12
        linear = {"workload": f"E [{lc.N}, {lc.D}] x C [{lc.V}, {lc.D}] bf16, loss + dE + dC "
                              "(fp32), logits never stored",
                  "steps": klin, "ms_per_step": round(lms, 3), "TFLOP/s": round(tfs, 1),
                  "algorithmic_flops": flops, "peak_TFLOP/s": 2500.0,
                  "frac_of_peak": round(tfs / 2500.0, 4), "loss": round(loss.item(), 6)}
        print(f"# linear CE: {lms:.3f} ms/step, {tfs:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del E, Cw, lws, dE, dC

    if args.copy_calibration:
        # a plain device copy of known size for scaling the HBM counters
        src = logits.view(torch.uint8).reshape(-1)[: 1 << 31]
        dst = grad.view(torch.uint8).reshape(-1)[: 1 << 31]
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy calibration: {src.numel()} bytes read, {dst.numel()} written",
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(logits, target, args.cpu_seconds)

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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "page-scale CE, fused forward+backward (ce_fused_fwd_bwd)",
                   "T": T, "V": V, "logits_dtype": "bf16", "grad_dtype": "bf16",
                   "reduction": "mean", "ignored_rows": case.n_ignored,
                   "confident_rows": case.n_margin, "logits": "N(0, 3^2), seed 1003"},
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic(), "algorithmic_bytes": nbytes,
                     "kernel": "k_fused_lds", "kernel_us": round(kms * 1e3, 1)},
        "cpu_baseline": cpu,
        "split_v": split,
        "unfused": unfused,
        "linear_ce": linear,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
