"""Benchmark of the Ulysses per-rank hot path on one MI355X.

One step = one Ulysses attention layer, forward and backward, for all sp
virtual ranks of the workload held on this GPU (default: the long-context
workload, B=1, N=131072, H=32, sp=8, d=128, bf16, causal):
  seq_to_head(q, k, v)  (one launch) 8 shards [16384, 32, 128] -> 8 shares [131072, 4, 128]
  attn_fwd over the 8 shares         saves lse only
  head_to_seq(o), seq_to_head(dO)
  attn_bwd over the 8 shares         D pre-pass, then dK/dV + dQ kernels (two calls)
  head_to_seq(dq, dk, dv)  (one launch)
Inputs are seeded synthetic tensors already resident in HBM. The timed steps
(wall clock between two device synchronisations) carry HIP events around the
backward call alone, the roofline's kernel; a second pass of as many steps
times every call with HIP events on the stream it runs on.

value = causal attention FLOPs counted as 14 * d * pairs (4 d forward, 10 d
backward; pairs = sum over documents of L (L + 1) / 2 per row and head)
divided by the whole step's time, in TFLOP/s. The config also carries the
same time counted as 12 * d * pairs (no recompute of S counted), the permute
bandwidth next to a plain device-to-device copy of one tensor of the same
size timed in the same run, and the per-call averages.

With --variant ring the step is ring attention instead (the other
sequence-parallel mode): the same q, k, v, dO sequence shards, no layout
change; sp forward ring steps (each rank's queries against the key/value
chunk passed to it, partial results merged by log-sum-exp), the D pre-pass,
then sp backward ring steps. Same FLOP count, same value definition.

With --variant tiledmlp it times ALST's tiled MLP instead: the Llama-7B
SwiGLU FFN (hidden 4096, inter 11008) over every virtual rank's token shard
of the workload (sp x B x N/sp tokens, one call with the shared weights, the
same work as sp rank calls plus the sum of their weight gradients), in tiles
of --mlp-tile tokens: forward and backward per step. value = FLOPs counted as
22 * hidden * inter per token (forward 6, backward 12, plus the forward's
gate and up products recomputed per tile, 4) per second.

With --variant loss it times the sequence-parallel loss aggregation on the
workload's tokens instead (sp ranks x B rows x N/sp tokens: per-token fp32
losses and int64 labels, 30% of them -100): value = bytes read (12 per
token) per second, against the HBM peak.

Prints one JSON line. --gpus above 1 exits: this build measures one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

import numpy as np
import torch

import workloads
import ulysses_sequence_parallelism_seq_amd as uly
from ulysses_sequence_parallelism_seq_amd.traffic import read_traffic

TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "attn_bwd_long_traffic.txt")

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk/CU)
PEAK_HBM_GBS = 8000.0


def causal_pairs(w: workloads.Workload) -> int:
    cu = workloads.workload_cu_seqlens(w)
    lengths = [w.N] if cu is None else np.diff(cu).tolist()
    if w.causal:
        return sum(L * (L + 1) // 2 for L in lengths)
    return sum(L * L for L in lengths)


def make_inputs(w: workloads.Workload, dev):
    """Full-H sequence shards of q, k, v, dO drawn on the device from one seeded generator."""
    g = torch.Generator(device=dev).manual_seed(w.seed)
    shape = workloads.seq_shard_shape(w)
    out = []
    for _ in range(4):
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if w.scale != 1.0:
            x.mul_(w.scale)
        out.append(x.to(workloads.torch_dtype(w.dtype)))
        del x
    return out


def make_buffers(w: workloads.Workload, dev):
    """Inputs (sequence shards) and every buffer one step writes, allocated once."""
    seq_in = make_inputs(w, dev)
    head_shape = (w.sp, w.B, w.N, w.Hl, w.d)
    dt = workloads.torch_dtype(w.dtype)
    return {
        "seq_in": seq_in,
        "head_in": [torch.empty(head_shape, dtype=dt, device=dev) for _ in range(4)],
        "head_out": [torch.empty(head_shape, dtype=dt, device=dev),
                     torch.empty((w.sp, w.B, w.Hl, w.N), dtype=torch.float32, device=dev)]
                    + [torch.empty(head_shape, dtype=dt, device=dev) for _ in range(3)],
        "seq_out": [torch.empty_like(seq_in[0]) for _ in range(4)],
        "fws": torch.empty(uly.ulysses_attn_fwd_workspace_bytes(), dtype=torch.uint8, device=dev),
        "ws": torch.empty(uly.ulysses_attn_bwd_workspace_bytes(w.sp, w.B, w.N, w.Hl, w.d, dt),
                          dtype=torch.uint8, device=dev),
    }


class Timer:
    """HIP-event timing of each named call (per-call median); with `only`, of those names alone."""

    def __init__(self, stream, only=None):
        self.stream = stream
        self.only = only
        self.pending = []

    def run(self, name, fn):
        if self.only is not None and name not in self.only:
            return fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        out = fn()
        b.record(self.stream)
        self.pending.append((name, a, b))
        return out

    def averages(self):
        """Median duration (ms) of each named call, and how many were timed."""
        acc = {}
        for name, a, b in self.pending:
            acc.setdefault(name, []).append(a.elapsed_time(b))
        return {k: statistics.median(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def timed_steps(one_step, steps, stream, live):
    """Wall time (s) of `steps` steps between two device synchronisations, with HIP events only
    around the calls named in `live` (the roofline's kernel), and their medians; then the per-call
    medians of a second pass of as many steps with events around every call. (An event pair
    adds a gap of a few microseconds: around all 13 calls, 7% of a 1.5 ms llama7b step.)"""
    live_timer = Timer(stream, only=set(live))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step(live_timer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timer = Timer(stream)
    for _ in range(steps):
        one_step(timer)
    torch.cuda.synchronize()
    avg, counts = timer.averages()
    live_avg, live_counts = live_timer.averages()
    avg.update(live_avg)
    counts.update(live_counts)
    return elapsed, avg, counts


def step(w, bufs, packing, timer=None):
    run = timer.run if timer else (lambda name, fn: fn())
    qs, ks, vs, dos = bufs["seq_in"]
    qh, kh, vh, doh = bufs["head_in"]
    o, lse, dq, dk, dv = bufs["head_out"]
    os_, dqs, dks, dvs = bufs["seq_out"]
    ws = bufs["ws"]
    # q, k and v go into the exchange together: one launch for the three
    run("seq_to_head_x3", lambda: uly.ulysses_seq_to_head_n([qs, ks, vs], [qh, kh, vh]))
    run("attn_fwd", lambda: uly.ulysses_attn_fwd(qh, kh, vh, packing, w.causal, out=o, lse=lse,
                                                 workspace=bufs["fws"]))
    run("head_to_seq", lambda: uly.ulysses_head_to_seq(o, out=os_))
    run("seq_to_head", lambda: uly.ulysses_seq_to_head(dos, out=doh))

    def bwd():  # ulysses_attn_bwd in its two steps: the D pre-pass, then the dK/dV and dQ kernels
        run("attn_bwd_prepare", lambda: uly.ulysses_attn_bwd_prepare(o, doh, lse, ws))
        run("attn_bwd_prepared", lambda: uly.ulysses_attn_bwd_prepared(qh, kh, vh, doh, lse, ws, packing,
                                                                       w.causal, dq=dq, dk=dk, dv=dv))
    run("attn_bwd", bwd)
    run("head_to_seq_x3", lambda: uly.ulysses_head_to_seq_n([dq, dk, dv], [dqs, dks, dvs]))


def make_ring_buffers(w: workloads.Workload, dev):
    """Ring variant: the sequence shards are the ring's chunks; fp32 running sums and bf16 outputs."""
    seq_in = make_inputs(w, dev)
    shape = workloads.seq_shard_shape(w)
    dt = workloads.torch_dtype(w.dtype)
    f32 = lambda: torch.empty(shape, dtype=torch.float32, device=dev)  # noqa: E731
    return {
        "seq_in": seq_in,
        "o": torch.empty(shape, dtype=dt, device=dev),
        "o_acc": f32(),
        "lse": torch.empty((w.sp, w.B, w.H, w.Ns), dtype=torch.float32, device=dev),
        "grads": [torch.empty(shape, dtype=dt, device=dev) for _ in range(3)],
        "accs": [f32() for _ in range(3)],
        "ws": torch.empty(uly.ulysses_ring_attn_bwd_workspace_bytes(w.sp, w.B, w.Ns, w.H, w.d),
                          dtype=torch.uint8, device=dev),
        "fws": torch.empty(uly.ulysses_attn_fwd_workspace_bytes(), dtype=torch.uint8, device=dev),
    }


def ring_step(w, bufs, timer=None):
    run = timer.run if timer else (lambda name, fn: fn())
    q, k, v, do = bufs["seq_in"]
    o, o_acc, lse, ws = bufs["o"], bufs["o_acc"], bufs["lse"], bufs["ws"]
    dq, dk, dv = bufs["grads"]
    dqa, dka, dva = bufs["accs"]
    for i in range(w.sp):
        run("ring_fwd_step", lambda: uly.ulysses_ring_attn_fwd_step(q, k, v, i, w.causal, o, o_acc, lse,
                                                                     bufs["fws"]))
    run("ring_bwd_prepare", lambda: uly.ulysses_ring_attn_bwd_prepare(o, do, lse, ws))
    for i in range(w.sp):
        run("ring_bwd_step", lambda: uly.ulysses_ring_attn_bwd_step(q, k, v, do, lse, ws, i, w.causal,
                                                                     dqa, dka, dva, dq, dk, dv))


def _cpu_model() -> str:
    """The host CPU's model name, from lscpu (else /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        return "unknown"


def cpu_baseline(w: workloads.Workload, target_s: float):
    """The float64 oracle, fwd + bwd, timed on a causal prefix of one head (a
    bounded sample of about target_s seconds), and the time of the whole
    configuration extrapolated from it by the exact ratio of causal pairs."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=os.cpu_count())
    except Exception:  # threadpoolctl missing: report the visible cores
        threads = os.cpu_count()

    def run(M):
        q, k, v, do = workloads.qkv_do((1, M, 1, w.d), w.seed, w.dtype, w.scale)
        t0 = time.perf_counter()
        oracle.attn_fwd(q, k, v, None, True)
        oracle.attn_bwd(q, k, v, do, None, True)
        return time.perf_counter() - t0

    # cost grows as M^2: grow the prefix until a run takes a third of the target,
    # then size the measured run to take about target_s
    M = 2048
    t = run(M)
    while t < target_s / 3 and M < w.N:
        M = min(2 * M, w.N)
        t = run(M)
    M2 = max(2048, min(int(M * (target_s / max(t, 1e-3)) ** 0.5) // 256 * 256, w.N))
    if M2 > M:
        M, t = M2, run(M2)
    pairs_sample = M * (M + 1) // 2
    flops = 14 * w.d * pairs_sample
    pairs_head = causal_pairs(w)
    pairs_config = pairs_head * w.sp * w.B * w.Hl
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": _cpu_model(),
        "openblas_num_threads": os.environ.get("OPENBLAS_NUM_THREADS", "unset"),
        "omp_num_threads": os.environ.get("OMP_NUM_THREADS", "unset"),
        "kind": "oracle",
        "sample": f"float64 oracle fwd+bwd of one head, causal prefix of {M} of the {w.N} tokens "
                  f"({t:.1f} s; FLOPs counted as 14*d*pairs like the GPU value)",
        "sample_s": round(t, 2),
        "extrapolated_one_head_s": round(t * pairs_head / pairs_sample, 1),
        "extrapolated_config_s": round(t * pairs_config / pairs_sample, 1),
        "extrapolation": f"extrapolated by the exact causal pair ratio: one head {pairs_head} pairs, the whole "
                         f"configuration ({w.sp * w.B * w.Hl} rank x row x head units) {pairs_config} pairs, "
                         f"against {pairs_sample} in the sample",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--variant", default="ulysses", choices=["ulysses", "ring", "loss", "tiledmlp"])
    ap.add_argument("--mlp-tile", type=int, default=4096)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the sequence-parallel exchange across GPUs is not part of this build", file=sys.stderr)
        sys.exit(2)

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cu = workloads.workload_cu_seqlens(w)
    if args.variant == "loss":
        return loss_main(args, w, dev)
    if args.variant == "tiledmlp":
        return mlp_main(args, w, dev)
    if args.variant == "ring":
        if cu is not None or w.dtype != "bf16":
            print("the ring variant runs bf16 workloads with one document per row", file=sys.stderr)
            sys.exit(2)
        return ring_main(args, w, dev)
    packing = None if cu is None else uly.DocPacking(cu, w.N, dev)

    bufs = make_buffers(w, dev)
    seq_in = bufs["seq_in"]
    stream = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        step(w, bufs, packing)
    torch.cuda.synchronize()

    elapsed, avg, counts = timed_steps(lambda timer: step(w, bufs, packing, timer), args.steps, stream,
                                       live=("attn_bwd",))

    # reference for the permute: a plain device-to-device copy of one tensor of the same size
    copy_dst = torch.empty_like(seq_in[0])
    copy_timer = Timer(stream)
    for _ in range(5):
        copy_timer.run("copy", lambda: copy_dst.copy_(seq_in[0]))
    torch.cuda.synchronize()
    copy_ms = copy_timer.averages()[0]["copy"]
    del copy_dst

    ms_per_step = elapsed * 1e3 / args.steps
    pairs = causal_pairs(w) * w.sp * w.B * w.Hl  # all virtual ranks, batch rows, local heads
    flops_step = 14 * w.d * pairs
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    attn_ms = avg["attn_fwd"] + avg["attn_bwd"]
    esize = 2 if w.dtype == "bf16" else 4
    tensor_bytes = w.B * w.N * w.H * w.d * esize
    permute_gbs = 2 * tensor_bytes / (statistics.mean([avg["seq_to_head"], avg["head_to_seq"]]) * 1e-3) / 1e9
    bwd_tflops = 10 * w.d * pairs / (avg["attn_bwd"] * 1e-3) / 1e12
    traffic = read_traffic(TRAFFIC_FILE) if args.workload == "long" else None
    # compulsory bytes of one backward call: read q, k, v, o, dO, lse; write dq, dk, dv
    min_bwd_bytes = 8 * w.sp * w.B * w.N * w.Hl * w.d * esize + w.sp * w.B * w.Hl * w.N * 4
    fwd_tflops = 4 * w.d * pairs / (avg["attn_fwd"] * 1e-3) / 1e12

    result = {
        "metric": "causal attn fwd+bwd TFLOP/s per GPU (% bf16 MFMA peak); permute GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v/dO on the device)",
        "config": {
            "workload": f"{w.name}: B={w.B} N={w.N} H={w.H} sp={w.sp} (all {w.sp} virtual ranks on one GPU) "
                        f"Hl={w.Hl} d={w.d} {w.dtype} causal={w.causal} docs={w.docs}",
            "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "attn_fwd_ms": round(avg["attn_fwd"], 3),
            "attn_bwd_ms": round(avg["attn_bwd"], 3),
            "attn_bwd_prepare_ms": round(avg["attn_bwd_prepare"], 4),
            "attn_bwd_prepared_ms": round(avg["attn_bwd_prepared"], 3),
            # the D pre-pass reads O and dO (2 d esize per row) and lse, writes -D and lse2 (8 bytes)
            "attn_bwd_prepare_gbs": round(w.sp * w.B * w.Hl * w.N * (2 * w.d * esize + 12)
                                          / (avg["attn_bwd_prepare"] * 1e-3) / 1e9, 1),
            "timing": f"value: wall clock of {args.steps} steps with HIP events around attn_bwd only (its time: their median); other per-call times: HIP events around every call on the launch stream, medians over {args.steps} more steps",
            "attn_fwd_tflops": round(fwd_tflops, 1),
            "attn_bwd_tflops": round(bwd_tflops, 1),
            "attn_only_tflops": round(flops_step / (attn_ms * 1e-3) / 1e12, 1),
            "permute_ms": round(statistics.mean([avg["seq_to_head"], avg["head_to_seq"]]), 4),
            "permute_gbs": round(permute_gbs, 1),
            "permute_pct_of_hbm_peak": round(100 * permute_gbs / PEAK_HBM_GBS, 1),
            "d2d_copy_gbs": round(2 * tensor_bytes / (copy_ms * 1e-3) / 1e9, 1),
            # HBM bytes of one permute call from the rocprofv3 counters (calibrated on a plain
            # device copy), against the algorithmic read + write of every element
            "permute_counter_bytes": None if traffic is None else {
                k: round(v) for k, v in traffic["permute"].items()},
            "permute_counter_gbs": None if traffic is None else {
                k: round(v / (avg["seq_to_head" if k.endswith("head") else "head_to_seq"] * 1e-3) / 1e9, 1)
                for k, v in traffic["permute"].items()},
            "permute_algorithmic_bytes": 2 * tensor_bytes,
            # q, k, v (dq, dk, dv) in one launch of ulysses_seq_to_head_n (head_to_seq_n)
            "permute_x3_ms": {k: round(avg[k], 4) for k in ("seq_to_head_x3", "head_to_seq_x3")},
            "permute_x3_gbs": {k: round(3 * 2 * tensor_bytes / (avg[k] * 1e-3) / 1e9, 1)
                               for k in ("seq_to_head_x3", "head_to_seq_x3")},
            "value_12d_no_recompute": round(12 * w.d * pairs / (ms_per_step * 1e-3) / 1e12, 2),
            "flops_per_step": flops_step,
            "calls_timed": counts,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_bwd (D pre-pass + dK/dV + dQ kernels of one ulysses_attn_bwd call)",
            "achieved": round(bwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None if traffic is None else round(traffic["bytes"]),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated on a plain "
                            "device-to-device copy of known size)",
            "compulsory_bytes": min_bwd_bytes,
            "flops_per_launch": 10 * w.d * pairs,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def loss_main(args, w, dev):
    shape = (w.sp, w.B, w.Ns)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    token_loss = torch.rand(shape, generator=g, device=dev) * 8.0
    labels = torch.randint(0, 32000, shape, generator=g, device=dev, dtype=torch.int64)
    labels[torch.rand(shape, generator=g, device=dev) < 0.3] = -100
    out = uly.ulysses_sp_loss(token_loss, labels)
    ws = torch.empty(max(int(uly.library().ulysses_sp_loss_workspace_bytes(*shape)), 8), dtype=torch.uint8,
                     device=dev)
    calls = 200 * max(1, args.steps)
    stream = torch.cuda.current_stream(dev)
    for _ in range(20 * max(1, args.warmup)):
        uly.ulysses_sp_loss(token_loss, labels, workspace=ws, loss=out[0], rank_loss=out[1], good_tokens=out[2])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(calls):
        uly.ulysses_sp_loss(token_loss, labels, workspace=ws, loss=out[0], rank_loss=out[1], good_tokens=out[2])
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / calls
    nbytes = 12 * w.sp * w.B * w.Ns
    gbs = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "SP loss aggregation GB/s (bytes read per second)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": calls,
        "warmup": 20 * max(1, args.warmup),
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+int64 in, f64 sums",
        "data": "synthetic (seeded per-token losses, 30% of labels -100)",
        "config": {
            "workload": f"{w.name}'s tokens: sp={w.sp} ranks x B={w.B} x {w.Ns} tokens",
            "tokens": w.sp * w.B * w.Ns,
            "launches_per_call": 2,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "ulysses_sp_loss (partial + final kernels of one call)",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": None,
            "bytes_per_launch": nbytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        tl, lab = token_loss.cpu().numpy(), labels.cpu().numpy()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.sp_loss(tl, lab)
            reps += 1
        t = (time.perf_counter() - t0) / reps
        result["cpu_baseline"] = {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle", "sample": f"the float64 oracle on the same tokens, {reps} calls"}
    print(json.dumps(result), flush=True)


def mlp_main(args, w, dev):
    h, inter, tile = workloads.MLP_HIDDEN, workloads.MLP_INTER, args.mlp_tile
    tokens = w.sp * w.B * w.Ns
    g = torch.Generator(device=dev).manual_seed(w.seed)
    x = torch.randn((tokens, h), generator=g, device=dev).bfloat16()
    dy = torch.randn((tokens, h), generator=g, device=dev).bfloat16()
    wg = (torch.randn((inter, h), generator=g, device=dev) * h ** -0.5).bfloat16()
    wu = (torch.randn((inter, h), generator=g, device=dev) * h ** -0.5).bfloat16()
    wd = (torch.randn((h, inter), generator=g, device=dev) * inter ** -0.5).bfloat16()
    ws = torch.empty(uly.ulysses_tiled_mlp_workspace_bytes(tokens, h, inter, tile), dtype=torch.uint8, device=dev)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dwg = torch.empty((inter, h), device=dev)
    dwu = torch.empty((inter, h), device=dev)
    dwd = torch.empty((h, inter), device=dev)
    stream = torch.cuda.current_stream(dev)

    def one_step(timer=None):
        run = timer.run if timer else (lambda name, fn: fn())
        run("mlp_fwd", lambda: uly.ulysses_tiled_mlp_fwd(x, wg, wu, wd, tile, ws, y))
        run("mlp_bwd", lambda: uly.ulysses_tiled_mlp_bwd(x, wg, wu, wd, dy, tile, ws, dx, dwg, dwu, dwd))

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    elapsed, avg, counts = timed_steps(one_step, args.steps, stream, live=("mlp_bwd",))
    ms_per_step = elapsed * 1e3 / args.steps
    hi = h * inter * tokens
    flops_step = 22 * hi
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    bwd_tflops = 16 * hi / (avg["mlp_bwd"] * 1e-3) / 1e12
    result = {
        "metric": "tiled MLP fwd+bwd TFLOP/s per GPU (% bf16 MFMA peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0, 1/fan_in) weights, on the device)",
        "config": {
            "workload": f"SwiGLU FFN hidden={h} inter={inter} over {w.name}'s token shards: sp={w.sp} x B={w.B} x "
                        f"{w.Ns} = {tokens} tokens, tiles of {tile} tokens, bf16",
            "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "mlp_fwd_ms": round(avg["mlp_fwd"], 3),
            "mlp_bwd_ms": round(avg["mlp_bwd"], 3),
            "mlp_fwd_tflops": round(6 * hi / (avg["mlp_fwd"] * 1e-3) / 1e12, 1),
            "mlp_bwd_tflops": round(bwd_tflops, 1),
            "value_18hi_no_recompute": round(18 * hi / (ms_per_step * 1e-3) / 1e12, 2),
            "flops_per_step": flops_step,
            "calls_timed": counts,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "ulysses_tiled_mlp_bwd (per tile: gate/up recompute, dA, dX, dWd, dWg, dWu GEMMs)",
            "achieved": round(bwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": 16 * hi,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = mlp_cpu_baseline(h, inter, tokens, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def mlp_cpu_baseline(h, inter, tokens, target_s):
    """The float64 MLP oracle, fwd + bwd, on a bounded sample of tokens (about
    target_s seconds), extrapolated to every token by the token ratio (its work
    is linear in the tokens)."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    x, wg, wu, wd, dy = workloads.mlp_inputs(64, h, inter, 1)

    def run(T):
        xs = x.repeat((T + 63) // 64, 1)[:T]
        dys = dy.repeat((T + 63) // 64, 1)[:T]
        t0 = time.perf_counter()
        oracle.mlp_fwd(xs, wg, wu, wd)
        oracle.mlp_bwd(xs, wg, wu, wd, dys)
        return time.perf_counter() - t0

    T = 64
    t = run(T)
    while t < target_s / 3 and T < tokens:
        T = min(2 * T, tokens)
        t = run(T)
    flops = 18 * h * inter * T  # the whole-shard oracle recomputes nothing
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": _cpu_model(),
        "openblas_num_threads": os.environ.get("OPENBLAS_NUM_THREADS", "unset"),
        "kind": "oracle",
        "sample": f"float64 MLP oracle fwd+bwd of {T} tokens ({t:.1f} s; FLOPs counted as 18*hidden*inter "
                  f"per token, its own work)",
        "sample_s": round(t, 2),
        "extrapolated_config_s": round(t * tokens / T, 1),
        "extrapolation": f"extrapolated by the token ratio {tokens}/{T}",
    }


def ring_main(args, w, dev):
    bufs = make_ring_buffers(w, dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        ring_step(w, bufs)
    torch.cuda.synchronize()
    elapsed, avg, counts = timed_steps(lambda timer: ring_step(w, bufs, timer), args.steps, stream,
                                       live=("ring_bwd_prepare", "ring_bwd_step"))
    ms_per_step = elapsed * 1e3 / args.steps
    pairs = causal_pairs(w) * w.B * w.H  # the whole sequence, every head
    flops_step = 14 * w.d * pairs
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    fwd_ms = w.sp * avg["ring_fwd_step"]
    bwd_ms = avg["ring_bwd_prepare"] + w.sp * avg["ring_bwd_step"]
    bwd_tflops = 10 * w.d * pairs / (bwd_ms * 1e-3) / 1e12
    result = {
        "metric": "ring attention fwd+bwd TFLOP/s per GPU (% bf16 MFMA peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v/dO on the device)",
        "config": {
            "workload": f"{w.name} as a ring: B={w.B} N={w.N} H={w.H} sp={w.sp} chunks of {w.Ns} tokens "
                        f"(all {w.sp} virtual ranks on one GPU) d={w.d} {w.dtype} causal={w.causal}",
            "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "ring_fwd_ms": round(fwd_ms, 3),
            "ring_bwd_ms": round(bwd_ms, 3),
            "ring_fwd_step_ms": round(avg["ring_fwd_step"], 3),
            "ring_bwd_step_ms": round(avg["ring_bwd_step"], 3),
            "ring_bwd_prepare_ms": round(avg["ring_bwd_prepare"], 3),
            "ring_fwd_tflops": round(4 * w.d * pairs / (fwd_ms * 1e-3) / 1e12, 1),
            "ring_bwd_tflops": round(bwd_tflops, 1),
            "flops_per_step": flops_step,
            "calls_timed": counts,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": f"ring backward (D pre-pass + {w.sp} ring steps of dK/dV + dQ kernels)",
            "achieved": round(bwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": 10 * w.d * pairs,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
