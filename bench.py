"""Benchmark of the selective-SSM scan on one MI355X.

Default: the forward scan at the Mamba-370m layer shape (batch 8, length 2048,
2048 channels, 16 states, fp32, outputs y and the final state).  One step is
one forward pass over one batch of synthetic inputs already resident in HBM;
three input sets are rotated so that the 256 MB last-level cache cannot hold a
step's inputs.  Before the W warmup steps the step runs untimed for about 0.25 s
so that the GPU has left its idle clock state (the count is reported as
``config.prewarm_steps``); then exactly K steps are timed.  Prints ONE JSON
line (rank 0).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

``--workload`` also accepts the other shapes and options (mamba-2.8b-layer-fwd,
decode-state-update, million-length-fwd, million-length-bwd,
mamba-370m-layer-bwd, the 370m forward with the exact zero-order hold, with one
step size per token, bidirectional or with the fused convolution, the 370m
backward with the exact hold or the fused convolution, and the decode step with
the exact hold); their lines use the same keys and are for reference, the
default workload is the headline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# Vector-ALU rates of MI355X: the published fp32 vector peak, 157.3 TFLOP/s, is
# 78.6e12 FP32 lane operations/s (an FMA counts two flops); exp2, log2 and rcp
# run at a quarter of that rate (measured on gfx950: about 8.4 SIMD cycles per
# wave64 v_exp_f32 against about 2 for a plain FP32 operation).
VALU_OPS_PER_S = 157.3e12 / 2
TRANS_OPS_PER_S = VALU_OPS_PER_S / 4
WORKLOAD_NAMES = ["mamba-370m-layer-fwd", "mamba-2.8b-layer-fwd", "decode-state-update",
                  "million-length-fwd", "million-length-bwd", "mamba-370m-layer-bwd",
                  "mamba-370m-layer-fwd-zoh", "mamba-370m-layer-fwd-token-delta",
                  "mamba-370m-layer-bidirectional", "decode-state-update-zoh",
                  "mamba-370m-layer-fwd-conv4", "mamba-370m-layer-bwd-conv4", "mamba-370m-layer-bwd-zoh"]
METRIC = "selective-scan fwd tokens·channels/s and HBM GB/s (% of peak), Mamba-370m shape"
# The only throughput figure the source pages give for the method is relative and
# names no hardware, precision or workload: context beside the kernel's rate, not
# a number it can be compared with (reading guide of arXiv 2312.00752, "Sonuçlar").
PAGES_CLAIM = {"claim": "inference throughput up to 5x that of Transformers of similar size",
               "hardware": None, "workload": None, "comparable": False}
UNIT = "tokens*channels/s"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba-370m-layer-fwd", choices=WORKLOAD_NAMES)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=3, help="input sets rotated between steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def _source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "selective_state_space_10_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key: str, sha: str, launches_per_step: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("bytes_per_launch")


PREWARM_S = 0.25  # untimed seconds of the same step before the warmup steps


def _prewarm(fn, rotate_inputs, seconds=PREWARM_S):
    """Run the step untimed for about ``seconds`` so that the GPU has left its
    idle clock state before anything is timed; returns the number of steps."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(4):
            fn(rotate_inputs[n % len(rotate_inputs)])
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def _time_launches(fn, steps, warmup, rotate_inputs):
    """Per-launch HIP-event durations on the launch stream, plus the wall time
    of the whole timed region (both synchronised on both sides)."""
    import torch
    stream = torch.cuda.current_stream()
    _time_launches.prewarm_steps = _prewarm(fn, rotate_inputs)
    for i in range(warmup):
        fn(rotate_inputs[i % len(rotate_inputs)])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        fn(rotate_inputs[i % len(rotate_inputs)])
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    return start.elapsed_time(stop) / steps, sum(per) / len(per), wall


def _cpu_baseline_fwd(p_cpu, min_seconds=10.0):
    """The fp64 C oracle's forward over the same inputs, on all host cores it may
    use, repeated until at least ``min_seconds`` of wall time have passed."""
    from oracle import oracle_c
    threads = oracle_c.default_threads()
    kw = {k: p_cpu[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    conv = {k: oracle_c._f64(v) for k, v in kw.items()}
    reps, total = 0, 0.0
    while total < min_seconds:
        t0 = time.perf_counter()
        oracle_c.scan_fwd(**conv, delta_softplus=True, nthreads=threads)
        total += time.perf_counter() - t0
        reps += 1
    Bsz, L, D = p_cpu["u"].shape
    N = p_cpu["A"].shape[1]
    return {"value": reps * Bsz * L * D / total, "unit": UNIT, "cores": threads, "kind": "oracle",
            "sample": f"{reps} full forward steps of the same workload ({Bsz}x{L}x{D}x{N}, "
                      f"fp64 C oracle, inputs upcast from the fp32 draws), {total:.1f} s wall",
            "seconds": round(total, 3)}


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters:
    each launch reads and writes ``nbytes``."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"calibration": "copy", "bytes_read_per_launch": nbytes,
            "bytes_written_per_launch": nbytes, "launches": reps}


def _r3w1_ceiling(sets, steps):
    """A measured ceiling for the forward's access pattern: a streaming
    elementwise op that reads three (B,L,D) arrays and writes one
    (torch.addcmul(u, delta, z)), on the same rotated input sets."""
    import torch
    out = torch.empty_like(sets[0]["u"])
    for p in sets:
        torch.addcmul(p["u"], p["delta"], p["z"], out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        p = sets[i % len(sets)]
        torch.addcmul(p["u"], p["delta"], p["z"], out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 4 * out.numel() * out.element_size()
    return {"kind": "read-3/write-1 elementwise op (torch.addcmul) on the same (B,L,D) arrays",
            "achieved": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": ms}


def bench_fwd(args, idx, name, zoh=False, per_token=False, bidirectional=False, conv=0):
    """Forward scan of workload ``idx``; options: the exact zero-order-hold
    input term, one step size per token (delta drawn as (B, L)), or both scan
    directions summed (two launches, the second accumulating into y)."""
    import torch

    import selective_state_space_10_amd as m
    from workloads import WORKLOADS, algorithmic_bytes_fwd, workload_inputs
    w = WORKLOADS[idx]
    want_hf = "h_final" in w.outputs and not bidirectional
    sets = [workload_inputs(idx, device="cuda", seed=idx + 100 * r) for r in range(args.rotate)]
    if per_token:  # one raw step size per token: the first channel's draw
        sets = [dict(p, delta=p["delta"][:, :, 0].contiguous()) for p in sets]
    if conv:  # u is the convolution's input x; taps and bias of width ``conv``
        from workloads import conv_inputs
        for r, p in enumerate(sets):
            p["conv_w"], p["conv_b"] = conv_inputs(w.dim, conv, seed=idx + 100 * r, device="cuda")
    torch.cuda.synchronize()

    def step(p):
        if conv:
            m.scan_fwd_conv(p["u"], p["conv_w"], p["conv_b"], p["delta"], p["A"], p["B"], p["C"],
                            p["D"], p["z"], p["delta_bias"], True, None,
                            return_final_state=want_hf, zoh=zoh)
        elif bidirectional:
            m.bidirectional_scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                 p["delta_bias"], True, zoh=zoh)
        else:
            m.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                       p["delta_bias"], True, None, return_final_state=want_hf, zoh=zoh)

    ms_step, ms_launch, wall = _time_launches(step, args.steps, args.warmup, sets)
    Bsz, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    io_bytes = 4 if w.io_dtype == torch.float32 else 2
    nbytes = algorithmic_bytes_fwd(Bsz, L, D, N, io_bytes, h_final=want_hf)
    if per_token:  # delta is (B, L) instead of (B, L, D)
        nbytes -= Bsz * L * (D - 1) * io_bytes
    if conv:  # x replaces u; taps and bias are read once
        nbytes += D * (conv + 1) * 4
    achieved = nbytes / (ms_launch * 1e-3) / 1e9
    sha = _source_sha("scan_fwd.hip", "device_common.hpp", "kernels.hpp")
    traffic = _traffic(f"fwd:{name}", sha)
    line = {
        "metric": (METRIC if idx == 1 and name == "mamba-370m-layer-fwd"
                   else f"selective-scan fwd tokens*channels/s, {name}"),
        "value": Bsz * L * D / (ms_step * 1e-3),
        "unit": UNIT, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if io_bytes == 4 else "bf16 storage, f32 compute",
        "data": "synthetic (seeded Gaussian inputs of the layer's shape, rotated over "
                f"{args.rotate} resident sets)",
        "config": {"workload": name, "batch": Bsz, "seqlen": L, "dim": D, "dstate": N,
                   "io_dtype": str(w.io_dtype).replace("torch.", ""), "outputs": list(w.outputs),
                   "gpu": torch.cuda.get_device_name(), "wall_s": round(wall, 4),
                   "prewarm_steps": _time_launches.prewarm_steps,
                   "options": {"zoh": zoh, "delta_per_token": per_token,
                               "bidirectional": bidirectional, "conv_width": conv}},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic if not (zoh or per_token or bidirectional or conv) else None,
                     "algorithmic_bytes": nbytes,
                     "kernel_ms": ms_launch, "source_sha": sha},
    }
    if bidirectional:
        line["roofline"]["note"] = ("two launches per step; algorithmic bytes are one read of "
                                    "the inputs and one write of y")
    if not (zoh or per_token or bidirectional or conv):
        line["roofline"]["alu"] = _alu_floor(Bsz, L, D, N, ms_launch)
    if not (per_token or conv):
        ceil = _r3w1_ceiling(sets, max(args.steps, 10))
        ceil["frac"] = achieved / ceil["achieved"]  # the scan's rate over the measured ceiling
        line["roofline"]["ceiling"] = ceil
    if not args.no_cpu_baseline and name == "mamba-370m-layer-fwd":
        pc = workload_inputs(idx, device="cuda", seed=idx)
        pc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in pc.items()}
        line["cpu_baseline"] = _cpu_baseline_fwd(pc)
    if name == "mamba-370m-layer-fwd":
        line["context"] = PAGES_CLAIM
    return line


def _alu_floor(Bsz, L, D, N, ms_launch):
    """The forward's vector-ALU floor: per state update 4 FP32 operations
    (dt*A', dt*u*B, the state FMA, the C*h FMA) and one exp2; per (b,t,d), shared
    by the N states, 10 FP32 operations (step size and softplus 4, SiLU 2, dt*u,
    D*u, the skip add, the gate) and 4 transcendentals (softplus: exp2, log2;
    SiLU: exp2, rcp)."""
    upd, td = Bsz * L * D * N, Bsz * L * D
    floor_s = (upd * (4 / VALU_OPS_PER_S + 1 / TRANS_OPS_PER_S)
               + td * (10 / VALU_OPS_PER_S + 4 / TRANS_OPS_PER_S))
    achieved = upd / (ms_launch * 1e-3) / 1e9
    peak = upd / floor_s / 1e9
    return {"kind": "vector-ALU floor of the plain forward (4 FP32 ops + 1 exp2 per state update, "
                    "10 FP32 ops + 4 transcendentals per (b,t,d)) at the published fp32 vector rate, "
                    "transcendentals at a quarter of it",
            "achieved": achieved, "peak": peak, "unit": "Gupdates/s", "frac": achieved / peak,
            "floor_ms": floor_s * 1e3}


def bench_decode(args, zoh=False):
    import torch

    import selective_state_space_10_amd as m
    from workloads import WORKLOADS, algorithmic_bytes_decode, decode_inputs
    w = WORKLOADS[3]
    d = decode_inputs(w.batch, w.dim, w.dstate, w.steps, w.io_dtype, seed=3, device="cuda")
    states = [d["state"].clone() for _ in range(4)]  # rotated so the state is not cache-resident
    tok = list(range(w.steps))

    def step(t):
        st = states[t % len(states)]
        m.state_update(st, d["u"][t], d["delta"][t], d["A"], d["B"][t], d["C"][t], d["D"],
                       d["z"][t], d["delta_bias"], True, zoh=zoh)

    ms_step, ms_launch, wall = _time_launches(step, args.steps, args.warmup, tok)
    prewarm = _time_launches.prewarm_steps
    nbytes = algorithmic_bytes_decode(w.batch, w.dim, w.dstate, 2)
    achieved = nbytes / (ms_launch * 1e-3) / 1e9

    def step_one(t):  # the literal 64-step run on one state: it can stay in the 256 MB MALL
        m.state_update(states[0], d["u"][t], d["delta"][t], d["A"], d["B"][t], d["C"][t], d["D"],
                       d["z"][t], d["delta_bias"], True, zoh=zoh)

    _, ms_one, _ = _time_launches(step_one, w.steps, args.warmup, tok)
    return {"metric": "decode state update tokens*channels/s", "unit": UNIT,
            "value": w.batch * w.dim / (ms_step * 1e-3), "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 storage, f32 compute",
            "data": "synthetic", "config": {"workload": "decode-state-update" + ("-zoh" if zoh else ""),
                                            "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                                            "prewarm_steps": prewarm,
                                            "options": {"zoh": zoh}},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "algorithmic_bytes": nbytes, "kernel_ms": ms_launch,
                         "mall_resident": {"kind": "one state buffer, 64 consecutive steps",
                                           "achieved": nbytes / (ms_one * 1e-3) / 1e9,
                                           "unit": "GB/s", "kernel_ms": ms_one}}}


def _alu_floor_bwd(Bsz, L, D, N, ms_launch):
    """The backward's vector-ALU floor: per state update 14 FP32 operations and
    one exp2 (recompute: dt*A', dt*u*B, the state FMA; adjoint: e*C + lambda and
    the decay product; C*h for dz; the dB and dC contributions and their adds in
    the sums over channels; lambda*B for du; lambda*h_prev, its A-weighted sum for
    ddelta and its dt-weighted sum for dA); per (b,t,d), shared by the N states,
    24 FP32 operations and 6 transcendentals (softplus and its derivative
    sigma(s), sigma(z) for the gate and its derivative, the input gradients
    du, ddelta, dz, and the dD and dbias sums).  A sequence split's first pass
    is extra work the floor does not count."""
    upd, td = Bsz * L * D * N, Bsz * L * D
    floor_s = (upd * (14 / VALU_OPS_PER_S + 1 / TRANS_OPS_PER_S)
               + td * (24 / VALU_OPS_PER_S + 6 / TRANS_OPS_PER_S))
    achieved = upd / (ms_launch * 1e-3) / 1e9
    peak = upd / floor_s / 1e9
    return {"kind": "vector-ALU floor of the backward (14 FP32 ops + 1 exp2 per state update, "
                    "24 FP32 ops + 6 transcendentals per (b,t,d)) at the published fp32 vector rate, "
                    "transcendentals at a quarter of it",
            "achieved": achieved, "peak": peak, "unit": "Gupdates/s", "frac": achieved / peak,
            "floor_ms": floor_s * 1e3}


def bench_bwd(args, idx, name, conv=0, zoh=False):
    """Backward of workload ``idx`` (one forward with chunk states runs first,
    outside the timed steps); ``conv``: with the fused convolution of that width;
    ``zoh``: with the exact zero-order hold."""
    import torch

    import selective_state_space_10_amd as m
    from workloads import WORKLOADS, cotangent, workload_inputs
    w = WORKLOADS[idx]
    p = workload_inputs(idx, device="cuda")
    if conv:
        from workloads import conv_inputs
        cw, cb = conv_inputs(w.dim, conv, seed=idx, device="cuda")
        y, _, cs = m.scan_fwd_conv(p["u"], cw, cb, p["delta"], p["A"], p["B"], p["C"], p["D"],
                                   p["z"], p["delta_bias"], True, None, save_chunk_states=True)
    else:
        y, _, cs = m.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                              p["delta_bias"], True, None, save_chunk_states=True, zoh=zoh)
    dy = cotangent(y, idx)
    del y

    def step(_):
        if conv:
            m.scan_bwd_conv(p["u"], cw, cb, p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                            p["delta_bias"], True, None, cs, dy)
        else:
            m.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                       p["delta_bias"], True, None, cs, dy, zoh=zoh)

    ms_step, ms_launch, wall = _time_launches(step, args.steps, args.warmup, [0])
    Bsz, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    io = 4 if w.io_dtype == torch.float32 else 2
    # u, delta, z, dy in; du, ddelta, dz out; B, C in and dB, dC out; chunk states in; A, D,
    # bias in and dA, dD, dbias out
    nbytes = (7 * Bsz * L * D * io + 4 * Bsz * L * N * io + cs.numel() * 4
              + D * N * 4 * 2 + D * 4 * 4)
    achieved = nbytes / (ms_launch * 1e-3) / 1e9
    return {"metric": f"selective-scan bwd tokens*channels/s, {name}", "unit": UNIT,
            "value": Bsz * L * D / (ms_step * 1e-3), "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": "f32" if io == 4 else "bf16 storage, f32 compute",
            "data": "synthetic", "config": {"workload": name, "batch": Bsz,
                                            "seqlen": L, "dim": D, "dstate": N,
                                            "prewarm_steps": _time_launches.prewarm_steps},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "algorithmic_bytes": nbytes, "kernel_ms": ms_launch,
                         **({} if conv or zoh else {"alu": _alu_floor_bwd(Bsz, L, D, N, ms_launch)})}}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    import selective_state_space_10_amd as m
    m.load()
    wl = args.workload
    if wl == "mamba-370m-layer-fwd":
        line = bench_fwd(args, 1, wl)
    elif wl == "mamba-370m-layer-fwd-zoh":
        line = bench_fwd(args, 1, wl, zoh=True)
    elif wl == "mamba-370m-layer-fwd-token-delta":
        line = bench_fwd(args, 1, wl, per_token=True)
    elif wl == "mamba-370m-layer-bidirectional":
        line = bench_fwd(args, 1, wl, bidirectional=True)
    elif wl == "mamba-2.8b-layer-fwd":
        line = bench_fwd(args, 2, wl)
    elif wl == "million-length-fwd":
        args.rotate = 1
        line = bench_fwd(args, 4, wl)
    elif wl == "decode-state-update":
        line = bench_decode(args)
    elif wl == "decode-state-update-zoh":
        line = bench_decode(args, zoh=True)
    elif wl == "mamba-370m-layer-bwd":
        line = bench_bwd(args, 1, wl)
    elif wl == "mamba-370m-layer-fwd-conv4":
        line = bench_fwd(args, 1, wl, conv=4)
    elif wl == "mamba-370m-layer-bwd-conv4":
        line = bench_bwd(args, 1, wl, conv=4)
    elif wl == "mamba-370m-layer-bwd-zoh":
        line = bench_bwd(args, 1, wl, zoh=True)
    else:
        line = bench_bwd(args, 4, wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
