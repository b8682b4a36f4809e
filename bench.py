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
the same with the fused width-4 convolution (mamba-2.8b-layer-fwd-conv4),
the 32K-context forward at the 2.8b width (mamba-2.8b-32k-fwd),
decode-state-update, million-length-fwd, million-length-bwd,
mamba-370m-layer-bwd, the backward at the 2.8b shape (mamba-2.8b-layer-bwd),
the 370m forward with the exact zero-order hold, with one
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
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# Nominal vector-ALU rates of MI355X: the published fp32 vector peak, 157.3
# TFLOP/s, is 78.6e12 FP32 lane operations/s (256 CUs x 4 SIMDs x 32 lanes per
# clock x 2.4 GHz; an FMA counts two flops), transcendentals a quarter of it.
# The ALU floors are priced with the rates the probes measure in the same run
# (plain v_fma_f32 and v_exp_f32, wall time, 4 waves per SIMD); these nominal
# figures are reported beside them.
VALU_OPS_PER_S_NOMINAL = 157.3e12 / 2
TRANS_OPS_PER_S_NOMINAL = VALU_OPS_PER_S_NOMINAL / 4
WORKLOAD_NAMES = ["mamba-370m-layer-fwd", "mamba-2.8b-layer-fwd", "decode-state-update",
                  "million-length-fwd", "million-length-bwd", "mamba-370m-layer-bwd",
                  "mamba-370m-layer-fwd-zoh", "mamba-370m-layer-fwd-token-delta",
                  "mamba-370m-layer-bidirectional", "decode-state-update-zoh",
                  "mamba-370m-layer-fwd-conv4", "mamba-370m-layer-bwd-conv4", "mamba-370m-layer-bwd-zoh",
                  "mamba-2.8b-32k-fwd", "mamba-2.8b-layer-fwd-conv4", "mamba-2.8b-layer-bwd"]
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
    ap.add_argument("--alu-calibration", action="store_true",
                    help="only time the vector-ALU probes (v_fma_f32, v_exp_f32, their 4:1 mix, "
                         "v_mul_f32) at 1-4 waves per SIMD and print their rates")
    return ap.parse_args()


def _source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "selective_state_space_10_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# sources whose hash identifies the kernels of each kind of line
SHA_FILES = {"fwd": ("scan_fwd.hip", "device_common.hpp", "kernels.hpp"),
             "bwd": ("scan_bwd.hip", "device_common.hpp", "kernels.hpp"),
             "decode": ("state_update.hip", "device_common.hpp", "kernels.hpp")}


def _traffic(workload: str, sha: str):
    """HBM bytes per step (all launches of the step: FETCH_SIZE and WRITE_SIZE
    scaled by a plain copy's counters) from the committed rocprofv3 summary
    profiles/hbm_traffic.json, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("bytes_per_step")


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
    _time_launches.median_ms = statistics.median(per)
    return start.elapsed_time(stop) / steps, sum(per) / len(per), wall


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# oracle work per timed sample: about a second on all host cores, and about a
# second on one core for the single-thread sample (state updates)
_CPU_UPDATES_MULTI = 2e9
_CPU_UPDATES_SINGLE = 1e8


def _channel_block(D, per_channel_updates, budget):
    """Channels [0, n) of a sample of about ``budget`` state updates (a multiple
    of 8, at least 8, at most D)."""
    n = int(budget // per_channel_updates) // 8 * 8
    return max(8, min(D, n))


def _slice_ch(p, n):
    """CPU fp64-ready copies of a workload's tensors restricted to channels [0, n)."""
    import torch
    out = {}
    for k, v in p.items():
        if not isinstance(v, torch.Tensor):
            out[k] = v
        elif k in ("u", "z", "dy", "x") or (k == "delta" and v.dim() == 3):
            out[k] = v[..., :n].cpu()
        elif k in ("A", "D", "delta_bias", "conv_w", "conv_b"):
            out[k] = v[:n].cpu()
        else:  # B, C (shared by the channels), a per-token delta
            out[k] = v.cpu()
    return out


def _cpu_baseline(runs, units_of, describe, repeats=3):
    """The fp64 C oracle as it stands, timed on the host: ``runs`` maps a
    thread count to a callable running one sample (the same work for every
    count), ``units_of`` maps it to the sample's tokens*channels.  Reports the
    median of ``repeats`` runs on all usable cores (the value) and on one."""
    import statistics
    from oracle import oracle_c
    threads = oracle_c.default_threads()
    res = {}
    for nthr in sorted({threads, 1}, reverse=True):
        fn = runs(nthr)
        ts = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        res[nthr] = (statistics.median(ts), ts, units_of(nthr))
    t, ts, units = res[threads]
    out = {"value": units / t, "unit": UNIT, "cores": threads, "kind": "oracle",
           "sample": describe(threads), "statistic": f"median of {repeats}",
           "seconds": round(sum(ts), 3), "cpu_model": _cpu_model()}
    t1, ts1, units1 = res[1]
    out["single_thread"] = {"value": units1 / t1, "unit": UNIT, "cores": 1,
                            "sample": describe(1), "statistic": f"median of {repeats}",
                            "seconds": round(sum(ts1), 3)}
    return out


def _cpu_baseline_fwd(p, Bsz, L, D, N, zoh=False, bidirectional=False, conv=0, repeats=3):
    """Forward oracle (with the line's options) on channel blocks of the
    workload's own inputs: the whole workload where it fits the multi-core
    budget, a block of channels for the single-core sample."""
    from oracle import oracle_c
    nch = {0: _channel_block(D, Bsz * L * N, _CPU_UPDATES_MULTI),
           1: _channel_block(D, Bsz * L * N, _CPU_UPDATES_SINGLE)}
    samples = {}

    def runs(nthr):
        n = nch[1] if nthr == 1 else nch[0]
        if n not in samples:
            samples[n] = {k: oracle_c._f64(v) if hasattr(v, "dim") else v
                          for k, v in _slice_ch(p, n).items()}
        q = samples[n]
        kw = {k: q.get(k) for k in ("delta", "A", "B", "C", "D", "z", "delta_bias")}
        if conv:
            return lambda: oracle_c.scan_fwd_conv(q["u"], q["conv_w"], q["conv_b"], **kw,
                                                  delta_softplus=True, nthreads=nthr, zoh=zoh)
        if bidirectional:
            def both():
                oracle_c.scan_fwd(q["u"], **kw, delta_softplus=True, nthreads=nthr, zoh=zoh)
                oracle_c.scan_fwd(q["u"], **dict(kw, D=None), delta_softplus=True, nthreads=nthr,
                                  zoh=zoh, reverse=True)
            return both
        return lambda: oracle_c.scan_fwd(q["u"], **kw, delta_softplus=True, nthreads=nthr, zoh=zoh)

    def units(nthr):
        return Bsz * L * (nch[1] if nthr == 1 else nch[0])

    def describe(nthr):
        n = nch[1] if nthr == 1 else nch[0]
        what = "the whole workload" if n == D else f"channels 0..{n - 1} of {D}"
        return (f"fp64 C oracle forward over {what} ({Bsz}x{L}x{n}x{N}, the workload's own inputs "
                f"upcast to fp64), {nthr} thread(s)")
    return _cpu_baseline(runs, units, describe, repeats)


def _cpu_baseline_bwd(p, dy, Bsz, L, D, N, zoh=False, conv=0, repeats=3):
    """Backward oracle (recomputing its forward) on channel blocks; its sums
    over channels (dB, dC) cover the block only, which does not change the
    work per token and channel."""
    from oracle import oracle_c
    nch = {0: _channel_block(D, 3 * Bsz * L * N, _CPU_UPDATES_MULTI),
           1: _channel_block(D, 3 * Bsz * L * N, _CPU_UPDATES_SINGLE)}
    samples = {}

    def runs(nthr):
        n = nch[1] if nthr == 1 else nch[0]
        if n not in samples:
            samples[n] = {k: oracle_c._f64(v) if hasattr(v, "dim") else v
                          for k, v in _slice_ch(dict(p, dy=dy), n).items()}
        q = samples[n]
        kw = {k: q.get(k) for k in ("delta", "A", "B", "C", "D", "z", "delta_bias")}
        if conv:
            return lambda: oracle_c.scan_bwd_conv(q["u"], q["conv_w"], q["conv_b"], **kw,
                                                  delta_softplus=True, dy=q["dy"], nthreads=nthr,
                                                  zoh=zoh)
        return lambda: oracle_c.scan_bwd(q["u"], **kw, delta_softplus=True, dy=q["dy"],
                                         nthreads=nthr, zoh=zoh)

    def units(nthr):
        return Bsz * L * (nch[1] if nthr == 1 else nch[0])

    def describe(nthr):
        n = nch[1] if nthr == 1 else nch[0]
        what = "the whole workload" if n == D else f"channels 0..{n - 1} of {D}"
        return (f"fp64 C oracle backward (with its own forward recompute) over {what} "
                f"({Bsz}x{L}x{n}x{N}), {nthr} thread(s)")
    return _cpu_baseline(runs, units, describe, repeats)


def _cpu_baseline_decode(d, Bsz, D, N, zoh=False, repeats=3):
    """Decode oracle (single-threaded as written): one step of the whole
    (B, D, N) state, repeated; the all-core figure is the same run."""
    from oracle import oracle_c
    q = {k: (oracle_c._f64(v.cpu()) if hasattr(v, "dim") else v) for k, v in d.items()}

    def runs(nthr):
        return lambda: oracle_c.state_update(q["state"], q["u"][0], q["delta"][0], q["A"],
                                             q["B"][0], q["C"][0], q["D"], q["z"][0],
                                             q["delta_bias"], True, zoh=zoh)
    out = _cpu_baseline(runs, lambda nthr: Bsz * D,
                        lambda nthr: f"fp64 C oracle state update, one step of the whole "
                                     f"{Bsz}x{D}x{N} state (the oracle is single-threaded)",
                        repeats)
    out["cores"] = 1
    return out


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


PROBE_KINDS = {0: "v_fma_f32", 1: "v_exp_f32", 2: "1 v_exp_f32 + 4 v_fma_f32 (independent)",
               3: "v_mul_f32", 4: "recurrence pattern (mul, exp, mul, fma, fma)"}


def _probe_lib():
    import ctypes

    from selective_state_space_10_amd import build as b
    if not os.path.exists(b.PROBE_LIB):
        raise ImportError(f"{b.PROBE_LIB} is missing (build the package first)")
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.ssm_probe_valu.restype = ctypes.c_int
    lib.ssm_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    lib.ssm_probe_instructions_per_lane.restype = ctypes.c_int64
    lib.ssm_probe_instructions_per_lane.argtypes = [ctypes.c_int, ctypes.c_int64]
    lib.ssm_probe_wave_placement.restype = ctypes.c_int
    lib.ssm_probe_wave_placement.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    return lib


def _probe_rate(lib, kind, W, iters, reps):
    """Lane operations per second of probe ``kind`` at W waves per SIMD: the
    median HIP-event time of ``reps`` launches after one untimed launch."""
    import ctypes
    import statistics

    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 1024, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    wgs = ctypes.c_int(0)
    times = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.ssm_probe_valu(kind, W, iters, out.data_ptr(), out.numel(), ctypes.byref(wgs),
                                ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        if st != 0:
            raise RuntimeError(f"probe launch failed with status {st}")
        torch.cuda.synchronize()
        if r:  # the first launch loads the code object
            times.append(e0.elapsed_time(e1) * 1e-3)
    t = statistics.median(times)
    per_lane = lib.ssm_probe_instructions_per_lane(kind, iters)
    return wgs.value * 256 * W * per_lane / t, t, per_lane * W


_RATES = {}


def _measured_alu_rates():
    """Plain FP32 (v_fma_f32) and transcendental (v_exp_f32) lane-operation
    rates measured now by the probes at 4 waves per SIMD (about 20 ms)."""
    if not _RATES:
        lib = _probe_lib()
        _RATES["plain"] = _probe_rate(lib, 0, 4, 10000, 3)[0]
        _RATES["trans"] = _probe_rate(lib, 1, 4, 4000, 3)[0]
    return _RATES["plain"], _RATES["trans"]


def _alu_block(kind, upd, td, per_upd, per_td, ms_launch):
    """A vector-ALU floor: ``per_upd`` = (plain, transcendental) instructions per
    state update, ``per_td`` the same per (b,t,d), priced at the measured rates
    (each class at its own peak, so the floor is a lower bound of the time)."""
    plain, trans = _measured_alu_rates()
    floor_s = (upd * (per_upd[0] / plain + per_upd[1] / trans)
               + td * (per_td[0] / plain + per_td[1] / trans))
    nominal_s = (upd * (per_upd[0] / VALU_OPS_PER_S_NOMINAL + per_upd[1] / TRANS_OPS_PER_S_NOMINAL)
                 + td * (per_td[0] / VALU_OPS_PER_S_NOMINAL + per_td[1] / TRANS_OPS_PER_S_NOMINAL))
    achieved = upd / (ms_launch * 1e-3) / 1e9
    peak = upd / floor_s / 1e9
    return {"kind": kind, "achieved": achieved, "peak": peak, "unit": "Gupdates/s",
            "frac": achieved / peak, "floor_ms": floor_s * 1e3,
            "rates": {"plain_lane_ops_per_s": plain, "trans_lane_ops_per_s": trans,
                      "source": "measured in this run: v_fma_f32 and v_exp_f32 probes "
                                "(libssm_alu_probe.so), one workgroup per CU, 4 waves per SIMD, "
                                "HIP-event wall time"},
            "nominal": {"plain_lane_ops_per_s": VALU_OPS_PER_S_NOMINAL,
                        "trans_lane_ops_per_s": TRANS_OPS_PER_S_NOMINAL,
                        "floor_ms": nominal_s * 1e3, "frac": nominal_s * 1e3 / ms_launch}}


def alu_calibration(reps=5):
    """Wall-time rates of the vector-ALU probes (libssm_alu_probe.so): one
    workgroup per compute unit, W = 1..4 waves per SIMD, each launch timed with
    HIP events on the stream it runs on; the median of ``reps`` launches."""
    import ctypes

    import torch
    lib = _probe_lib()
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    stream = torch.cuda.current_stream()
    rows = []
    for kind, name in PROBE_KINDS.items():
        iters = 2000 if kind in (2, 4) else 4000 if kind == 1 else 10000
        for W in (1, 2, 3, 4):
            rate, t, wave_instr_per_simd = _probe_rate(lib, kind, W, iters, reps)
            rows.append({"kind": name, "waves_per_simd": W, "seconds": t,
                         "lane_ops_per_s": rate,
                         "ns_per_wave_instruction_per_simd": t * 1e9 / wave_instr_per_simd,
                         "cycles_at_2p4ghz": t * 2.4e9 / wave_instr_per_simd})
    # where the waves of the scan's workgroup shapes land: SIMD of each wave
    placement = []
    for threads, lds in ((768, 86016), (960, 106496), (384, 43008), (512, 126976), (768, 0)):
        nw = threads // 64
        buf = torch.full((cus * nw,), -1, dtype=torch.int32, device="cuda")
        st = lib.ssm_probe_wave_placement(threads, lds, cus, buf.data_ptr(), buf.numel(),
                                          ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"placement probe failed with status {st}")
        torch.cuda.synchronize()
        simd = (buf.view(cus, nw) & 3).cpu()
        patterns = {}
        for row in simd.tolist():
            patterns[tuple(row)] = patterns.get(tuple(row), 0) + 1
        common = sorted(patterns.items(), key=lambda kv: -kv[1])[:3]
        placement.append({"threads": threads, "lds_bytes": lds,
                          "simd_of_wave_most_common": [list(k) for k, _ in common],
                          "workgroups_with_that_pattern": [v for _, v in common],
                          "waves_per_simd_max": int(max(torch.bincount(r, minlength=4).max()
                                                        for r in simd))})
    return {"calibration": "valu", "device": props.name, "cus": cus, "placement": placement,
            "method": "one workgroup per CU, W waves per SIMD, 8 independent chains per lane, "
                      "HIP-event wall time of one launch (median of 5 after one untimed)",
            "rows": rows}


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
    ms_median = _time_launches.median_ms
    Bsz, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    io_bytes = 4 if w.io_dtype == torch.float32 else 2
    nbytes = algorithmic_bytes_fwd(Bsz, L, D, N, io_bytes, h_final=want_hf)
    if per_token:  # delta is (B, L) instead of (B, L, D)
        nbytes -= Bsz * L * (D - 1) * io_bytes
    if conv:  # x replaces u; taps and bias are read once
        nbytes += D * (conv + 1) * 4
    achieved = nbytes / (ms_launch * 1e-3) / 1e9
    sha = _source_sha(*SHA_FILES["fwd"])
    traffic = _traffic(name, sha)
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
                     "traffic": traffic,
                     "algorithmic_bytes": nbytes,
                     "kernel_ms": ms_launch, "kernel_ms_median": ms_median, "source_sha": sha},
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
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline_fwd(sets[0], Bsz, L, D, N, zoh=zoh,
                                                 bidirectional=bidirectional, conv=conv,
                                                 repeats=1 if idx == 4 else 3)
    if name == "mamba-370m-layer-fwd":
        line["context"] = PAGES_CLAIM
    return line


def _alu_floor(Bsz, L, D, N, ms_launch):
    """The forward's vector-ALU floor: per state update 4 FP32 operations
    (dt*A', dt*u*B, the state FMA, the C*h FMA) and one exp2; per (b,t,d), shared
    by the N states, 10 FP32 operations (step size and softplus 4, SiLU 2, dt*u,
    D*u, the skip add, the gate) and 4 transcendentals (softplus: exp2, log2;
    SiLU: exp2, rcp)."""
    return _alu_block("vector-ALU floor of the plain forward (4 FP32 ops + 1 exp2 per state update, "
                      "10 FP32 ops + 4 transcendentals per (b,t,d)), each class at its measured rate",
                      Bsz * L * D * N, Bsz * L * D, (4, 1), (10, 4), ms_launch)


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
    ms_median = _time_launches.median_ms
    nbytes = algorithmic_bytes_decode(w.batch, w.dim, w.dstate, 2)
    achieved = nbytes / (ms_launch * 1e-3) / 1e9

    def step_one(t):  # the literal 64-step run on one state: it can stay in the 256 MB MALL
        m.state_update(states[0], d["u"][t], d["delta"][t], d["A"], d["B"][t], d["C"][t], d["D"],
                       d["z"][t], d["delta_bias"], True, zoh=zoh)

    _, ms_one, _ = _time_launches(step_one, w.steps, args.warmup, tok)
    extra = {}
    if not args.no_cpu_baseline:
        extra["cpu_baseline"] = _cpu_baseline_decode(d, w.batch, w.dim, w.dstate, zoh=zoh)
    return {**extra, "metric": "decode state update tokens*channels/s", "unit": UNIT,
            "value": w.batch * w.dim / (ms_step * 1e-3), "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 storage, f32 compute",
            "data": "synthetic", "config": {"workload": "decode-state-update" + ("-zoh" if zoh else ""),
                                            "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                                            "prewarm_steps": prewarm,
                                            "options": {"zoh": zoh}},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": _traffic("decode-state-update" + ("-zoh" if zoh else ""),
                                             _source_sha(*SHA_FILES["decode"])),
                         "algorithmic_bytes": nbytes, "kernel_ms": ms_launch,
                         "kernel_ms_median": ms_median,
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
    return _alu_block("vector-ALU floor of the backward (14 FP32 ops + 1 exp2 per state update, "
                      "24 FP32 ops + 6 transcendentals per (b,t,d)), each class at its measured rate",
                      Bsz * L * D * N, Bsz * L * D, (14, 1), (24, 6), ms_launch)


def bench_bwd(args, idx, name, conv=0, zoh=False):
    """Backward of workload ``idx`` (one forward with chunk states runs first,
    outside the timed steps); ``conv``: with the fused convolution of that width;
    ``zoh``: with the exact zero-order hold."""
    import torch

    import selective_state_space_10_amd as m
    from workloads import WORKLOADS, algorithmic_bytes_bwd, cotangent, workload_inputs
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
    ms_median = _time_launches.median_ms
    Bsz, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    io = 4 if w.io_dtype == torch.float32 else 2
    # u, delta, z, dy in; du, ddelta, dz out; B, C in and dB, dC out; chunk states in; A, D,
    # bias in and dA, dD, dbias out
    nbytes = algorithmic_bytes_bwd(Bsz, L, D, N, io, m.chunk_len())
    assert cs.numel() * 4 == Bsz * -(-L // m.chunk_len()) * N * D * 4
    achieved = nbytes / (ms_launch * 1e-3) / 1e9
    extra = {}
    if not args.no_cpu_baseline:
        pb = dict(p, conv_w=cw, conv_b=cb) if conv else p
        extra["cpu_baseline"] = _cpu_baseline_bwd(pb, dy, Bsz, L, D, N, zoh=zoh, conv=conv,
                                                  repeats=1 if idx == 4 else 3)
    return {**extra, "metric": f"selective-scan bwd tokens*channels/s, {name}", "unit": UNIT,
            "value": Bsz * L * D / (ms_step * 1e-3), "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": "f32" if io == 4 else "bf16 storage, f32 compute",
            "data": "synthetic", "config": {"workload": name, "batch": Bsz,
                                            "seqlen": L, "dim": D, "dstate": N,
                                            "prewarm_steps": _time_launches.prewarm_steps},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": _traffic(name, _source_sha(*SHA_FILES["bwd"])),
                         "algorithmic_bytes": nbytes, "kernel_ms": ms_launch,
                         "kernel_ms_median": ms_median,
                         **({} if conv or zoh else {"alu": _alu_floor_bwd(Bsz, L, D, N, ms_launch)})}}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    if args.alu_calibration:
        print(json.dumps(alu_calibration()), flush=True)
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
    elif wl == "mamba-2.8b-32k-fwd":
        line = bench_fwd(args, 5, wl)
    elif wl == "decode-state-update":
        line = bench_decode(args)
    elif wl == "decode-state-update-zoh":
        line = bench_decode(args, zoh=True)
    elif wl == "mamba-370m-layer-bwd":
        line = bench_bwd(args, 1, wl)
    elif wl == "mamba-370m-layer-fwd-conv4":
        line = bench_fwd(args, 1, wl, conv=4)
    elif wl == "mamba-2.8b-layer-fwd-conv4":
        line = bench_fwd(args, 2, wl, conv=4)
    elif wl == "mamba-370m-layer-bwd-conv4":
        line = bench_bwd(args, 1, wl, conv=4)
    elif wl == "mamba-2.8b-layer-bwd":
        line = bench_bwd(args, 2, wl)
    elif wl == "mamba-370m-layer-bwd-zoh":
        line = bench_bwd(args, 1, wl, zoh=True)
    else:
        line = bench_bwd(args, 4, wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
