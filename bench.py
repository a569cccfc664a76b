#!/usr/bin/env python3
"""Benchmark of the per-tensor-scaled FP8 path on one MI355X.

One step = the whole hot path on the FC1 forward layer of the Transformer
Engine chapter's example (hidden 4096, ffn 16384; tokens = 4 x 2048):
  1. fused amax + delayed-scaled E4M3 cast of X [8192 x 4096] bf16,
  2. fused amax + delayed-scaled E4M3 cast-transpose of W [4096 x 16384] bf16,
  3. FP8 GEMM  C[8192 x 16384] = X_q · W_qᵀ with fp32 accumulation and the
     ×1/(s_x·s_w) epilogue, bf16 output,
  4. the amax-history update of both tensors (next step's scales).
Inputs are synthetic (seeded), resident in HBM before timing starts.

Printed on stdout: ONE JSON line.  `value` is GEMM FLOP / step time (TFLOP/s
of the whole step); `roofline` is the GEMM kernel alone (HIP events around
each launch on its stream); `extra` holds the delayed-scaling stream
(32 x 8192x4096, bf16 and fp32 inputs, HBM GB/s of the fused amax+cast), one HYBRID linear-layer
training step at the FC1 shape (forward, dgrad, wgrad, each launch timed), the
fine-grained MoE grouped GEMM, one GPU's parts of an E5M2 gradient all-reduce,
MXFP8 (block-32 quantisation and the block-scaled GEMM) on the FC1 shape, and
the vendor library's GEMMs on that shape; `cpu_baseline` times the CPU oracle on a
bounded slice of the same step.

Run order: the FC1 inputs and the CPU oracle (host work), the extras, the FC1
GEMM in the other accumulation mode, then the FC1 steps (W warm-up, K timed),
so that those start from the clock of a GPU under sustained matrix-core load.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 GEMM TFLOPS (% MFMA peak) at 8192x4096x16384; cast+amax HBM GB/s"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16/FP16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
# Untimed iterations before each extra's timed ones: the GEMMs slow down over their first launches after
# other work, then settle (the board's power control), within about 10-30 launches.
EXTRA_WARMUP = 10
# Untimed launches before the other accumulation mode's timed ones (see headline()).
OTHER_WARMUP = 40
# Matrix-core peak of the instruction each accumulation mode runs on.
PEAK_BY_ACCUM = {"exact": PEAK_BF16_TFLOPS, "mfma_fp8": PEAK_FP8_TFLOPS}

# HBM traffic per launch of the FC1 GEMM from two counter runs (FETCH_SIZE, WRITE_SIZE), each scaled by what
# the same counter reads for a 256 MiB device copy (profiles/gemm_fc1_8192x16384x4096_hbm_traffic.md).  Valid
# only for the kernel sources they were taken on: GEMM_SOURCES hashed in order must give GEMM_TRAFFIC_SHA256.
GEMM_SOURCES = ("gemm.hip", "gemm_dispatch.hpp", "gemm_kernel.hpp", "gemm_tile.hpp", "device_common.hpp")
GEMM_TRAFFIC_SHA256 = "2a8df5447029215bb2bf6d580f5b78871c0b499c58e48f090d1eb685663bfed5"
GEMM_TRAFFIC = {"exact": {"read_bytes": 805546341, "write_bytes": 268523191},
                "mfma_fp8": {"read_bytes": 805601577, "write_bytes": 268710760}}


def gemm_traffic(accum):
    """Counter-measured HBM bytes per launch, or None once the GEMM sources differ from the measured ones."""
    import hashlib

    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "fp8_precision_numerics_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != GEMM_TRAFFIC_SHA256:
        return None
    t = GEMM_TRAFFIC[accum]
    return t["read_bytes"] + t["write_bytes"]


def _percentiles(xs, ps):
    """Nearest-rank percentiles of xs."""
    s = sorted(xs)
    return [s[min(len(s) - 1, max(0, int(round(p / 100 * len(s) + 0.5)) - 1))] for p in ps]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--quick", action="store_true", help="headline step only (no extras, no CPU baseline)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--with-stream", action="store_true",
                   help="with --quick: also run the 32-step delayed-scaling stream (for counter runs of the cast)")
    p.add_argument("--stream-dtype", default="bf16", choices=["bf16", "f32"])
    p.add_argument("--accum", default="exact", choices=["exact", "mfma_fp8"],
                   help="GEMM accumulation mode of the timed step (the other mode is timed as an extra)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device-to-device copy (3 times): the known-size reference "
                        "for scaling the HBM traffic counters of a profiler run")
    return p.parse_args()


class EventTimer:
    """Pairs of HIP events recorded on the current stream around a launch."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        s = self.torch.cuda.Event(enable_timing=True)
        s.record()
        self._s = s
        return self

    def __exit__(self, *exc):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((self._s, e))

    def ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs]


def headline_prepare(torch, fm, args):
    """Inputs and state of the FC1 step, resident on the device (run before the
    extras, so that no host work separates the last extra from the timed step)."""
    from synth import fc1_forward

    dev = torch.device("cuda:0")
    M, K, N = 8192, 4096, 16384
    log("generating FC1 inputs (X 8192x4096, W 4096x16384, 4 priors each) ...")
    d = fc1_forward(M, K, N)
    to_dev = lambda h: torch.from_numpy(h.data.view("int16")).to(dev).view(torch.bfloat16)  # noqa: E731
    stX = fm.DelayedScalingState("e4m3", 16, device=dev)
    stW = fm.DelayedScalingState("e4m3", 16, device=dev)
    for pX, pW in zip(d["X_priors"], d["W_priors"]):
        stX.quantize(to_dev(pX))
        stX.update()
        stW.quantize(to_dev(pW))
        stW.update()
    X, W = to_dev(d["X"]), to_dev(d["W"])
    del d
    # Consecutive steps read different input buffers, so the casts stream cold
    # HBM rather than the 256 MB memory-side cache: NSETS copies of X and W
    # (rows of X, columns of W rotated, i.e. the same values and statistics)
    # of 192 MiB each, 576 MiB in all.
    NSETS = 3
    Xs = [X] + [torch.roll(X, shifts=997 * j, dims=0).contiguous() for j in range(1, NSETS)]
    Ws = [W] + [torch.roll(W, shifts=1009 * j, dims=1).contiguous() for j in range(1, NSETS)]
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    qwT = torch.empty((N, K), dtype=torch.uint8, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    return {"M": M, "K": K, "N": N, "NSETS": NSETS, "stX": stX, "stW": stW, "Xs": Xs, "Ws": Ws, "qx": qx,
            "qwT": qwT, "c": c, "X": X, "W": W}


def headline(torch, fm, args, ctx):
    M, K, N, NSETS = ctx["M"], ctx["K"], ctx["N"], ctx["NSETS"]
    stX, stW, Xs, Ws, qx, qwT, c = ctx["stX"], ctx["stW"], ctx["Xs"], ctx["Ws"], ctx["qx"], ctx["qwT"], ctx["c"]
    t_gemm = EventTimer(torch)

    # One delayed-scaling step per tensor per call (cast, then the history step
    # that sets the next step's scale); the GEMM takes the inverse scales the
    # casts used.
    def casts(i):
        stX.quantize_update(Xs[i % NSETS], q=qx)
        stW.quantize_update(Ws[i % NSETS], q_t=qwT)

    def gemm():
        fm.fp8_gemm(qx, "e4m3", qwT, "e4m3", stX.scale_inv_used, stW.scale_inv_used, c, accum=args.accum)

    flops = 2.0 * M * N * K
    # The same GEMM in the other accumulation mode, alone, on the codes of one
    # cast step, timed first: the FC1 steps then start from the clock of a GPU
    # under sustained matrix-core load.  Whichever GEMM loop runs first after
    # lighter work slows for some tens of launches while the board's power
    # control settles (up to ~14 %), so this loop gets a long warm-up of its own.
    casts(0)
    other = "mfma_fp8" if args.accum == "exact" else "exact"
    t_other = EventTimer(torch)
    for i in range(OTHER_WARMUP + args.steps):
        if i < OTHER_WARMUP:
            fm.fp8_gemm(qx, "e4m3", qwT, "e4m3", stX.scale_inv_used, stW.scale_inv_used, c, accum=other)
            continue
        with t_other:
            fm.fp8_gemm(qx, "e4m3", qwT, "e4m3", stX.scale_inv_used, stW.scale_inv_used, c, accum=other)
    for i in range(args.warmup):
        casts(i)
        gemm()
    torch.cuda.synchronize()
    # Timed region.  A timing event left in the stream idles the GPU for about
    # 10 us where it sits (MI355X kernel trace: a gap at each event boundary,
    # none between the launches of the untimed steps, whatever the event's
    # release scope), so the GEMM is bracketed by events on every other step
    # only: its mean duration over those launches, measured live on its stream,
    # gives the roofline, and the steps between keep the launches back to back.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        casts(args.warmup + i)
        if i % 2 == 0:
            with t_gemm:
                gemm()
        else:
            gemm()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    gemm_ms = statistics.mean(t_gemm.ms())
    # The casts, each between events, in the same steps run after the timed
    # region: the per-call cost of each (its events' gaps included).
    t_cx, t_cw = EventTimer(torch), EventTimer(torch)
    for i in range(args.steps):
        j = args.warmup + args.steps + i
        with t_cx:
            stX.quantize_update(Xs[j % NSETS], q=qx)
        with t_cw:
            stW.quantize_update(Ws[j % NSETS], q_t=qwT)
        gemm()
    torch.cuda.synchronize()
    cx_ms, cw_ms = statistics.mean(t_cx.ms()), statistics.mean(t_cw.ms())
    log(f"step {total_ms / args.steps:.3f} ms; gemm {gemm_ms * 1e3:.1f} us ({flops / gemm_ms / 1e9:.0f} TFLOP/s, "
        f"{len(t_gemm.pairs)} of {args.steps} launches timed); cast X + history step {cx_ms * 1e3:.1f} us; "
        f"cast-transpose W + history step {cw_ms * 1e3:.1f} us")
    # Median: a rare stall of the whole GPU (one launch of ~21 ms seen among 50, the next ones slower while
    # the clock recovers) would otherwise dominate the mean, which is reported beside it.
    other_ms = statistics.median(t_other.ms())
    other_mean_ms = statistics.mean(t_other.ms())
    log(f"gemm in {other} mode: {other_ms * 1e3:.1f} us median ({flops / other_ms / 1e9:.0f} TFLOP/s), "
        f"{other_mean_ms * 1e3:.1f} us mean")
    out = {
        "accum": args.accum,
        "gemm_other_mode": {"accum": other, "us": other_ms * 1e3, "us_mean": other_mean_ms * 1e3,
                            "tflops": flops / other_ms / 1e9,
                            "frac_of_its_peak": flops / other_ms / 1e9 / PEAK_BY_ACCUM[other],
                            "frac_of_fp8_peak": flops / other_ms / 1e9 / PEAK_FP8_TFLOPS},
        "ms_per_step": total_ms / args.steps,
        "value": flops / (total_ms / args.steps) / 1e9,
        "gemm_ms": gemm_ms,
        "gemm_ms_median": statistics.median(t_gemm.ms()),
        "gemm_us_p10_p50_p90": [round(float(x), 1) for x in _percentiles([v * 1e3 for v in t_gemm.ms()], (10, 50, 90))],
        "gemm_tflops": flops / gemm_ms / 1e9,
        "gemm_frac_of_fp8_peak": flops / gemm_ms / 1e9 / PEAK_FP8_TFLOPS,
        "cast_x_us": cx_ms * 1e3,
        "cast_x_gbs": M * K * 3 / (cx_ms * 1e-3) / 1e9,
        "cast_transpose_w_us": cw_ms * 1e3,
        "cast_transpose_w_gbs": K * N * 3 / (cw_ms * 1e-3) / 1e9,
        "scale_x": stX.scale.item(),
        "scale_w": stW.scale.item(),
        "input_sets": NSETS,
        "input_bytes_rotated": NSETS * (M * K + K * N) * 2,
    }
    del Xs, Ws, qx, qwT, c
    ctx.clear()
    torch.cuda.empty_cache()
    return out


def stream_bench(torch, fm, dtype, passes=3):
    """Delayed-scaling stream: 32 distinct 8192x4096 tensors resident in HBM
    (2 GiB bf16 / 4 GiB fp32, beyond the 256 MB last-level cache)."""
    from synth import stream_step
    import concurrent.futures as cf

    dev = torch.device("cuda:0")
    R, C = 8192, 4096
    log(f"generating the 32-step stream ({dtype}) ...")
    with cf.ThreadPoolExecutor(4) as ex:
        hs = list(ex.map(lambda t: stream_step(t, R, C, dtype), range(32)))
    xs = []
    for h in hs:
        arr = torch.from_numpy(h.data.view("int16") if dtype == "bf16" else h.data).to(dev)
        xs.append(arr.view(torch.bfloat16) if dtype == "bf16" else arr)
    del hs
    q = torch.empty((R, C), dtype=torch.uint8, device=dev)
    # reporting pass: per-step scale and saturation count
    st = fm.DelayedScalingState("e4m3", 16, device=dev)
    per_step = []
    for t, x in enumerate(xs):
        scale_used = st.scale.item()
        st.quantize(x, q=q, count_saturation=True)
        st.update()
        per_step.append({"t": t, "scale": scale_used, "amax": st.amax.item(), "saturated": int(st.sat.item())})
    # timing: per-call events around each eager step (fp8_quantize_update: the
    # cast and the history step, with the host launch cost), and the whole
    # 32-step sequence captured once in a HIP graph and replayed, which is what
    # the GPU sustains -- with the fused call, and with the two separate calls
    timer = EventTimer(torch)
    for p in range(passes):
        st = fm.DelayedScalingState("e4m3", 16, device=dev)
        for x in xs:
            with timer:
                st.quantize_update(x, q=q, count_saturation=True)
    torch.cuda.synchronize()
    ms = timer.ms()[32:] if passes > 1 else timer.ms()

    def graph_step_ms(fused):
        st = fm.DelayedScalingState("e4m3", 16, device=dev)

        def one(x):
            if fused:
                st.quantize_update(x, q=q, count_saturation=True)
            else:
                st.quantize(x, q=q, count_saturation=True)
                st.update()

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):              # warm the path up off the capture
            for x in xs[:2]:
                one(x)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for x in xs:
                one(x)
        graph.replay()
        torch.cuda.synchronize()
        out = []
        for _ in range(passes):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / len(xs))
        del graph
        return statistics.mean(out)

    step = graph_step_ms(True)
    step_separate = graph_step_ms(False)
    ceiling = hbm_ceiling(torch, fm, xs, q, passes)
    bytes_per_step = R * C * ((2 if dtype == "bf16" else 4) + 1)
    avg = statistics.mean(ms)
    log(f"stream {dtype}: cast + history step {avg * 1e3:.1f} us/call (eager, events per call) = "
        f"{bytes_per_step / (avg * 1e-3) / 1e9:.0f} GB/s; graph-replayed step {step * 1e3:.1f} us = "
        f"{bytes_per_step / (step * 1e-3) / 1e9:.0f} GB/s (separate cast and update calls: {step_separate * 1e3:.1f} us)")
    del xs, q
    torch.cuda.empty_cache()
    return {"dtype": dtype, "us_per_call_eager": avg * 1e3, "gbs_per_call_eager": bytes_per_step / (avg * 1e-3) / 1e9,
            "us_per_step_graph": step * 1e3, "gbs": bytes_per_step / (step * 1e-3) / 1e9,
            "us_per_step_graph_separate_calls": step_separate * 1e3,
            "frac_hbm_peak": bytes_per_step / (step * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "algorithmic_bytes_per_step": bytes_per_step, "hbm_ceiling": ceiling, "per_step": per_step}


def hbm_ceiling(torch, fm, xs, q, passes=3):
    """What HBM sustains on cold data, next to the cast: over the 32 resident
    stream tensors (more than the 256 MB memory-side cache holds), each pass
    captured once as a HIP graph of 32 back-to-back calls and replayed:
      copy   a plain device-to-device copy of the tensor (read + write its bytes),
      read   the amax alone (fp8_quantize with no codes requested: read only),
      cast   the fused amax + cast with a fixed scale (read, write 1 B per value),
    each in GB/s of the bytes it must move."""
    dev = xs[0].device
    n, eb = xs[0].numel(), xs[0].element_size()
    dst = torch.empty_like(xs[0])
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(fm.QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    scale = torch.ones(1, dtype=torch.float32, device=dev)
    passes_ = {
        "copy": (lambda x: dst.copy_(x), 2 * n * eb),
        "read": (lambda x: fm.fp8_quantize(x, "e4m3", amax=amax, workspace=ws), n * eb),
        "cast": (lambda x: fm.fp8_quantize(x, "e4m3", scale, q=q, amax=amax, workspace=ws), n * (eb + 1)),
    }
    out = {}
    for name, (fn, nbytes) in passes_.items():
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(xs[0])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for x in xs:
                fn(x)
        graph.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(passes):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / len(xs))
        del graph
        us = statistics.mean(per) * 1e3
        out[name] = {"us_per_call": us, "bytes_per_call": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9}
    out["cast_over_copy_gbs"] = out["cast"]["gbs"] / out["copy"]["gbs"]
    out["cast_over_read_gbs"] = out["cast"]["gbs"] / out["read"]["gbs"]
    log("hbm ceiling (32 distinct tensors, graph-replayed): " + ", ".join(
        f"{k} {v['us_per_call']:.1f} us {v['gbs']:.0f} GB/s" for k, v in out.items() if isinstance(v, dict)))
    del dst, ws
    return out


def linear_bench(torch, fm, iters=10):
    """One FP8 linear layer training step at the FC1 shape (tokens 8192, in 4096,
    out 16384) under HYBRID delayed scaling: forward (cast-transpose of X and W,
    Y = X W^T bf16), backward (cast-transpose of dY to E5M2, dX = dY W and
    dW = dY^T X in fp32), the three history updates.  Each launch is timed on its
    own, and the whole step once more as one region.  Also timed: the forward
    GEMM with Y re-quantised to E4M3 in its epilogue, and the cast of the bf16 Y
    that the unfused path would need instead."""
    from synth import dgrad_hybrid, fc1_forward

    dev = torch.device("cuda:0")
    T, I, O = 8192, 4096, 16384
    log("generating linear-layer inputs ...")
    d = dgrad_hybrid(T, O, I, priors=False)
    G = torch.from_numpy(d["dY"].data.view("int16")).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(d["W"].data.view("int16")).to(dev).view(torch.bfloat16)      # [out x in]
    del d
    X = torch.from_numpy(fc1_forward(T, I, O, priors=False)["X"].data.view("int16")).to(dev).view(torch.bfloat16)
    Y = torch.empty((T, O), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((T, I), dtype=torch.float32, device=dev)
    dW = torch.empty((O, I), dtype=torch.float32, device=dev)
    flops = 2.0 * T * I * O
    res = {}
    for accum in ("exact", "mfma_fp8"):
        layer = fm.Fp8Linear(T, I, O, accum=accum, device=dev)
        for _ in range(EXTRA_WARMUP):         # from the second step on, casts use amax-derived scales
            layer.forward(X, W, Y)
            layer.backward(G, dX, dW)
            layer.update()
        parts = {k: EventTimer(torch) for k in ("cast_x", "cast_w", "fwd_gemm", "cast_dy", "dgrad_gemm",
                                                "wgrad_gemm", "update")}
        whole = EventTimer(torch)
        sx, sw, sg = layer.state_x, layer.state_w, layer.state_g
        for _ in range(iters):
            with parts["cast_x"]:
                sx.quantize(X, q=layer.qx, q_t=layer.qx_t)
            with parts["cast_w"]:
                sw.quantize(W, q=layer.qw, q_t=layer.qw_t)
            with parts["fwd_gemm"]:
                fm.fp8_gemm(layer.qx, "e4m3", layer.qw, "e4m3", sx.scale_inv, sw.scale_inv, Y, accum=accum)
            with parts["cast_dy"]:
                sg.quantize(G, q=layer.qg, q_t=layer.qg_t)
            with parts["dgrad_gemm"]:
                fm.fp8_gemm(layer.qg, "e5m2", layer.qw_t, "e4m3", sg.scale_inv, sw.scale_inv, dX, accum=accum)
            with parts["wgrad_gemm"]:
                fm.fp8_gemm(layer.qg_t, "e5m2", layer.qx_t, "e4m3", sg.scale_inv, sx.scale_inv, dW, accum=accum)
            with parts["update"]:
                layer.update()
        for _ in range(iters):
            with whole:
                layer.forward(X, W, Y)
                layer.backward(G, dX, dW)
                layer.update()
        # the forward with Y re-quantised to E4M3 in the GEMM epilogue, against the
        # unfused alternative's extra pass (the cast of the bf16 Y)
        st_y = fm.DelayedScalingState("e4m3", 16, device=dev)
        yq = torch.empty((T, O), dtype=torch.uint8, device=dev)
        for _ in range(2):
            st_y.quantize(Y, q=yq)
            st_y.update()
        parts["fwd_gemm_requant"], parts["cast_y"] = EventTimer(torch), EventTimer(torch)
        for _ in range(iters):
            with parts["fwd_gemm_requant"]:
                fm.fp8_gemm_requant(layer.qx, "e4m3", layer.qw, "e4m3", sx.scale_inv, sw.scale_inv, "e4m3",
                                    st_y.scale, yq, amax=st_y.amax, sat=st_y.sat, accum=accum)
            with parts["cast_y"]:
                st_y.quantize(Y, q=yq)
        torch.cuda.synchronize()
        us = {k: statistics.mean(t.ms()) * 1e3 for k, t in parts.items()}
        step_us = statistics.mean(whole.ms()) * 1e3
        r = {"step_us": step_us, "step_tflops": 3 * flops / step_us / 1e6, "parts_us": us}
        for g in ("fwd_gemm", "dgrad_gemm", "wgrad_gemm"):
            r[g.replace("_gemm", "_tflops")] = flops / us[g] / 1e6
        log(f"linear step ({accum}): {step_us:.1f} us = {r['step_tflops']:.0f} TFLOP/s; "
            + ", ".join(f"{k} {v:.1f}" for k, v in us.items()))
        res[accum] = r
    # Gradients mix very large and very small magnitudes: the share of dY's
    # (nonzero) entries that its E5M2 cast flushes to +-0, against a cast of the
    # same tensor to E4M3 with E4M3's scale from the same amax history (what
    # choosing E4M3 for gradients would lose).  Reporting only, after the timing.
    sg = layer.state_g
    hist_max = float(sg.history.max().item())
    s4 = torch.tensor([448.0 / hist_max], dtype=torch.float32, device=dev)
    q4 = torch.empty((T, O), dtype=torch.uint8, device=dev)
    fm.fp8_quantize(G, "e4m3", s4, q=q4)
    nonzero = G != 0
    n_nz = int(nonzero.sum().item())
    f5 = int((((layer.qg & 0x7F) == 0) & nonzero).sum().item()) / n_nz
    f4 = int((((q4 & 0x7F) == 0) & nonzero).sum().item()) / n_nz
    res["dy_flushed_to_zero"] = {"e5m2": f5, "e4m3_same_history": f4, "scale_e5m2": float(sg.scale.item()),
                                 "scale_e4m3": float(s4.item()), "nonzero_entries": n_nz}
    log(f"dY [{T}x{O}] entries flushed to 0: E5M2 {f5 * 100:.3f} %, E4M3 with the same history {f4 * 100:.3f} %")
    del q4, nonzero, layer
    del G, W, X, Y, dX, dW
    torch.cuda.empty_cache()
    return res


def mx_bench(torch, fm, iters=20):
    """MXFP8 on the FC1 shape: the per-32-block quantisation of X (8192 x 4096)
    and of W^T (16384 x 4096), both bf16 -> E4M3 codes + exponent bytes, and the
    GEMM X W^T -> bf16 in both modes: exact (bf16 matrix cores, exact products,
    fp32 sums) and on the block-scaled FP8 matrix cores."""
    from synth import fc1_forward

    dev = torch.device("cuda:0")
    M, K, N = 8192, 4096, 16384
    d = fc1_forward(M, K, N, priors=False)
    X = torch.from_numpy(d["X"].data.view("int16")).to(dev).view(torch.bfloat16)
    Wt = torch.from_numpy(d["W"].data.view("int16")).to(dev).view(torch.bfloat16).t().contiguous()
    del d
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sx = torch.empty((K // 32, fm.mx_scale_ld(M)), dtype=torch.uint8, device=dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((K // 32, fm.mx_scale_ld(N)), dtype=torch.uint8, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = {k: EventTimer(torch) for k in ("quantize_x", "quantize_w", "gemm_exact", "gemm_mfma_fp8",
                                        "plain_exact_same_codes")}
    one = torch.ones(1, dtype=torch.float32, device=dev)
    for i in range(iters + EXTRA_WARMUP):
        timed = i >= EXTRA_WARMUP
        with (t["quantize_x"] if timed else _Null()):
            fm.fp8_quantize_mx(X, "e4m3", qx, sx)
        with (t["quantize_w"] if timed else _Null()):
            fm.fp8_quantize_mx(Wt, "e4m3", qw, sw)
        with (t["gemm_exact"] if timed else _Null()):
            fm.fp8_gemm_mx(qx, "e4m3", sx, qw, "e4m3", sw, c, accum="exact")
        with (t["gemm_mfma_fp8"] if timed else _Null()):
            fm.fp8_gemm_mx(qx, "e4m3", sx, qw, "e4m3", sw, c, accum="mfma_fp8")
        # reference: the per-tensor exact GEMM on the same codes (no block scales)
        with (t["plain_exact_same_codes"] if timed else _Null()):
            fm.fp8_gemm(qx, "e4m3", qw, "e4m3", one, one, c, accum="exact")
    torch.cuda.synchronize()
    us = {k: statistics.mean(v.ms()) * 1e3 for k, v in t.items()}
    flops = 2.0 * M * N * K
    res = {"us": us,
           "gemm_exact_tflops": flops / us["gemm_exact"] / 1e6,
           "gemm_exact_frac_of_fp8_peak": flops / us["gemm_exact"] / 1e6 / PEAK_FP8_TFLOPS,
           "gemm_exact_frac_of_bf16_peak": flops / us["gemm_exact"] / 1e6 / PEAK_BF16_TFLOPS,
           "gemm_mfma_fp8_tflops": flops / us["gemm_mfma_fp8"] / 1e6,
           "gemm_mfma_fp8_frac_of_fp8_peak": flops / us["gemm_mfma_fp8"] / 1e6 / PEAK_FP8_TFLOPS,
           "quantize_x_gbs": M * K * (2 + 1 + 1 / 32) / us["quantize_x"] / 1e3,
           "quantize_w_gbs": N * K * (2 + 1 + 1 / 32) / us["quantize_w"] / 1e3}
    log(f"mxfp8: quantize X {us['quantize_x']:.1f} us ({res['quantize_x_gbs']:.0f} GB/s), W {us['quantize_w']:.1f} us "
        f"({res['quantize_w_gbs']:.0f} GB/s); gemm exact {us['gemm_exact']:.1f} us "
        f"({res['gemm_exact_tflops']:.0f} TFLOP/s), fp8 cores {us['gemm_mfma_fp8']:.1f} us "
        f"({res['gemm_mfma_fp8_tflops']:.0f} TFLOP/s); per-tensor exact GEMM on the same codes "
        f"{us['plain_exact_same_codes']:.1f} us")
    del X, Wt, qx, sx, qw, sw, c
    torch.cuda.empty_cache()
    return res


def allreduce_bench(torch, fm, iters=20, ranks=8):
    """One GPU's parts of an FP8 (E5M2) all-reduce of the FC1 weight gradient
    (4096 x 16384 fp32) over `ranks` ranks: its amax pass, the shared scale, the
    cast with that scale, and the fp32 sum of the `ranks` payloads of one
    reduce-scattered chunk (67.1M / ranks codes each)."""
    dev = torch.device("cuda:0")
    n = 4096 * 16384
    chunk = n // ranks
    g = torch.empty(n, dtype=torch.float32, device=dev).normal_(0.0, 1e-4, generator=torch.Generator(dev).manual_seed(7))
    amaxes = torch.zeros(ranks, dtype=torch.float32, device=dev)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    scale_inv = torch.empty(1, dtype=torch.float32, device=dev)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    out = torch.empty(chunk, dtype=torch.float32, device=dev)
    ws = torch.empty(fm.QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    # the received chunk: `ranks` payloads, here the codes of this rank's own gradient chunks
    recv = q.view(ranks, chunk)
    t = {k: EventTimer(torch) for k in ("amax", "shared_scale", "cast", "dequant_sum")}
    for i in range(iters + 3):
        timed = i >= 3
        with (t["amax"] if timed else _Null()):
            fm.fp8_quantize(g, "e5m2", None, amax=amaxes[0:1], workspace=ws)
        with (t["shared_scale"] if timed else _Null()):
            fm.fp8_shared_scale(amaxes, "e5m2", scale, scale_inv)
        with (t["cast"] if timed else _Null()):
            fm.fp8_quantize(g, "e5m2", scale, q=q, workspace=ws)
        with (t["dequant_sum"] if timed else _Null()):
            fm.fp8_dequant_sum(recv, "e5m2", scale_inv, out)
    torch.cuda.synchronize()
    us = {k: statistics.mean(v.ms()) * 1e3 for k, v in t.items()}
    gbs = {"amax": n * 4 / us["amax"] / 1e3, "cast": n * 5 / us["cast"] / 1e3,
           "dequant_sum": (ranks * chunk + 4 * chunk) / us["dequant_sum"] / 1e3}
    log(f"fp8 all-reduce parts (E5M2, {ranks} ranks, 67.1M-value gradient): amax {us['amax']:.1f} us "
        f"({gbs['amax']:.0f} GB/s), shared scale {us['shared_scale']:.1f} us, cast {us['cast']:.1f} us "
        f"({gbs['cast']:.0f} GB/s), sum of {ranks} payloads {us['dequant_sum']:.1f} us ({gbs['dequant_sum']:.0f} GB/s)")
    del g, q, out, recv
    torch.cuda.empty_cache()
    return {"ranks": ranks, "values": n, "us": us, "gbs": gbs}


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def moe_bench(torch, fm, iters=20):
    from synth import moe_grouped

    dev = torch.device("cuda:0")
    log("generating MoE inputs ...")
    d = moe_grouped()
    G, N, K = d["B"].shape
    total = int(d["m_offsets"][-1])
    A = torch.from_numpy(d["A"].data.view("int16")).to(dev).view(torch.bfloat16)
    B = torch.from_numpy(d["B"].data.reshape(G * N, K).view("int16")).to(dev).view(torch.bfloat16)
    offs = torch.from_numpy(d["m_offsets"].astype("int32")).to(dev)
    counts = d["counts"].tolist()
    del d
    qa = torch.empty((total, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((total, K // 128), dtype=torch.float32, device=dev)
    qb = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((G * N // 128, K // 128), dtype=torch.float32, device=dev)
    c = torch.empty((total, N), dtype=torch.bfloat16, device=dev)
    ta, tb = EventTimer(torch), EventTimer(torch)
    tg = {"exact": EventTimer(torch), "mfma_fp8": EventTimer(torch)}
    for i in range(iters + EXTRA_WARMUP):
        if i < EXTRA_WARMUP:
            fm.fp8_quantize_blockwise(A, 1, "e4m3", qa, sa)
            fm.fp8_quantize_blockwise(B, 128, "e4m3", qb, sb)
            for accum in tg:
                fm.fp8_grouped_gemm(qa, sa, qb.view(G, N, K), sb.view(G, N // 128, K // 128), offs, c, accum=accum)
            continue
        with ta:
            fm.fp8_quantize_blockwise(A, 1, "e4m3", qa, sa)
        with tb:
            fm.fp8_quantize_blockwise(B, 128, "e4m3", qb, sb)
        for accum, timer in tg.items():
            with timer:
                fm.fp8_grouped_gemm(qa, sa, qb.view(G, N, K), sb.view(G, N // 128, K // 128), offs, c, accum=accum)
    torch.cuda.synchronize()
    flops = 2.0 * total * N * K
    gem = {}
    for accum, timer in tg.items():
        g_ms = statistics.mean(timer.ms())
        gem[accum] = {"us": g_ms * 1e3, "tflops": flops / g_ms / 1e9,
                      "frac_of_its_peak": flops / g_ms / 1e9 / PEAK_BY_ACCUM[accum]}
    a_ms, b_ms = statistics.mean(ta.ms()), statistics.mean(tb.ms())
    log(f"moe grouped: gemm exact {gem['exact']['us']:.1f} us ({gem['exact']['tflops']:.0f} TFLOP/s), "
        f"mfma_fp8 {gem['mfma_fp8']['us']:.1f} us ({gem['mfma_fp8']['tflops']:.0f} TFLOP/s); "
        f"blockwise A {a_ms * 1e3:.1f} us, W {b_ms * 1e3:.1f} us")
    del A, B, qa, sa, qb, sb, c
    torch.cuda.empty_cache()
    return {"token_counts": counts, "grouped_gemm": gem, "blockwise_a_us": a_ms * 1e3,
            "blockwise_w_us": b_ms * 1e3,
            "blockwise_a_gbs": total * K * 3 / (a_ms * 1e-3) / 1e9,
            "blockwise_w_gbs": G * N * K * 3 / (b_ms * 1e-3) / 1e9}


def vendor_reference(torch, iters=20):
    """hipBLASLt (through torch) on the FC1 shape, timed the same way: the
    practical rate of this GPU for a plain fp16/bf16 GEMM and for an FP8 GEMM
    with per-tensor scales.  Context for the roofline fractions only; no part
    of the path uses it."""
    dev = torch.device("cuda:0")
    M, N, K = 8192, 16384, 4096
    flops = 2.0 * M * N * K
    out = {}

    def t(fn):
        for _ in range(3):
            fn()
        timer = EventTimer(torch)
        for _ in range(iters):
            with timer:
                fn()
        torch.cuda.synchronize()
        return statistics.mean(timer.ms())

    for name, dt in (("fp16", torch.float16), ("bf16", torch.bfloat16)):
        a = torch.randn(M, K, device=dev, dtype=dt)
        b = torch.randn(N, K, device=dev, dtype=dt)
        ms = t(lambda: torch.matmul(a, b.t()))
        out[f"matmul_{name}"] = {"us": ms * 1e3, "tflops": flops / ms / 1e9}
        del a, b
    try:
        a = torch.randn(M, K, device=dev).to(torch.float8_e4m3fn)
        b = torch.randn(N, K, device=dev).to(torch.float8_e4m3fn)
        one = torch.ones((), device=dev)
        ms = t(lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
        out["scaled_mm_e4m3"] = {"us": ms * 1e3, "tflops": flops / ms / 1e9}
        del a, b
    except Exception as e:  # noqa: BLE001
        out["scaled_mm_e4m3"] = f"unavailable: {type(e).__name__}"
    torch.cuda.empty_cache()
    log("vendor library on the same shape: " + ", ".join(
        f"{k} {v['us']:.1f} us ({v['tflops']:.0f} TFLOP/s)" for k, v in out.items() if isinstance(v, dict)))
    return out


def cpu_baseline(rows=8192, min_seconds=10.0, max_steps=3):
    """The CPU oracle on the headline step (by default all of it; `rows` bounds
    it to a slice of X): delayed-scaled cast of `rows` rows of X, cast of the
    whole W, the dequantised GEMM of those rows (fp64 BLAS) and the history
    updates, repeated as consecutive steps until `min_seconds` have passed (at
    most `max_steps`; each takes about 5 s of host work on an MI355X machine's CPU).
    Reported in TFLOP/s of the GEMM FLOPs per step."""
    import numpy as np

    from oracle import gemm, scaling
    from synth import fc1_forward

    d = fc1_forward(8192, 4096, 16384, priors=False)
    x = scaling.widen(d["X"].data[:rows], "bf16")
    w = scaling.widen(d["W"].data, "bf16")
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        blas = threads
    sx = scaling.DelayedScaling("e4m3", 16)
    sw = scaling.DelayedScaling("e4m3", 16)
    steps = 0
    t0 = time.perf_counter()
    while steps < max_steps and (steps == 0 or time.perf_counter() - t0 < min_seconds):
        qx, ax, _ = scaling.quantize(x, sx.scale, "e4m3")
        qw, aw, _ = scaling.quantize(w, sw.scale, "e4m3")
        c = gemm.dequant_gemm(qx, "e4m3", qw, "e4m3", sx.scale_inv, sw.scale_inv)
        sx.update(ax)
        sw.update(aw)
        steps += 1
        assert np.isfinite(c).all()
    dt = (time.perf_counter() - t0) / steps
    flops = 2.0 * rows * 16384 * 4096
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas), "kind": "oracle",
            "sample": f"oracle (numpy) on {rows} of 8192 rows, {steps} consecutive steps: amax+cast of X[{rows}x4096] "
                      f"and of all of W[4096x16384] (1 thread), fp64 dequantised GEMM {rows}x4096x16384 "
                      f"(BLAS, {blas} threads of {threads} available), history updates; {dt:.1f} s per step"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the path is single-GPU; see the design notes for how it would shard).", file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_precision_numerics_amd as fm

    fm.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    # Order: the FC1 inputs and the CPU oracle first (host work), then the
    # extras, then the timed FC1 step straight after the extras' last GPU work,
    # so that its W warm-up steps start from the clock a GPU settles at under
    # sustained matrix-core load (over the first tens of launches after idle
    # the GEMM runs slower, down to ~1000 us, before it settles at 740-770 us).
    ctx = headline_prepare(torch, fm, args)
    cpu = None
    if not args.quick and not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline()
    extra = {}
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = src.numel()
        del src, dst
    if not args.quick or args.with_stream:
        extra["stream"] = stream_bench(torch, fm, args.stream_dtype)
    if not args.quick:
        other = "f32" if args.stream_dtype == "bf16" else "bf16"
        extra["stream_" + other] = stream_bench(torch, fm, other)
    if not args.quick:
        # The vendor GEMMs go first: after them this GEMM runs ~5 % slower for
        # some tens of launches; after this library's own kernels it does not.
        extra["vendor_reference"] = vendor_reference(torch)
        extra["linear_step"] = linear_bench(torch, fm)
        extra["moe_grouped"] = moe_bench(torch, fm)
        extra["grad_allreduce_parts"] = allreduce_bench(torch, fm)
        extra["mxfp8"] = mx_bench(torch, fm)
    head = headline(torch, fm, args, ctx)
    extra = {"headline": head, **extra}
    line = {
        "metric": METRIC,
        "value": round(head["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "fc1_forward_delayed_scaling", "M": 8192, "K": 4096, "N": 16384,
                   "inputs": "bf16 X (N(0,1), 0.1% x100 outliers), bf16 W N(0,0.02)", "fp8": "e4m3 x e4m3",
                   "out": "bf16", "history_len": 16, "amax_rule": "max", "accum": args.accum},
        # Priced against the dense FP8 matrix-core peak the metric names, whichever
        # instruction the accumulation mode runs on; the fraction of that
        # instruction's own peak is reported beside it.
        "roofline": {"bound": "mfma", "achieved": round(head["gemm_tflops"], 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(head["gemm_tflops"] / PEAK_FP8_TFLOPS, 4),
                     "traffic": gemm_traffic(args.accum),
                     "kernel": "gemm_kernel (%s accumulation: %s matrix cores)"
                               % (args.accum, "bf16" if args.accum == "exact" else "fp8"),
                     "instruction_peak": PEAK_BY_ACCUM[args.accum],
                     "frac_of_instruction_peak": round(head["gemm_tflops"] / PEAK_BY_ACCUM[args.accum], 4)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
