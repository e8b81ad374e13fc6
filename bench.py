"""Throughput of the four-layer bidirectional LSTM stack on one MI355X.

One step = one bilstm_forward over a batch of synthetic windows (the whole hot path: four
projections and eight direction recurrences). Default workload: 32 windows x 589 frames.

Prints one JSON line: frames/s over the timed steps, per-phase times from the plan's HIP
events, the recurrence's roofline figures and per-step latency against its on-chip bound,
the projection's fraction of FP32-MFMA peak, and the oracle timed on the host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_FP32_MFMA_TFLOPS = 157.3      # MI355X dense FP32 matrix peak (published)
PEAK_FP32_VECTOR_TFLOPS = 157.3    # MI355X FP32 vector peak (published)
CLOCK_GHZ = 2.4
# FP32 FMA per clock per CU implied by the published vector peak:
# 157.3e12 / (256 CUs x 2.4e9 Hz x 2 flop) = 128
FMA_PER_CLK_PER_CU = 128

RECUR_FMA_PER_FRAME_DIR = 512 * 128                   # R·h per step per direction
HEAD_FLOP_PER_FRAME = 2 * (256 * 128 + 128 * 128 + 128 * 7)   # segmentation heads
HEAD_BYTES_PER_FRAME = 256 * 4 + 7 * 4                          # stack output read, log-probs written


def projection_flops(frames: int) -> float:
    """Algorithmic FLOPs of the four projections: 2·M·1024·K summed over K = 60, 256, 256, 256."""
    return 2.0 * frames * 1024 * (60 + 3 * 256)


def recurrence_flops_per_layer(frames: int) -> float:
    """Algorithmic FLOPs of one layer's recurrence, both directions: 2·65,536 per frame and direction."""
    return 2.0 * 2 * frames * RECUR_FMA_PER_FRAME_DIR


def kernel_source_digest() -> str:
    """Digest of the recurrence kernel's sources, to tell whether recorded counters still apply."""
    h = hashlib.sha256()
    for name in ("kernels_recurrence.hip", "bilstm_internal.h"):
        with open(os.path.join(ROOT, "bidirectional_lstm_sequence_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str, info: dict):
    """HBM bytes per recurrence launch from the rocprofv3 counters recorded in profiles/.

    Returns (bytes, detail), or (None, None) unless the counters were taken on this kernel
    source, workload, kernel (streamed or not) and recurrence split. Counter collection runs
    kernels one at a time, so the streamed recurrence is counted in the streamed plan without
    layer overlap (the next layer's projection starts after this layer's recurrence, so no
    kernel waits for one that starts after it); the recurrence kernel, its gates and its outputs
    are the same as in the default streamed plan."""
    path = os.path.join(ROOT, "profiles", "recurrence_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, None
    if (rec.get("source_sha256") != kernel_source_digest() or rec.get("workload") != workload
            or rec.get("streamed") != bool(info["pipeline"]) or rec.get("groups") != info["recur_groups"]
            or rec.get("tile") != info["recur_tile"] or rec.get("concurrent") != info["concurrent"]):
        return None, None
    detail = {"bytes_per_launch": rec["fetch_bytes"] + rec["write_bytes"], "fetch_bytes": rec["fetch_bytes"],
              "write_bytes": rec["write_bytes"], "algorithmic_bytes": rec.get("algorithmic_bytes"),
              "kernel": rec["kernel"], "windows_per_launch": rec["windows_per_launch"],
              "counter_run": rec["command"], "source": "profiles/recurrence_traffic.json"}
    return detail["bytes_per_launch"], detail


def cpu_baseline(x, layers, steps, max_threads=16, target_windows=None):
    """The oracle (fp64, unchanged) on the host: the all-threads rate over a bounded sample of
    windows, and the single-core rate of its single-threaded routine on one window."""
    import oracle
    oracle.build(force=False)
    host_cores = os.cpu_count() or 1
    threads = max(1, min(max_threads, host_cores))
    windows = target_windows or min(x.shape[0], 2 * threads)
    idx = list(range(windows))
    t0 = time.perf_counter()
    oracle.stack(x, layers, windows=idx, threads=threads)
    wall = time.perf_counter() - t0
    used = min(threads, windows)
    t1 = time.perf_counter()
    oracle.stack(x, layers, windows=[0], threads=1)
    one = time.perf_counter() - t1
    return {"value": windows * steps / wall, "unit": "frames/s", "cores": used, "kind": "oracle",
            "sample": f"{windows} of the {x.shape[0]} windows ({windows * steps} frames), one window per "
                      f"task on {used} threads, fp64 single-threaded routine per window; wall {wall:.2f} s",
            "host_cores": host_cores,
            "single_core": {"value": steps / one, "unit": "frames/s", "sample": f"window 0 ({steps} frames) on "
                            f"one thread; wall {one:.2f} s"}}


PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)


def split_bf16_rates(split: dict, products: int) -> dict:
    """A split-precision projection runs `products` bf16 products per FP32 product: its rate in
    bf16 MFMA flops, against the bf16 dense peak (its own dtype's), beside the FP32-equivalent
    rate in `achieved_tflops`."""
    if "achieved_tflops" not in split:
        return {}
    bf16 = products * split["achieved_tflops"]
    return {"note": "achieved_tflops and frac: FP32-equivalent flops over time against the FP32 MFMA peak; "
                    f"bf16_tflops and frac_of_bf16_peak: the {products} bf16 products per FP32 one that the "
                    "matrix pipes run, against the bf16 dense peak",
            "bf16_tflops": bf16, "bf16_peak_tflops": PEAK_BF16_MFMA_TFLOPS,
            "frac_of_bf16_peak": bf16 / PEAK_BF16_MFMA_TFLOPS}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="b32", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--groups", type=int, default=0)
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--concurrent", type=int, default=-1)
    ap.add_argument("--slices", type=int, default=0)
    ap.add_argument("--projection", type=int, default=0, choices=(0, 1, 2, 3, 4),
                    help="0 the plan's rule (default), 1 vendor GEMM, 2 and 3 own split-precision kernel "
                         "(two or three bf16 parts), 4 own FP32-MFMA kernel")
    ap.add_argument("--pipeline", type=int, default=0, choices=(0, 1, 2, 3, 4, 5),
                    help="streamed gates: 0 auto, 1 off, 2 on, 3 on without and 4 on with layer overlap, "
                         "5 on with every kernel after the previous one (for counter collection)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--fma-probe", action="store_true",
                    help="only measure the FP32 FMA issue rate the recurrence's bound rests on: shader clocks per "
                         "wave64 FMA per SIMD with 1, 2 and 4 waves per SIMD, on one CU and on every CU")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only measure the matrix-core rates the projection's peaks rest on: bf16 32x32x16 and "
                         "FP32 32x32x2 MFMAs on every CU with zero, constant and random operands")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times), to calibrate the HBM "
                         "byte counters of a profiler run against a known size")
    args = ap.parse_args()

    if args.copy_calibration > 0:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}))
        return 0

    if args.mfma_probe:
        import bidirectional_lstm_sequence_amd as bl
        rows = []
        for kind, name, peak in ((0, "bf16 32x32x16", PEAK_BF16_MFMA_TFLOPS), (1, "fp32 32x32x2", PEAK_FP32_MFMA_TFLOPS)):
            for data, dname in ((0, "zeros"), (1, "ones"), (2, "uniform [-1, 1)")):
                r = bl.probe_mfma_rate(kind, data, 0, 20000 if kind == 0 else 5000)
                rows.append({"mfma": name, "operands": dname, **r, "peak_tflops": peak, "frac": r["tflops"] / peak})
        print(json.dumps({"mfma_probe": rows, "note": "two 256-thread workgroups per CU on every CU, 16 MFMAs per "
                          "round over 4 independent accumulators, operands in registers; the second of two launches"}))
        return 0

    if args.fma_probe:
        import torch
        import bidirectional_lstm_sequence_amd as bl
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        rows = []
        for wg in (1, 64, cus):
            for wps in (1, 2, 4):
                r = bl.probe_fma_rate(0, wps, wg, 20000)
                rows.append({"workgroups": wg, "waves_per_simd": wps, **r,
                             "fma_per_clk_per_cu": 4 * 64 / r["clocks_per_fma"]})
        print(json.dumps({"fma_probe": rows, "note": "128 FP32 FMAs per lane per round over 8 accumulators "
                          "(v_fmac_f32, register operands), 20000 rounds; median workgroup"}))
        return 0

    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the stack would shard by windows (each GPU its own "
                                   "windows, no collective on the hot path), but no multi-GPU path is built",
                          "n_gpus": args.gpus}))
        return 2

    import torch
    import bidirectional_lstm_sequence_amd as bl

    wl = workloads.WORKLOADS[args.workload]
    x, layers = workloads.make_workload(wl)
    frames = wl.batch * wl.steps
    plan = bl.Plan(layers, wl.batch, wl.steps, groups=args.groups, tile=args.tile,
                   concurrent=args.concurrent, slices=args.slices, projection=args.projection,
                   pipeline=args.pipeline)
    info = plan.info()
    xd = torch.from_numpy(x).cuda()
    yd = torch.empty((wl.batch, wl.steps, 256), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        plan.forward(xd, yd)
    plan.check()

    # timed region: exactly K forwards, bracketed by synchronisation and by one pair of HIP
    # events on the caller's stream (the plan joins its projection stream back into it; an
    # event after every forward would serialise the forwards a little more). The last forward
    # runs with the plan's phase events on, which time each phase and the recurrence launch.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for k in range(args.steps):
        if k == args.steps - 1:
            plan.set_phase_events(True)
        plan.forward(xd, yd)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    plan.check()
    total_ms = ev0.elapsed_time(ev1)
    value = frames * args.steps / (total_ms / 1e3)
    timed_phases = plan.phase_times()

    # The dominant kernel's average launch duration over the timed region. With streamed gates
    # every recurrence launch runs on the caller's stream, back to back (each waits inside for
    # its first chunk; the projections run on the plan's own stream), so the two HIP events that
    # bracket the timed region, on that stream, hold exactly the forwards' recurrence launches:
    # their average is the region's time over the launches in it (an upper bound: it includes
    # the few microseconds between launches). Otherwise (projections and recurrences alternate
    # on the stream) the launch bracketed by the plan's phase events in the last timed forward.
    fused = bool(info["stream_fused"])
    layers_per_launch = 4 if fused else 1
    launches_per_forward = 1 if fused else 4
    events_ms = (sum(timed_phases["recurrence_launch_ms"]) if fused
                 else statistics.mean(timed_phases["recurrence_launch_ms"]))
    back_to_back = bool(info["pipeline"]) and info["concurrent"] == 2 and info["recur_launches"] == 1 \
        and info["slices"] == 1
    if back_to_back:
        launch_dur_ms = total_ms / args.steps / launches_per_forward
        launch_source = (f"timed region over its {args.steps * launches_per_forward} recurrence launches (HIP events "
                         "on the caller's stream, where they run back to back)")
    else:
        launch_dur_ms = events_ms
        launch_source = "the plan's HIP events around the launch in the last timed forward"
    slice_windows = info["slice_windows"] if info["slices"] > 1 else wl.batch
    launch_dirs = 2 if info["concurrent"] == 2 else 1
    flop_per_launch = layers_per_launch * launch_dirs * recurrence_flops_per_layer(slice_windows * wl.steps) / 2

    # Each kernel alone, outside the timed region, on the whole batch: the projection of every
    # layer (bilstm_project) and the recurrence of every layer (bilstm_recur), each between HIP
    # events on the caller's stream; medians over repetitions.
    reps = max(3, min(9, args.steps))
    gates = torch.empty((frames, 1024), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(yd)
    proj_ms = [[] for _ in range(4)]
    rec_ms = [[] for _ in range(4)]
    layer_in = [xd.view(frames, 60)] + [yd.view(frames, 256)] * 3
    for _ in range(reps):
        for l in range(4):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(stream)
            plan.project(l, layer_in[l], gates)
            e1.record(stream)
            plan.recur(l, gates, y2)
            e2.record(stream)
            torch.cuda.synchronize()
            proj_ms[l].append(e0.elapsed_time(e1))
            rec_ms[l].append(e1.elapsed_time(e2))
    plan.check()
    proj_med = [statistics.median(v) for v in proj_ms]
    rec_med = [statistics.median(v) for v in rec_ms]
    plan.close()

    # The plan's projection inside an unstreamed forward of its own (whole batch, one slice),
    # between the plan's phase events: each layer's projection phase is its kernel plus the
    # launch gap, as the kernel trace sees it, without the per-call completion event (a
    # system-scope fence) that each bilstm_project call above pays.
    def projection_phases(mode):
        pplan = bl.Plan(layers, wl.batch, wl.steps, pipeline=1, slices=1, projection=mode)
        y3 = torch.empty_like(yd)
        pplan.forward(xd, y3)
        pplan.set_phase_events(True)
        ms = [[] for _ in range(4)]
        for _ in range(reps):
            pplan.forward(xd, y3)
            for l, v in enumerate(pplan.phase_times()["projection_ms"]):
                ms[l].append(v)
        pplan.check()
        pplan.close()
        return [statistics.median(v) for v in ms]
    proj_phase_med = projection_phases(info["projection"])

    # the other projection modes, each alone on the whole batch: the vendor GEMM (hipBLASLt,
    # FP32, bias epilogue), the own kernel in split precision (two and three bf16 parts) and, when
    # the plan chose a split, the own FP32 kernel
    def other_projection(mode):
        ms = [[] for _ in range(4)]
        try:
            oplan = bl.Plan(layers, wl.batch, wl.steps, projection=mode)
            for _ in range(reps + 1):
                for l in range(4):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    oplan.project(l, layer_in[l], gates)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    ms[l].append(e0.elapsed_time(e1))
            oplan.close()
        except Exception as e:  # measurement only
            return {"error": str(e)}
        med = [statistics.median(v[1:]) for v in ms]
        tf = projection_flops(frames) / (sum(med) / 1e3) / 1e12
        return {"ms_per_layer": med, "achieved_tflops": tf, "frac": tf / PEAK_FP32_MFMA_TFLOPS,
                "tflops_per_layer": [2.0 * frames * 1024 * k / (v / 1e3) / 1e12
                                     for k, v in zip((60, 256, 256, 256), med)]}
    library_projection = other_projection(1)
    split_projection = other_projection(2)
    split3_projection = other_projection(3)
    fp32_projection = other_projection(4) if info["projection"] != 4 else None

    # the fused segmentation heads after the stack, alone, on this workload's stack output
    heads = bl.Heads(workloads.make_heads(wl.seed))
    logp = torch.empty((wl.batch, wl.steps, 7), dtype=torch.float32, device="cuda")
    heads_ms = []
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        heads.forward(yd, logp)
        e1.record(stream)
        torch.cuda.synchronize()
        heads_ms.append(e0.elapsed_time(e1))
    heads.close()
    heads_med = statistics.median(heads_ms[1:])
    heads_tflops = HEAD_FLOP_PER_FRAME * frames / (heads_med / 1e3) / 1e12

    # recurrence: the dominant kernel. Its achieved rate is the algorithmic FLOPs of one launch
    # over that launch's duration in the timed region (events on the stream it runs on).
    rec_tflops = flop_per_launch / (launch_dur_ms / 1e3) / 1e12
    rec_layer_ms = statistics.mean(rec_med)
    us_per_step = rec_layer_ms * 1e3 / wl.steps
    traffic, traffic_detail = recorded_traffic(wl.name, info)
    groups, tile = info["recur_groups"], info["recur_tile"]
    fma_clk = RECUR_FMA_PER_FRAME_DIR * tile / groups / FMA_PER_CLK_PER_CU
    xchg_ns = None
    if not args.no_probe:
        try:
            xchg_ns = bl.probe_exchange(0, True, 2000)["one_way_ns"]
        except Exception as e:  # measurement only
            print(f"exchange probe failed: {e}", file=sys.stderr)
    bound_us = fma_clk / (CLOCK_GHZ * 1e3) + ((xchg_ns or 0.0) / 1e3 if groups > 1 else 0.0)

    # projection: fraction of FP32-MFMA peak over the four projections, from the phases of an
    # unstreamed forward; per call (bilstm_project between the caller's events) beside it
    proj_total_ms = sum(proj_phase_med)
    proj_tflops = projection_flops(frames) / (proj_total_ms / 1e3) / 1e12
    proj_layer_tflops = [2.0 * frames * 1024 * k / (ms / 1e3) / 1e12
                         for k, ms in zip((60, 256, 256, 256), proj_phase_med)]
    call_tflops = projection_flops(frames) / (sum(proj_med) / 1e3) / 1e12

    out = {
        "metric": "frames/sec through 4-layer BiLSTM (H=128) at B=32,T=589; per-step latency",
        "value": value,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {1: "f32", 2: "f32 (projection: two-part bf16 split, 3 products, FP32 accumulate)",
                  3: "f32 (projection: three-part bf16 split, 6 products, FP32 accumulate)",
                  4: "f32"}[info["projection"]],
        "data": "synthetic: seeded U(-1/sqrt(128), 1/sqrt(128)) weights, N(0,1) input windows",
        "config": {"workload": f"{wl.name}: {wl.batch} windows x {wl.steps} frames, 4-layer BiLSTM "
                               f"H=128, input 60", "batch": wl.batch, "seq_len": wl.steps,
                   "recurrence_split": {"groups": groups, "tile": tile, "tiles": info["recur_tiles"],
                                        "concurrent": info["concurrent"]},
                   "slices": info["slices"], "slice_windows": info["slice_windows"],
                   "streamed_gates": {"on": bool(info["pipeline"]), "chunk_steps": info["stream_chunk"],
                                      "layers_overlap": bool(info["stream_overlap"]),
                                      "one_recurrence_launch": fused}},
        "roofline": {"kernel": (f"recurrence_stream_kernel<{tile}>" if info["pipeline"]
                                else f"recurrence_kernel<{groups}, {tile}>") +
                               f" ({launch_dirs} direction(s), {layers_per_launch} layer(s) per launch"
                               f"{', streamed gates' if info['pipeline'] else ''})",
                     "bound": "alu", "achieved": rec_tflops, "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                     "frac": rec_tflops / PEAK_FP32_VECTOR_TFLOPS,
                     "traffic": traffic,
                     "launch_ms": launch_dur_ms,
                     "launch_ms_source": launch_source,
                     "launch_ms_last_forward_events": events_ms,
                     "flop_per_launch": flop_per_launch,
                     "layers_per_launch": layers_per_launch,
                     "windows_per_launch": slice_windows,
                     "traffic_detail": traffic_detail},
        "recurrence_step": {"us_per_step": us_per_step, "bound_us": bound_us,
                            "frac_of_bound": bound_us / us_per_step, "exchange_one_way_ns": xchg_ns,
                            "bound_terms": f"FMA {fma_clk:.0f} clk at {FMA_PER_CLK_PER_CU} FMA/clk/CU, "
                                           f"{CLOCK_GHZ} GHz" + (" + one exchange" if groups > 1 else "")},
        "projection": dict({"mode": {2: "split, two bf16 parts", 3: "split, three bf16 parts",
                                     4: "FP32 MFMA"}.get(info["projection"], str(info["projection"])),
                            "ms_total": proj_total_ms, "ms_per_layer": proj_phase_med, "achieved_tflops": proj_tflops,
                            "tflops_per_layer": proj_layer_tflops,
                            "peak_tflops": PEAK_FP32_MFMA_TFLOPS, "frac": proj_tflops / PEAK_FP32_MFMA_TFLOPS,
                            "method": "each layer's projection phase in an unstreamed forward of the same projection "
                                      "(whole batch, the plan's phase events; medians)",
                            "per_call": {"ms_per_layer": proj_med, "achieved_tflops": call_tflops,
                                         "frac": call_tflops / PEAK_FP32_MFMA_TFLOPS,
                                         "method": "bilstm_project between HIP events on the caller's stream, "
                                                   "including the call's completion event"}},
                           **(split_bf16_rates({"achieved_tflops": proj_tflops}, 3 if info["projection"] == 2 else 6)
                              if info["projection"] in (2, 3) else {})),
        "projection_vendor_gemm": library_projection,
        "projection_split_bf16x3": dict(split_projection, **split_bf16_rates(split_projection, 3)),
        "projection_split_bf16x6": dict(split3_projection, **split_bf16_rates(split3_projection, 6)),
        **({"projection_fp32": fp32_projection} if fp32_projection is not None else {}),
        "heads": {"ms": heads_med, "achieved_tflops": heads_tflops, "peak_tflops": PEAK_FP32_MFMA_TFLOPS,
                  "frac": heads_tflops / PEAK_FP32_MFMA_TFLOPS,
                  "hbm_gbs": HEAD_BYTES_PER_FRAME * frames / (heads_med / 1e3) / 1e9,
                  "note": "linear0 + LeakyReLU, linear1 + LeakyReLU, classifier + log-softmax, fused; "
                          "not part of the timed step"},
        "kernels_alone_ms": {"projection": proj_med, "recurrence": rec_med},
        "phases_ms_first_slice": {"projection": timed_phases["projection_ms"],
                                  "recurrence": timed_phases["recurrence_ms"]},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, layers, wl.steps)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
