#!/usr/bin/env python3
"""Benchmark of the Llama-block library on one MI355X.

One step = one llama_block_forward over one batch of synthetic input (every
stage of the block: RMSNorm, q/k/v + RoPE + cache append, causal GQA
attention, o projection + residual, RMSNorm, gate/up + SiLU*up, down +
residual).

Default run (N = 1):
  * prefill: Llama-3-8B-width block, B=2 x S=2048 from position 0 -> the
    headline `value` in tokens/s;
  * decode:  Llama-3-8B-width block, 32 sequences x 1 new token at position
    8191 over 8191 cached positions -> reported under "decode" (us/step);
  * configs: the tiny fp32 block (latency), the SmolLM2-width prefill and the
    70B-width prefill, each with its stage times and roofline;
  * cpu_baseline: the fp64 oracle on the host cores on every row of the
    prefill workload, and per workload under cpu_baselines (the 70B width on
    its first 256 tokens).
Per-stage GPU times come from the library's HIP-event profiler on the
forward's stream: a first pass times every stage and finds the dominant one;
the timed region of `value` then records events only around that stage, whose
average duration gives `roofline`.

Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense fp16/bf16 matrix peak
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
METRIC = "block prefill tokens/s + decode µs/step; % bf16 MFMA peak / % HBM BW"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stage_work(w, positions=None, active_experts=None):
    """Algorithmic work per forward, per profiled stage: flops (matrix products,
    causal attention over visible (query, key) pairs only) and HBM bytes (each
    operand read once, each result written once).  positions: the start
    position of each sequence (default: w.start_pos for all).  For a
    mixture-of-experts block the FFN stages add the router and the routed
    experts (M * top_k rows); their weights count once per expert that the
    forward used (active_experts, default all)."""
    M, d, dh, H, G, dff = w.M, w.d, w.d_head, w.H, w.n_kv, w.d_ff
    qd, kvd = H * dh, G * dh
    e = 2  # bytes per bf16/fp16 element
    starts = list(positions) if positions is not None else [w.start_pos] * w.B
    vis = sum(p + s + 1 for p in starts for s in range(w.S))       # visible pairs per head
    kv_read = sum(G * (p + w.S) * dh * 2 * e for p in starts)       # K and V, every visible row
    out = {
        "rmsnorm_1": {"flops": 0, "bytes": M * d * (e + e)},
        "qkv_rope_append": {"flops": 2 * M * (qd + 2 * kvd) * d,
                            "bytes": (qd + 2 * kvd) * d * e + M * d * e + M * (qd + 4 * kvd) * e},
        "attention": {"flops": 4 * dh * vis * H,
                      "bytes": kv_read + 2 * M * qd * e},
        "o_proj_residual": {"flops": 2 * M * d * qd,
                            "bytes": d * qd * e + M * qd * e + M * d * (e + 4)},
        "rmsnorm_2": {"flops": 0, "bytes": M * d * (4 + e)},
        "gate_up_swiglu": {"flops": 2 * M * 2 * dff * d,
                           "bytes": 2 * dff * d * e + M * d * e + M * dff * e},
        "down_residual": {"flops": 2 * M * d * dff,
                          "bytes": d * dff * e + M * dff * e + M * d * (4 + e)},
    }
    if w.n_experts > 0:
        E, K, fe = w.n_experts, w.top_k, w.d_ff_expert
        act = E if active_experts is None else active_experts
        MK = M * K
        gu, dn = out["gate_up_swiglu"], out["down_residual"]
        # router, gathered rows, experts' gate/up, their z
        gu["flops"] += 2 * M * E * d + 2 * MK * 2 * fe * d
        gu["bytes"] += E * d * e + M * E * 4 + 2 * MK * d * e + act * 2 * fe * d * e + MK * fe * e
        # experts' down into fp32 rows, the combine
        dn["flops"] += 2 * MK * d * fe
        dn["bytes"] += act * d * fe * e + MK * fe * e + 2 * MK * d * 4 + M * d * 4
    return out


PER_CALL = 50  # forwards timed one by one for the median / p10 / p90


def make_tensors(w, on_device=False):
    """The workload's tensors: drawn on the host by workloads.generate (the
    oracle's inputs), or on the device for model-sized blocks (same
    distributions, other random streams) when on_device."""
    import workloads
    if w.n_experts > 0 or on_device:
        g = workloads.generate_stack_on_device(w, 1)
        return dict(g["layers"][0], x=g["x"])
    return workloads.generate(w)


def run_gpu(w, steps, warmup, positions=None, tensors=None, per_call=True):
    import torch

    import decoder_only_transformer_amd as lbmod

    cap = (w.capacity + 7) // 8 * 8
    cfg = lbmod.make_config(w.d, w.H, w.n_kv, w.d_head, w.d_ff, w.M, cap, w.theta, w.eps, w.dtype)
    t = tensors if tensors is not None else make_tensors(w)
    if w.n_experts > 0:
        blk = lbmod.LlamaMoeBlock(cfg, t, w.moe)
    else:
        blk = lbmod.LlamaBlock(cfg, {n: t[n].to("cuda") for n in lbmod.WEIGHT_NAMES})
    k, v = lbmod.new_kv_cache(w.B, w.n_kv, cap, w.d_head, w.torch_dtype)
    if w.start_pos > 0:
        k[:, :, : w.start_pos, :] = t["k_prefix"].to("cuda")
        v[:, :, : w.start_pos, :] = t["v_prefix"].to("cuda")
    x = t["x"].to("cuda")
    out = torch.empty_like(x)
    del t
    torch.cuda.empty_cache()
    sp = list(positions) if positions is not None else w.start_pos
    for _ in range(warmup):
        blk.forward(x, sp, (k, v), out)

    def timed(stages):
        """`steps` back-to-back forwards with the library's timing-only HIP
        events at the boundaries of `stages` (recorded on the forward's
        stream, the current torch stream); wall ms/step and per-stage ms."""
        if stages:
            lbmod.llama_block_profile(blk.handle, stages)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            blk.forward(x, sp, (k, v), out)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        avg = {}
        if stages:
            stage_ms, calls = lbmod.llama_block_profile_read(blk.handle)
            lbmod.llama_block_profile(blk.handle, 0)
            avg = {n: stage_ms[n] / max(calls, 1) for n in stage_ms if n in stages}
        return (t1 - t0) * 1e3 / steps, avg

    # 1) every stage timed: the per-stage breakdown and the dominant stage
    ms_all, avg_all = timed(list(lbmod.STAGE_NAMES))
    dom = max(avg_all, key=lambda n: avg_all[n])
    # 2) the timed region of the headline: events only around the dominant
    #    stage, so the other kernels run back to back as in production
    ms, avg_dom = timed([dom])
    # 3) the same forwards without any event, for comparison
    ms_plain, _ = timed([])
    # 4) per-call spread: each forward between its own pair of events, as is
    #    and after a 512 MB read that evicts the 256 MB MALL and the L2s (a
    #    read, so that no dirty lines are left to be written back during the
    #    timed call)
    calls = {"calls": PER_CALL}
    scratch = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    for tag, flush in ((("", False), ("flushed_", True)) if per_call else ()):
        ev = []
        for _ in range(PER_CALL):
            if flush:
                scratch.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            blk.forward(x, sp, (k, v), out)
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        d = sorted(a.elapsed_time(b) for a, b in ev)
        q = lambda f: d[min(len(d) - 1, int(round(f * (len(d) - 1))))]
        calls.update({tag + "median_ms": round(q(0.5), 4), tag + "p10_ms": round(q(0.1), 4),
                      tag + "p90_ms": round(q(0.9), 4)})
    del scratch
    active = None
    if w.n_experts > 0:
        active = int(torch.unique(blk.routing(w.M)[0]).numel())
        calls["active_experts"] = active
    blk.close()
    del k, v, x, out
    torch.cuda.empty_cache()
    return ms, avg_all, dom, avg_dom[dom], ms_plain, ms_all, calls


def run_stack(w, n_layers, steps, warmup):
    """Model-level decode: one step of a stack of n_layers blocks (each with
    its own weights and cache) and the final RMSNorm, eagerly (host
    positions) and as a replay of the captured step (device positions).
    Returns (eager ms/step, graph ms/step)."""
    import torch

    import decoder_only_transformer_amd as lbmod
    import workloads

    cap = (w.capacity + 7) // 8 * 8
    cfg = lbmod.make_config(w.d, w.H, w.n_kv, w.d_head, w.d_ff, w.M, cap, w.theta, w.eps, w.dtype)
    t = workloads.generate_stack_on_device(w, n_layers)
    stack = lbmod.LlamaStack(cfg, [{n: lt[n] for n in lbmod.WEIGHT_NAMES} for lt in t["layers"]],
                             t["final_norm"])
    kv = []
    for lt in t["layers"]:
        k, v = lbmod.new_kv_cache(w.B, w.n_kv, cap, w.d_head, w.torch_dtype, fill=None)
        if w.start_pos > 0:
            k[:, :, :w.start_pos] = lt.pop("k_prefix")
            v[:, :, :w.start_pos] = lt.pop("v_prefix")
        kv.append((k, v))
    x = t["x"]
    out = torch.empty_like(x)
    del t
    torch.cuda.empty_cache()

    def clock(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    eager = lambda: stack.forward(x, w.start_pos, kv, out)
    clock(eager, warmup)
    ms_eager = clock(eager, steps)
    # the captured step reads its positions from the device; at the end of the
    # cache they stay clamped to the last start, so every replay does the work
    # of the eager step at w.start_pos
    positions = torch.full((w.B,), w.start_pos, dtype=torch.int32, device="cuda")
    graph = stack.capture(x, positions, kv, out)
    clock(graph.launch, warmup)
    ms_graph = clock(graph.launch, steps)
    stack.close()
    del kv, x, out, positions
    torch.cuda.empty_cache()
    return ms_eager, ms_graph


def roofline(w, avg_ms, dom, dom_ms, bound, positions=None, active_experts=None):
    """Per-stage figures from the all-stage pass; the roofline entry from the
    dominant stage's own timed region."""
    work = stage_work(w, positions, active_experts)
    stages = {}
    for n, ms in avg_ms.items():
        s = ms * 1e-3
        stages[n] = {"ms": round(ms, 4),
                     "tflops": round(work[n]["flops"] / s / 1e12, 2) if s > 0 else None,
                     "gbs": round(work[n]["bytes"] / s / 1e9, 1) if s > 0 else None}
    s = dom_ms * 1e-3
    if bound == "mfma":
        a = work[dom]["flops"] / s / 1e12
        r = {"bound": "mfma", "achieved": round(a, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(a / MFMA_PEAK_TFLOPS, 4), "traffic": None, "kernel": dom,
             "kernel_ms": round(dom_ms, 4)}
    else:
        a = work[dom]["bytes"] / s / 1e9
        r = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom,
             "kernel_ms": round(dom_ms, 4)}
    return r, stages


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama3_8b.txt")
KERNEL_SOURCES = os.path.join(ROOT, "decoder_only_transformer_amd", "csrc")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCES)):
        with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` on `workload` from the counter summary
    under profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by its reading on a
    plain copy of known size), or None when there is none or when the kernel
    sources have changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha, rows = None, {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            if p[0] == "sources_sha256":
                sha = p[1]
            elif p[0] == "stage" and len(p) >= 4:
                rows[(p[1], p[2])] = float(p[3])
    if sha != kernel_sources_sha256():
        return None
    v = rows.get((workload, stage))
    return None if v is None else int(round(v))


def copy_only(mib):
    """A plain device copy of known size (out = in * 1, fp32), three times: the
    counter reading that scales FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}),
          flush=True)


def vendor_gemm(w, reps=20):
    """The vendor GEMM library (torch.mm on ROCm, hipBLASLt) on the four
    prefill products of workload w, fp16 operands, fp32 accumulation: A [M][K]
    times W[N][K]^T, timed with events over `reps` calls after 3 warm-ups.
    Context for the library's own GEMM kernels, not part of the step."""
    import torch
    M, d, qd, kvd, dff = w.M, w.d, w.H * w.d_head, w.n_kv * w.d_head, w.d_ff
    shapes = {"qkv": (qd + 2 * kvd, d), "o": (d, qd), "gate_up": (2 * dff, d), "down": (d, dff)}
    g = torch.Generator(device="cuda").manual_seed(0)
    out = {}
    for name, (N, K) in shapes.items():
        a = torch.randn(M, K, device="cuda", generator=g).mul_(1.0).half()
        b = (torch.randn(N, K, device="cuda", generator=g) * 0.02).half()
        for _ in range(3):
            c = torch.mm(a, b.t())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = torch.mm(a, b.t())
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"M": M, "N": N, "K": K, "ms": round(ms, 4),
                     "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        del a, b, c
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, tensors, rows=None, repeats=1):
    """The fp64 oracle, as it stands, on the host: one forward of workload w on
    `tensors` (its own inputs, cache prefix included), every token row or the
    flat token rows `rows` (the oracle then computes only what those rows
    see), timed `repeats` times (median).  Tokens/s counts the rows computed."""
    import oracle
    cfg = oracle.cfg_of(w)
    wts = {n: oracle._f64(tensors[n]) for n in oracle.WEIGHT_NAMES}
    x = oracle._f64(tensors["x"])
    times = []
    for _ in range(repeats):
        kc, vc = oracle.empty_cache(w)
        if w.start_pos > 0:
            kc[:, :, :w.start_pos, :] = oracle._f64(tensors["k_prefix"])
            vc[:, :, :w.start_pos, :] = oracle._f64(tensors["v_prefix"])
        t0 = time.perf_counter()
        oracle.block_forward(cfg, x, wts, w.start_pos, kc, vc, rows=rows)
        times.append(time.perf_counter() - t0)
        del kc, vc
    times.sort()
    dt = times[len(times) // 2]
    n = w.M if rows is None else len(rows)
    sample = (f"{w.name}: all {n} token rows (B={w.B}, S={w.S}, start_pos={w.start_pos})"
              if rows is None else
              f"{w.name}: the first {n} token rows of the {w.S}-token sequence (the oracle computes "
              f"only what they see)")
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3), "runs": repeats,
            "sample": sample + ", fp64 naive loops"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_prefill")
    ap.add_argument("--decode-workload", default="llama3_8b_decode")
    ap.add_argument("--decode-steps", type=int, default=0, help="default: 5 x --steps")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the model-level stack decode")
    ap.add_argument("--no-moe", action="store_true", help="skip the mixture-of-experts block")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged decode")
    ap.add_argument("--no-vendor", action="store_true", help="skip the vendor-library GEMM figures")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny fp32, SmolLM2-width and 70B-width entries")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the block's hot path is single-GPU "
              "(no collectives); multi-GPU runs are not supported.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_only:
        copy_only(args.copy_only)
        return

    w = workloads.get(args.workload)
    log(f"[bench] prefill {w.name}: warmup {args.warmup}, steps {args.steps}")
    t_pre = make_tensors(w)
    ms, avg, dom, dom_ms, ms_plain, ms_all, per_call = run_gpu(w, args.steps, args.warmup, tensors=t_pre)
    roof, stages = roofline(w, avg, dom, dom_ms, "mfma")
    roof["traffic"] = measured_traffic(w.name, roof["kernel"])
    total_flops = sum(v["flops"] for v in stage_work(w).values())
    result = {
        "metric": METRIC,
        "value": round(w.M / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_without_events": round(ms_plain, 4),
        "ms_per_step_all_stage_events": round(ms_all, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "io_dtype": w.dtype,
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "start_pos": w.start_pos, "d": w.d,
                   "H": w.H, "n_kv": w.n_kv, "d_head": w.d_head, "d_ff": w.d_ff,
                   "theta": w.theta, "parallelism": "single-gpu"},
        "block_tflops": round(total_flops / (ms * 1e-3) / 1e12, 2),
        "block_mfma_frac": round(total_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
        "roofline": roof,
        "stages": stages,
        "per_call": per_call,
    }
    log(f"[bench] prefill {ms:.3f} ms/step, {result['value']:.0f} tokens/s")
    if not args.no_vendor:
        result["vendor_gemm"] = vendor_gemm(w)
        log(f"[bench] vendor GEMM: {result['vendor_gemm']}")

    if not args.no_decode:
        wd = workloads.get(args.decode_workload)
        dsteps = args.decode_steps or 5 * args.steps
        log(f"[bench] decode {wd.name}: warmup {args.warmup}, steps {dsteps}")
        t_dec = make_tensors(wd)
        dms, davg, ddom, ddom_ms, dms_plain, dms_all, dper_call = run_gpu(wd, dsteps, args.warmup, tensors=t_dec)
        droof, dstages = roofline(wd, davg, ddom, ddom_ms, "hbm")
        droof["traffic"] = measured_traffic(wd.name, droof["kernel"])
        total_bytes = sum(v["bytes"] for v in stage_work(wd).values())
        result["decode"] = {
            "workload": wd.name, "B": wd.B, "start_pos": wd.start_pos, "steps": dsteps,
            "us_per_step": round(dms * 1e3, 2),
            "us_per_step_without_events": round(dms_plain * 1e3, 2),
            "us_per_step_all_stage_events": round(dms_all * 1e3, 2),
            "tokens_per_s": round(wd.M / (dms * 1e-3), 1),
            "block_gbs": round(total_bytes / (dms * 1e-3) / 1e9, 1),
            "block_hbm_frac": round(total_bytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": droof, "stages": dstages, "per_call": dper_call,
        }
        log(f"[bench] decode {dms * 1e3:.1f} us/step")

    if not args.no_decode and not args.no_ragged:
        # one sequence: the per-token latency case
        wb = workloads.get("llama3_8b_decode_b1")
        log(f"[bench] decode {wb.name}: warmup {args.warmup}, steps {dsteps}")
        bms, bavg, bdom, bdom_ms, bms_plain, _, bper = run_gpu(wb, dsteps, args.warmup)
        broof, bstages = roofline(wb, bavg, bdom, bdom_ms, "hbm")
        bbytes = sum(v["bytes"] for v in stage_work(wb).values())
        result["decode_b1"] = {
            "workload": wb.name, "B": wb.B, "start_pos": wb.start_pos, "steps": dsteps,
            "us_per_step": round(bms * 1e3, 2), "us_per_step_without_events": round(bms_plain * 1e3, 2),
            "block_gbs": round(bbytes / (bms * 1e-3) / 1e9, 1),
            "block_hbm_frac": round(bbytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "dominant_stage": broof, "stages": bstages, "per_call": bper,
        }
        log(f"[bench] decode one sequence {bms * 1e3:.1f} us/step")

        # the same decode with every sequence at its own position (ragged
        # batch): positions spread evenly from 1024 to the workload's last one
        pos = [1024 + (wd.start_pos - 1024) * b // max(wd.B - 1, 1) for b in range(wd.B)]
        log(f"[bench] ragged decode: positions {pos[0]}..{pos[-1]}")
        rms, ravg, rdom, rdom_ms, rms_plain, rms_all, _ = run_gpu(wd, dsteps, args.warmup, pos, tensors=t_dec)
        rroof, rstages = roofline(wd, ravg, rdom, rdom_ms, "hbm", pos)
        rroof["traffic"] = None  # counters are taken for the uniform decode only
        rbytes = sum(v["bytes"] for v in stage_work(wd, pos).values())
        result["decode_ragged"] = {
            "workload": wd.name, "B": wd.B, "positions": f"{pos[0]}..{pos[-1]} evenly spread",
            "steps": dsteps, "us_per_step": round(rms * 1e3, 2),
            "us_per_step_without_events": round(rms_plain * 1e3, 2),
            "tokens_per_s": round(wd.M / (rms * 1e-3), 1),
            "block_gbs": round(rbytes / (rms * 1e-3) / 1e9, 1),
            "block_hbm_frac": round(rbytes / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": rroof, "stages": rstages,
        }
        log(f"[bench] ragged decode {rms * 1e3:.1f} us/step")

    if not args.no_moe:
        # mixture-of-experts block (shared expert + top-k routed experts)
        result["moe"] = []
        for name, bound in (("llama4_moe_prefill", "mfma"), ("llama4_moe_decode", "hbm")):
            wm = workloads.get(name)
            msteps = args.steps if bound == "mfma" else 5 * args.steps
            log(f"[bench] moe {name}: warmup {args.warmup}, steps {msteps}")
            mms, mavg, mdom, mdom_ms, mms_plain, _, mper = run_gpu(wm, msteps, args.warmup)
            act = mper.get("active_experts")
            mroof, mstages = roofline(wm, mavg, mdom, mdom_ms, bound, active_experts=act)
            work = stage_work(wm, active_experts=act)
            fl = sum(v["flops"] for v in work.values())
            by = sum(v["bytes"] for v in work.values())
            entry = {"workload": name, "B": wm.B, "S": wm.S, "start_pos": wm.start_pos, "n_experts": wm.n_experts,
                     "top_k": wm.top_k, "d_ff_expert": wm.d_ff_expert, "d_ff_shared": wm.d_ff,
                     "active_experts": act, "steps": msteps, "ms_per_step": round(mms, 4),
                     "ms_per_step_without_events": round(mms_plain, 4),
                     "tokens_per_s": round(wm.M / (mms * 1e-3), 1),
                     "block_tflops": round(fl / (mms * 1e-3) / 1e12, 2),
                     "block_mfma_frac": round(fl / (mms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                     "block_gbs": round(by / (mms * 1e-3) / 1e9, 1),
                     "block_hbm_frac": round(by / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "dominant_stage": mroof, "stages": mstages}
            result["moe"].append(entry)
            log(f"[bench] moe {name}: {mms:.3f} ms/step")

    if not args.no_stack:
        # model-level decode: every block of the model, then the final norm
        # (no embedding, no output projection)
        result["stack_decode"] = []
        for name, n_layers in (("llama3_8b_decode", 32), ("smollm2_135m_decode", 30),
                               ("smollm2_135m_decode_b1", 30)):
            ws = workloads.get(name)
            log(f"[bench] stack decode {name} x {n_layers} blocks")
            se, sg = run_stack(ws, n_layers, args.steps, args.warmup)
            sbytes = n_layers * sum(v["bytes"] for v in stage_work(ws).values())
            result["stack_decode"].append({
                "workload": name, "blocks": n_layers, "B": ws.B, "start_pos": ws.start_pos,
                "eager_ms_per_step": round(se, 4), "graph_ms_per_step": round(sg, 4),
                "tokens_per_s": round(ws.B / (min(se, sg) * 1e-3), 1),
                "gbs": round(sbytes / (min(se, sg) * 1e-3) / 1e9, 1),
                "hbm_frac": round(sbytes / (min(se, sg) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            log(f"[bench] stack decode {name}: eager {se:.3f} ms, graph {sg:.3f} ms")

    # the other workloads of the benchmark suite: the tiny fp32 block (latency),
    # the SmolLM2-width prefill and the 70B-width prefill (weights drawn on the
    # device), each with its stage times and roofline
    extra = {}
    if not args.no_configs:
        result["configs"] = []
        for name, bound, steps, on_dev in (("tiny_f32", "latency", 5 * args.steps, False),
                                           ("smollm2_135m_prefill", "mfma", 5 * args.steps, False),
                                           ("llama3_70b_prefill", "mfma", max(args.steps // 2, 3), True)):
            wc = workloads.get(name)
            log(f"[bench] {name}: warmup {args.warmup}, steps {steps}")
            tc = make_tensors(wc, on_device=on_dev)
            cms, cavg, cdom, cdom_ms, cms_plain, _, _ = run_gpu(wc, steps, args.warmup, tensors=tc, per_call=False)
            work = stage_work(wc)
            fl = sum(v["flops"] for v in work.values())
            entry = {"workload": name, "B": wc.B, "S": wc.S, "start_pos": wc.start_pos, "d": wc.d, "H": wc.H,
                     "n_kv": wc.n_kv, "d_head": wc.d_head, "d_ff": wc.d_ff, "dtype": wc.dtype, "steps": steps,
                     "ms_per_step": round(cms, 4), "us_per_step": round(cms * 1e3, 2),
                     "ms_per_step_without_events": round(cms_plain, 4),
                     "tokens_per_s": round(wc.M / (cms * 1e-3), 1)}
            if bound == "mfma":
                croof, cstages = roofline(wc, cavg, cdom, cdom_ms, "mfma")
                entry.update({"block_tflops": round(fl / (cms * 1e-3) / 1e12, 2),
                              "block_mfma_frac": round(fl / (cms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                              "roofline": croof, "stages": cstages})
            else:
                _, cstages = roofline(wc, cavg, cdom, cdom_ms, "mfma")
                entry.update({"bound": "latency (1.5 MFLOP per call)", "stages": cstages})
            result["configs"].append(entry)
            extra[name] = tc
            log(f"[bench] {name}: {cms * 1e3:.1f} us/step")

    if not args.no_cpu_baseline:
        # the fp64 oracle on the host cores, per workload: the headline one on
        # every row of the 8B-width prefill, the others beside their GPU entries
        log("[bench] cpu baseline: oracle on every row of the 8B-width prefill")
        result["cpu_baseline"] = cpu_baseline(w, t_pre)
        log(f"[bench] cpu baseline {result['cpu_baseline']['seconds']} s")
        cb = {"llama3_8b_prefill": result["cpu_baseline"]}
        if not args.no_decode:
            log("[bench] cpu baseline: decode (median of 3)")
            cb[wd.name] = cpu_baseline(wd, t_dec, repeats=3)
        for name, tc in extra.items():
            wc = workloads.get(name)
            if wc.M <= 4096 and name != "llama3_70b_prefill":
                log(f"[bench] cpu baseline: {name} (median of 3)")
                cb[name] = cpu_baseline(wc, tc, repeats=3)
            else:
                log(f"[bench] cpu baseline: {name}, first 256 tokens")
                cb[name] = cpu_baseline(wc, tc, rows=list(range(256)))
        result["cpu_baselines"] = cb
        for name, v in cb.items():
            log(f"[bench] cpu baseline {name}: {v['seconds']} s, {v['value']} tokens/s")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
