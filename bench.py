#!/usr/bin/env python3
"""Benchmark: batch-1 decode of one 256-expert MXFP4 MoE layer on one MI355X.

Workload (the layer the pages' model uses at decode: 256 routed experts plus
one shared expert, hidden 4096, expert intermediate 2048, top-8, 13,369,344
bytes per FP4 expert): one step = route one token's fp32 logits (top-8,
renormalised) + the SwiGLU MLP of the 8 selected experts and the shared
expert on MXFP4 weights + the weighted combine to a bf16 output, issued as one
moe_layer_decode call: one kernel at full width (the layer flagged for the
single launch, which the library takes on a device whose CUs hold the whole
grid; --two-launch asks for the two-kernel step instead).  Each step uses fresh seeded logits and
activations; every expert is resident in HBM.  The model has many such layers
(43): the timed steps rotate over --layers resident layers (8 by default,
27.5 GB), each with its own experts and shared expert, so consecutive steps
share no weights and none of a step's bytes can come from the 256 MB
last-level cache; single-layer steady and cold latencies are reported beside.

Prints one JSON line: tokens/s of the whole step, the achieved HBM bandwidth
of the dominant kernel (the single launch; with two launches, the gate/up
GEMV) against the 8 TB/s peak, and the CPU oracle timed on the host on a
bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "decode-b1"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="graph: the timed steps are captured into one HIP graph and replayed; "
                         "eager: one launch sequence per step from the host")
    ap.add_argument("--workload", choices=("decode-b1", "decode-b64", "prefill", "slotcache", "slotcache-prefill"),
                    default="decode-b1",
                    help="decode-b1 (default, the headline line): batch-1 decode of a resident 256-expert "
                         "layer; decode-b64: 64 tokens, top-6, Zipf-skewed routing, grouped by expert; "
                         "prefill: 4096 tokens, top-8, MXFP8 x MXFP4 scaled MFMA; "
                         "slotcache: 512 tokens x 8 layers through the 512-slot cache with the (2,4) ladder; "
                         "slotcache-prefill: 4096-token prompt chunks through the same 8 layers by whole-layer "
                         "streaming into two layer buffers of the cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=8,
                    help="decode-b1: resident layers the timed steps rotate over (step s runs layer s mod L)")
    ap.add_argument("--tp-share", type=int, default=1,
                    help="decode-b1 on rank 0's share of G-way tensor parallelism (experts cut along I)")
    ap.add_argument("--single-launch", action="store_true",
                    help="decode-b1: layers flagged MOE_LAYER_SINGLE_LAUNCH (routing through combine in one kernel; "
                         "hidden 4096 with I 2048, or I 256 with --tp-share 8); the default at full width")
    ap.add_argument("--two-launch", action="store_true",
                    help="decode-b1 at full width: the two-launch step (gate/up, then down + combine) instead of "
                         "the single launch")
    ap.add_argument("--slot-tier", action="store_true",
                    help="slotcache workload with a 100-slot 2-bit device tier and LFU eviction "
                         "(decay 0.95, counts seeded from a separate 64-token routing trace)")
    ap.add_argument("--prefetch", type=int, default=0, metavar="R",
                    help="slotcache workload with an R-entry staging ring fed, two layers ahead, by "
                         "12-expert predictions of controlled recall (computed before the timed loop)")
    ap.add_argument("--prefetch-recall", type=float, default=0.75,
                    help="share of the true top-k each prediction holds")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (known bytes for HBM counter scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="lower bound on the oracle's timed CPU work (whole tokens)")
    return ap.parse_args()


def kernel_hash(files=("decode_b1.hip", "b1_dev.h", "route_dev.h", "common.h")) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mxfp4_routed_expert_renorm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


B64_KERNEL_FILES = ("prefill.hip", "common.h")
FUSED_KERNEL_FILES = ("decode_fused.hip", "handoff_dev.h", "b1_dev.h", "route_dev.h", "common.h")


def traffic_from_profiles(khash: str, record: str = "traffic_gateup_decode_b1.json"):
    """HBM bytes per launch of the gate/up kernel from committed counter runs,
    or None when absent or taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", record)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_hash") != khash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Host threads this process may use, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_tokens(min_seconds: float, first_step: int, stride: int):
    """Whole tokens of the batch-1 decode workload through the oracle, until
    at least min_seconds of timed oracle work; inputs are generated untimed.
    Returns (tokens, seconds)."""
    from mxfp4_routed_expert_renorm_amd import workloads as W
    from oracle import moe_oracle as O

    cfg = W.WORKLOADS[DEFAULT_WORKLOAD]
    seed = cfg["seed"]
    H, I, k = cfg["H"], cfg["I"], cfg["k"]
    toks, t_used = 0, 0.0
    while t_used < min_seconds or toks == 0:
        d = W.make_layer_inputs(cfg, seed, step=first_step + toks * stride, with_bank=False)
        lg = d["logits"]
        ids, _ = O.route(lg, k)
        recs = {int(e): W.fp4_record(seed, W.S_BANK, int(e), H, I) for e in ids[0]}
        shared = W.fp4_record(seed, W.S_SHARED, 0, H, I)
        x = O.bf16_bits_to_f64(d["x"])
        t0 = time.perf_counter()
        ids, w = O.route(lg, k)
        out = O.layer_forward(x, ids, w, lambda e: recs[int(e)], H, I, shared_rec=shared)
        O.round_to_bf16(out)
        t_used += time.perf_counter() - t0
        toks += 1
    return toks, t_used


def cpu_baseline(min_seconds: float, threads: int = 1):
    """The oracle as it stands, on whole tokens of the same workload, BLAS
    limited to one thread per worker; with threads > 1, that many host threads
    each run whole tokens at once (NumPy releases the interpreter lock in its
    array work) and the rates of the threads add up."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        if threads == 1:
            toks, t_used = _oracle_tokens(min_seconds, 0, 1)
            return {"value": toks / t_used, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{toks} token(s) of the batch-1 decode workload (route + 9 experts dequantised "
                              f"and evaluated in float64 + combine), one thread; input generation excluded; "
                              f"{t_used:.1f} s"}
        with ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(lambda i: _oracle_tokens(min_seconds, i, threads), range(threads)))
    value = sum(n / t for n, t in res)
    ntok = sum(n for n, _ in res)
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{ntok} token(s) of the batch-1 decode workload on {threads} threads at once (each thread: "
                      f"whole tokens, route + 9 experts dequantised and evaluated in float64 + combine, BLAS one "
                      f"thread); value = the sum of the threads' tokens per second of their own timed work; input "
                      f"generation excluded; at least {min_seconds:.0f} s per thread"}


def step_latency(torch, step, steps, flush_bytes=1 << 30, flush=True):
    """Per-step latency with HIP events on the launch stream, eager: "steady"
    back to back, and (flush) "cold" with an untimed 1 GiB write before every
    step, which leaves none of the step's weights in the 256 MB MALL."""
    import numpy as np
    scratch = torch.empty(flush_bytes if flush else 1, dtype=torch.uint8, device="cuda")
    out = {}
    for name, flush_it in (("steady", False), ("cold", True))[:2 if flush else 1]:
        evs = []
        for s in steps:
            if flush_it:
                scratch.fill_(s & 0xff)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(s)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
        out[name] = {"p10": round(float(np.percentile(us, 10)), 3), "median": round(float(np.median(us)), 3),
                     "p90": round(float(np.percentile(us, 90)), 3), "n": len(us)}
    del scratch
    return out


def measured_read_peak(torch, lib, gib=4, reps=5):
    """GB/s of the library's streaming-read reference over a 4 GiB buffer."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.moe_debug_stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        lib.moe_debug_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbps = reps * buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    return round(gbps, 1)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MoE layer here runs on a single MI355X "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if (args.prefetch or args.slot_tier) and args.workload != "slotcache":
        print("--prefetch and --slot-tier apply to --workload slotcache", file=sys.stderr)
        sys.exit(2)
    if args.prefetch < 0:
        print("--prefetch takes a ring size >= 0", file=sys.stderr)
        sys.exit(2)
    if args.workload == "decode-b64":
        return bench_decode_b64(args)
    if args.workload == "slotcache":
        return bench_slotcache(args)
    if args.workload == "slotcache-prefill":
        return bench_slotcache_prefill(args)
    if args.workload == "prefill":
        return bench_prefill(args)
    return bench_decode_b1(args)


def resident_bank(W, lib, torch, cfg, seed, dev, layer=0):
    """A layer's 256 FP4 records (slot = expert id) and its shared record, in
    HBM.  Layer l's expert e is record l * E + e of the seeded bank (layer 0 is
    the workload's own bank), its shared expert record l of the shared stream."""
    E, H, I = cfg["E"], cfg["H"], cfg["I"]
    rec_bytes = lib.moe_fp4_expert_bytes(H, I)
    bank = torch.empty((E, rec_bytes), dtype=torch.uint8, device=dev)
    host = np.empty((16, rec_bytes), np.uint8)
    for e0 in range(0, E, 16):
        W.fp4_bank(seed, W.S_BANK, 16, H, I, out=host, first_index=layer * E + e0)
        bank[e0:e0 + 16].copy_(torch.from_numpy(host))
    shared = torch.from_numpy(W.fp4_record(seed, W.S_SHARED, layer, H, I)).to(dev)
    return bank, shared, rec_bytes


def calibration_copy(torch, dev):
    """One 256 MiB device-to-device copy: the reference launch that scales the
    FETCH_SIZE / WRITE_SIZE counters of the same profiling run to bytes."""
    src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def bench_decode_b1(args):

    import torch

    from mxfp4_routed_expert_renorm_amd import binding as lib
    from mxfp4_routed_expert_renorm_amd import workloads as W

    cfg = W.WORKLOADS[DEFAULT_WORKLOAD]
    seed = cfg["seed"]
    E, H, I, k, T = cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"]
    K, Wm = args.steps, args.warmup
    nsteps = K + Wm
    dev = torch.device("cuda:0")
    rec_bytes = lib.moe_fp4_expert_bytes(H, I)

    t0 = time.time()
    G = args.tp_share
    NL = max(1, args.layers)
    print(f"[bench] generating {NL} layers of {E}+1 experts ({NL * (E + 1) * rec_bytes / 1e9:.2f} GB) and "
          f"{nsteps} steps of inputs", file=sys.stderr, flush=True)
    layers_mem = []
    for l in range(NL):
        bank, shared, rec_bytes = resident_bank(W, lib, torch, cfg, seed, dev, layer=l)
        if G > 1:  # rank 0's slice of every expert: I/G rows of w1, w3 and columns of w2
            rec_bytes = lib.moe_fp4_expert_bytes(H, I // G)
            share = torch.empty((E, rec_bytes), dtype=torch.uint8, device=dev)
            shared_share = torch.empty((1, rec_bytes), dtype=torch.uint8, device=dev)
            lib.moe_tp_slice(bank, H, I, G, 0, share)
            lib.moe_tp_slice(shared[None, :], H, I, G, 0, shared_share)
            torch.cuda.synchronize()
            del bank
            bank, shared = share, shared_share[0]
        layers_mem.append((bank, shared))
    if G > 1:
        I = I // G
    xs = np.stack([W.make_layer_inputs(cfg, seed, s, with_bank=False)["x"][0] for s in range(nsteps)])
    lgs = np.stack([W.make_layer_inputs(cfg, seed, s, with_bank=False)["logits"][0] for s in range(nsteps)])
    x_d = torch.from_numpy(xs).to(dev).view(torch.bfloat16)          # [steps, H]
    lg_d = torch.from_numpy(lgs).to(dev)                             # [steps, E]
    ids_d = torch.empty((nsteps, k), dtype=torch.int32, device=dev)
    w_d = torch.empty((nsteps, k), dtype=torch.float32, device=dev)
    out_d = torch.empty((nsteps, H), dtype=torch.bfloat16, device=dev)
    ws = lib.expert_workspace(H, I, T, k, True, device=dev)
    # full width: the single launch unless asked for two (it needs every
    # workgroup resident at once, which the library checks; a 1/G share runs
    # two launches unless asked, being faster that way)
    single = args.single_launch or (G == 1 and not args.two_launch)
    lflags = lib.MOE_LAYER_SINGLE_LAUNCH if single else 0
    layers = [lib.make_layer(H, I, fp4_base=bk, fp4_stride=rec_bytes, num_slots=E, shared=sh, flags=lflags)
              for bk, sh in layers_mem]
    torch.cuda.synchronize()
    print(f"[bench] inputs resident in HBM after {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    def step(s):
        # route + expert MLP + combine of one token on layer s mod L: one kernel launch (or two)
        lib.moe_layer_decode(layers[s % NL], lg_d[s], x_d[s:s + 1], k, ids_d[s], w_d[s], out_d[s:s + 1], ws)

    def step_one_layer(s):
        lib.moe_layer_decode(layers[0], lg_d[s], x_d[s:s + 1], k, ids_d[s], w_d[s], out_d[s:s + 1], ws)

    if args.calibrate_copy:
        calibration_copy(torch, dev)

    off = lib.moe_expert_workspace_sync_offset(H, I, T, k, True)

    def err_word():
        return int(ws[off + 1024:off + 1028].view(torch.int32).item())

    step(0)
    torch.cuda.synchronize()
    if single and err_word() != 0:
        # the single launch's handoff gave up (its grid was not all resident):
        # the two-launch step instead, on a fresh workspace
        print("[bench] the single launch's handoff gave up on the first step; running two launches",
              file=sys.stderr, flush=True)
        ws = lib.expert_workspace(H, I, T, k, True, device=dev)
        layers = [lib.make_layer(H, I, fp4_base=bk, fp4_stride=rec_bytes, num_slots=E, shared=sh, flags=0)
                  for bk, sh in layers_mem]
        step(0)
        torch.cuda.synchronize()

    elapsed = run_steps(args, torch, step, K, Wm)
    print(f"[bench] timed {K} steps in {elapsed * 1e3:.2f} ms ({args.mode})", file=sys.stderr, flush=True)

    # profiled pass over the same steps: HIP events on the launch stream around
    # each of the library's kernels
    lib.moe_profile_begin(8 * K + 16)
    for s in range(Wm, nsteps):
        step(s)
    prof = lib.moe_profile_end()
    k1 = k + 1
    # algorithmic bytes of one step: the 9 experts' records (codes + scales of
    # w1, w3, w2), the logits row, the activation row, the bf16 SwiGLU outputs
    # written and read back, the ids and weights, the bf16 output row
    step_alg_bytes = k1 * rec_bytes + E * 4 + H * 2 + 2 * k1 * I * 2 + k * 8 + H * 2
    # a single launch that gave up a wait set the workspace's error word: its
    # outputs would be meaningless, so such a run reports nothing
    err = err_word()
    if err != 0:
        raise SystemExit(f"[bench] the single launch's handoff gave up (error word {err}); no result")
    per_kernel = {n: round(v[0] / v[1] * 1e3, 3) for n, v in prof.items()}
    print(f"[bench] kernel averages (us): {per_kernel}", file=sys.stderr, flush=True)
    if "fused" in prof:  # the single launch: the whole step is one kernel
        ms, n = prof["fused"]
        dom_kernel = ("fused_b1_kernel (routing through combine, one launch)" if G == 1 else
                      f"fused_b1s_kernel (routing through combine of a 1/{G} share, I = {I}, one launch)")
        # the step's algorithmic bytes (the SwiGLU outputs cross workgroups
        # through memory: written once and read back)
        dom_bytes = step_alg_bytes
        khash = kernel_hash(FUSED_KERNEL_FILES)
        traffic = traffic_from_profiles(khash, "traffic_fused_decode_b1.json") if G == 1 else None
    else:
        ms, n = prof["gateup"]      # the dominant kernel of the two launches
        dom_kernel = ("gateup_b1_kernel (routing + batch-1 gate/up GEMV + SwiGLU)" if G == 1 else
                      f"gateup_b1s_kernel (routing + batch-1 gate/up GEMV + SwiGLU of a 1/{G} share, I = {I})")
        # the 9 experts' w1 and w3 codes and scales, the logits row, the
        # activation row, the bf16 SwiGLU outputs written
        dom_bytes = k1 * 2 * (H * I // 2 + H * I // 32) + E * 4 + H * 2 + k1 * I * 2
        khash = kernel_hash()
        traffic = traffic_from_profiles(khash) if G == 1 else None
    dom_avg_s = ms / n / 1e3
    achieved = dom_bytes / dom_avg_s / 1e9

    tokens = K * T
    value = tokens / elapsed
    step_bytes = k1 * rec_bytes
    result = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (% of peak), MXFP4 256-expert decode",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4-w/bf16-x/f32-acc",
        "data": "synthetic (seeded; fresh logits and activations every step)",
        "config": {"workload": cfg["name"] + (f"-tp{G}-share0" if G > 1 else "") +
                   (f"-{NL}layers-rotated" if NL > 1 else "") + ("-single-launch" if "fused" in prof else ""),
                   "experts": E,
                   "shared_experts": 1, "hidden": H, "expert_intermediate": I, "top_k": k, "tokens_per_step": T,
                   "layers": NL, "layer_of_step": "s mod layers",
                   "expert_bytes": rec_bytes, "weight_bytes_per_step": step_bytes, "launch": args.mode,
                   "tp_share": G},
        "step_hbm_GBps": round(step_bytes * value / 1e9, 1),
        "step_hbm_frac": round(step_bytes * value / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": dom_kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_avg_s * 1e6, 3),
                     "kernel_hash": khash},
        "kernel_avg_us": per_kernel,
    }
    result["step_latency_us"] = step_latency(torch, step, range(Wm, nsteps), flush=False)
    if NL > 1:  # one resident layer: its shared expert and repeats can sit in the last-level cache
        result["single_layer_step_latency_us"] = step_latency(torch, step_one_layer, range(Wm, nsteps))
    peak_m = measured_read_peak(torch, lib)
    result["hbm_read_peak_measured_GBps"] = peak_m
    result["roofline"]["frac_vs_measured_peak"] = round(achieved / peak_m, 4)
    if not args.no_cpu_baseline and G == 1:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cb = cpu_baseline(args.cpu_seconds)
        n = host_threads()
        allc = cpu_baseline(args.cpu_seconds, n)
        cb["all_cores"] = {"value": allc["value"], "cores": n, "sample": allc["sample"]}
        cb["cpu_model"] = cpu_model()
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


def upload_graph(torch, g):
    """hipGraphUpload of a captured graph's executable on the current stream, so
    its first replay does not also pay for moving the graph to the device."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    st = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError(f"hipGraphUpload failed with status {st}")


def run_steps(args, torch, step, K, Wm):
    """Warm up, then time K steps: graph-replayed (one capture of all K) or eager."""
    nsteps = K + Wm
    if args.mode == "graph":
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for s in range(min(3, nsteps)):
                step(s)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm):
            for s in range(Wm):
                step(s)
        with torch.cuda.graph(g_timed):
            for s in range(Wm, nsteps):
                step(s)
        g_warm.replay()
        upload_graph(torch, g_timed)  # the executable graph goes to the device outside the timed region
        torch.cuda.synchronize()
        ta = time.perf_counter()
        g_timed.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - ta
    for s in range(Wm):
        step(s)
    torch.cuda.synchronize()
    ta = time.perf_counter()
    for s in range(Wm, nsteps):
        step(s)
    torch.cuda.synchronize()
    return time.perf_counter() - ta


def bench_decode_b64(args):
    """64 tokens per step, top-6, Zipf(1.1)-skewed routing, the shared expert;
    the (token, rank) pairs are grouped by expert so each selected expert
    streams once per step."""
    import torch

    from mxfp4_routed_expert_renorm_amd import binding as lib
    from mxfp4_routed_expert_renorm_amd import workloads as W

    cfg = W.WORKLOADS["decode-b64"]
    seed = cfg["seed"]
    E, H, I, k, T = cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"]
    K, Wm = args.steps, args.warmup
    nsteps = K + Wm
    dev = torch.device("cuda:0")
    bank, shared, rec_bytes = resident_bank(W, lib, torch, cfg, seed, dev)
    ins = [W.make_layer_inputs(cfg, seed, s, with_bank=False) for s in range(nsteps)]
    x_d = torch.from_numpy(np.stack([d["x"] for d in ins])).to(dev).view(torch.bfloat16)     # [steps, T, H]
    lg_d = torch.from_numpy(np.stack([d["logits"] for d in ins])).to(dev)                    # [steps, T, E]
    ids_d = torch.empty((nsteps, T, k), dtype=torch.int32, device=dev)
    w_d = torch.empty((nsteps, T, k), dtype=torch.float32, device=dev)
    out_d = torch.empty((nsteps, T, H), dtype=torch.bfloat16, device=dev)
    ws = lib.expert_workspace(H, I, T, k, True, device=dev)
    layer = lib.make_layer(H, I, fp4_base=bank, fp4_stride=rec_bytes, num_slots=E, shared=shared)
    torch.cuda.synchronize()

    def step(s):
        lib.moe_route(lg_d[s], k, ids_d[s], w_d[s])
        lib.moe_expert_forward(layer, x_d[s], T, k, ids_d[s], None, w_d[s], out_d[s], ws)

    if args.calibrate_copy:
        calibration_copy(torch, dev)

    step(0)
    torch.cuda.synchronize()
    elapsed = run_steps(args, torch, step, K, Wm)
    lib.moe_profile_begin(16 * K + 16)
    for s in range(Wm, nsteps):
        step(s)
    prof = lib.moe_profile_end()
    ids_h = ids_d[Wm:].cpu().numpy()
    distinct = np.array([len(np.unique(ids_h[s])) for s in range(K)])
    step_bytes = (distinct + 1) * rec_bytes                       # selected experts + shared, once each
    value = K * T / elapsed
    gbps = step_bytes.sum() / elapsed / 1e9
    result = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (% of peak), MXFP4 256-expert decode (batch 64)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4-w/bf16-x/f32-acc",
        "data": "synthetic (seeded; fresh Zipf-skewed logits and activations every step)",
        "config": {"workload": cfg["name"], "experts": E, "shared_experts": 1, "hidden": H,
                   "expert_intermediate": I, "top_k": k, "tokens_per_step": T, "launch": args.mode,
                   "distinct_experts_per_step_mean": round(float(distinct.mean()), 2)},
        "step_hbm_GBps": round(gbps, 1), "step_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "roofline": b64_roofline(prof, distinct, T, k, H, I),
        "kernel_avg_us": {n: round(v[0] / v[1] * 1e3, 3) for n, v in prof.items()},
    }
    print(json.dumps(result), flush=True)


def b64_roofline(prof, distinct, T, k, H, I):
    """Gate/up kernel of the batched decode: every selected record's w1 and w3
    (codes and scales) once, the tokens' activations once, h written once."""
    gu_unit = 2 * (H * I // 2 + H * I // 32)
    P = T * (k + 1)
    alg = float((distinct + 1).mean()) * gu_unit + T * H * 2 + P * I * 2
    us = prof["gateup"][0] / prof["gateup"][1] * 1e3
    achieved = alg / (us * 1e-6) / 1e9
    khash = kernel_hash(B64_KERNEL_FILES)
    return {"bound": "hbm", "kernel": "dgemm_kernel<2> (batched gate/up on bf16 MFMA + SwiGLU)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profiles(khash, "traffic_gateup_decode_b64.json"),
            "algorithmic_bytes_per_launch": int(alg), "avg_launch_us": round(us, 3), "kernel_hash": khash}


def bench_prefill(args):
    """4096 tokens through the resident 256-expert layer (+ shared), top-8:
    route, then MXFP8 activations x MXFP4 weights on the scaled MFMA, grouped
    by expert, SwiGLU and requantisation fused, combine to bf16."""
    import torch

    from mxfp4_routed_expert_renorm_amd import binding as lib
    from mxfp4_routed_expert_renorm_amd import workloads as W

    cfg = W.WORKLOADS["prefill"]
    seed = cfg["seed"]
    E, H, I, k, T = cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"]
    K, Wm = args.steps, args.warmup
    nsteps = K + Wm
    dev = torch.device("cuda:0")
    bank, shared, rec_bytes = resident_bank(W, lib, torch, cfg, seed, dev)
    ins = [W.make_layer_inputs(cfg, seed, s, with_bank=False) for s in range(nsteps)]
    x_d = torch.from_numpy(np.stack([d["x"] for d in ins])).to(dev).view(torch.bfloat16)     # [steps, T, H]
    lg_d = torch.from_numpy(np.stack([d["logits"] for d in ins])).to(dev)                    # [steps, T, E]
    ids_d = torch.empty((T, k), dtype=torch.int32, device=dev)
    w_d = torch.empty((T, k), dtype=torch.float32, device=dev)
    out_d = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.moe_prefill_workspace_bytes(H, I, T, k, True), dtype=torch.uint8, device=dev)
    layer = lib.make_layer(H, I, fp4_base=bank, fp4_stride=rec_bytes, num_slots=E, shared=shared)
    torch.cuda.synchronize()

    def step(s):
        lib.moe_route(lg_d[s], k, ids_d, w_d)
        lib.moe_prefill_forward(layer, x_d[s], k, ids_d, w_d, out_d, ws)

    step(0)
    torch.cuda.synchronize()
    elapsed = run_steps(args, torch, step, K, Wm)
    lib.moe_profile_begin(16 * K + 16)
    for s in range(Wm, nsteps):
        step(s)
    prof = lib.moe_profile_end()
    kus = {n: round(v[0] / v[1] * 1e3, 3) for n, v in prof.items()}
    pairs = T * (k + 1)
    flops = pairs * 2 * 3 * H * I                       # gate, up, down per (token, expert)
    gemm_s = (prof["gemm_gateup"][0] / prof["gemm_gateup"][1] + prof["gemm_down"][0] / prof["gemm_down"][1]) / 1e3
    wbytes = (E + 1) * rec_bytes
    result = {
        "metric": "MoE-layer prefill tokens/s + MFMA fraction, MXFP4 256-expert layer (4096 tokens)",
        "value": round(K * T / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp8-x/mxfp4-w/f32-acc",
        "data": "synthetic (seeded; fresh logits and activations every step)",
        "config": {"workload": cfg["name"], "experts": E, "shared_experts": 1, "hidden": H,
                   "expert_intermediate": I, "top_k": k, "tokens_per_step": T, "launch": args.mode},
        "roofline": {"bound": "mfma", "kernel": "gemm_gateup_kernel + gemm_down_kernel",
                     "achieved": round(flops / gemm_s / 1e12, 1), "peak": 5000.0, "unit": "TFLOP/s",
                     "frac": round(flops / gemm_s / 1e12 / 5000.0, 4),
                     "frac_vs_fp4_peak": round(flops / gemm_s / 1e12 / 10100.0, 4),
                     "flops_per_step": flops, "traffic": None},
        "weight_bytes_per_step": wbytes,
        "gemm_weight_GBps": round(wbytes / gemm_s / 1e9, 1),
        "gemm_weight_hbm_frac": round(wbytes / gemm_s / 1e9 / HBM_PEAK_GBPS, 4),
        "kernel_avg_us": kus,
        "kernel_us_per_step": {n: round(v[0] / K * 1e3, 3) for n, v in prof.items()},
    }
    print(json.dumps(result), flush=True)


def bench_slotcache(args):
    """512 batch-1 tokens through 8 layers of 256 experts with a 512-slot HBM
    cache, the (2,4) ladder and pinned host banks; per (token, layer): route,
    moe_cache_ensure (one host sync, miss copies on a side stream), expert
    MLP over the slot arena.  Cold start, as the workload defines it."""
    import torch

    from mxfp4_routed_expert_renorm_amd import binding as lib
    from mxfp4_routed_expert_renorm_amd import workloads as W

    cfg = W.WORKLOADS["slotcache"]
    seed = cfg["seed"]
    L, E, H, I, k, T, S = cfg["L"], cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"], cfg["slots"]
    a, b = cfg["ladder"]
    dev = torch.device("cuda:0")
    rb4, rb2 = lib.moe_fp4_expert_bytes(H, I), lib.moe_int2_expert_bytes(H, I)
    t0 = time.time()
    print(f"[bench] pinning {L * E * (rb4 + rb2) / 1e9:.1f} GB of host banks", file=sys.stderr, flush=True)
    fp4_host = lib.PinnedBuffer(L * E * rb4)
    int2_host = lib.PinnedBuffer(L * E * rb2)
    for p in range(L * E):
        W.fp4_record(seed, W.S_BANK, p, H, I, out=fp4_host.array[p * rb4:(p + 1) * rb4])
        if p % 256 == 255:
            print(f"[bench] {p + 1}/{L * E} host records", file=sys.stderr, flush=True)
    # the 2-bit fallback copies are made from the FP4 records (clip search on
    # the GPU, moe_int2_from_fp4), 64 records at a time
    nb = 64
    src_d = torch.empty((nb, rb4), dtype=torch.uint8, device=dev)
    dst_d = torch.empty((nb, rb2), dtype=torch.uint8, device=dev)
    for p0 in range(0, L * E, nb):
        n = min(nb, L * E - p0)
        src_d[:n].copy_(torch.from_numpy(fp4_host.array[p0 * rb4:(p0 + n) * rb4]).view(n, rb4))
        lib.moe_int2_from_fp4(src_d[:n], H, I, dst_d[:n])
        torch.from_numpy(int2_host.array[p0 * rb2:(p0 + n) * rb2]).view(n, rb2).copy_(dst_d[:n])
    del src_d, dst_d
    print(f"[bench] 2-bit copies of the {L * E} records made", file=sys.stderr, flush=True)
    R = args.prefetch
    arena = torch.empty((S + R) * rb4, dtype=torch.uint8, device=dev)
    tier = {}
    if args.slot_tier:
        # LFU counts seeded from the picks of a separate 64-token trace, routed by the library
        warm = torch.from_numpy(W.slotcache_logits(seed + 1, L, E, 64, cfg["zipf"]).reshape(64 * L, E)).to(dev)
        wids_d = torch.empty((64 * L, k), dtype=torch.int32, device=dev)
        ww_d = torch.empty((64 * L, k), dtype=torch.float32, device=dev)
        lib.moe_route(warm, k, wids_d, ww_d)
        wids = wids_d.cpu().numpy().reshape(64, L, k)
        counts = np.zeros(L * E, np.float32)
        for l in range(L):
            np.add.at(counts, l * E + wids[:, l].reshape(-1), 1.0)
        tier = {"int2_slots": 100, "policy": "lfu", "lfu_decay": 0.95, "lfu_seed": counts}
    staging = torch.empty(tier.get("int2_slots", b - a) * rb2, dtype=torch.uint8, device=dev)
    logits = W.slotcache_logits(seed, L, E, T, cfg["zipf"]).reshape(T * L, E)
    lg_d = torch.from_numpy(logits).to(dev)
    xs = np.stack([W.slotcache_x(seed, t, l, H)[0] for t in range(T) for l in range(L)])
    x_d = torch.from_numpy(xs).to(dev).view(torch.bfloat16)                               # [T*L, H]
    ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    w = torch.empty((1, k), dtype=torch.float32, device=dev)
    prec = torch.empty((1, k), dtype=torch.int8, device=dev)
    out_d = torch.empty((T * L, H), dtype=torch.bfloat16, device=dev)
    ws = lib.expert_workspace(H, I, 1, k, False, device=dev)
    copy_stream = torch.cuda.Stream()
    pf_stream = torch.cuda.Stream()
    pred = {}
    if R:
        # The pages' predictor is a trained network (out of scope): stand-in predictions hold a
        # seeded share of the true top-k of the call two layers ahead plus the experts ranked
        # next, 12 in all, from the library's top-(k+12) routing before the timed loop.
        tids_d = torch.empty((T * L, k + 12), dtype=torch.int32, device=dev)
        tw_d = torch.empty((T * L, k + 12), dtype=torch.float32, device=dev)
        lib.moe_route(lg_d, k + 12, tids_d, tw_d)
        tids = tids_d.cpu().numpy().reshape(T, L, k + 12)
        for t in range(T):
            for l in range(L):
                t2, l2 = t + (l + 2) // L, (l + 2) % L
                if t2 < T:
                    pred[(t, l)] = (l2, W.predicted_experts(seed, (t2, l2), tids[t2, l2], k, m=12,
                                                            recall=args.prefetch_recall))
    # host-link peak for this copy pattern: 64 records back to back from the pinned bank
    src = torch.from_numpy(fp4_host.array[:64 * rb4])
    dst = arena[:64 * rb4]
    torch.cuda.synchronize()
    tc = time.perf_counter()
    with torch.cuda.stream(copy_stream):
        for r in range(64):
            dst[r * rb4:(r + 1) * rb4].copy_(src[r * rb4:(r + 1) * rb4], non_blocking=True)
    torch.cuda.synchronize()
    h2d_peak = 64 * rb4 / (time.perf_counter() - tc) / 1e9
    print(f"[bench] setup {time.time() - t0:.1f} s; pinned copy rate {h2d_peak:.1f} GB/s",
          file=sys.stderr, flush=True)

    # token-to-token repeat rate of the trace's routing (the share of a token's
    # top-k, per layer, that the previous token also picked), from the
    # library's routing of every row before the timed loop
    rids_d = torch.empty((T * L, k), dtype=torch.int32, device=dev)
    rw_d = torch.empty((T * L, k), dtype=torch.float32, device=dev)
    lib.moe_route(lg_d, k, rids_d, rw_d)
    rids = rids_d.cpu().numpy().reshape(T, L, k)
    repeat = float(np.mean([len(set(rids[t, l]) & set(rids[t - 1, l])) / k
                            for t in range(1, T) for l in range(L)]))
    cache = lib.Cache(L, E, H, I, S, k, a, b, 1, fp4_host, int2_host, arena, staging, prefetch_slots=R, **tier)
    layer = cache.layer()
    t_tok = []
    torch.cuda.synchronize()
    ta = time.perf_counter()
    for t in range(T):
        for l in range(L):
            row = t * L + l
            if (t, l) in pred:
                cache.prefetch(*pred[(t, l)], copy=pf_stream)
            lib.moe_route(lg_d[row:row + 1], k, ids, w)
            cache.ensure(l, 1, ids, w, prec, copy=copy_stream)
            lib.moe_expert_forward(layer, x_d[row:row + 1], 1, k, ids, prec, w, out_d[row:row + 1], ws)
        t_tok.append(time.perf_counter())
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - ta
    st = cache.stats()
    cache.destroy()
    steady = (t_tok[-1] - t_tok[T // 2 - 1]) / (T - T // 2)
    uses = st["hits"] + st["misses"] + st["int2_uses"] + st["drops"]
    result = {
        "metric": "MoE tokens/s through 8 slot-cached layers (host-link bound), MXFP4 + 2-bit ladder",
        "value": round(T / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": T, "warmup": 0,
        "ms_per_step": round(elapsed / T * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4+int2-w/bf16-x/f32-acc",
        "data": "synthetic (seeded; per-layer Zipf(1.1) logits, fresh activations per token and layer; "
                "2-bit copies made from the FP4 records by clip search)",
        "config": {"workload": cfg["name"] + ("-int2tier100-lfu" if tier else "") + (f"-ring{R}" if R else ""),
                   "layers": L, "experts": E,
                   "slots": S, "top_k": k, "ladder": [a, b], "tokens": T, "cold_start": True,
                   "int2_slots": tier.get("int2_slots", 0), "policy": tier.get("policy", "lru"),
                   "lfu_decay": tier.get("lfu_decay"),
                   "lfu_seed": "64-token routing trace of a separate seed" if tier else None,
                   "prefetch_slots": R,
                   "prediction": (f"12 experts: {int(round(args.prefetch_recall * k))} of the true top-{k} and "
                                  "the experts ranked next, two layers ahead, precomputed from the routing "
                                  "(stand-in for a trained predictor)") if R else None},
        "steady_state_ms_per_token": round(steady * 1e3, 4),
        "cache": {**st, "hit_rate": round(st["hits"] / uses, 4)},
        "routing_repeat_rate": round(repeat, 4),
        "h2d_GBps": round(st["bytes_h2d"] / elapsed / 1e9, 2),
        "h2d_bytes_per_token": int(st["bytes_h2d"] / T),
        "pinned_copy_GBps_measured": round(h2d_peak, 1),
        "host_syncs_per_token": L,
    }
    fp4_host.free()
    int2_host.free()
    print(json.dumps(result), flush=True)


def bench_slotcache_prefill(args):
    """Prompt chunks of 4096 tokens through the 8 slot-cached layers above the
    prefill crossover (T * k >= E): per layer, route on the GPU, stream the
    next layer's 256 experts from the pinned bank into the other layer buffer
    of the cache (side stream, overlapping this layer's compute), then the
    prefill GEMM on this layer's buffer.  Bound by the host link: 3.42 GB per
    layer against a few ms of compute."""
    import torch

    from mxfp4_routed_expert_renorm_amd import binding as lib
    from mxfp4_routed_expert_renorm_amd import workloads as W

    cfg = W.WORKLOADS["slotcache"]
    seed = cfg["seed"]
    L, E, H, I, k, S = cfg["L"], cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["slots"]
    T = 4096
    chunks = max(1, min(args.steps, 4))
    assert lib.moe_prefill_streams(T, k, E)
    dev = torch.device("cuda:0")
    rb4 = lib.moe_fp4_expert_bytes(H, I)
    t0 = time.time()
    print(f"[bench] pinning {L * E * rb4 / 1e9:.1f} GB of host bank", file=sys.stderr, flush=True)
    fp4_host = lib.PinnedBuffer(L * E * rb4)
    for p in range(L * E):
        W.fp4_record(seed, W.S_BANK, p, H, I, out=fp4_host.array[p * rb4:(p + 1) * rb4])
        if p % 256 == 255:
            print(f"[bench] {p + 1}/{L * E} host records", file=sys.stderr, flush=True)
    arena = torch.empty(S * rb4, dtype=torch.uint8, device=dev)
    # per (chunk, layer): Zipf-skewed logits and bf16 activations, resident before timing
    lg = W.slotcache_logits(seed + 7, L, E, (chunks + 1) * T, cfg["zipf"]).reshape(chunks + 1, T, L, E)
    lg_d = torch.from_numpy(lg).to(dev)
    x_d = torch.from_numpy(np.stack([W.bf16_normal(seed, (W.S_X, c, l), (T, H))
                                     for c in range(chunks + 1) for l in range(L)])).to(dev).view(torch.bfloat16)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.moe_prefill_workspace_bytes(H, I, T, k, False), dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()
    cache = lib.Cache(L, E, H, I, S, k, k, k, 1, fp4_host, None, arena, None)
    print(f"[bench] setup {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    lg_rows = lg_d.permute(0, 2, 1, 3).contiguous()                                   # [chunks+1, L, T, E]

    def run(c_first, n):
        calls = [(c, l) for c in range(c_first, c_first + n) for l in range(L)]
        cache.stream_layer(calls[0][1], copy=copy_stream)
        for i, (c, l) in enumerate(calls):
            lib.moe_route(lg_rows[c, l], k, ids, w)
            if i + 1 < len(calls):
                cache.stream_layer(calls[i + 1][1], copy=copy_stream)
            lay = cache.layer_buffer(l)
            lib.moe_prefill_forward(lay, x_d[c * L + l], k, ids, w, out, ws)

    run(0, 1)                                  # warm-up chunk
    torch.cuda.synchronize()
    b0 = cache.stats()["bytes_h2d"]
    ta = time.perf_counter()
    run(1, chunks)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - ta
    st = cache.stats()
    moved = st["bytes_h2d"] - b0
    # the same chunk's compute alone, with every layer's buffer already streamed: the GEMM share
    lib.moe_profile_begin(64 * L)
    for l in range(2):
        cache.stream_layer(l, copy=copy_stream)
    torch.cuda.synchronize()
    for l in range(2):
        lib.moe_route(lg_rows[1, l], k, ids, w)
        lib.moe_prefill_forward(cache.layer_buffer(l), x_d[L + l], k, ids, w, out, ws)
    torch.cuda.synchronize()
    prof = lib.moe_profile_end()
    compute_ms = sum(v[0] for v in prof.values()) / 2
    # host-link peak for this copy size: one layer's records in one copy
    src = torch.from_numpy(fp4_host.array[:E * rb4])
    tc = time.perf_counter()
    with torch.cuda.stream(copy_stream):
        arena[:E * rb4].copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h2d_peak = E * rb4 / (time.perf_counter() - tc) / 1e9
    cache.destroy()
    fp4_host.free()
    rate = moved / elapsed / 1e9
    result = {
        "metric": "prefill tokens/s through 8 slot-cached layers by whole-layer streaming (host-link bound)",
        "value": round(chunks * T / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": chunks, "warmup": 1,
        "ms_per_step": round(elapsed / chunks * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp8-x/mxfp4-w/f32-acc",
        "data": "synthetic (seeded; per-layer Zipf(1.1) logits, fresh activations per chunk and layer)",
        "config": {"workload": cfg["name"].replace("decode", "prefill-stream"), "layers": L, "experts": E,
                   "slots": S, "top_k": k, "chunk_tokens": T, "layer_buffers": 2,
                   "crossover": f"T*k >= E ({T}*{k} >= {E})"},
        "h2d_bytes_per_chunk": int(moved / chunks),
        "h2d_GBps": round(rate, 2),
        "pinned_copy_GBps_measured": round(h2d_peak, 1),
        "link_frac": round(rate / h2d_peak, 4),
        "compute_ms_per_layer": round(compute_ms, 3),
        "copy_ms_per_layer": round(E * rb4 / rate / 1e6, 3),
        "cache": st,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
