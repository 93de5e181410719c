#!/usr/bin/env python3
"""Benchmark: batch-1 decode of one 256-expert MXFP4 MoE layer on one MI355X.

Workload (the layer the pages' model uses at decode: 256 routed experts plus
one shared expert, hidden 4096, expert intermediate 2048, top-8, 13,369,344
bytes per FP4 expert): one step = route one token's fp32 logits (top-8,
renormalised) + the SwiGLU MLP of the 8 selected experts and the shared
expert on MXFP4 weights + the weighted combine to a bf16 output.  Each step
uses fresh seeded logits and activations; every expert is resident in HBM.

Prints one JSON line: tokens/s of the whole step, the achieved HBM bandwidth
of the dominant kernel (gate/up GEMV) against the 8 TB/s peak, and the CPU
oracle timed on the host on a bounded sample.
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

HBM_PEAK_GBPS = 8000.0
CFG_INDEX = 1


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="graph: the timed steps are captured into one HIP graph and replayed; "
                         "eager: one launch sequence per step from the host")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (known bytes for HBM counter scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="lower bound on the oracle's timed CPU work (whole tokens)")
    return ap.parse_args()


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode_b1.hip", "common.h"):
        with open(os.path.join(ROOT, "mxfp4_routed_expert_renorm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(khash: str):
    """HBM bytes per launch of the gate/up kernel from committed counter runs,
    or None when absent or taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic_gateup_decode_b1.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_hash") != khash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(min_seconds: float):
    """The oracle as it stands, on whole tokens of the same workload, until at
    least min_seconds of CPU work; BLAS pinned to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from mxfp4_routed_expert_renorm_amd import workloads as W
    from oracle import moe_oracle as O

    cfg = W.CONFIGS[CFG_INDEX]
    seed = W.config_seed(CFG_INDEX)
    H, I, k = cfg["H"], cfg["I"], cfg["k"]
    toks, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < min_seconds or toks == 0:
            d = W.make_layer_inputs(cfg, seed, step=toks, with_bank=False)
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
    return {"value": toks / t_used, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{toks} token(s) of the batch-1 decode workload (route + 9 experts dequantised "
                      f"and evaluated in float64 + combine), BLAS limited to one thread; "
                      f"input generation excluded; {t_used:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MoE layer here runs on a single MI355X "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mxfp4_routed_expert_renorm_amd import binding as lib
    from mxfp4_routed_expert_renorm_amd import workloads as W

    cfg = W.CONFIGS[CFG_INDEX]
    seed = W.config_seed(CFG_INDEX)
    E, H, I, k, T = cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"]
    K, Wm = args.steps, args.warmup
    nsteps = K + Wm
    dev = torch.device("cuda:0")
    rec_bytes = lib.moe_fp4_expert_bytes(H, I)

    t0 = time.time()
    print(f"[bench] generating {E}+1 experts ({(E + 1) * rec_bytes / 1e9:.2f} GB) and {nsteps} steps of inputs",
          file=sys.stderr, flush=True)
    bank = torch.empty((E, rec_bytes), dtype=torch.uint8, device=dev)
    host = np.empty((16, rec_bytes), np.uint8)
    for e0 in range(0, E, 16):
        W.fp4_bank(seed, W.S_BANK, 16, H, I, out=host, first_index=e0)
        bank[e0:e0 + 16].copy_(torch.from_numpy(host))
    shared = torch.from_numpy(W.fp4_record(seed, W.S_SHARED, 0, H, I)).to(dev)
    xs = np.stack([W.make_layer_inputs(cfg, seed, s, with_bank=False)["x"][0] for s in range(nsteps)])
    lgs = np.stack([W.make_layer_inputs(cfg, seed, s, with_bank=False)["logits"][0] for s in range(nsteps)])
    x_d = torch.from_numpy(xs).to(dev).view(torch.bfloat16)          # [steps, H]
    lg_d = torch.from_numpy(lgs).to(dev)                             # [steps, E]
    ids_d = torch.empty((nsteps, k), dtype=torch.int32, device=dev)
    w_d = torch.empty((nsteps, k), dtype=torch.float32, device=dev)
    out_d = torch.empty((nsteps, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.moe_expert_workspace_bytes(H, I, T, k, True), dtype=torch.uint8, device=dev)
    layer = lib.make_layer(H, I, fp4_base=bank, fp4_stride=rec_bytes, num_slots=E, shared=shared)
    torch.cuda.synchronize()
    print(f"[bench] inputs resident in HBM after {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    def step(s):
        lib.moe_route(lg_d[s:s + 1], k, ids_d[s], w_d[s])
        lib.moe_expert_forward(layer, x_d[s:s + 1], T, k, ids_d[s], None, w_d[s], out_d[s:s + 1], ws)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    step(0)
    torch.cuda.synchronize()

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
        torch.cuda.synchronize()
        ta = time.perf_counter()
        g_timed.replay()
        torch.cuda.synchronize()
        tb = time.perf_counter()
    else:
        for s in range(Wm):
            step(s)
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for s in range(Wm, nsteps):
            step(s)
        torch.cuda.synchronize()
        tb = time.perf_counter()
    elapsed = tb - ta
    print(f"[bench] timed {K} steps in {elapsed * 1e3:.2f} ms ({args.mode})", file=sys.stderr, flush=True)

    # profiled pass over the same steps: HIP events on the launch stream around
    # each of the library's kernels
    lib.moe_profile_begin(8 * K + 16)
    for s in range(Wm, nsteps):
        step(s)
    prof = lib.moe_profile_end()
    gu_ms, gu_n = prof["gateup"]
    gu_avg_s = gu_ms / gu_n / 1e3
    k1 = k + 1
    # algorithmic bytes of one gate/up launch: w1 and w3 (codes + scales) of the
    # 9 experts, the activation row, and the fp32 SwiGLU outputs
    gu_bytes = k1 * 2 * (H * I // 2 + H * I // 32) + H * 2 + k1 * I * 4
    achieved = gu_bytes / gu_avg_s / 1e9
    khash = kernel_hash()
    traffic = traffic_from_profiles(khash)
    per_kernel = {n: round(v[0] / v[1] * 1e3, 3) for n, v in prof.items()}
    print(f"[bench] kernel averages (us): {per_kernel}", file=sys.stderr, flush=True)

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
        "config": {"workload": cfg["name"], "experts": E, "shared_experts": 1, "hidden": H,
                   "expert_intermediate": I, "top_k": k, "tokens_per_step": T,
                   "expert_bytes": rec_bytes, "weight_bytes_per_step": step_bytes, "launch": args.mode},
        "step_hbm_GBps": round(step_bytes * value / 1e9, 1),
        "step_hbm_frac": round(step_bytes * value / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "gateup_b1_kernel (batch-1 gate/up GEMV + SwiGLU)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_avg_s * 1e6, 3),
                     "kernel_hash": khash},
        "kernel_avg_us": per_kernel,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
