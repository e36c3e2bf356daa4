#!/usr/bin/env python3
"""Benchmark of the sparse MoE FFN layer (Step-3.5-Flash shape) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

One step = one moe_layer_forward over one batch of synthetic tokens (router,
dispatch, gate/up GEMM, down GEMM, combine), with every input already resident
in HBM.  W untimed steps, then K timed steps between two device
synchronisations, each with HIP events the library records on its stream around
the gate/up stage (the roofline kernel); a per-stage breakdown comes from a
separate, untimed pass with every stage boundary recorded.  Prints one JSON
line.

Workloads (seeded synthetic inputs, shapes from the llm-atlas "Step-3.5-Flash"
config fields): decode (32 tokens, default), verify (256 tokens, Zipf expert
popularity), prefill (16384 tokens), int4_decode (32 tokens, INT4-g32 weights),
mtp_decode (32 tokens through a last layer: SwiGLU limits 7 routed / 16 shared,
activations drawn 8x wider so that the limits act), page_router_decode (32
tokens under the page's router configuration: sigmoid scores, a seeded
per-expert router bias, weights x3), step3_decode / step3_prefill (Step-3's
MoE shape: hidden 7168, 48 experts, top-3, width 5120, no renormalisation; 32
and 4096 tokens), dense_decode / dense_prefill (the dense SwiGLU FFN of width
11264 as one expert; 32 and 16384 tokens), tiny (parity-sized).
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

METRIC = "MoE-layer tokens/s + % of HBM BW (decode) / % of bf16 MFMA peak (prefill)"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E (published)
PEAK_BF16 = 2.5e15         # flop/s, MI355X dense bf16 MFMA (published)
HOT_ROWS = 32              # the library's threshold for a hot expert's LDS tiles
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_layer_amd", "csrc")
# sources of the gate/up stage's kernels per workload: LDS-tiled GEMMs from 16
# rows per expert, weight-streaming GEMMs below
_STREAM = os.path.join(CSRC, "moe_gemm_stream.hip")
_TILED = os.path.join(CSRC, "moe_gemm_tiled.hip")
GEMM_SRC = {"prefill": [_TILED], "step3_prefill": [_TILED], "dense_prefill": [_TILED],
            "dense_decode": [_TILED]}   # one expert with 32 rows: LDS-tiled as well
# workloads whose roofline is the MFMA peak (the LDS-tiled regime); the rest are HBM-bound
MFMA_BOUND = ("prefill", "step3_prefill", "dense_prefill")
WORKLOAD_NAMES = ["tiny", "decode", "verify", "prefill", "int4_decode", "mtp_decode",
                  "page_router_decode", "step3_decode", "step3_prefill", "dense_decode",
                  "dense_prefill"]
GEMM_SRC_DEFAULT = [_STREAM]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=WORKLOAD_NAMES)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the oracle on the host (e.g. under a profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the default decode workload: skip the prefill leg (16384 tokens) "
                         "that the line otherwise carries as its 'prefill' object")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (the "
                         "reference kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


def src_digest(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_counters(workload: str):
    """HBM traffic of the gate/up stage from committed rocprofv3 --pmc runs.

    profiles/gate_up_<workload>_counters.txt holds 'key: value' lines, among
    them src_sha (digests of the kernel sources the counters were taken on,
    comma-separated in GEMM_SRC order) and fetch_bytes / write_bytes per call
    already scaled by the copy-kernel calibration.  Returns None when absent
    or taken on other kernel code."""
    path = os.path.join(PROFILES, f"gate_up_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("src_sha") != ",".join(src_digest(p) for p in GEMM_SRC.get(workload, GEMM_SRC_DEFAULT)):
        return None
    try:
        return float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    except (KeyError, ValueError):
        return None


def device_info():
    """Name, CU count and peak shader clock of cuda:0 as the HIP runtime reports
    them, and the dense bf16 MFMA rate they imply (4096 flop per clock per CU)."""
    import ctypes as C
    import torch
    props = torch.cuda.get_device_properties(0)
    hip = C.CDLL("libamdhip64.so.7")
    hip.hipDeviceGetAttribute.argtypes = [C.POINTER(C.c_int), C.c_int, C.c_int]
    # hipDeviceAttribute_t values (hip_runtime_api.h): ClockRate (kHz) 5, MultiprocessorCount 63
    vals = {}
    for name, attr in (("clock_khz", 5), ("cus", 63)):
        v = C.c_int(0)
        vals[name] = v.value if hip.hipDeviceGetAttribute(C.byref(v), attr, 0) == 0 else None
    info = {"name": props.name, "arch": props.gcnArchName.split(":")[0], "cus": vals["cus"],
            "sclk_peak_mhz": None if vals["clock_khz"] is None else vals["clock_khz"] / 1000}
    if vals["cus"] and vals["clock_khz"]:
        info["bf16_dense_tflops_at_peak_sclk"] = round(vals["cus"] * 4096 * vals["clock_khz"] * 1e3 / 1e12, 1)
    return info


def cpu_baseline(inp, shape, target_s: float):
    """The oracle as it stands, on the host cores, on the first S tokens of the
    same batch (S doubled until the run takes about target_s seconds)."""
    import numpy as np
    import torch
    import threadpoolctl
    import moe_synth
    import oracle

    E = shape.experts
    x64 = moe_synth.host_f64(inp.x)
    wr = moe_synth.host_f64(inp.router_w)
    bias = None if inp.router_bias is None else inp.router_bias.cpu().numpy()
    int4 = shape.weight_dtype == "int4_g32"
    host = {}

    def fetch(e):        # device -> host copy, outside the timed region
        if e in host:
            return
        if int4:
            host[e] = tuple((inp.q[n][0][e].cpu().numpy(), inp.q[n][1][e].cpu().numpy())
                            for n in ("gate", "up", "down"))
        else:
            host[e] = (inp.w_gate[e].cpu(), inp.w_up[e].cpu(), inp.w_down[e].cpu())

    def experts(e):      # widening to float64 is part of the oracle's work
        if int4:
            return tuple(oracle.dequant_int4(q, s) for q, s in host[e])
        return tuple(t.to(torch.float64).numpy() for t in host[e])

    if int4:
        shared = tuple(oracle.dequant_int4(inp.q[n][0].cpu().numpy(), inp.q[n][1].cpu().numpy())
                       for n in ("s_gate", "s_up", "s_down"))
    else:
        shared = tuple(moe_synth.host_f64(t) for t in (inp.s_gate, inp.s_up, inp.s_down))
    info = threadpoolctl.threadpool_info()
    cores = max([d.get("num_threads", 1) for d in info] or [1])
    T = x64.shape[0]
    s, elapsed, spent = 1, 0.0, 0.0
    while True:
        idx, *_ = oracle.route(x64[:s], wr, bias, shape.top_k, shape.score, shape.renormalize,
                               shape.routed_scale, shape.bias_mode)
        for e in np.unique(idx):
            fetch(int(e))
        t0 = time.perf_counter()
        oracle.forward(x64[:s], wr, bias, experts, shared, shape.top_k, shape.score,
                       shape.renormalize, shape.routed_scale, shape.bias_mode,
                       swiglu_limit=shape.swiglu_limit, swiglu_limit_shared=shape.swiglu_limit_shared)
        elapsed = time.perf_counter() - t0
        spent += elapsed
        log(f"[bench]   oracle on {s} tokens: {elapsed:.1f} s")
        # stop at about target_s per run, and after about 3 x target_s in all
        if elapsed >= target_s or s >= T or spent + 2.2 * elapsed > 3 * target_s:
            break
        s = min(T, s * 2 if elapsed < target_s / 4 else max(s + 1, int(s * target_s / elapsed)))
        host.clear()
    return {"value": s / elapsed, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {s} of the {T} tokens of the same batch (float64 NumPy oracle, "
                      f"{elapsed:.1f} s; expert weights widened one expert at a time)"}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or 'unknown'."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


WL_DESC = {"tiny": "tiny parity layer", "decode": "Step-3.5-Flash MoE layer, decode batch",
           "verify": "Step-3.5-Flash MoE layer, MTP verify batch (64 streams x 4), Zipf experts",
           "prefill": "Step-3.5-Flash MoE layer, prefill chunk",
           "int4_decode": "Step-3.5-Flash MoE layer, decode batch, INT4-g32 weights",
           "mtp_decode": "Step-3.5-Flash last MoE layer (SwiGLU limits 7 / 16), decode batch",
           "page_router_decode": "Step-3.5-Flash MoE layer under the page's router config "
                                 "(sigmoid, router bias, x3), decode batch",
           "step3_decode": "Step-3 MoE layer shape, decode batch",
           "step3_prefill": "Step-3 MoE layer shape, 4096-token chunk",
           "dense_decode": "dense SwiGLU FFN (width 11264) as one expert, decode batch",
           "dense_prefill": "dense SwiGLU FFN (width 11264) as one expert, prefill chunk"}


def measure(workload: str, args, cpu_seconds: float) -> dict:
    """Times one workload (W warm-up steps, then K steps between two device
    synchronisations) and returns its JSON fields."""
    import torch
    import moe_synth
    from sparse_mixture_experts_layer_amd import _binding as B
    from sparse_mixture_experts_layer_amd.layer import MoELayer

    shape = moe_synth.WORKLOADS[workload]
    T, H, E, k, I, Is = (shape.tokens, shape.hidden, shape.experts, shape.top_k, shape.inter,
                         shape.shared_inter)
    log(f"[bench] workload {workload}: T={T} H={H} E={E} k={k} I={I} Is={Is} "
        f"weights={shape.weight_dtype}")
    t0 = time.time()
    inp = moe_synth.make_layer(shape, seed=args.seed, device="cuda")
    layer = MoELayer.from_shape(shape)
    layer.pack_inputs(inp)
    out = torch.empty((T, H), dtype=inp.x.dtype, device="cuda")
    ws = torch.empty(layer.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs + packing ready in {time.time() - t0:.1f}s "
        f"(packed {layer.packed_bytes / 1e9:.2f} GB, workspace {ws.numel() / 1e6:.1f} MB)")

    for _ in range(args.warmup):
        layer.forward(inp.x, inp.router_w, inp.router_bias, out=out, workspace=ws)
    torch.cuda.synchronize()
    # Timed region: K steps, each recording HIP events around its gate/up
    # stage only (the roofline kernel's duration, live); a record costs ~2 us
    # of a decode step, so the other stage boundaries are timed afterwards.
    GU = B.STAGES.index("gate_up")
    ev = B.StageEvents(sets=args.steps, only=(GU, GU + 1))
    t0 = time.perf_counter()
    for i in range(args.steps):
        layer.forward(inp.x, inp.router_w, inp.router_bias, out=out, workspace=ws,
                      stage_events=ev, event_set=i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    gu_ms = sum(ev.elapsed_ms(i, GU, GU + 1) for i in range(args.steps)) / args.steps
    # stage breakdown (reported, not timed): the same forward with every boundary
    nb = min(args.steps, 20)
    ev_all = B.StageEvents(sets=nb)
    for i in range(nb):
        layer.forward(inp.x, inp.router_w, inp.router_bias, out=out, workspace=ws,
                      stage_events=ev_all, event_set=i)
    torch.cuda.synchronize()
    stages = [ev_all.stage_ms(i) for i in range(nb)]
    stage_avg = [sum(s[j] for s in stages) / len(stages) for j in range(len(B.STAGES))]
    log(f"[bench] {workload}: {ms:.4f} ms/step; gate_up ms (timed region): {gu_ms:.4f}; "
        "stage ms (separate pass): "
        + ", ".join(f"{n}={v:.4f}" for n, v in zip(B.STAGES, stage_avg)))

    # routing of the (deterministic) batch: distinct experts touched
    _, route = layer.forward(inp.x, inp.router_w, inp.router_bias, out=out, workspace=ws,
                             return_route=True)
    counts = route.expert_counts.cpu()
    U = int((counts > 0).sum())
    P = T * k
    int4 = shape.weight_dtype == "int4_g32"
    wb = 0.5 + 2.0 / 32 if int4 else 2.0          # bytes per weight (INT4: nibble + fp16/32)
    ab = 4 if shape.act_dtype == "f32" else 2
    expert_b = 3 * I * H * wb
    b_alg = U * expert_b + 3 * Is * H * wb + E * H * 2 + 2 * T * H * ab
    f_alg = T * (2 * H * E + k * 6 * H * I + 6 * H * Is)
    t_layer = ms / 1e3
    Us = U
    if workload in MFMA_BOUND:
        gu_flops = 4.0 * H * (P * I + T * Is)
        achieved = gu_flops / (gu_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_BF16, 4),
                "traffic": read_counters(workload)}
        layer_frac = {"mfma_frac": round(f_alg / t_layer / PEAK_BF16, 4)}
    else:
        # The gate/up stage on the layer's stream is one streaming launch over
        # the experts it holds.  In load-imbalanced 256-1024-token batches
        # (bf16, under 16 rows per expert on average) the library moves routed
        # experts with HOT_ROWS or more rows to LDS-tiled GEMMs on its second
        # stream, outside this stage: their bytes are not this launch's.
        Us, Ps = U, P
        if (not int4 and shape.act_dtype == "bf16" and P / E < 16 and 256 <= T <= 1024):
            cold = (counts > 0) & (counts < HOT_ROWS)
            Us, Ps = int(cold.sum()), int(counts[cold].sum())
        gu_bytes = (Us * 2 * I * H + 2 * Is * H) * wb + T * H * ab + (Ps + T) * I * 2
        achieved = gu_bytes / (gu_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved * 1e9 / PEAK_HBM, 4),
                "traffic": read_counters(workload)}
        layer_frac = {"hbm_frac": round(b_alg / t_layer / PEAK_HBM, 4)}
    roof["kernel"] = "gate_up (grouped gate/up GEMM + SiLU*up)"
    if workload not in MFMA_BOUND and Us != U:
        roof["kernel"] += f" streaming launch: {Us} of {U} routed experts + shared"

    cpu = None
    if cpu_seconds > 0:
        log(f"[bench] timing the oracle on the host ({workload}) ...")
        cpu = cpu_baseline(inp, shape, cpu_seconds)
        log(f"[bench] oracle: {cpu}")

    res = {
        "value": round(T / t_layer, 1),
        "unit": "tokens/s",
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "dtype": "bf16" if not int4 else "bf16 x int4-g32",
        "data": (f"synthetic (seeded N(0,{shape.x_scale:g}^2) activations, N(0,1/fan_in) weights"
                 + {"zipf": ", Zipf-calibrated router bias", "bias": ", N(0,0.1^2) router bias"}
                 .get(shape.routing, "") + ")"),
        "config": {"workload": f"{workload}: {WL_DESC[workload]}", "tokens": T,
                   "hidden": H, "experts": E, "top_k": k, "expert_inter": I,
                   "shared_inter": Is, "weights": shape.weight_dtype,
                   "routing": shape.routing, "parallelism": "single GPU",
                   "renormalize": shape.renormalize,
                   **({"score": shape.score, "routed_scale": shape.routed_scale,
                       "bias_mode": shape.bias_mode}
                      if shape.score != "softmax" or shape.routed_scale != 1.0 else {}),
                   **({"swiglu_limits": [shape.swiglu_limit, shape.swiglu_limit_shared]}
                      if shape.swiglu_limit or shape.swiglu_limit_shared else {})},
        "roofline": roof,
        "layer": {**layer_frac, "alg_bytes": int(b_alg), "alg_flops": int(f_alg),
                  "experts_touched": U,
                  "gate_up_ms_timed": round(gu_ms, 5),
                  "stage_ms": {n: round(v, 5) for n, v in zip(B.STAGES, stage_avg)},
                  "stage_ms_note": f"{nb} steps after the timed region, every stage boundary recorded"},
        "cpu_baseline": cpu,
    }
    del inp, layer, out, ws, route
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is designed, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} bytes 5 times")
        return

    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    main_res = measure(args.workload, args, cpu_s)
    line = {"metric": METRIC, "value": main_res["value"], "unit": main_res["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None}
    for key in ("dtype", "data", "config", "roofline"):
        line[key] = main_res[key]
    line["device"] = {**device_info(),
                      "peaks_used": "published: HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s"}
    line["layer"] = main_res["layer"]
    line["cpu_baseline"] = main_res["cpu_baseline"]
    # The metric's second half: the 16384-token prefill chunk's MFMA fraction,
    # timed in the same process after the headline workload (same K and W).
    if args.workload == "decode" and not args.no_prefill:
        pf = measure("prefill", args, cpu_s)
        line["prefill"] = {key: pf[key] for key in ("value", "unit", "ms_per_step", "steps",
                                                    "warmup", "dtype", "config", "roofline",
                                                    "layer", "cpu_baseline")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
