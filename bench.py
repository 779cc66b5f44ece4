#!/usr/bin/env python3
"""Throughput of the 8-bit attention forward on one MI355X.

One step = one whole plug-and-play forward (statistics + smoothing/quantisation
kernels + the attention kernel) over one batch of seeded synthetic input that is
already resident in HBM.  Default workload: causal LLM prefill, B=4 H=32 N=4096
d=128, INT8 Q K^T + FP16 P~V.

Prints one JSON line: the throughput in attention TOPS (4*B*H*N^2*d per step,
halved for causal), the attention kernel's roofline position (its average
duration from HIP events on the launch stream), and the CPU oracle timed on a
bounded sample of the same workload.

--config picks another workload; --variant 1 runs the FP8 P~V variant on it
(with Q smoothing), --variant 2 the MXFP4 Q K^T variant, --smooth-v adds V
smoothing to either; --q-group 1 uses per-token INT8 Q scales.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TOPS at 1 MI355X (d=128,N=4096); % of INT8 MFMA peak"
# MI355X published dense matrix peaks, in tera-operations per second
INT8_PEAK_TOPS = 5000.0
FP16_PEAK_TOPS = 2500.0
FP8_PEAK_TOPS = 5000.0
FP4_PEAK_TOPS = 10100.0
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["quantized_bit_attention_amd/csrc/sage_attn.hip", "quantized_bit_attention_amd/csrc/sage_device.h",
                  "quantized_bit_attention_amd/csrc/sage_tiles.h"]
VARIANT_TAG = {0: "_int8qk_fp16pv", 1: "_int8qk_fp8pv", 2: "_mxfp4qk_fp8pv", 3: "_mxfp4qk_fp4pv"}


def mfma_ceiling_tops(variant: int) -> float:
    """The attention kernel's matrix-unit ceiling for its own operand types: half of the
    counted operations are Q K^T (INT8, or FP4 in variants 2 and 3), half P~ V (FP16 in
    variant 0, FP4 in variant 3, FP8 otherwise), so the ceiling is the harmonic combination
    of the two peaks."""
    qk = FP4_PEAK_TOPS if variant >= 2 else INT8_PEAK_TOPS
    pv = FP16_PEAK_TOPS if variant == 0 else FP4_PEAK_TOPS if variant == 3 else FP8_PEAK_TOPS
    return 1.0 / (0.5 / qk + 0.5 / pv)


def profile_name(cfg: dict, variant: int) -> str:
    """File-name stem of a workload's profile summaries; a variant other than the workload's
    own is appended as a suffix."""
    tag = "" if variant == cfg["variant"] else VARIANT_TAG[variant]
    return cfg["name"].replace("-", "_") + tag


def traffic_file(cfg: dict, variant: int) -> str:
    return os.path.join(ROOT, "profiles", f"attn_kernel_hbm_traffic_{profile_name(cfg, variant)}.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(cfg, variant):
    """HBM bytes per attention-kernel launch from the committed rocprofv3 counter summary of
    this workload and variant, or None when it is missing or was taken from another version
    of the kernel."""
    path = traffic_file(cfg, variant)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = the headline workload)")
    ap.add_argument("--variant", type=int, choices=(0, 1, 2, 3), default=None,
                    help="0: INT8 QK + FP16 P~V, 1: INT8 QK + Q smoothing + FP8 P~V, 2: MXFP4 QK + FP8 P~V, "
                         "3: MXFP4 QK + MXFP4 P~V (default: the workload's)")
    ap.add_argument("--smooth-v", action="store_true",
                    help="variants 1-3: subtract V's token mean before FP8 / MXFP4 and add it back")
    ap.add_argument("--q-group", type=int, default=0,
                    help="rows per Q scale (0: one per Q block; 1: per token)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32, help="heads of the workload the oracle runs")
    ap.add_argument("--bwd", action="store_true",
                    help="measure the 8-bit backward (dQ, dK, dV) of the workload instead of the forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_bit_attention_amd as sage
    import workloads

    if args.bwd:
        return bench_bwd(args)

    cfg = workloads.config(args.config)
    x = workloads.make_inputs(args.config)
    B, H, N, d = x["q"].shape
    causal = cfg["causal"]
    variant = cfg["variant"] if args.variant is None else args.variant
    smooth_v = bool(args.smooth_v)
    if smooth_v and variant == 0:
        print("bench.py: --smooth-v needs an FP8 / FP4 P~V variant (--variant 1, 2 or 3, or --config 5)",
              file=sys.stderr)
        sys.exit(2)
    q_group = args.q_group
    opts = dict(causal=bool(causal), variant=variant, blk_q=cfg["blk_q"], blk_k=cfg["blk_k"], smooth_v=smooth_v,
                q_group=q_group)
    ops = workloads.attention_ops(B, H, N, d, causal)

    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    ws = torch.empty(sage.workspace_bytes(B, H, N, d, variant, blk_q=cfg["blk_q"], blk_k=cfg["blk_k"],
                                          smooth_v=smooth_v, q_group=q_group),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        sage.attn(q, k, v, out=out, workspace=ws, **opts)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        sage.attn(q, k, v, out=out, workspace=ws, **opts)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # the attention kernel alone, as the step launches it (same stream, same launch
    # configuration): every variant quantises Q inside the kernel; variants 1-3 read the
    # quantised V
    if variant >= 2:
        qk = sage.quant_qk_mx(q, k)
    else:
        qk = sage.quant_qk(q, k, blk_q=cfg["blk_q"], blk_k=cfg["blk_k"], smooth_q=variant == 1, q_group=q_group)
    vq = (sage.quant_v_mx(v, smooth_v=smooth_v) if variant == 3 else
          sage.quant_v(v, smooth_v=smooth_v) if variant != 0 else None)
    if variant == 3:
        def kernel():
            sage.attn_qf16_fp4(q, qk, vq, causal=bool(causal), smooth_v=smooth_v, out=out)
    elif variant == 2:
        def kernel():
            sage.attn_qf16_mx(q, qk, vq, causal=bool(causal), smooth_v=smooth_v, out=out)
    elif variant == 0:
        def kernel():
            sage.attn_qf16(q, qk, v, out=out, causal=bool(causal), blk_q=cfg["blk_q"], blk_k=cfg["blk_k"],
                           q_group=q_group)
    else:
        def kernel():
            sage.attn_qf16_fp8(q, qk, vq, causal=bool(causal), blk_q=cfg["blk_q"], blk_k=cfg["blk_k"], smooth_q=True,
                               smooth_v=smooth_v, q_group=q_group, out=out)
    for _ in range(3):
        kernel()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(args.steps):
        kernel()
    a1.record(stream)
    torch.cuda.synchronize()
    attn_ms = a0.elapsed_time(a1) / args.steps

    if args.copy_calibration:
        # known traffic: reads 1 GiB, writes 1 GiB; its FETCH_SIZE / WRITE_SIZE scale the counters
        src_t = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t

    value = ops / (ms * 1e-3) / 1e12
    attn_tops = ops / (attn_ms * 1e-3) / 1e12
    # counter summaries exist per workload and variant, for the default options
    traffic = read_traffic(cfg, variant) if q_group == 0 and not smooth_v else None
    ceiling = mfma_ceiling_tops(variant)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int8+fp16", "int8+fp8", "mxfp4+fp8", "mxfp4")[variant],
        "data": "synthetic (seeded SplitMix64/Box-Muller; K with per-channel offsets)",
        "config": {"workload": f"{cfg['name']} B={B} H={H} N={N} d={d}", "B": B, "H": H, "N": N, "d": d,
                   "causal": causal, "variant": variant, "blk_q": cfg["blk_q"], "blk_k": cfg["blk_k"],
                   "smooth_v": int(smooth_v), "q_group": q_group or cfg["blk_q"], "kv_tile": sage.kv_tile(variant, d)},
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "attn_kernel_ms": round(attn_ms, 5),
        "attn_kernel_tops": round(attn_tops, 2),
        # the attention kernel against the matrix-unit ceiling of its own operand types
        # (variant 0: INT8 + FP16 = 3333 TOPS; 1: INT8 + FP8 = 5000; 2: FP4 + FP8 = 6689;
        # 3: FP4 + FP4 = 10100)
        "roofline": {"bound": "mfma", "achieved": round(attn_tops, 2), "peak": round(ceiling, 1),
                     "unit": "TOPS", "frac": round(attn_tops / ceiling, 4),
                     "frac_of_int8_peak": round(attn_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic},
    }

    if not args.no_cpu_baseline:
        import oracle

        orc = oracle.Oracle()
        nh = min(args.cpu_heads, B * H)
        heads = np.repeat(np.arange(nh, dtype=np.int32), N)
        rows = np.tile(np.arange(N, dtype=np.int32), nh)
        t0 = time.perf_counter()
        orc.attn_rows(x["q"], x["k"], x["v"], heads, rows, causal=causal, variant=variant,
                      blk_q=cfg["blk_q"], blk_k=cfg["blk_k"], bkv=sage.kv_tile(variant, d), smooth_v=int(smooth_v),
                      q_group=q_group or None)
        dt = time.perf_counter() - t0
        sample_ops = workloads.attention_ops(1, nh, N, d, causal)
        result["cpu_baseline"] = {"value": round(sample_ops / dt / 1e12, 6), "unit": "TOPS",
                                  "cores": orc.threads_used, "kind": "oracle",
                                  "sample": f"{nh} of {B * H} heads, all {N} rows, {dt:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_bwd(args):
    """The 8-bit backward of the workload: one step = stats + quantisation + preparation +
    dK/dV + dQ kernels on inputs resident in HBM.  Operations counted: the five products
    of the backward, 2*N^2*d each per head (10*B*H*N^2*d, halved for causal); the dQ kernel's
    recomputation of S and dP is not counted.  Ceiling: two INT8 products (5.0 POP/s) and
    three FP16 products (2.5 PFLOP/s) -> 3125 TOPS."""
    import numpy as np
    import torch

    import quantized_bit_attention_amd as sage
    import workloads

    cfg = workloads.config(args.config)
    x = workloads.make_inputs(args.config)
    B, H, N, d = x["q"].shape
    causal = bool(cfg["causal"])
    blk_q = max(cfg["blk_q"], 64)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev) for n in ("q", "k", "v"))
    rng = np.random.default_rng(12)
    dout = torch.from_numpy(rng.standard_normal(x["q"].shape).astype(np.float16)).to(dev)
    o, lse = sage.attn_fwd_train(q, k, v, causal=causal, blk_q=blk_q, blk_k=cfg["blk_k"])
    ws = torch.empty(sage._load().sage_attn_bwd_workspace_bytes(
        B, H, N, d, ctypes_params(sage, blk_q, cfg["blk_k"])), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    kw = dict(causal=causal, blk_q=blk_q, blk_k=cfg["blk_k"], workspace=ws)
    for _ in range(args.warmup):
        sage.attn_bwd(q, k, v, o, dout, lse, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        sage.attn_bwd(q, k, v, o, dout, lse, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ops = 2.5 * workloads.attention_ops(B, H, N, d, causal)  # 5 products of 2*N^2*d
    tops = ops / (ms * 1e-3) / 1e12
    ceiling = 1.0 / (0.4 / INT8_PEAK_TOPS + 0.6 / FP16_PEAK_TOPS)
    result = {
        "metric": "8-bit attention backward TOPS (10*B*H*N^2*d per step, halved for causal)",
        "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+fp16", "data": "synthetic (seeded SplitMix64/Box-Muller; dO from numpy PCG64 seed 12)",
        "config": {"workload": f"{cfg['name']} backward B={B} H={H} N={N} d={d}", "B": B, "H": H, "N": N, "d": d,
                   "causal": int(causal), "blk_q": blk_q, "blk_k": cfg["blk_k"]},
        "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": round(ceiling, 1), "unit": "TOPS",
                     "frac": round(tops / ceiling, 4), "traffic": None,
                     "scope": "whole backward call (per-kernel split in the rocprofv3 summary)"},
    }
    print(json.dumps(result), flush=True)


def ctypes_params(sage, blk_q, blk_k):
    import ctypes
    return ctypes.byref(sage._params(blk_q, blk_k, True, False, False, 0))


if __name__ == "__main__":
    main()
