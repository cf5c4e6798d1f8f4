#!/usr/bin/env python
"""Benchmark of the AWQ per-layer hot path on one MI355X; prints ONE JSON line.

A step is one pass of the whole path over one synthetic layer:
  activation statistics -> 21-point alpha search (scale tables, exact
  quantiser for every alpha, loss contraction on the matrix cores, argmin,
  final quantisation) -> INT4 packing -> W4A16 products at decode batch sizes
  M = 1, 8, 32 on the packed result.
Default workload: the large layer (D_in = 8192, D_out = 28672, N = 4096
calibration tokens, bf16, INT4, group 128), the largest layer of the five
that fits one GPU.

value  = alpha-candidates per second of the whole step (21 per step).
roofline: the loss contraction (dominant kernel), timed live with HIP events on
the stream it runs on; algorithmic work 2·N·D_in·D_out FLOP per alpha.
search_4096x4096: the same step on the attention-projection layer
(D_in = D_out = 4096, N = 2048), with its own loss-contraction roofline.
decode_gemm: the W4A16 product on the packed large layer at M = 1, 8, 32 with
inv_s = 1/s*, rotating 4 weight copies (> the 256 MB Infinity Cache) so that
weights stream from HBM.
prefill_gemm: the same packed layer at M = 512 and 2048 (matrix-core
dequantising product), TFLOP/s against the dense fp16 MFMA peak.
statistic_variants, group_sweep, zero_point, fp16_steps, clip_search: the
variants on the 4096x4096 layer (the W4A16 variants on 8192x28672).
cpu_baseline: the CPU oracle on a bounded column slice of the large layer.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "α-candidates/sec per layer + W4A16 GEMM TFLOP/s & GB/s (% roofline), 1 GPU"
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA
PEAK_F32_TFLOPS = 157.3      # MI355X fp32 matrix/vector
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
DECODE_SHAPE = (8192, 28672)
VARIANT_CONFIG = 2           # layer of the variant measurements

# Bytes per launch of the loss contraction past its L2 (HBM or Infinity
# Cache), from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
# dispatch), scaled by what the same counters read for a plain 1 GiB copy
# (reads x2.0, writes x1.0).  Keyed by layer config; valid only for the kernel
# source they were taken on.
_K_SEARCH = "weight_only_quantization_awq_amd/csrc/k_search.hip"
_K_SEARCH_SHA = "5a6aee55c975257282d9296e275aad6812875ac3825f692b5c2e4de65cfd3b0b"
LOSS_GEMM_COUNTERS = {
    5: {"fetch_kib": 30838579.5, "write_kib": 294.0, "fetch_factor": 2.0, "write_factor": 1.0,
        "source": _K_SEARCH, "sha256": _K_SEARCH_SHA, "clock_ghz": 1.61, "mfma_busy": 0.75},
    2: {"fetch_kib": 1065125.5, "write_kib": 21.0, "fetch_factor": 2.0, "write_factor": 1.0,
        "source": _K_SEARCH, "sha256": _K_SEARCH_SHA, "clock_ghz": 1.66, "mfma_busy": 0.69},
}
# The same counter runs also read the core clock during the kernel
# (GRBM_GUI_ACTIVE / duration / 8, calibrated on the MFMA issue loop) and the
# fraction of those cycles the matrix cores were busy
# (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / cycles).
# v_mfma_f32_32x32x16_f16 issue loop, 16 independent accumulators per wave,
# operands cycling through pseudo-random halves: 1.54-1.66 PFLOP/s measured on
# MI355X (2.29-2.36 with all-zero operands: the clock is power-held)
SUSTAINED_FP16_MFMA = 1600.0
# v_mfma_f32_32x32x16_bf16, same loop and operand recipe: 1.80 PFLOP/s
# (calib mfma kind 5)
SUSTAINED_BF16_MFMA = 1800.0
DECODE_MS = (1, 8, 32)
PREFILL_MS = (512, 2048)     # prefill batch sizes on the same packed large layer
EVENT_EVERY = 5              # timed steps that carry the phase events


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=5, help="layer config 1..5 of the headline step (default 5)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="only the headline step (no 4096x4096 step, variants, decode or prefill tables)")
    p.add_argument("--no-decode", action="store_true", help="skip the large-layer W4A16 decode/prefill tables")
    p.add_argument("--decode-reps", type=int, default=40)
    p.add_argument("--prefill-reps", type=int, default=10)
    p.add_argument("--cpu-cols", type=int, default=1024, help="output columns in the CPU-oracle sample")
    return p.parse_args()


def loss_gemm_record(config: int):
    """The counter record of the loss contraction for this layer, or None if absent or stale."""
    rec = LOSS_GEMM_COUNTERS.get(config)
    if rec is None:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as fh:
        if hashlib.sha256(fh.read()).hexdigest() != rec["sha256"]:
            return None
    return rec


def loss_gemm_traffic(config: int):
    """Counter-derived bytes per launch past the L2, or None if absent or stale."""
    rec = loss_gemm_record(config)
    if rec is None:
        return None
    return int(round(rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]))


def search_flops(case) -> float:
    return 2.0 * case.N * case.D_in * case.D_out * len(case.alphas)


def layer_step(torch, awq, synth, case, cfg, steps, warmup, dev):
    """Time `steps` whole-path steps on one layer (inputs resident in HBM).

    Returns the figures, the last search result and the packed words."""
    tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    X = torch.from_numpy(case.X).to(tdt).to(dev)
    W = torch.from_numpy(case.W).to(tdt).to(dev)
    n_alpha = len(case.alphas)
    ws = torch.empty(awq.search_workspace_size(case.N, case.D_in, case.D_out, tdt, case.bits, case.group, n_alpha),
                     dtype=torch.uint8, device=dev)
    f16_path = (tdt == torch.bfloat16) and case.N * case.D_out >= 65536
    # 16-bit path on bf16 matrix cores (with 64 correction rows): 2048 <= D_in <= 16384, N·D_in·D_out >= 2^39
    bf16_path = f16_path and 2048 <= case.D_in <= 16384 and case.N * case.D_in * case.D_out >= 2 ** 39
    sustained = SUSTAINED_BF16_MFMA if bf16_path else SUSTAINED_FP16_MFMA
    Xdec = {M: torch.from_numpy(synth.decode_x(M, case.D_in, seed=1050 + M)).to(torch.bfloat16).to(dev)
            for M in DECODE_MS}
    Ydec = {M: torch.empty(M, case.D_out, dtype=torch.float32, device=dev) for M in DECODE_MS}
    pack_bits = case.bits if case.bits <= 4 else None
    with_decode = pack_bits is not None and case.group % 32 == 0
    dws = {M: torch.empty(max(awq.w4a16_workspace_size(M, case.D_in, case.D_out, False), 16), dtype=torch.uint8,
                          device=dev) for M in DECODE_MS}
    last = {}

    def step(events=None):
        a = awq.act_stats(X)
        r = awq.search_layer(X, W, alphas=case.alphas, bits=case.bits, group=case.group, a=a, workspace=ws,
                             events=events)
        last["r"] = r
        if pack_bits is not None:
            packed = awq.pack(r.codes, bits=pack_bits)
            last["packed"] = packed
            if with_decode:
                for M in DECODE_MS:
                    awq.w4a16_gemm(Xdec[M], packed, r.scales, group=case.group, out=Ydec[M], workspace=dws[M])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Phase events (HIP events the library records on its stream at the phase
    # boundaries) on every EVENT_EVERY-th timed step: each recorded event
    # leaves a small bubble in the stream, so recording them on every step
    # would slow the step being measured.
    timed = [k for k in range(steps) if k % EVENT_EVERY == 0]
    evsets = {k: [torch.cuda.Event(enable_timing=True) for _ in range(5)] for k in timed}
    torch.cuda.synchronize()
    tstart = time.perf_counter()
    for k in range(steps):
        step(evsets.get(k))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - tstart
    res = last["r"]
    best = res.best_index()
    phases = np.array([[evs[i].elapsed_time(evs[i + 1]) for i in range(4)] for evs in evsets.values()])  # ms
    ph_mean = phases.mean(axis=0)
    gemm_ms = float(ph_mean[2])
    flops = search_flops(case)
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_F16_TFLOPS if f16_path else PEAK_F32_TFLOPS
    ms_per_step = elapsed / steps * 1e3
    value = n_alpha * steps / elapsed
    log(f"[bench] {case.name}: {steps} steps in {elapsed:.3f}s: {ms_per_step:.3f} ms/step, "
        f"alpha*={case.alphas[best]:.2f}; phases ms prep={ph_mean[0]:.3f} quant={ph_mean[1]:.3f} "
        f"loss_gemm={ph_mean[2]:.3f} reduce+select={ph_mean[3]:.3f}; loss_gemm {achieved:.1f} TFLOP/s")
    out = {
        "value": round(value, 3),
        "ms_per_step": round(ms_per_step, 4),
        "dtype": ("bf16" if bf16_path else "f16") if f16_path else "f32",
        "config": {
            "workload": f"{synth.CONFIG_NAMES[cfg]}, {n_alpha}-point alpha grid"
                        + (", + INT4 pack + W4A16 decode M=1,8,32" if with_decode else
                           (", + pack" if pack_bits else "")),
            "N": case.N, "D_in": case.D_in, "D_out": case.D_out, "bits": case.bits, "group": case.group,
            "n_alpha": n_alpha, "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": ("loss_gemm_f16_kernel<true> (X·D for all alphas, v_mfma_f32_32x32x16_bf16, fp32 accumulate, "
                       "+64 correction rows)" if bf16_path else
                       "loss_gemm_f16_kernel<false> (X·D for all alphas, v_mfma_f32_32x32x16_f16, fp32 accumulate)")
            if f16_path else "loss_gemm_f32_kernel (X·D for all alphas, v_mfma_f32_16x16x4_f32)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": loss_gemm_traffic(cfg) if f16_path else None,
            "traffic_kind": "bytes past L2 (HBM or Infinity Cache) per launch, FETCH_SIZE x2 + WRITE_SIZE x1",
            "algorithmic_bytes": 2 * (case.N * case.D_in + n_alpha * case.D_in * case.D_out) if f16_path else None,
            "counter_clock_GHz": (loss_gemm_record(cfg) or {}).get("clock_ghz") if f16_path else None,
            "mfma_busy_at_clock": (loss_gemm_record(cfg) or {}).get("mfma_busy") if f16_path else None,
            "flop_per_launch": flops,
            "launch_ms": round(gemm_ms, 4),
            # what the matrix cores sustain on this part with full-entropy FP16
            # operands (an issue loop with no memory traffic), for context only
            "sustained_mfma_TFLOP_s": sustained if f16_path else None,
            "frac_of_sustained": round(achieved / sustained, 4) if f16_path else None,
        },
        "phases_ms": {"prep": round(float(ph_mean[0]), 4), "quantise_all_alpha": round(float(ph_mean[1]), 4),
                      "loss_gemm": round(gemm_ms, 4), "reduce_select": round(float(ph_mean[3]), 4)},
        "alpha_star": float(case.alphas[best]),
    }
    del ws, X, W
    return out, res, last.get("packed")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); "
              "the search would shard by output columns with one 21-value all-reduce, which is not implemented.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    from weight_only_quantization_awq_amd import awq, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(int(os.environ.get("LOCAL_RANK", "0")))
    dev = torch.device("cuda")

    t0 = time.time()
    case = synth.config_case(args.config)
    log(f"[bench] generated {case.name} N={case.N} D_in={case.D_in} D_out={case.D_out} in {time.time() - t0:.1f}s")
    head, res, packed = layer_step(torch, awq, synth, case, args.config, args.steps, args.warmup, dev)

    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "alpha-candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "phases_ms": head["phases_ms"],
        "alpha_star": head["alpha_star"],
    }
    cpu_case = case if not args.no_cpu_baseline else None

    if not args.no_extras:
        if not args.no_decode and (case.D_in, case.D_out) == DECODE_SHAPE and packed is not None:
            out["decode_gemm"], out["prefill_gemm"] = decode_bench(args, torch, awq, synth, dev, packed, res)
        del packed, res
        torch.cuda.empty_cache()
        vcase = case if args.config == VARIANT_CONFIG else synth.config_case(VARIANT_CONFIG)
        if args.config != VARIANT_CONFIG:
            vhead, _, _ = layer_step(torch, awq, synth, vcase, VARIANT_CONFIG, 50, 25, dev)
            out["search_4096x4096"] = vhead
        torch.cuda.empty_cache()
        tdt = torch.bfloat16 if vcase.dtype == "bf16" else torch.float32
        X = torch.from_numpy(vcase.X).to(tdt).to(dev)
        W = torch.from_numpy(vcase.W).to(tdt).to(dev)
        ws = torch.empty(awq.search_workspace_size(vcase.N, vcase.D_in, vcase.D_out, tdt, vcase.bits, vcase.group,
                                                   len(vcase.alphas)), dtype=torch.uint8, device=dev)
        a = awq.act_stats(X)
        vres = awq.search_layer(X, W, alphas=vcase.alphas, bits=vcase.bits, group=vcase.group, a=a, workspace=ws)
        out["statistic_variants"] = variants_bench(args, torch, awq, vcase, X, W, ws, dev)
        out["group_sweep"] = group_sweep_bench(args, torch, awq, vcase, X, W)
        if vcase.group in (32, 64, 128, 256):
            out["clip_search"] = clip_bench(args, torch, awq, vcase, X, W, vres)
        if vcase.group != 256 and vcase.D_in % 256 == 0:
            out["clip_search_g256"] = clip_bench(args, torch, awq, vcase, X, W, vres, group=256)
        out["zero_point"] = {"search": variant_search_bench(args, torch, awq, vcase, X, W, zero_point=True)}
        out["fp16_steps"] = {"search": variant_search_bench(args, torch, awq, vcase, X, W, f16_steps=True)}
        out["variants_layer"] = synth.CONFIG_NAMES[VARIANT_CONFIG]
        del X, W, ws, vres
        torch.cuda.empty_cache()
        if not args.no_decode:
            out["zero_point"].update(variant_gemm_bench(args, torch, awq, synth, dev, zero_point=True))
            out["fp16_steps"].update(variant_gemm_bench(args, torch, awq, synth, dev, f16_steps=True))

    if cpu_case is not None:
        out["cpu_baseline"] = cpu_baseline(args, cpu_case)

    print(json.dumps(out), flush=True)


def _event_us(torch, fn, reps):
    """Mean microseconds per call of ``fn`` with HIP events around each call."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3


def variants_bench(args, torch, awq, case, X, W, ws, dev):
    """The max statistic, the weight statistic and the weight-term search on the benchmark layer."""
    elt = 2 if X.dtype == torch.bfloat16 else 4
    us_max = _event_us(torch, lambda: awq.act_stats(X, statistic="max"), 20)
    us_mean = _event_us(torch, lambda: awq.act_stats(X), 20)
    us_w = _event_us(torch, lambda: awq.weight_stats(W), 20)
    bx = case.N * case.D_in * elt + case.D_in * 4
    bw = case.D_in * case.D_out * elt + case.D_in * 4
    a = awq.act_stats(X)
    b = awq.weight_stats(W)
    us_ws = _event_us(torch, lambda: awq.search_layer(X, W, alphas=case.alphas, bits=case.bits, group=case.group,
                                                      a=a, b=b, workspace=ws), 10)
    res = {
        "act_stats_mean": {"us": round(us_mean, 2), "GB_s": round(bx / us_mean / 1e3, 1),
                           "frac_hbm": round(bx / us_mean / 1e3 / PEAK_HBM_GBS, 4)},
        "act_stats_max": {"us": round(us_max, 2), "GB_s": round(bx / us_max / 1e3, 1),
                          "frac_hbm": round(bx / us_max / 1e3 / PEAK_HBM_GBS, 4)},
        "weight_stats": {"us": round(us_w, 2), "GB_s": round(bw / us_w / 1e3, 1),
                         "frac_hbm": round(bw / us_w / 1e3 / PEAK_HBM_GBS, 4)},
        "search_weight_term": {"ms": round(us_ws / 1e3, 4),
                               "alpha_candidates_s": round(len(case.alphas) / (us_ws * 1e-6), 1)},
    }
    log(f"[bench] statistics: mean {us_mean:.1f} us, max {us_max:.1f} us, weight {us_w:.1f} us; "
        f"weight-term search {us_ws / 1e3:.3f} ms")
    return res


def group_sweep_bench(args, torch, awq, case, X, W):
    """The whole search (21 alpha) at group sizes 32, 64, 128, 256 on the benchmark layer."""
    res = []
    for g in (32, 64, 128, 256):
        if case.D_in % g:
            continue
        gws = torch.empty(awq.search_workspace_size(case.N, case.D_in, case.D_out, X.dtype, case.bits, g,
                                                    len(case.alphas)), dtype=torch.uint8, device=X.device)
        a = awq.act_stats(X)
        us = _event_us(torch, lambda: awq.search_layer(X, W, alphas=case.alphas, bits=case.bits, group=g, a=a,
                                                       workspace=gws), 8)
        res.append({"group": g, "ms": round(us / 1e3, 4), "alpha_candidates_s": round(len(case.alphas) / (us * 1e-6), 1)})
        del gws
    log("[bench] group sweep: " + ", ".join(f"g{r['group']} {r['ms']:.3f} ms" for r in res))
    return res


def variant_search_bench(args, torch, awq, case, X, W, zero_point=False, f16_steps=False):
    """The whole search with zero-point codes and/or FP16 steps on the benchmark layer."""
    gws = torch.empty(awq.search_workspace_size(case.N, case.D_in, case.D_out, X.dtype, case.bits, case.group,
                                                len(case.alphas)), dtype=torch.uint8, device=X.device)
    a = awq.act_stats(X)
    us = _event_us(torch, lambda: awq.search_layer(X, W, alphas=case.alphas, bits=case.bits, group=case.group,
                                                   a=a, workspace=gws, zero_point=zero_point,
                                                   f16_steps=f16_steps), 10)
    log(f"[bench] search (zero_point={zero_point}, f16_steps={f16_steps}): {us / 1e3:.3f} ms")
    return {"ms": round(us / 1e3, 4), "alpha_candidates_s": round(len(case.alphas) / (us * 1e-6), 1)}


def variant_gemm_bench(args, torch, awq, synth, dev, zero_point=False, f16_steps=False):
    """W4A16 with zero points and/or FP16 steps on 8192x28672 (random codes, 4 rotating copies): decode
    M = 1, 8, 32 and prefill M = 2048."""
    D_in, D_out = DECODE_SHAPE
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    copies = 4
    packs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (D_in // 8, D_out), dtype=torch.int32, device=dev, generator=g)
             for _ in range(copies)]
    sdt = torch.float16 if f16_steps else torch.float32
    scs = [(torch.rand(D_in // 128, D_out, device=dev, generator=g) * 0.01).to(sdt) for _ in range(copies)]
    zps = [torch.randint(0, 16, (D_in // 128, D_out), dtype=torch.uint8, device=dev, generator=g)
           if zero_point else None for _ in range(copies)]
    inv_s = torch.rand(D_in, device=dev, generator=g) + 0.5
    step_bytes = (2 if f16_steps else 4) + (1 if zero_point else 0)
    dec, pre = [], []
    for M in DECODE_MS + (2048,):
        Xd = torch.from_numpy(synth.decode_x(M, D_in, seed=3000 + M)).to(torch.bfloat16).to(dev)
        Y = torch.empty(M, D_out, dtype=torch.bfloat16, device=dev)
        need = (awq.load().awq_w4a16_workspace_size_ex(M, D_in, D_out, 128, awq.AWQ_F16) if f16_steps
                else awq.w4a16_workspace_size(M, D_in, D_out, True))
        gws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        it = iter(range(1 << 30))

        def call():
            i = next(it) % copies
            awq.w4a16_gemm(Xd, packs[i], scs[i], group=128, inv_s=inv_s, out=Y, workspace=gws, zeros=zps[i])

        us = _event_us(torch, call, args.decode_reps if M <= 32 else args.prefill_reps)
        if M <= 32:
            nbytes = D_in * D_out // 2 + (D_in // 128) * D_out * step_bytes + M * D_in * 2 + M * D_out * 2 + D_in * 4
            gbs = nbytes / (us * 1e-6) / 1e9
            dec.append({"M": M, "us": round(us, 3), "GB_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
        else:
            tf = 2.0 * M * D_in * D_out / (us * 1e-6) / 1e12
            pre.append({"M": M, "us": round(us, 2), "TFLOP_s": round(tf, 1), "frac_mfma": round(tf / PEAK_F16_TFLOPS, 4)})
        del Xd, Y, gws
    log(f"[bench] W4A16 (zero_point={zero_point}, f16_steps={f16_steps}): decode {[d['us'] for d in dec]} us, "
        f"prefill M=2048 {pre[0]['us']} us")
    return {"decode_gemm": dec, "prefill_gemm": pre}


def clip_bench(args, torch, awq, case, X, W, res, group=None):
    """Weight-clipping search after the scale search: 11 ratios 1 .. 0.5 on the benchmark layer."""
    group = case.group if group is None else group
    ratios = awq.default_clip_ratios(11, 0.5)
    s = res.s_best
    cws = torch.empty(awq.clip_workspace_size(case.N, case.D_in, group), dtype=torch.uint8, device=X.device)
    us = _event_us(torch, lambda: awq.clip_search(X, W, s, ratios=ratios, bits=case.bits, group=group,
                                                  workspace=cws), 10)
    G = case.D_in // group
    # algorithmic work: the quadratic forms d^T H_g d (2 group^2 per group, column and ratio) and the Gram
    # matrices (2 N group per input channel); the forms run as three FP16 products (hi/lo splits)
    forms = len(ratios) * G * case.D_out * 2.0 * group ** 2
    flops = forms + 2.0 * case.N * case.D_in * group
    tflops = flops / (us * 1e-6) / 1e12
    f16_exec = 3.0 * forms / (us * 1e-6) / 1e12
    log(f"[bench] clip search ({len(ratios)} ratios, group {group}): {us:.1f} us, {tflops:.1f} algorithmic TFLOP/s; "
        f"FP16 matrix work {f16_exec:.1f} TFLOP/s ({f16_exec / PEAK_F16_TFLOPS * 100:.1f}% of the fp16 peak)")
    return {"group": group, "n_ratio": len(ratios), "us": round(us, 2), "TFLOP_s": round(tflops, 2),
            "fp16_matrix_TFLOP_s": round(f16_exec, 2), "frac_fp16_mfma": round(f16_exec / PEAK_F16_TFLOPS, 4)}


def decode_bench(args, torch, awq, synth, dev, packed0, r):
    """W4A16 at the large layer's decode shapes on the headline step's packed
    result (inv_s = 1/s*), weights streamed from HBM."""
    D_in, D_out = DECODE_SHAPE
    scales0 = r.scales
    inv_s = (1.0 / r.s_best).contiguous()   # 1/s* prepared once, outside the timed region
    copies = 4  # 4 x 125 MB > 256 MB Infinity Cache
    packs = [packed0] + [packed0.clone() for _ in range(copies - 1)]
    scs = [scales0] + [scales0.clone() for _ in range(copies - 1)]
    res = []
    for M in DECODE_MS:
        Xd = torch.from_numpy(synth.decode_x(M, D_in)).to(torch.bfloat16).to(dev)
        Y = torch.empty(M, D_out, dtype=torch.bfloat16, device=dev)
        gws = torch.empty(max(awq.w4a16_workspace_size(M, D_in, D_out, True), 16), dtype=torch.uint8, device=dev)
        for i in range(8):
            awq.w4a16_gemm(Xd, packs[i % copies], scs[i % copies], group=128, inv_s=inv_s, out=Y, workspace=gws)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.decode_reps)]
        for i, (e0, e1) in enumerate(evs):
            e0.record()
            awq.w4a16_gemm(Xd, packs[i % copies], scs[i % copies], group=128, inv_s=inv_s, out=Y, workspace=gws)
            e1.record()
        torch.cuda.synchronize()
        us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
        # back to back: the same calls issued one after another between one pair of events, as
        # consecutive layers are in a serving loop (each call's launch overlaps the previous one)
        e0, e1 = evs[0]
        e0.record()
        for i in range(args.decode_reps):
            awq.w4a16_gemm(Xd, packs[i % copies], scs[i % copies], group=128, inv_s=inv_s, out=Y, workspace=gws)
        e1.record()
        torch.cuda.synchronize()
        us_stream = e0.elapsed_time(e1) * 1e3 / args.decode_reps
        # warm: one weight copy, resident in the 256 MB Infinity Cache after the first call
        for e0, e1 in evs:
            e0.record()
            awq.w4a16_gemm(Xd, packs[0], scs[0], group=128, inv_s=inv_s, out=Y, workspace=gws)
            e1.record()
        torch.cuda.synchronize()
        us_warm = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
        nbytes = D_in * D_out // 2 + (D_in // 128) * D_out * 4 + M * D_in * 2 + M * D_out * 2 + D_in * 4
        flops = 2.0 * M * D_in * D_out
        gbs = nbytes / (us * 1e-6) / 1e9
        res.append({"M": M, "us": round(us, 3), "GB_s": round(gbs, 1), "TFLOP_s": round(flops / (us * 1e-6) / 1e12, 3),
                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
                    "stream_us": round(us_stream, 3),
                    "stream_frac_hbm": round(nbytes / (us_stream * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "warm_us": round(us_warm, 3), "warm_GB_s": round(nbytes / (us_warm * 1e-6) / 1e9, 1)})
        log(f"[bench] W4A16 M={M}: {us:.2f} us, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS * 100:.1f}% of HBM); "
            f"back to back {us_stream:.2f} us; warm (one copy, Infinity Cache) {us_warm:.2f} us")
        del Xd, Y, gws
    pre = []
    for M in PREFILL_MS:
        Xd = torch.from_numpy(synth.decode_x(M, D_in, seed=2000 + M)).to(torch.bfloat16).to(dev)
        Y = torch.empty(M, D_out, dtype=torch.bfloat16, device=dev)
        gws = torch.empty(awq.w4a16_workspace_size(M, D_in, D_out, True), dtype=torch.uint8, device=dev)
        for i in range(3):
            awq.w4a16_gemm(Xd, packs[i % copies], scs[i % copies], group=128, inv_s=inv_s, out=Y, workspace=gws)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.prefill_reps)]
        for i, (e0, e1) in enumerate(evs):
            e0.record()
            awq.w4a16_gemm(Xd, packs[i % copies], scs[i % copies], group=128, inv_s=inv_s, out=Y, workspace=gws)
            e1.record()
        torch.cuda.synchronize()
        us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
        tflops = 2.0 * M * D_in * D_out / (us * 1e-6) / 1e12
        pre.append({"M": M, "us": round(us, 2), "TFLOP_s": round(tflops, 1),
                    "frac_mfma": round(tflops / PEAK_F16_TFLOPS, 4)})
        log(f"[bench] W4A16 prefill M={M}: {us:.1f} us, {tflops:.0f} TFLOP/s "
            f"({tflops / PEAK_F16_TFLOPS * 100:.1f}% of the fp16 MFMA peak)")
        del Xd, Y, gws
    return res, pre


def cpu_baseline(args, case):
    """The oracle, as it stands, on a column slice of the benchmark layer."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
    except Exception:  # pragma: no cover
        threadpool_info = None
    cols = min(args.cpu_cols, case.D_out)
    Wc = np.ascontiguousarray(case.W[:, :cols])
    reps, t = 0, 0.0
    while reps < 5 and (reps == 0 or t < 10.0):    # about 10 s of host work
        t0 = time.perf_counter()
        r = oracle.search_layer(case.X, Wc, case.alphas, case.bits, case.group)
        if case.bits <= 4 and case.D_in % 8 == 0:
            oracle.pack_int4(r["codes"])
        t += time.perf_counter() - t0
        reps += 1
    t /= reps
    threads = None
    if threadpool_info is not None:
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(i.get("num_threads", 1) for i in info)
    value = len(case.alphas) / (t * case.D_out / cols)
    log(f"[bench] oracle on {cols}/{case.D_out} columns: {t:.1f}s -> {value:.4f} alpha-candidates/s (full layer)")
    return {"value": round(value, 5), "unit": "alpha-candidates/s", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": (f"the whole layer ({case.N} tokens, {case.D_in}x{case.D_out})" if cols == case.D_out else
                       f"the layer restricted to its first {cols} of {case.D_out} output columns (the loss is a sum "
                       f"over columns and groups never cross columns), all {case.N} tokens")
                      + f", {len(case.alphas)} alphas, + pack; mean of {reps} runs of {t:.2f}s"
                      + ("" if cols == case.D_out else f", scaled by {case.D_out / cols:g}")}


if __name__ == "__main__":
    main()
