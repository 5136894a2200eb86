#!/usr/bin/env python3
"""Throughput of the MI355X flash-CCE ORPO head: one step = forward (logits + online softmax +
merge) -> ORPO loss (segmented means + epilogue + cotangent) -> backward (recompute + coefficients
+ dh and dW GEMMs) over one synthetic batch whose inputs are already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]

Prints one JSON line. The default workload is the e4b-shaped head (d=2560, V=262144, softcap 30,
M=8192 tokens as 16 chosen/rejected pairs). Runs on one GPU only.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PEAK_BF16 = 2.5e15       # MI355X dense bf16 MFMA, FLOP/s
PEAK_F32 = 157.3e12      # MI355X fp32 (vector and MFMA)
PEAK_FP8 = 5.0e15        # MI355X dense fp8 MFMA, FLOP/s
HBM_PEAK = 8.0e12        # bytes/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="e4b-bf16-softcap30",
                    help="workload name (lm_head_cross_amd.synth.WORKLOADS) or its integer key")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload at this many tokens M (its pairs scaled with M); "
                         "0 = the workload's own M")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    ap.add_argument("--trace-steps", type=int, default=5,
                    help="steps of the separate traced pass (per-kernel HIP events) after the timed region")
    ap.add_argument("--objective", default="orpo",
                    choices=["orpo", "simpo", "dpo", "ipo", "hinge", "grpo"],
                    help="the loss between the head's forward and backward")
    ap.add_argument("--skip-eps", type=float, default=0.0,
                    help="backward coefficient filter threshold (0 = exact backward)")
    ap.add_argument("--fp8", action="store_true",
                    help="the FP8 head (row-wise E4M3 logit operands; an approximation, reported "
                         "with its distance from the exact head)")
    ap.add_argument("--no-dw", action="store_true",
                    help="frozen head: the backward computes dh only (no dW), as for the 4-bit head")
    ap.add_argument("--q4-stage", action="store_true",
                    help="4-bit workloads: each step dequantises W once into bf16 rows and runs the "
                         "bf16 kernels on them (instead of dequantising every tile in the kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--mfma-peak", nargs="?", const="both", default=None,
                    choices=["both", "zeros", "random"],
                    help="instead of the head: the bf16 MFMA rate this GPU sustains (microbenchmark), "
                         "with zero and/or random operands")
    return ap.parse_args()


def workload_for(config: str, tokens: int = 0):
    """The named workload, or (tokens > 0) the same head, distributions and lengths at M = tokens,
    its pairs scaled with M (at least one; branch lengths shrink to fit when they do not)."""
    from lm_head_cross_amd import synth
    cfg = synth.workload(config)
    if tokens:
        if tokens < 0:
            raise ValueError("--tokens must be positive")
        pairs = max(1, round(cfg.pairs * tokens / cfg.M))
        cfg = cfg.replace(M=tokens, pairs=pairs, name=f"{cfg.name}-M{tokens}")
    return cfg


def _objective_inputs(objective: str, cfg, off: np.ndarray, n_valid_per_span: np.ndarray, M: int,
                      seed: int) -> dict:
    """Seeded synthetic inputs of the sibling objectives (parameters and cached reference values);
    timing only. SimPO beta 2, gamma 0.5; DPO beta 0.1 with reference sums near the head's scale;
    IPO beta 0.5 with reference means near the head's; hinge beta 0.1 with reference sums;
    GRPO clip 0.2, KL weight 0.04, groups of 4 completions; the sampling and reference policies'
    log-probs are filled in by main() from the policy's own forward plus seeded noise."""
    import numpy as np
    rng = np.random.default_rng(9000 + seed)
    if objective == "simpo":
        return {"beta": 2.0, "gamma": 0.5}
    if objective in ("dpo", "hinge"):
        ref = -7.7 * n_valid_per_span + rng.normal(0.0, 5.0, size=n_valid_per_span.shape)
        return {"beta": 0.1, "ref_sums": ref}
    if objective == "ipo":
        return {"beta": 0.5, "ref_sums": -7.7 + rng.normal(0.0, 0.1, size=n_valid_per_span.shape)}
    if objective == "grpo":
        S = len(off) - 1
        rewards = rng.normal(size=S + (-S) % 4)
        r = rewards.reshape(-1, 4)
        adv = ((r - r.mean(axis=1, keepdims=True)) / (r.std(axis=1, keepdims=True) + 1e-6)).reshape(-1)[:S]
        return {"clip_eps": 0.2, "beta": 0.04, "advantages": adv.astype(np.float32),
                "old_noise": rng.normal(0.0, 0.1, size=M).astype(np.float32),
                "ref_noise": rng.normal(0.0, 0.2, size=M).astype(np.float32)}
    return {}


def cpu_baseline(inp, rows: int, objective: str, want_dw: bool):
    """The float64 oracle as it stands, on a bounded sample of the same batch, on the host cores
    this process may run on (BLAS threads pinned to that count)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    n_cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=n_cores):
        res = _cpu_baseline(inp, rows, objective, want_dw)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    res["cores"] = int(min(threads, n_cores))
    res["affinity_cores"] = n_cores
    return res


def _cpu_baseline(inp, rows: int, objective: str, want_dw: bool):
    import numpy as np
    from oracle import objectives as ob
    from oracle import orpo_oracle as orc
    from lm_head_cross_amd import synth

    cfg = inp.cfg
    if cfg.q4:
        W = orc.dequant_q4(inp.wq, synth.bf16_bits(inp.scales), synth.bf16_bits(inp.biases), 64)
    else:
        W = inp.w.float().numpy()
    h = inp.h[:rows].float().numpy()
    labels = inp.labels[:rows].copy()
    # The sample is treated as one pair (the loss epilogue is a negligible part of the oracle's
    # time; the three [rows, V] x d products dominate).
    labels[labels == synth.IGNORE_INDEX] = 0
    t0 = time.perf_counter()
    if objective == "orpo" and cfg.scope == "full":     # prompt, chosen, rejected thirds
        off = np.array([0, rows // 3, 2 * rows // 3, rows], dtype=np.int32)
        out = orc.head_step_full(h, W, labels, off, cfg.softcap, cfg.lam, want_dW=want_dw)
    elif objective == "orpo":
        off = np.array([0, rows // 2, rows], dtype=np.int32)
        out = orc.head_step(h, W, labels, off, cfg.softcap, cfg.lam, want_dW=want_dw)
    else:
        off = np.array([0, rows // 2, rows], dtype=np.int32)
        logp, lse = orc.forward(h, W, labels, cfg.softcap)
        sums, n = ob.span_stats(logp, labels, off)
        if objective == "simpo":
            ep = ob.simpo_epilogue(sums[0::2] / n[0::2], sums[1::2] / n[1::2], 2.0, 0.5)
            g = ob.pairwise_cotangent("simpo", ep, n, labels, off)
        elif objective == "dpo":
            ep = ob.dpo_epilogue(sums[0::2], sums[1::2], sums[0::2] - 1.0, sums[1::2], 0.1)
            g = ob.pairwise_cotangent("dpo", ep, n, labels, off)
        elif objective == "ipo":
            m = sums / n
            ep = ob.ipo_epilogue(m[0::2], m[1::2], m[0::2] - 0.1, m[1::2], 0.5)
            g = ob.pairwise_cotangent("ipo", ep, n, labels, off)
        elif objective == "hinge":
            ep = ob.hinge_epilogue(sums[0::2], sums[1::2], sums[0::2] + 1.0, sums[1::2], 0.1)
            g = ob.pairwise_cotangent("hinge", ep, n, labels, off)
        else:
            ep = ob.grpo_loss(logp, logp - 0.1, logp + 0.1, labels, off, np.array([1.0, -1.0]), 0.2, 0.04)
            g = ep["g"]
        orc.backward(h, W, labels, lse, g, cfg.softcap, want_dW=want_dw)
        out = ep
    dt = time.perf_counter() - t0
    assert math.isfinite(out["loss"])
    return {
        "value": rows / dt, "unit": "tokens/s", "kind": "oracle",
        "sample": f"first {rows} tokens of the same batch (full V={cfg.V}, d={cfg.d}), float64 "
                  f"forward + {objective} loss + backward{' + dW' if want_dw else ''}; {dt:.1f} s",
    }


def mfma_peak(which: str = "both"):
    """The bf16 MFMA rate the GPU sustains with independent back-to-back 32x32x16 MFMAs on every
    SIMD (no memory traffic), with zero and with random operands: the achievable ceiling at the
    clock the chip runs, beside the 2.5 PFLOP/s nominal figure. Prints one JSON line."""
    import ctypes
    import torch
    from lm_head_cross_amd import build as B

    if not os.path.exists(B.PEAK_LIB):
        raise RuntimeError(f"{B.PEAK_LIB} is missing: run lm_head_cross_amd/build.py first")
    L = ctypes.CDLL(B.PEAK_LIB)
    L.mfma_peak_run.restype = ctypes.c_int
    L.mfma_peak_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]
    dev = torch.device("cuda:0")
    n_wg, iters = 512, 500                # 2 rounds of one workgroup per CU, ~0.5 s at 2 PFLOP/s
    flop = n_wg * 8 * iters * 8 * 32768.0
    out = torch.empty(n_wg * 512, dtype=torch.float32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    res = {}
    kinds = {"zeros": lambda: torch.zeros(128 * 8, dtype=torch.bfloat16, device=dev),
             "random": lambda: torch.randn(128 * 8, device=dev, generator=g).to(torch.bfloat16)}
    for name in (["zeros", "random"] if which == "both" else [which]):
        src = kinds[name]()
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        for _ in range(2):   # warm-up
            assert L.mfma_peak_run(n_wg, iters, ctypes.c_void_p(src.data_ptr()),
                                   ctypes.c_void_p(out.data_ptr()), stream) == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        reps = 5
        for _ in range(reps):
            assert L.mfma_peak_run(n_wg, iters, ctypes.c_void_p(src.data_ptr()),
                                   ctypes.c_void_p(out.data_ptr()), stream) == 0
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        assert bool(torch.isfinite(out).all())
        res[name] = {"ms_per_launch": round(ms, 3), "tflops": round(flop / ms / 1e9, 1)}
        print(f"[mfma-peak] {name}: {ms:.3f} ms, {flop / ms / 1e9:.1f} TFLOP/s", file=sys.stderr,
              flush=True)
    print(json.dumps({"metric": "bf16 MFMA microbenchmark (32x32x16, 8 independent chains per wave, "
                                "2 waves per SIMD, no memory traffic)", "unit": "TFLOP/s",
                      "nominal_peak": 2500.0, **res,
                      "frac_of_nominal": {k: round(v["tflops"] / 2500.0, 4) for k, v in res.items()}}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this head is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    if args.mfma_peak:
        mfma_peak(args.mfma_peak)
        return
    import numpy as np
    import torch
    from lm_head_cross_amd import head as H
    from lm_head_cross_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = workload_for(args.config, args.tokens)
    print(f"[bench] generating {cfg.name} M={cfg.M} d={cfg.d} V={cfg.V}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg, seed=args.seed, label_device="cuda")
    h = inp.h.to(dev)
    if cfg.q4:
        w = torch.from_numpy(inp.wq.view(np.int32)).to(dev)
        sc, bi = inp.scales.to(dev), inp.biases.to(dev)
    else:
        w, sc, bi = inp.w.to(dev), None, None
    labels = torch.from_numpy(inp.labels).to(dev)
    off = torch.from_numpy(inp.seg_offsets).to(dev)
    torch.cuda.synchronize()
    inputs_bytes = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    obj = None
    if args.objective != "orpo":
        if cfg.scope == "full":
            print("sibling objectives take (chosen, rejected) spans: use a response-scope workload",
                  file=sys.stderr)
            sys.exit(2)
        n_span = np.array([int((inp.labels[a:b] != synth.IGNORE_INDEX).sum())
                           for a, b in zip(inp.seg_offsets[:-1], inp.seg_offsets[1:])], dtype=np.float64)
        o = _objective_inputs(args.objective, cfg, inp.seg_offsets, n_span, cfg.M, args.seed)
        obj = {k: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v) for k, v in o.items()}
        if args.objective == "grpo":   # old / reference log-probs: the policy's own, perturbed
            pre = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, scales=sc, biases=bi,
                             want_dW=False)
            pre.forward()
            obj["old_logp"] = pre.logp + obj.pop("old_noise")
            obj["ref_logp"] = pre.logp + obj.pop("ref_noise")
            del pre
    if args.fp8 and (cfg.q4 or cfg.dtype != "bf16"):
        print("--fp8 approximates a bf16 head: pick a bf16 workload", file=sys.stderr)
        sys.exit(2)
    if args.q4_stage and not cfg.q4:
        print("--q4-stage stages a 4-bit head: pick a q4 workload", file=sys.stderr)
        sys.exit(2)
    want_dw = not cfg.q4 and not args.no_dw      # the 4-bit head is frozen: dh only
    step = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, scales=sc, biases=bi,
                      want_dW=want_dw, scope=cfg.scope, objective=args.objective, obj=obj,
                      skip_eps=args.skip_eps, fp8=args.fp8, q4_stage=args.q4_stage)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step.step()
    torch.cuda.synchronize()
    loss0 = float(step.out[0].item())
    assert math.isfinite(loss0), "non-finite loss"

    # Headline: exactly `steps` steps, nothing traced; events on the launch stream mark the step
    # boundaries for the per-step median.
    stream = torch.cuda.current_stream(dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step.step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    peak = torch.cuda.max_memory_allocated()
    free_b, total_b = torch.cuda.mem_get_info(dev)
    reserved = torch.cuda.memory_reserved(dev)
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]

    # Per-kernel times: a separate traced pass (HIP event pairs around every launch).
    n_tr = max(1, args.trace_steps)
    H.trace_enable(max(64, 200 * n_tr))
    H.trace_reset()
    for _ in range(n_tr):
        step.step()
    torch.cuda.synchronize()
    tr = H.trace_collect()
    H.trace_enable(0)

    ms = (t1 - t0) * 1e3 / args.steps
    n_valid = inp.n_valid
    tok_s = n_valid / (ms / 1e3)
    peak_flops = PEAK_F32 if cfg.dtype == "f32" else PEAK_BF16
    # Algorithmic work credited: valid tokens only (padding and ignored rows are processed, not
    # credited), 8 V d FLOP each (fwd 2, bwd 6; 6 V d for a dh-only backward: the 4-bit head, or
    # --no-dw).
    work = (8 if want_dw else 6) * n_valid * cfg.V * cfg.d
    if args.fp8:
        # The logit GEMMs (forward 2 V d, recompute 2 V d) run at the fp8 rate, dh and dW (4 V d;
        # dh alone 2 V d) at the bf16 rate: the step's peak is the harmonic mix.
        g_flop = 4.0 if want_dw else 2.0
        peak_flops = (4.0 + g_flop) / (4.0 / PEAK_FP8 + g_flop / PEAK_BF16)
    mfma_frac = work / (ms / 1e3) / peak_flops

    # Dominant kernel: the kind with the most traced time; achieved = its algorithmic FLOPs per
    # launch over its average launch time (HIP events on the library's launch stream).
    from lm_head_cross_amd import prof_summary
    kinds = {k: v for k, v in tr.items() if v[0] > 0}
    dom = max(kinds, key=lambda k: kinds[k][1])
    n_l, tot_ms, fl = kinds[dom]
    avg_ms = tot_ms / n_l
    achieved = (fl / n_l) / (avg_ms / 1e3)
    dom_peak = peak_flops
    if args.fp8:   # the dominant kernel's own mix: fp8 logits, bf16 gradient products
        dom_peak = {"fwd": PEAK_FP8, "coeff": PEAK_FP8, "dhdw": PEAK_BF16,
                    "bwd": 6.0 / (2.0 / PEAK_FP8 + 4.0 / PEAK_BF16)}.get(dom, PEAK_BF16)
    traffic = None
    # The counters were taken on the ORPO step of this workload (dh only: its own file), exact.
    tfile = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                         f"{cfg.name}{'-dh-only' if args.no_dw else ''}_traffic.txt")
    t = prof_summary.read_traffic(tfile)
    if (t is not None and t[0] == dom and not args.fp8 and args.skip_eps == 0
            and args.objective == "orpo" and not args.q4_stage):
        traffic = round(t[1])
    per_kernel = {k: {"launches_per_step": v[0] / n_tr, "avg_ms": v[1] / max(v[0], 1),
                      "ms_per_step": v[1] / n_tr,
                      "tflops": (v[2] / (v[1] / 1e3) / 1e12) if v[1] > 0 and v[2] > 0 else None}
                  for k, v in kinds.items()}

    # Coefficient filter: its distance from the exact backward on this batch (measured once, after
    # the timed region and after the peak-memory reading).
    fidelity = None
    if args.skip_eps > 0:
        ex = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, scales=sc, biases=bi,
                        want_dW=want_dw, scope=cfg.scope, objective=args.objective, obj=obj)
        ex.step()
        torch.cuda.synchronize()
        rel = lambda a, b: float(torch.linalg.norm(a - b) / torch.linalg.norm(b))
        fidelity = {"dh_rel": rel(step.dh, ex.dh),
                    "dW_rel": None if step.dW is None else rel(step.dW, ex.dW),
                    "against": "the exact backward on the same batch (HIP, skip_eps = 0)"}
        del ex

    # The FP8 head: its distance from the exact head on this batch.
    fp8_fid = None
    if args.fp8:
        ex = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, want_dW=want_dw,
                        scope=cfg.scope, objective=args.objective, obj=obj)
        ex.step()
        torch.cuda.synchronize()
        rel = lambda a, b: float(torch.linalg.norm(a.float() - b.float()) / torch.linalg.norm(b.float()))
        m = labels != synth.IGNORE_INDEX
        fp8_fid = {"logp_rel": rel(step.logp[m], ex.logp[m]), "lse_rel": rel(step.lse, ex.lse),
                   "loss_rel": abs(float(step.out[0]) - float(ex.out[0])) / abs(float(ex.out[0])),
                   "dh_rel": rel(step.dh, ex.dh),
                   "dW_rel": None if step.dW is None else rel(step.dW, ex.dW),
                   "against": "the exact bf16 head on the same batch (HIP)"}
        del ex

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline:
        # About 4e12 FLOP of float64 oracle work (10-30 s on the host), rounded to 128 tokens.
        auto = int(4e12 / (6 * cfg.V * cfg.d)) // 128 * 128
        rows = args.cpu_rows or max(128, min(cfg.M, auto))
        print(f"[bench] oracle cpu baseline on {rows} rows", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, rows, args.objective, want_dw)

    line = {
        "metric": "ORPO head fwd+bwd tokens/s (d=2560,V=262144); % bf16 MFMA peak; peak GB",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "median_ms_per_step": round(float(np.median(step_ms)), 3),
        "mean_ms_per_step_events": round(float(np.mean(step_ms)), 3),
        "median_tokens_per_s": round(n_valid / (float(np.median(step_ms)) / 1e3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else ("fp8e4m3 logits, bf16 gradients" if args.fp8 else "bf16"),
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "M": cfg.M, "valid_tokens": n_valid, "d": cfg.d, "V": cfg.V,
            "pairs": cfg.pairs, "softcap": cfg.softcap, "lambda": cfg.lam, "nll_scope": cfg.scope,
            "objective": args.objective, "skip_eps": args.skip_eps, "fp8": args.fp8,
            "dW": want_dw,
            "w_format": "q4g64" if cfg.q4 else ("f32" if cfg.dtype == "f32" else "bf16"),
            "q4_stage": args.q4_stage,
            "parallelism": "single GPU",
        },
        "mfma_frac_of_peak": round(mfma_frac, 4),
        "algorithmic_tflops": round(work / (ms / 1e3) / 1e12, 1),
        "peak_hbm_gb": round(peak / 1e9, 3),
        "hip_mem_used_gb": round((total_b - free_b) / 1e9, 3),
        "torch_reserved_gb": round(reserved / 1e9, 3),
        "mem_note": "peak_hbm_gb = torch.cuda.max_memory_allocated over the timed steps (inputs, "
                    "outputs and workspaces all allocated through torch); hip_mem_used_gb = "
                    "hipMemGetInfo's total - free after them (torch's reserved pool plus the "
                    "runtime's own allocations)",
        "kernels_traced_steps": n_tr,
        "inputs_gb": round(inputs_bytes / 1e9, 3),
        "workspace_gb": round(step.workspace_bytes() / 1e9, 3),
        "loss": loss0,
        "kernels": per_kernel,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved / 1e12, 1),
            "peak": round(dom_peak / 1e12, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / dom_peak, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
        },
        "cpu_baseline": cpu,
    }
    if args.fp8:
        line["fp8_fidelity"] = fp8_fid
        line["peak_note"] = ("fp8 logit GEMMs at 5.0 PFLOP/s, bf16 gradient GEMMs at 2.5: the step's "
                             "peak is their harmonic mix")
    if args.skip_eps > 0:
        line["skip_fidelity"] = fidelity
        line["roofline"]["work"] = "the exact method's FLOP (blocks the filter skips included)"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
