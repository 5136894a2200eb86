"""Helpers shared by the GPU parity tests: run the HIP head through the C ABI and compare with the
oracle. The tolerance gates: logp and lse within 1e-3 relative (norm-wise), each branch mean and the
loss terms within 1e-3 relative, dh and dW within 1e-2 relative Frobenius error."""
from __future__ import annotations

import sys

import numpy as np
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from oracle import orpo_oracle as orc

TOL_LOGP = 1e-3
TOL_SCALAR = 1e-3
TOL_GRAD = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU test needs a GPU"
    return torch.device("cuda:0")


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def srel(a, b) -> float:
    return abs(float(a) - float(b)) / max(abs(float(b)), 1e-300)


def gpu_weights(inp: synth.HeadInputs, d):
    if inp.cfg.q4:
        w = torch.from_numpy(inp.wq.view(np.int32)).to(d)
        return w, inp.scales.to(d), inp.biases.to(d)
    return inp.w.to(d), None, None


def oracle_weight(inp: synth.HeadInputs) -> np.ndarray:
    if inp.cfg.q4:
        return orc.dequant_q4(inp.wq, synth.bf16_bits(inp.scales), synth.bf16_bits(inp.biases), 64)
    return inp.w.float().numpy().astype(np.float64)


def run_gpu(inp: synth.HeadInputs, want_dW=None, g_override=None):
    """fwd -> loss -> bwd on the GPU; returns numpy results (and the GPU tensors under 't')."""
    d = dev()
    cfg = inp.cfg
    if want_dW is None:
        want_dW = not cfg.q4
    h = inp.h.to(d)
    w, sc, bi = gpu_weights(inp, d)
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    logp, lse, fws = H.head_fwd(h, w, labels, cfg.softcap, scales=sc, biases=bi, return_ws=True)
    out, g, lws = H.orpo_loss(logp, labels, off, cfg.V, cfg.lam, return_ws=True, scope=cfg.scope)
    gg = g if g_override is None else g_override.to(d)
    dh, dW = H.head_bwd(h, w, labels, lse, gg, cfg.softcap, want_dW=want_dW, scales=sc, biases=bi)
    torch.cuda.synchronize()
    P = cfg.pairs
    o = out.cpu().numpy()
    return {
        "logp": logp.cpu().numpy(), "lse": lse.cpu().numpy(), "g": g.cpu().numpy(),
        "loss": o[0], "nll": o[1], "or": o[2], "accuracy": o[3], "margin": o[4],
        "lw": o[5:5 + P], "lr": o[5 + P:5 + 2 * P],
        "pm": o[5 + 2 * P:5 + 3 * P] if cfg.scope == "full" else None,
        "dh": dh.cpu().numpy(), "dW": None if dW is None else dW.cpu().numpy(),
        "fwd_status": H.read_status(fws), "loss_status": H.read_status(lws),
    }


def run_oracle(inp: synth.HeadInputs, want_dW=None):
    if want_dW is None:
        want_dW = not inp.cfg.q4
    W = oracle_weight(inp)
    h = inp.h.float().numpy().astype(np.float64)
    step = orc.head_step_full if inp.cfg.scope == "full" else orc.head_step
    return step(h, W, inp.labels, inp.seg_offsets, inp.cfg.softcap, inp.cfg.lam, want_dW=want_dW)


def assert_parity(gpu, ora, label=""):
    errs = {
        "logp": rel(gpu["logp"], ora["logp"]),
        "lse": rel(gpu["lse"], ora["lse"]),
        "lw": rel(gpu["lw"], ora["lw"]),
        "lr": rel(gpu["lr"], ora["lr"]),
        "loss": srel(gpu["loss"], ora["loss"]),
        "nll": srel(gpu["nll"], ora["nll"]),
        "or": srel(gpu["or"], ora["or"]),
        "margin": abs(gpu["margin"] - ora["margin"]) / max(1.0, abs(ora["margin"])),
        "g": rel(gpu["g"], ora["g"]),
        "dh": rel(gpu["dh"], ora["dh"]),
    }
    if ora.get("dW") is not None and gpu.get("dW") is not None:
        errs["dW"] = rel(gpu["dW"], ora["dW"])
    if gpu.get("pm") is not None:
        errs["pm"] = rel(gpu["pm"], ora["pm"])
    say(f"[parity {label}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k in ("logp", "lse", "lw", "lr", "loss", "nll", "g", "pm"):
        if k in errs:
            assert errs[k] <= TOL_SCALAR, (k, errs[k])
    # The odds-ratio term and the margin are gated by what the 1e-3 branch-mean gate implies for
    # them: |d log_odds| <= F(lw)|d lw| + F(lr)|d lr| with F(l) = 1/(1 - e^l) and |d softplus(-z)/dz|
    # = 1 - sigmoid(z), so a branch-mean error of TOL * |ell| allows these absolute errors.
    lw, lr = np.asarray(ora["lw"]), np.asarray(ora["lr"])
    F = lambda x: 1.0 / -np.expm1(np.minimum(x, -1e-12))
    dz = TOL_SCALAR * (F(lw) * np.abs(lw) + F(lr) * np.abs(lr))
    one_minus_sig = 1.0 / (1.0 + np.exp(np.asarray(ora["log_odds"])))
    assert abs(gpu["or"] - ora["or"]) <= np.mean(one_minus_sig * dz) + 1e-12, "or"
    assert abs(gpu["margin"] - ora["margin"]) <= np.mean(dz) + 1e-12, "margin"
    for k in ("dh", "dW"):
        if k in errs:
            assert errs[k] <= TOL_GRAD, (k, errs[k])
    # Per-branch means individually, not only norm-wise.
    for a, b in zip(np.concatenate([gpu["lw"], gpu["lr"]]), np.concatenate([ora["lw"], ora["lr"]])):
        assert srel(a, b) <= TOL_SCALAR
    assert gpu["accuracy"] == ora["accuracy"] or abs(gpu["lw"] - gpu["lr"]).min() < 1e-4
    return errs
