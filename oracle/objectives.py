"""Float64 CPU oracle for the sibling objectives that reuse the head's forward and backward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run anything in this package. It shares no code with the HIP path.

Every objective here consumes the head's per-token log-probs and produces a scalar loss and the
per-token cotangent g = dL/dlogp that the head's backward turns into dh and dW. The definitions are
the pages' own, written out in float64 (reductions with math.fsum), with the chain rule term by
term. Parity pins: `tests/test_oracle_objectives.py`.
"""
from __future__ import annotations

import math

import numpy as np

from .orpo_oracle import IGNORE_INDEX, OracleError, _sigmoid, _softplus


def span_stats(logp, labels, seg_offsets, ignore_index: int = IGNORE_INDEX):
    """Per span s = [off[s], off[s+1]): (sum of logp over its valid tokens, their count). A span
    without a valid token is a data error."""
    logp = np.asarray(logp, dtype=np.float64)
    labels = np.asarray(labels).astype(np.int64)
    off = np.asarray(seg_offsets).astype(np.int64)
    if off.ndim != 1 or off.shape[0] < 2:
        raise OracleError("need at least one span")
    if off[0] < 0 or off[-1] > logp.shape[0] or np.any(np.diff(off) < 0):
        raise OracleError("segment offsets must be monotone within [0, M]")
    ns = off.shape[0] - 1
    sums = np.zeros(ns)
    n = np.zeros(ns, dtype=np.int64)
    for s in range(ns):
        ts = [t for t in range(off[s], off[s + 1]) if labels[t] != ignore_index]
        if not ts:
            raise OracleError(f"span {s} has no valid token")
        sums[s] = math.fsum(logp[t] for t in ts)
        n[s] = len(ts)
    return sums, n


def span_cotangent(dL_dspan, labels, seg_offsets, per_token_scale=None,
                   ignore_index: int = IGNORE_INDEX):
    """g_t = dL/dspan_s * scale_s for a valid token t of span s (scale 1 for a sum, 1/n for a
    mean), else 0."""
    labels = np.asarray(labels).astype(np.int64)
    off = np.asarray(seg_offsets).astype(np.int64)
    g = np.zeros(labels.shape[0])
    for s in range(off.shape[0] - 1):
        sc = 1.0 if per_token_scale is None else per_token_scale[s]
        for t in range(off[s], off[s + 1]):
            if labels[t] != ignore_index:
                g[t] = dL_dspan[s] * sc
    return g


# --------------------------------------------------------------------------------------------
# SimPO
# --------------------------------------------------------------------------------------------
def simpo_epilogue(lw, lr, beta: float, gamma: float):
    """SimPO from the length-normalised branch means (Training — design, §8.3 "Objective variants
    and data"): L_p = softplus(-beta ((lw - lr) - gamma)), loss = mean over pairs. Metrics:
    accuracy = mean 1[lw > lr], margin = mean (lw - lr). dL/dlw = -beta (1 - sigma(u)) / P with
    u = beta ((lw - lr) - gamma), dL/dlr = -dL/dlw."""
    lw = np.asarray(lw, dtype=np.float64)
    lr = np.asarray(lr, dtype=np.float64)
    P = lw.shape[0]
    lp = np.zeros(P)
    dw = np.zeros(P)
    for p in range(P):
        u = beta * ((lw[p] - lr[p]) - gamma)
        lp[p] = _softplus(-u)
        dw[p] = -beta * _sigmoid(-u) / P
    return {"loss": math.fsum(lp) / P, "accuracy": float(np.mean(lw > lr)),
            "margin": math.fsum(lw - lr) / P, "dL_dw": dw, "dL_dr": -dw}


# --------------------------------------------------------------------------------------------
# DPO
# --------------------------------------------------------------------------------------------
def dpo_epilogue(sw, sr, ref_w, ref_r, beta: float):
    """DPO from per-sequence log-prob sums (the sibling project's design, "Stage P1 — DPO":
    seq_logprob is the sum of log-probs over the completion's positions; with Delta = beta
    [(s_w - ref_w) - (s_r - ref_r)] the loss is -log sigma(Delta), only the policy terms carry
    gradient; reference sums are cached inputs). loss = mean over pairs. Metrics: accuracy = mean
    1[Delta > 0], margin = mean Delta (the reward margin). dL/ds_w = -beta (1 - sigma(Delta)) / P,
    dL/ds_r = -dL/ds_w."""
    sw, sr, ref_w, ref_r = (np.asarray(x, dtype=np.float64) for x in (sw, sr, ref_w, ref_r))
    P = sw.shape[0]
    lp = np.zeros(P)
    delta = np.zeros(P)
    dw = np.zeros(P)
    for p in range(P):
        delta[p] = beta * ((sw[p] - ref_w[p]) - (sr[p] - ref_r[p]))
        lp[p] = _softplus(-delta[p])
        dw[p] = -beta * _sigmoid(-delta[p]) / P
    return {"loss": math.fsum(lp) / P, "accuracy": float(np.mean(delta > 0)),
            "margin": math.fsum(delta) / P, "delta": delta, "dL_dw": dw, "dL_dr": -dw}


# --------------------------------------------------------------------------------------------
# IPO and hinge (SLiC)
# --------------------------------------------------------------------------------------------
# The pages name both as siblings on the shared log-prob engine (Training — design, §8.3
# "Objective variants and data") and give no formula. Reading: each is the published loss on the
# log-ratio margin h = (v_w - ref_w) - (v_r - ref_r), with reference values optional (zero gives
# the reference-free form that SimPO uses). IPO takes SimPO's length-normalised means (the
# squared loss is scale-sensitive, and length normalisation keeps its target margin meaningful
# across lengths); hinge takes DPO's per-sequence sums, as SLiC's calibration loss does.
def ipo_epilogue(lw, lr, ref_w, ref_r, beta: float):
    """IPO: L_p = (h_p - 1 / (2 beta))^2 with h_p = (lw - ref_w) - (lr - ref_r) on the branch
    means; loss = mean over pairs (beta > 0). Metrics: accuracy = mean 1[h > 0], margin = mean h.
    dL/dlw = 2 (h - 1 / (2 beta)) / P, dL/dlr = -dL/dlw."""
    if not beta > 0:
        raise OracleError("IPO needs beta > 0")
    lw, lr, ref_w, ref_r = (np.asarray(x, dtype=np.float64) for x in (lw, lr, ref_w, ref_r))
    P = lw.shape[0]
    target = 1.0 / (2.0 * beta)
    hm = np.zeros(P)
    lp = np.zeros(P)
    dw = np.zeros(P)
    for p in range(P):
        hm[p] = (lw[p] - ref_w[p]) - (lr[p] - ref_r[p])
        lp[p] = (hm[p] - target) ** 2
        dw[p] = 2.0 * (hm[p] - target) / P
    return {"loss": math.fsum(lp) / P, "accuracy": float(np.mean(hm > 0)),
            "margin": math.fsum(hm) / P, "h": hm, "dL_dw": dw, "dL_dr": -dw}


def hinge_epilogue(sw, sr, ref_w, ref_r, beta: float):
    """Hinge / SLiC: L_p = max(0, 1 - beta h_p) with h_p = (sw - ref_w) - (sr - ref_r) on the
    per-sequence sums; loss = mean over pairs. Metrics: accuracy = mean 1[h > 0], margin = mean h.
    dL/dsw = -beta / P where 1 - beta h > 0, else 0 (the flat side's zero at the kink itself),
    dL/dsr = -dL/dsw."""
    sw, sr, ref_w, ref_r = (np.asarray(x, dtype=np.float64) for x in (sw, sr, ref_w, ref_r))
    P = sw.shape[0]
    hm = np.zeros(P)
    lp = np.zeros(P)
    dw = np.zeros(P)
    for p in range(P):
        hm[p] = (sw[p] - ref_w[p]) - (sr[p] - ref_r[p])
        u = 1.0 - beta * hm[p]
        lp[p] = u if u > 0 else 0.0
        dw[p] = -beta / P if u > 0 else 0.0
    return {"loss": math.fsum(lp) / P, "accuracy": float(np.mean(hm > 0)),
            "margin": math.fsum(hm) / P, "h": hm, "dL_dw": dw, "dL_dr": -dw}


MEAN_KINDS = ("simpo", "ipo")     # length-normalised branch values; the others use sums


def pairwise_cotangent(kind: str, ep, n, labels, seg_offsets, ignore_index: int = IGNORE_INDEX):
    """Per-token g for the pairwise objectives (spans: chosen 2p, rejected 2p+1): a mean (SimPO,
    IPO) spreads dL/dell_b as 1/n_b per token, a sum (DPO, hinge) passes it unchanged."""
    P = len(ep["dL_dw"])
    dl = np.zeros(2 * P)
    dl[0::2], dl[1::2] = ep["dL_dw"], ep["dL_dr"]
    scale = 1.0 / np.asarray(n, dtype=np.float64) if kind in MEAN_KINDS else None
    return span_cotangent(dl, labels, seg_offsets, scale, ignore_index)


# --------------------------------------------------------------------------------------------
# GRPO
# --------------------------------------------------------------------------------------------
def grpo_loss(logp, old_logp, ref_logp, labels, seg_offsets, adv, clip_eps: float, beta: float,
              ignore_index: int = IGNORE_INDEX):
    """GRPO's clipped policy-gradient loss with the k3 KL leash (the sibling project's design,
    "Stage P3 — GRPO", (d)): per completion token t of completion s, rho = exp(logp - old),
    l_t = -min(rho A_s, clip(rho, 1 - eps, 1 + eps) A_s) + beta k3_t with
    k3_t = exp(ref - logp) - (ref - logp) - 1, masked to the completion's valid tokens. Reduction
    (the pages leave it open; GRPO's own form): mean over each completion's tokens, then mean over
    completions. Gradient: d l_t / d logp_t = -A rho where the unclipped term is the minimum (ties
    included), 0 where the clipped one is (it is then constant in rho), plus beta (1 - exp(ref -
    logp)). Returns loss, pg (the policy-gradient part), kl (mean k3), clip_frac (share of valid
    tokens where the clipped term is the strict minimum) and g."""
    logp, old_logp, ref_logp = (np.asarray(x, dtype=np.float64) for x in (logp, old_logp, ref_logp))
    labels = np.asarray(labels).astype(np.int64)
    off = np.asarray(seg_offsets).astype(np.int64)
    adv = np.asarray(adv, dtype=np.float64)
    S = off.shape[0] - 1
    if adv.shape[0] != S:
        raise OracleError("one advantage per completion")
    g = np.zeros(logp.shape[0])
    pg_s, kl_s = np.zeros(S), np.zeros(S)
    clipped = 0
    total = 0
    for s in range(S):
        ts = [t for t in range(off[s], off[s + 1]) if labels[t] != ignore_index]
        if not ts:
            raise OracleError(f"completion {s} has no valid token")
        pg_t, kl_t = [], []
        for t in ts:
            rho = math.exp(logp[t] - old_logp[t])
            a = adv[s]
            unclipped = rho * a
            clipped_v = min(max(rho, 1.0 - clip_eps), 1.0 + clip_eps) * a
            pg_t.append(-min(unclipped, clipped_v))
            d = ref_logp[t] - logp[t]
            kl_t.append(math.exp(d) - d - 1.0)
            dpg = -a * rho if unclipped <= clipped_v else 0.0
            clipped += unclipped > clipped_v
            g[t] = (dpg + beta * (1.0 - math.exp(d))) / (len(ts) * S)
        total += len(ts)
        pg_s[s] = math.fsum(pg_t) / len(ts)
        kl_s[s] = math.fsum(kl_t) / len(ts)
    pg = math.fsum(pg_s) / S
    kl = math.fsum(kl_s) / S
    return {"loss": pg + beta * kl, "pg": pg, "kl": kl, "clip_frac": clipped / total, "g": g}


def group_advantages(rewards, group: int, eps: float = 1e-6):
    """Group-relative advantage (same section, (c)): A_i = (r_i - mean(r_group)) / (std(r_group) +
    eps) over consecutive groups of `group` completions (population std)."""
    r = np.asarray(rewards, dtype=np.float64).reshape(-1, group)
    return ((r - r.mean(axis=1, keepdims=True)) / (r.std(axis=1, keepdims=True) + eps)).reshape(-1)
