"""Float64 CPU oracle for the flash-CCE ORPO head.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run anything in this package. It shares no code with the HIP path:
it never imports `lm_head_cross_amd`, and it takes plain NumPy arrays (bf16 values arrive already
widened to float32, which is exact; 4-bit weights arrive as their packed words and bf16 bit
patterns).

Everything here is the plain definition, written out in float64: full logit rows per row block
(never an online softmax), a library log-sum-exp over the full row, `math.fsum` for branch sums,
and the chain rule written term by term for the gradients. The flash-CCE head reaches the same
values up to floating-point reassociation (the pages' "Training — design", §2 "Oracles and the
parity ladder": the kernel's difference from a full-logits reference is reassociation, not error).

Parity pins: every function below is pinned by `tests/test_oracle.py` to closed forms, worked
values, invariances, finite differences and brute force; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

IGNORE_INDEX = -100
# Clamp on 1 - e^x inside log1mexp. The pages give only "a small eps"; 1e-12 binds only when
# the branch mean log-prob is above -1e-12 (a branch the model already predicts with certainty).
LOG1MEXP_EPS = 1e-12


class OracleError(ValueError):
    pass


# --------------------------------------------------------------------------------------------
# Inputs
# --------------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """A bf16 bit pattern is the top half of the float32 with the same value."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dequant_q4(wq, scale_bits, bias_bits, group_size: int = 64) -> np.ndarray:
    """Affine 4-bit dequantisation, w = scale * q + bias per group of `group_size` along d.

    Training — design (older revision), §"Memory & speed optimization", the flash-CCE Metal kernel
    note: the classifier is the quantised head, dequantised affinely in-kernel; Steel flash-CCE —
    handoff, "Gotchas" item 4: a 32-bit word holds 32/bits codes. Code j of a row sits in word
    j // 8 at bits [4*(j % 8), 4*(j % 8) + 4).
    """
    wq = np.asarray(wq, dtype=np.uint32)
    V, n_words = wq.shape
    d = n_words * 8
    if d % group_size:
        raise OracleError("d must be a multiple of the group size")
    q = np.empty((V, d), dtype=np.float64)
    for i in range(8):
        q[:, i::8] = ((wq >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.float64)
    s = bf16_bits_to_f64(scale_bits)
    b = bf16_bits_to_f64(bias_bits)
    if s.shape != (V, d // group_size) or b.shape != s.shape:
        raise OracleError("scale/bias shape must be [V, d / group_size]")
    grp = np.arange(d) // group_size
    return s[:, grp] * q + b[:, grp]


# --------------------------------------------------------------------------------------------
# Forward: raw logits, softcap, log-sum-exp, per-token log-prob
# --------------------------------------------------------------------------------------------
def softcap(raw: np.ndarray, cap: float) -> np.ndarray:
    """z = cap * tanh(raw / cap); cap <= 0 means no softcap.

    Training — design (older revision), "Implementation spec — fused linear-CE log-prob head":
    Gemma's final-logit softcapping; Steel flash-CCE — handoff, Glossary D "Softcap".
    """
    if cap > 0:
        return cap * np.tanh(raw / cap)
    return raw


def softcap_slope(raw: np.ndarray, cap: float) -> np.ndarray:
    """dz/draw = sech^2(raw / cap) = 1 - tanh^2(raw / cap) (1 without a softcap). Same passages."""
    if cap > 0:
        t = np.tanh(raw / cap)
        return 1.0 - t * t
    return np.ones_like(raw)


def _check_labels(labels: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    valid = labels != ignore_index
    if np.any(valid & ((labels < 0) | (labels >= V))):
        raise OracleError("label outside [0, V) that is not the ignore index")
    return valid


def forward(h, W, labels, cap: float = 0.0, ignore_index: int = IGNORE_INDEX, rows: int = 64):
    """Per-token log-prob and log-sum-exp from full logit rows.

    logp_t = z_t[y_t] - logsumexp_v z_tv with z = softcap(h_t . W_v) (Training — design, §5.1
    "The head": CE and the target log-prob are the same quantity). Ignored tokens get logp = 0;
    lse is returned for every row. Returns (logp [M], lse [M]) in float64.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels).astype(np.int64)
    M, V = h.shape[0], W.shape[0]
    if h.ndim != 2 or W.ndim != 2 or h.shape[1] != W.shape[1] or labels.shape != (M,):
        raise OracleError("shape mismatch")
    if V < 1:
        raise OracleError("V must be >= 1")
    valid = _check_labels(labels, V, ignore_index)
    logp = np.zeros(M)
    lse = np.zeros(M)
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        z = softcap(h[r0:r1] @ W.T, cap)
        zmax = z.max(axis=1)
        lse[r0:r1] = zmax + np.log(np.exp(z - zmax[:, None]).sum(axis=1))
        for i in range(r1 - r0):
            t = r0 + i
            if valid[t]:
                logp[t] = z[i, labels[t]] - lse[t]
    return logp, lse


# --------------------------------------------------------------------------------------------
# Segmented per-branch mean
# --------------------------------------------------------------------------------------------
def branch_means(logp, labels, seg_offsets, ignore_index: int = IGNORE_INDEX):
    """ell_b = (sum of logp over the valid tokens of branch b) / (their count).

    Training — design, §1 "The objective": ell is the length-normalised mean over response tokens
    ("Mean, not sum"). Branch b covers positions [off[b], off[b+1]); branch 2p is the chosen and
    2p+1 the rejected response of pair p. Returns (ell [2P], n [2P]).
    """
    logp = np.asarray(logp, dtype=np.float64)
    labels = np.asarray(labels).astype(np.int64)
    off = np.asarray(seg_offsets).astype(np.int64)
    M = logp.shape[0]
    nb = off.shape[0] - 1
    if nb < 2 or nb % 2:
        raise OracleError("need an even number (>= 2) of branches")
    if off[0] < 0 or off[-1] > M or np.any(np.diff(off) < 0):
        raise OracleError("segment offsets must be monotone within [0, M]")
    ell = np.zeros(nb)
    n = np.zeros(nb, dtype=np.int64)
    for b in range(nb):
        ts = [t for t in range(off[b], off[b + 1]) if labels[t] != ignore_index]
        if not ts:
            raise OracleError(f"branch {b} has no valid token")
        n[b] = len(ts)
        ell[b] = math.fsum(logp[t] for t in ts) / len(ts)
    return ell, n


# --------------------------------------------------------------------------------------------
# Scalar ORPO epilogue
# --------------------------------------------------------------------------------------------
def log1mexp(x: float) -> tuple[float, bool]:
    """log(1 - e^x) for x <= 0, with 1 - e^x clamped below at LOG1MEXP_EPS.

    Training — design, §1 "The objective", implementation note: log1mexp is log(clip(1 - exp(x),
    eps, 1)). Evaluated with the two-branch form (log(-expm1 x) above -ln 2, log1p(-e^x) below) so
    that it stays accurate at both ends. Returns (value, clamped).
    """
    v = -math.expm1(x)
    if not v >= LOG1MEXP_EPS:          # also catches NaN
        return math.log(LOG1MEXP_EPS), True
    if x > -math.log(2.0):
        return math.log(v), False
    return math.log1p(-math.exp(x)), False


def _softplus(x: float) -> float:
    return max(x, 0.0) + math.log1p(math.exp(-abs(x)))


def _sigmoid(x: float) -> float:
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def orpo_epilogue(ell, lam: float):
    """ORPO loss, metrics and dL/d(ell) from the branch means.

    Training — design, §1 "The objective": L = L_NLL(y_w) + lam * L_OR with
    L_OR = -log sigmoid(log_odds), log_odds = (lw - lr) - (log1mexp(lw) - log1mexp(lr)); the
    response-scope NLL is -lw. Batch reduction (older revision, "File-by-file changes", orpoLoss):
    nll = mean(-lw), or = mean(softplus(-log_odds)), loss = nll + lam * or. Metrics (orpoMetrics):
    accuracy = mean 1[lw > lr]; margin = mean log_odds (older revision, the IFEval experiment:
    "val margin" is the mean chosen-minus-rejected log-odds).

    Gradient: d/d ell [ell - log1mexp(ell)] = 1/(1 - e^ell), the "1/(1-P)" factor of the OR
    gradient (Training — design, §4 "Recommended defaults and regularization geometry", schedule
    row; older revision, the implementer notes that also call log1mexp the NaN hazard to clamp or
    split in two branches); it is 1 where the clamp binds (the clamp has zero slope). Returns a dict with loss, nll, or, accuracy, margin, lw [P], lr [P], log_odds [P] and
    dL_dell [2P].
    """
    ell = np.asarray(ell, dtype=np.float64)
    if ell.ndim != 1 or ell.shape[0] < 2 or ell.shape[0] % 2:
        raise OracleError("ell must hold 2P branch means")
    P = ell.shape[0] // 2
    lw, lr = ell[0::2], ell[1::2]
    log_odds = np.zeros(P)
    lor = np.zeros(P)
    dldw = np.zeros(P)
    dldr = np.zeros(P)
    for p in range(P):
        a, ca = log1mexp(lw[p])
        b, cb = log1mexp(lr[p])
        z = (lw[p] - lr[p]) - (a - b)
        log_odds[p] = z
        lor[p] = _softplus(-z)
        one_minus_sig = _sigmoid(-z)
        f_w = 1.0 if ca else -1.0 / math.expm1(lw[p])
        f_r = 1.0 if cb else -1.0 / math.expm1(lr[p])
        dldw[p] = (-1.0 - lam * one_minus_sig * f_w) / P
        dldr[p] = (lam * one_minus_sig * f_r) / P
    nll = math.fsum(-lw) / P
    orv = math.fsum(lor) / P
    dl = np.zeros(2 * P)
    dl[0::2] = dldw
    dl[1::2] = dldr
    return {
        "loss": nll + lam * orv,
        "nll": nll,
        "or": orv,
        "accuracy": float(np.mean(lw > lr)),
        "margin": math.fsum(log_odds) / P,
        "lw": lw.copy(),
        "lr": lr.copy(),
        "log_odds": log_odds,
        "dL_dell": dl,
    }


def token_cotangent(dL_dell, n, labels, seg_offsets, ignore_index: int = IGNORE_INDEX):
    """g_t = dL/dlogp_t = (dL/d ell_b) / n_b for a valid token t of branch b, else 0 (chain rule
    through the branch mean)."""
    labels = np.asarray(labels).astype(np.int64)
    off = np.asarray(seg_offsets).astype(np.int64)
    g = np.zeros(labels.shape[0])
    for b in range(off.shape[0] - 1):
        for t in range(off[b], off[b + 1]):
            if labels[t] != ignore_index:
                g[t] = dL_dell[b] / n[b]
    return g


# --------------------------------------------------------------------------------------------
# Full-scope NLL (prompt + chosen response)
# --------------------------------------------------------------------------------------------
def span_means_full(logp, labels, seg_offsets, ignore_index: int = IGNORE_INDEX):
    """Per pair p: the spans [prompt, chosen, rejected] = segments 3p, 3p+1, 3p+2 of seg_offsets
    (3P+1 entries). Returns (mean [3P], n [3P]); a prompt span may hold no valid token (its mean is
    then reported as 0 and has no weight), the two responses may not."""
    logp = np.asarray(logp, dtype=np.float64)
    labels = np.asarray(labels).astype(np.int64)
    off = np.asarray(seg_offsets).astype(np.int64)
    M = logp.shape[0]
    ns = off.shape[0] - 1
    if ns < 3 or ns % 3:
        raise OracleError("need 3P (>= 3) spans: prompt, chosen, rejected per pair")
    if off[0] < 0 or off[-1] > M or np.any(np.diff(off) < 0):
        raise OracleError("segment offsets must be monotone within [0, M]")
    mean = np.zeros(ns)
    n = np.zeros(ns, dtype=np.int64)
    for b in range(ns):
        ts = [t for t in range(off[b], off[b + 1]) if labels[t] != ignore_index]
        if not ts:
            if b % 3 == 0:
                continue
            raise OracleError(f"response span {b} has no valid token")
        n[b] = len(ts)
        mean[b] = math.fsum(logp[t] for t in ts) / len(ts)
    return mean, n


def orpo_epilogue_full(mean, n, lam: float):
    """ORPO with the full-scope NLL, from the span means of span_means_full.

    Training — design, §1 "The objective", the sft_scope `full` option: the chosen sequence's NLL
    is the token mean over its supervised prompt positions and its response, combined from the two
    span means as NLL_full = -((P-1) pm + M lw) / ((P-1) + M), where P-1 is the number of
    supervised prompt positions (here n_q, the prompt span's valid tokens), M the response's (n_w)
    and pm the prompt span's mean. The odds-ratio term keeps the response-only means lw, lr in both
    scopes, and lam weights only it. Batch reduction as for the response scope: mean over pairs.

    Gradient: dNLL_full/dpm = -n_q / (n_q + n_w), dNLL_full/dlw = -n_w / (n_q + n_w), plus the OR
    term's d/dlw and d/dlr exactly as in orpo_epilogue. Returns the dict of orpo_epilogue with
    `nll` the full-scope value, plus pm [P], n_q [P] and dL_dmean [3P].
    """
    mean = np.asarray(mean, dtype=np.float64)
    n = np.asarray(n).astype(np.int64)
    if mean.ndim != 1 or mean.shape[0] < 3 or mean.shape[0] % 3:
        raise OracleError("need 3P span means")
    P = mean.shape[0] // 3
    ell = np.zeros(2 * P)
    ell[0::2] = mean[1::3]
    ell[1::2] = mean[2::3]
    ep = orpo_epilogue(ell, lam)       # OR term, metrics, and its d/dlw, d/dlr
    pm, n_q, n_w = mean[0::3], n[0::3], n[1::3]
    nll_p = np.zeros(P)
    dl = np.zeros(3 * P)
    for p in range(P):
        tot = n_q[p] + n_w[p]
        nll_p[p] = -(n_q[p] * pm[p] + n_w[p] * ep["lw"][p]) / tot
        dl[3 * p] = -(n_q[p] / tot) / P
        # orpo_epilogue's chosen term is (-1 - lam (1 - sigma) f_w) / P; swap its -1 for -n_w / tot
        dl[3 * p + 1] = ep["dL_dell"][2 * p] + (1.0 - n_w[p] / tot) / P
        dl[3 * p + 2] = ep["dL_dell"][2 * p + 1]
    nll = math.fsum(nll_p) / P
    out = dict(ep)
    out.update(loss=nll + lam * ep["or"], nll=nll, pm=pm.copy(), n_q=n_q.copy(), dL_dmean=dl)
    del out["dL_dell"]
    return out


def token_cotangent_full(dL_dmean, n, labels, seg_offsets, ignore_index: int = IGNORE_INDEX):
    """g_t = (dL/dmean_s) / n_s for a valid token t of span s (prompt, chosen or rejected), else 0."""
    labels = np.asarray(labels).astype(np.int64)
    off = np.asarray(seg_offsets).astype(np.int64)
    g = np.zeros(labels.shape[0])
    for s_ in range(off.shape[0] - 1):
        for t in range(off[s_], off[s_ + 1]):
            if labels[t] != ignore_index and n[s_] > 0:
                g[t] = dL_dmean[s_] / n[s_]
    return g


# --------------------------------------------------------------------------------------------
# Backward: coeff, dh, dW
# --------------------------------------------------------------------------------------------
def backward(h, W, labels, lse, g, cap: float = 0.0, ignore_index: int = IGNORE_INDEX,
             want_dW: bool = True, rows: int = 64, logit_operands=None):
    """dh = coeff . W and dW = coeff^T . h with coeff_tv = g_t (1[v = y_t] - p_tv) sech^2(raw_tv/cap).

    Training — design (older revision), "Implementation spec — fused linear-CE log-prob head",
    backward: recompute each logit from the saved lse, softmax = exp(softcap(raw) - lse), per-logit
    cotangent g (onehot - softmax), times sech^2 under a softcap; Steel flash-CCE — handoff,
    Glossary D "softmax-onehot coeff". dW is the same chain rule for the weight operand of
    raw = h . W^T. Returns (dh [M, d], dW [V, d] or None) in float64.

    logit_operands = (h_l, W_l): the logits (and so p, the softcap slope and lse's consistency)
    come from raw = h_l . W_l^T while the gradient products keep h and W; the low-precision head
    passes its dequantised FP8 operands here (see oracle/fp8.py for that reading).
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels).astype(np.int64)
    lse = np.asarray(lse, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    M, V = h.shape[0], W.shape[0]
    valid = _check_labels(labels, V, ignore_index)
    if logit_operands is None:
        h_l, W_l = h, W
    else:
        h_l = np.asarray(logit_operands[0], dtype=np.float64)
        W_l = np.asarray(logit_operands[1], dtype=np.float64)
        if h_l.shape != h.shape or W_l.shape != W.shape:
            raise OracleError("logit operands must have the shapes of h and W")
    dh = np.zeros_like(h)
    dW = np.zeros_like(W) if want_dW else None
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        raw = h_l[r0:r1] @ W_l.T
        p = np.exp(softcap(raw, cap) - lse[r0:r1, None])
        onehot = np.zeros_like(raw)
        for i in range(r1 - r0):
            if valid[r0 + i]:
                onehot[i, labels[r0 + i]] = 1.0
        coeff = g[r0:r1, None] * (onehot - p) * softcap_slope(raw, cap)
        dh[r0:r1] = coeff @ W
        if want_dW:
            dW += coeff.T @ h[r0:r1]
    return dh, dW


def backward_filtered(h, W, labels, lse, g, cap: float, eps: float,
                      ignore_index: int = IGNORE_INDEX, tok_block: int = 256, k_slice: int = 64,
                      logit_operands=None):
    """The backward with the coefficient filter: dh and dW from coefficients whose negligible
    blocks are dropped.

    Steel flash-CCE — handoff, Glossary E "Backward approximations": the coefficient filter skips
    the gradient GEMM's chunks whose whole coefficient block is below eps (ORPO training — design,
    the flash-CCE status notes, give its default 1e-5 and its measured effect on real data). The
    chunks here are the K slices of the two gradient GEMMs: for dh (K = vocabulary) a block is
    tok_block tokens x k_slice vocabulary entries, for dW (K = tokens) tok_block vocabulary entries
    x k_slice tokens, aligned to multiples of their sizes from index 0. A block is dropped when
    max |coeff| over it is < eps. eps = 0 is the exact backward. Returns (dh, dW, kept_dh, kept_dw)
    with the kept fractions of the blocks. logit_operands as for backward().
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels).astype(np.int64)
    lse = np.asarray(lse, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    M, V = h.shape[0], W.shape[0]
    valid = _check_labels(labels, V, ignore_index)
    h_l, W_l = (h, W) if logit_operands is None else (np.asarray(logit_operands[0], dtype=np.float64),
                                                      np.asarray(logit_operands[1], dtype=np.float64))
    raw = h_l @ W_l.T
    p = np.exp(softcap(raw, cap) - lse[:, None])
    onehot = np.zeros_like(raw)
    for t in range(M):
        if valid[t]:
            onehot[t, labels[t]] = 1.0
    coeff = g[:, None] * (onehot - p) * softcap_slope(raw, cap)
    a = np.abs(coeff)

    def block_mask(rows_per, cols_per):
        keep = np.zeros_like(a, dtype=bool)
        n_keep = n_all = 0
        for r0 in range(0, M, rows_per):
            for c0 in range(0, V, cols_per):
                k = a[r0:r0 + rows_per, c0:c0 + cols_per].max() >= eps
                keep[r0:r0 + rows_per, c0:c0 + cols_per] = k
                n_keep += int(k)
                n_all += 1
        return keep, n_keep / max(n_all, 1)

    keep_dh, f_dh = block_mask(tok_block, k_slice)       # (tokens, vocabulary) blocks
    keep_dw, f_dw = block_mask(k_slice, tok_block)       # (tokens, vocabulary) = (64, 256) blocks
    dh = np.where(keep_dh, coeff, 0.0) @ W
    dW = np.where(keep_dw, coeff, 0.0).T @ h
    return dh, dW, f_dh, f_dw


# --------------------------------------------------------------------------------------------
# The whole head step
# --------------------------------------------------------------------------------------------
def head_step(h, W, labels, seg_offsets, cap: float, lam: float,
              ignore_index: int = IGNORE_INDEX, want_dW: bool = True):
    """forward -> branch means -> ORPO epilogue -> per-token cotangent -> dh, dW."""
    logp, lse = forward(h, W, labels, cap, ignore_index)
    ell, n = branch_means(logp, labels, seg_offsets, ignore_index)
    ep = orpo_epilogue(ell, lam)
    g = token_cotangent(ep["dL_dell"], n, labels, seg_offsets, ignore_index)
    dh, dW = backward(h, W, labels, lse, g, cap, ignore_index, want_dW)
    out = dict(ep)
    out.update(logp=logp, lse=lse, ell=ell, n=n, g=g, dh=dh, dW=dW)
    return out


def loss_value(h, W, labels, seg_offsets, cap: float, lam: float,
               ignore_index: int = IGNORE_INDEX) -> float:
    """The scalar loss alone (used by the finite-difference pins)."""
    logp, _ = forward(h, W, labels, cap, ignore_index)
    ell, _ = branch_means(logp, labels, seg_offsets, ignore_index)
    return orpo_epilogue(ell, lam)["loss"]


def head_step_full(h, W, labels, seg_offsets, cap: float, lam: float,
                   ignore_index: int = IGNORE_INDEX, want_dW: bool = True):
    """head_step with the full-scope NLL: seg_offsets holds [prompt, chosen, rejected] per pair."""
    logp, lse = forward(h, W, labels, cap, ignore_index)
    mean, n = span_means_full(logp, labels, seg_offsets, ignore_index)
    ep = orpo_epilogue_full(mean, n, lam)
    g = token_cotangent_full(ep["dL_dmean"], n, labels, seg_offsets, ignore_index)
    dh, dW = backward(h, W, labels, lse, g, cap, ignore_index, want_dW)
    out = dict(ep)
    out.update(logp=logp, lse=lse, mean=mean, n=n, g=g, dh=dh, dW=dW)
    return out


def loss_value_full(h, W, labels, seg_offsets, cap: float, lam: float,
                    ignore_index: int = IGNORE_INDEX) -> float:
    """The full-scope scalar loss alone (used by the finite-difference pins)."""
    logp, _ = forward(h, W, labels, cap, ignore_index)
    mean, n = span_means_full(logp, labels, seg_offsets, ignore_index)
    return orpo_epilogue_full(mean, n, lam)["loss"]
