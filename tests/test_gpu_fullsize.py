"""GPU parity at the full workload sizes, where the full float64 oracle would take hours:

  * forward: per-token logp and lse on a sampled row set (tokens from every branch and padding),
    computed by the oracle on those rows only;
  * loss: the oracle's float64 branch means + ORPO epilogue + cotangent on the GPU's own logp vector;
  * backward: a g-sparse probe — orpo_head_bwd with g zero except on a few sampled tokens S, so dh's
    rows in S and the whole dW depend only on S, and the oracle computes them from S alone; every
    other dh row must be exactly zero.

Runs the same HeadStep (and launch configuration) that bench.py times.
"""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from oracle import orpo_oracle as orc
from tests.gpu_helpers import (TOL_GRAD, TOL_SCALAR, dev, mfma_operand_weight, oracle_weight, rel,
                               row_gate, say, token_gate)

pytestmark = pytest.mark.gpu


def _sample_rows(inp, n_per_branch=2, seed=0):
    rng = np.random.default_rng(seed)
    off = inp.seg_offsets
    rows = []
    for b in range(len(off) - 1):
        rows += list(rng.integers(off[b], off[b + 1], size=n_per_branch))
    if off[-1] < inp.cfg.M:
        rows.append(inp.cfg.M - 1)                       # a padding row
    return np.unique(np.array(rows, dtype=np.int64))


@pytest.mark.parametrize("name", ["minicpm-like-bf16", "e4b-bf16-softcap30",
                                  "q4g64-minicpm-shape-softcap30", "q4g64-e4b-shape-softcap30",
                                  "q4g64-minicpm-shape-softcap30+stage",
                                  "q4g64-e4b-shape-softcap30+stage",
                                  "12b-like-bf16-softcap30", "e4b-bf16-softcap30-fullnll"])
def test_full_size_sampled_parity(name):
    # "+stage": the 4-bit head staged as bf16 rows each step (HeadStep q4_stage, bench --q4-stage).
    name, _, variant = name.partition("+")
    cfg = synth.workload(name)
    say(f"[fullsize] {cfg.name}{'+' + variant if variant else ''} M={cfg.M} d={cfg.d} V={cfg.V}")
    inp = synth.make_inputs(cfg, seed=0, label_device="cuda")
    d = dev()
    h = inp.h.to(d)
    if cfg.q4:
        w = torch.from_numpy(inp.wq.view(np.int32)).to(d)
        sc, bi = inp.scales.to(d), inp.biases.to(d)
    else:
        w, sc, bi = inp.w.to(d), None, None
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    step = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, scales=sc, biases=bi,
                      want_dW=not cfg.q4, scope=cfg.scope, q4_stage=variant == "stage")
    step.forward()
    step.loss()
    torch.cuda.synchronize()
    assert H.read_status(step.fws) == 0 and H.read_status(step.lws) == 0
    logp = step.logp.cpu().numpy().astype(np.float64)
    lse = step.lse.cpu().numpy().astype(np.float64)
    out = step.out.cpu().numpy()
    g = step.g.cpu().numpy().astype(np.float64)

    W = oracle_weight(inp)
    hh = inp.h.float().numpy().astype(np.float64)

    # Forward on sampled rows: norm-wise against the definition, per token against the oracle on
    # the operands the kernels multiply (the same weights except for the 4-bit head, whose
    # dequantised values the kernels round to bf16).
    rows = _sample_rows(inp)
    ref_logp, ref_lse = orc.forward(hh[rows], W, inp.labels[rows], cfg.softcap)
    e_logp, e_lse = rel(logp[rows], ref_logp), rel(lse[rows], ref_lse)
    W_op = mfma_operand_weight(inp) if cfg.q4 else W
    if cfg.q4:
        op_logp, op_lse = orc.forward(hh[rows], W_op, inp.labels[rows], cfg.softcap)
    else:
        op_logp, op_lse = ref_logp, ref_lse
    m_logp = token_gate("logp", logp[rows], op_logp)
    m_lse = token_gate("lse", lse[rows], op_lse)
    say(f"[fullsize {cfg.name}] rows={len(rows)} logp={e_logp:.2e} lse={e_lse:.2e} "
        f"max|dlogp|={m_logp:.2e} max|dlse|={m_lse:.2e}")
    assert e_logp <= TOL_SCALAR and e_lse <= TOL_SCALAR

    # Loss epilogue on the GPU's logp vector, in float64.
    P = cfg.pairs
    if cfg.scope == "full":
        mean, n = orc.span_means_full(logp, inp.labels, inp.seg_offsets)
        ep = orc.orpo_epilogue_full(mean, n, cfg.lam)
        gref = orc.token_cotangent_full(ep["dL_dmean"], n, inp.labels, inp.seg_offsets)
        assert np.allclose(out[5 + 2 * P:5 + 3 * P], ep["pm"], rtol=1e-9, atol=1e-12)
    else:
        ell, n = orc.branch_means(logp, inp.labels, inp.seg_offsets)
        ep = orc.orpo_epilogue(ell, cfg.lam)
        gref = orc.token_cotangent(ep["dL_dell"], n, inp.labels, inp.seg_offsets)
    for i, k in enumerate(("loss", "nll", "or", "accuracy", "margin")):
        assert abs(out[i] - ep[k]) <= 1e-9 * max(1.0, abs(ep[k])), k
    assert np.allclose(out[5:5 + P], ep["lw"], rtol=1e-9, atol=1e-12)
    assert np.allclose(out[5 + P:5 + 2 * P], ep["lr"], rtol=1e-9, atol=1e-12)
    assert rel(g, gref) <= 1e-6

    # g-sparse backward probe.
    probe = _sample_rows(inp, n_per_branch=1, seed=1)
    probe = probe[inp.labels[probe] != -100][:6]
    gs = np.zeros(cfg.M, dtype=np.float32)
    gs[probe] = g[probe]
    step.g.copy_(torch.from_numpy(gs).to(d))
    step.backward()
    torch.cuda.synchronize()
    dh = step.dh.cpu().numpy()
    pl, plse = orc.forward(hh[probe], W, inp.labels[probe], cfg.softcap)
    rdh, rdW = orc.backward(hh[probe], W, inp.labels[probe], plse, gs[probe].astype(np.float64),
                            cfg.softcap, want_dW=not cfg.q4)
    e_dh = rel(dh[probe], rdh)
    others = np.setdiff1d(np.arange(cfg.M), probe)
    assert np.all(dh[others] == 0.0)
    if cfg.q4:   # per row against the probe on the MFMA's operands
        _, plse_op = orc.forward(hh[probe], W_op, inp.labels[probe], cfg.softcap)
        rdh_op, _ = orc.backward(hh[probe], W_op, inp.labels[probe], plse_op,
                                 gs[probe].astype(np.float64), cfg.softcap, want_dW=False)
    else:
        rdh_op = rdh
    r_dh = row_gate("dh", dh[probe], rdh_op)
    msg = f"[fullsize {cfg.name}] probe={len(probe)} dh={e_dh:.2e} dh_row={r_dh:.2e}"
    assert e_dh <= TOL_GRAD
    if not cfg.q4:
        dW = step.dW.cpu().numpy()
        e_dW = rel(dW, rdW)
        r_dW = row_gate("dW", dW, rdW)
        msg += f" dW={e_dW:.2e} dW_row={r_dW:.2e}"
        assert e_dW <= TOL_GRAD
    say(msg)


def test_full_size_sibling_objectives_on_gpu_logp():
    # At the e4b size: every sibling objective's float64 epilogue on the GPU (loss, metrics, branch
    # values and the per-token g) against the oracle's on the same logp vector. The head kernels
    # they share are covered above; here it is the objectives' reductions over 8192 tokens.
    from oracle import objectives as ob
    cfg = synth.workload("e4b-bf16-softcap30")
    say(f"[fullsize objectives] {cfg.name} M={cfg.M}")
    inp = synth.make_inputs(cfg, seed=0, label_device="cuda")
    d = dev()
    h, w = inp.h.to(d), inp.w.to(d)
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    logp_t, _ = H.head_fwd(h, w, labels, cfg.softcap)
    torch.cuda.synchronize()
    logp = logp_t.cpu().numpy().astype(np.float64)
    sums, n = ob.span_stats(logp, inp.labels, inp.seg_offsets)
    means = sums / n
    rng = np.random.default_rng(5)
    P = cfg.pairs
    for kind, beta, gamma, ref in (("simpo", 2.0, 0.5, None),
                                   ("dpo", 0.1, 0.0, sums + rng.normal(0, 5.0, 2 * P)),
                                   ("ipo", 0.5, 0.0, means + rng.normal(0, 0.1, 2 * P)),
                                   ("hinge", 0.02, 0.0, sums + rng.normal(0, 30.0, 2 * P))):
        r = np.zeros(2 * P) if ref is None else ref
        if kind == "simpo":
            ep, vals = ob.simpo_epilogue(means[0::2], means[1::2], beta, gamma), means
        elif kind == "dpo":
            ep, vals = ob.dpo_epilogue(sums[0::2], sums[1::2], r[0::2], r[1::2], beta), sums
        elif kind == "ipo":
            ep, vals = ob.ipo_epilogue(means[0::2], means[1::2], r[0::2], r[1::2], beta), means
        else:
            ep, vals = ob.hinge_epilogue(sums[0::2], sums[1::2], r[0::2], r[1::2], beta), sums
            assert np.min(np.abs(1.0 - beta * ep["h"])) > 1e-6       # no pair at the kink
        ref_t = None if ref is None else torch.from_numpy(ref).to(d)
        out, g = H.pref_loss(kind, logp_t, labels, off, cfg.V, beta, gamma, ref_sums=ref_t)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        for i, k in enumerate(("loss", "accuracy", "margin")):
            assert abs(o[i] - ep[k]) <= 1e-12 * max(1.0, abs(ep[k])), (kind, k)
        assert np.allclose(o[3:3 + P], vals[0::2], rtol=1e-12) and np.allclose(o[3 + P:], vals[1::2], rtol=1e-12)
        g_o = ob.pairwise_cotangent(kind, ep, n, inp.labels, inp.seg_offsets)
        e = rel(g.cpu().numpy(), g_o)
        say(f"[fullsize objectives] {kind}: loss {o[0]:.6g} g rel {e:.1e}")
        assert e < 1e-6
    # GRPO over the same spans as completions (old / reference policies: the logp plus noise).
    old = (logp + rng.normal(0, 0.1, cfg.M)).astype(np.float32)
    refl = (logp + rng.normal(0, 0.2, cfg.M)).astype(np.float32)
    S = len(inp.seg_offsets) - 1
    adv = ob.group_advantages(rng.normal(size=S), 4).astype(np.float32)
    out, g = H.grpo_loss(logp_t, torch.from_numpy(old).to(d), torch.from_numpy(refl).to(d),
                         torch.from_numpy(adv).to(d), labels, off, cfg.V, 0.2, 0.04)
    torch.cuda.synchronize()
    r = ob.grpo_loss(logp, old, refl, inp.labels, inp.seg_offsets, adv, 0.2, 0.04)
    o = out.cpu().numpy()
    for i, k in enumerate(("loss", "pg", "kl")):
        assert abs(o[i] - r[k]) <= 1e-9 * max(1.0, abs(r[k])), ("grpo", k)
    assert abs(o[3] - r["clip_frac"]) < 1e-12
    e = rel(g.cpu().numpy(), r["g"])
    say(f"[fullsize objectives] grpo: loss {o[0]:.6g} g rel {e:.1e}")
    assert e < 1e-6
