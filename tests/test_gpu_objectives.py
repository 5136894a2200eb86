"""GPU parity for the sibling objectives (SimPO, DPO, IPO, hinge, GRPO) that reuse the head's forward and
backward: their float64 epilogues on the GPU's own log-probs against the oracle's, and a whole
forward -> objective -> backward step against the oracle's. Inputs the objectives need beyond the
head's (reference sums, the sampling and reference policies' log-probs, advantages) are drawn from
seeded noise around the oracle's own log-probs, never from the HIP path."""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from oracle import objectives as ob
from oracle import orpo_oracle as orc
from tests.gpu_helpers import TOL_GRAD, TOL_SCALAR, dev, rel, say

pytestmark = pytest.mark.gpu


def _problem(M, d, V, cap, seed, n_spans):
    rng = np.random.default_rng(seed)
    h = synth.to_bf16(rng.standard_normal((M, d)))
    w = synth.to_bf16((rng.standard_normal((V, d)) * (3.0 / np.sqrt(d))).astype(np.float32))
    used = (M * 7) // 8
    cuts = np.sort(rng.choice(np.arange(1, used), size=n_spans - 1, replace=False))
    off = np.concatenate([[0], cuts, [used]]).astype(np.int32)
    labels = rng.integers(0, V, size=M).astype(np.int32)
    labels[used:] = -100
    for s in range(n_spans):
        if off[s + 1] - off[s] >= 3:
            labels[off[s] + 1] = -100
    hh = h.float().numpy().astype(np.float64)
    W = w.float().numpy().astype(np.float64)
    logp, lse = orc.forward(hh, W, labels, cap)
    return dict(h=h, w=w, hh=hh, W=W, labels=labels, off=off, logp=logp, lse=lse, cap=cap, V=V,
                rng=rng)


def _gpu_logp(pb):
    d = dev()
    h, w = pb["h"].to(d), pb["w"].to(d)
    lab = torch.from_numpy(pb["labels"]).to(d)
    logp, lse = H.head_fwd(h, w, lab, pb["cap"])
    return h, w, lab, logp, lse


def _backward_parity(pb, h, w, lab, lse, g_gpu, g_ref, label):
    dh, dW = H.head_bwd(h, w, lab, lse, g_gpu, pb["cap"])
    rdh, rdW = orc.backward(pb["hh"], pb["W"], pb["labels"], pb["lse"], g_ref, pb["cap"])
    e_dh, e_dW = rel(dh.cpu().numpy(), rdh), rel(dW.cpu().numpy(), rdW)
    say(f"[objective {label}] dh={e_dh:.2e} dW={e_dW:.2e}")
    assert e_dh <= TOL_GRAD and e_dW <= TOL_GRAD


def _oracle_pair(kind, sums, n, ref, beta, gamma):
    """The oracle's epilogue for `kind` on span sums/counts; returns (epilogue, branch values)."""
    means = sums / n
    if kind == "simpo":
        return ob.simpo_epilogue(means[0::2], means[1::2], beta, gamma), means
    r = np.zeros_like(sums) if ref is None else ref
    if kind == "ipo":
        return ob.ipo_epilogue(means[0::2], means[1::2], r[0::2], r[1::2], beta), means
    if kind == "hinge":
        return ob.hinge_epilogue(sums[0::2], sums[1::2], r[0::2], r[1::2], beta), sums
    return ob.dpo_epilogue(sums[0::2], sums[1::2], r[0::2], r[1::2], beta), sums


@pytest.mark.parametrize("kind,with_ref", [("simpo", False), ("dpo", True), ("ipo", True),
                                           ("ipo", False), ("hinge", True), ("hinge", False)])
def test_pairwise_objective_step(kind, with_ref):
    d = dev()
    seed = {"simpo": 42, "dpo": 41, "ipo": 43, "hinge": 44}[kind] + (10 if with_ref else 0)
    pb = _problem(700, 192, 3001, 30.0, seed=seed, n_spans=6)
    say(f"[case] {kind} ref={with_ref} M=700 d=192 V=3001")
    h, w, lab, logp, lse = _gpu_logp(pb)
    off_t = torch.from_numpy(pb["off"]).to(d)
    sums_o, n = ob.span_stats(pb["logp"], pb["labels"], pb["off"])
    beta, gamma = {"simpo": (2.0, 0.3), "dpo": (0.1, 0.0), "ipo": (0.5, 0.0),
                   "hinge": (0.2, 0.0)}[kind]
    if kind == "hinge" and not with_ref:
        beta = 1e-3   # reference-free sums differ by ~1e3 here: a mix of sloped and flat pairs
    ref = None
    if with_ref:
        # Cached reference values of the objective's kind: noise around the oracle's own.
        scale = {"dpo": 3.0, "hinge": 3.0, "ipo": 0.2}[kind]
        base = sums_o / n if kind in ob.MEAN_KINDS else sums_o
        ref = base + pb["rng"].normal(0.0, scale, size=sums_o.shape)
    ep_o, _ = _oracle_pair(kind, sums_o, n, ref, beta, gamma)
    if kind == "hinge":   # every pair away from the kink (the two sides' g differ), both sides used
        u = 1.0 - beta * ep_o["h"]
        assert np.min(np.abs(u)) > 1e-2 and np.any(u > 0), u
    ref_t = None if ref is None else torch.from_numpy(ref).to(d)
    out, g, ws = H.pref_loss(kind, logp, lab, off_t, pb["V"], beta, gamma, ref_sums=ref_t,
                             return_ws=True)
    torch.cuda.synchronize()
    assert H.read_status(ws) == 0
    o = out.cpu().numpy()
    g_o = ob.pairwise_cotangent(kind, ep_o, n, pb["labels"], pb["off"])
    errs = {"loss": abs(o[0] - ep_o["loss"]) / max(abs(ep_o["loss"]), 1e-12),
            "g": rel(g.cpu().numpy(), g_o),
            "margin": abs(o[2] - ep_o["margin"]) / max(1.0, abs(ep_o["margin"]))}
    say(f"[objective {kind}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["loss"] <= TOL_SCALAR and errs["g"] <= TOL_SCALAR and errs["margin"] <= TOL_SCALAR
    _backward_parity(pb, h, w, lab, lse, g, g_o, kind)

    # The float64 epilogue on the GPU's own logp vector, against the oracle's on the same vector.
    lv = logp.cpu().numpy().astype(np.float64)
    sums, n2 = ob.span_stats(lv, pb["labels"], pb["off"])
    ep, vals = _oracle_pair(kind, sums, n2, ref, beta, gamma)
    for i, k in enumerate(("loss", "accuracy", "margin")):
        assert abs(o[i] - ep[k]) <= 1e-12 * max(1.0, abs(ep[k])), k
    assert np.allclose(o[3:6], vals[0::2], rtol=1e-12) and np.allclose(o[6:9], vals[1::2], rtol=1e-12)
    assert rel(g.cpu().numpy(), ob.pairwise_cotangent(kind, ep, n2, pb["labels"], pb["off"])) < 1e-6


def test_dpo_policy_equals_reference_on_gpu():
    # Reference sums = the oracle's own sums: Delta ~ 0 up to the GPU's logp error, L ~ ln 2.
    d = dev()
    pb = _problem(400, 64, 1000, 0.0, seed=7, n_spans=4)
    h, w, lab, logp, lse = _gpu_logp(pb)
    sums_o, _ = ob.span_stats(pb["logp"], pb["labels"], pb["off"])
    out, g = H.pref_loss("dpo", logp, lab, torch.from_numpy(pb["off"]).to(d), pb["V"], 0.5,
                         ref_sums=torch.from_numpy(sums_o).to(d))
    o = out.cpu().numpy()
    assert abs(o[0] - np.log(2.0)) < 1e-5 and abs(o[2]) < 1e-4
    # beta = 0: no gradient at all.
    out, g = H.pref_loss("dpo", logp, lab, torch.from_numpy(pb["off"]).to(d), pb["V"], 0.0,
                         ref_sums=torch.from_numpy(sums_o).to(d))
    assert abs(out[0].item() - np.log(2.0)) <= 1e-15 and torch.count_nonzero(g).item() == 0


def test_grpo_step():
    d = dev()
    pb = _problem(700, 192, 3001, 30.0, seed=43, n_spans=8)
    say("[case] grpo M=700 d=192 V=3001")
    h, w, lab, logp, lse = _gpu_logp(pb)
    rng = pb["rng"]
    old = pb["logp"] + rng.normal(0.0, 0.25, size=pb["logp"].shape)
    refl = pb["logp"] + rng.normal(0.0, 0.3, size=pb["logp"].shape)
    adv = ob.group_advantages(rng.normal(size=8), 4)
    eps, beta = 0.2, 0.04
    f32 = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float32)).to(d)
    old32, ref32, adv32 = np.float32(old), np.float32(refl), np.float32(adv)
    off_t = torch.from_numpy(pb["off"]).to(d)
    out, g, ws = H.grpo_loss(logp, f32(old32), f32(ref32), f32(adv32), lab, off_t, pb["V"], eps, beta,
                             return_ws=True)
    torch.cuda.synchronize()
    assert H.read_status(ws) == 0
    o = out.cpu().numpy()
    r_o = ob.grpo_loss(pb["logp"], old32, ref32, pb["labels"], pb["off"], adv32, eps, beta)
    errs = {"loss": abs(o[0] - r_o["loss"]) / max(1.0, abs(r_o["loss"])),
            "kl": abs(o[2] - r_o["kl"]) / max(1e-3, abs(r_o["kl"])), "g": rel(g.cpu().numpy(), r_o["g"])}
    say("[objective grpo] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" clip={o[3]:.3f}")
    assert errs["loss"] <= TOL_SCALAR and errs["kl"] <= 1e-2 and errs["g"] <= 1e-2
    _backward_parity(pb, h, w, lab, lse, g, r_o["g"], "grpo")

    # The float64 epilogue on the GPU's own logp vector: exact up to rounding order.
    lv = logp.cpu().numpy().astype(np.float64)
    r = ob.grpo_loss(lv, old32, ref32, pb["labels"], pb["off"], adv32, eps, beta)
    for i, k in enumerate(("loss", "pg", "kl", "clip_frac")):
        assert abs(o[i] - r[k]) <= 1e-12 * max(1.0, abs(r[k])), k
    assert rel(g.cpu().numpy(), r["g"]) < 1e-6

    # One-sample groups: zero advantage, no policy-gradient term.
    out, g = H.grpo_loss(logp, f32(old32), f32(ref32), f32(np.zeros(8)), lab, off_t, pb["V"], eps, beta)
    assert out[1].item() == 0.0


def test_objective_status_bits():
    d = dev()
    pb = _problem(400, 64, 1000, 0.0, seed=9, n_spans=4)
    labels = pb["labels"].copy()
    labels[pb["off"][1]:pb["off"][2]] = -100
    lab = torch.from_numpy(labels).to(d)
    logp, _ = H.head_fwd(pb["h"].to(d), pb["w"].to(d), lab, 0.0)
    off_t = torch.from_numpy(pb["off"]).to(d)
    out, g, ws = H.pref_loss("simpo", logp, lab, off_t, 1000, 1.0, return_ws=True)
    assert H.read_status(ws) & 2 and np.isnan(out[0].item())
    z = torch.zeros(400, dtype=torch.float32, device=d)
    out, g, ws = H.grpo_loss(logp, z, z, torch.zeros(4, device=d), lab, off_t, 1000, 0.2, 0.1,
                             return_ws=True)
    assert H.read_status(ws) & 2 and np.isnan(out[0].item())
    bad = pb["off"].copy()
    bad[1], bad[2] = bad[2], bad[1]
    out, g, ws = H.grpo_loss(logp, z, z, torch.zeros(4, device=d), lab,
                             torch.from_numpy(bad).to(d), 1000, 0.2, 0.1, return_ws=True)
    assert H.read_status(ws) & 4 and torch.isnan(g).all().item()
