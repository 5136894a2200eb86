"""Pins for the sibling-objective oracle (oracle/objectives.py): the degenerate cases the pages
list as correctness gates, closed forms, and central finite differences of each loss through the
head (w.r.t. h and W) or w.r.t. the log-probs. A plausible slip (a sign, a dropped 1/n, a sum
taken as a mean, the clipped branch's gradient, the KL derivative) fails at least one of them."""
import math

import numpy as np
import pytest

from oracle import objectives as ob
from oracle import orpo_oracle as orc

LN2 = math.log(2.0)


def _rng(s):
    return np.random.default_rng(777 + s)


# ----------------------------------------------------------------------------- SimPO
def test_simpo_beta_zero_and_margin_at_gamma():
    ep = ob.simpo_epilogue([-1.0, -2.0], [-3.0, -1.5], 0.0, 0.7)
    assert ep["loss"] == LN2 and np.all(ep["dL_dw"] == 0) and np.all(ep["dL_dr"] == 0)
    # (lw - lr) = gamma => u = 0 => L = ln 2, dL/dlw = -beta / 2 / P.
    ep = ob.simpo_epilogue([-1.0], [-1.5], 2.5, 0.5)
    assert ep["loss"] == pytest.approx(LN2, rel=1e-15)
    assert ep["dL_dw"][0] == pytest.approx(-1.25, rel=1e-15) and ep["dL_dr"][0] == pytest.approx(1.25)


def test_simpo_closed_form():
    # lw = -1, lr = -2, gamma = 0.5, beta = 2: u = 1, L = ln(1 + e^-1); accuracy 1, margin 1.
    ep = ob.simpo_epilogue([-1.0], [-2.0], 2.0, 0.5)
    assert ep["loss"] == pytest.approx(math.log1p(math.exp(-1.0)), rel=1e-15)
    assert ep["accuracy"] == 1.0 and ep["margin"] == 1.0
    assert ep["dL_dw"][0] == pytest.approx(-2.0 / (1.0 + math.e), rel=1e-14)


# ----------------------------------------------------------------------------- DPO
def test_dpo_policy_equals_reference_gives_ln2():
    sw, sr = np.array([-12.0, -30.5]), np.array([-14.0, -29.0])
    ep = ob.dpo_epilogue(sw, sr, sw, sr, 0.1)
    assert ep["loss"] == LN2 and ep["margin"] == 0.0 and ep["accuracy"] == 0.0
    assert np.allclose(ep["dL_dw"], -0.1 / 2 / 2, rtol=1e-15)


def test_dpo_beta_zero_has_no_gradient():
    ep = ob.dpo_epilogue([-3.0], [-9.0], [-4.0], [-2.0], 0.0)
    assert ep["loss"] == LN2 and ep["dL_dw"][0] == 0.0 and ep["dL_dr"][0] == 0.0


def test_dpo_closed_form():
    # Delta = 0.5 [(-10 + 11) - (-20 + 18)] = 1.5; L = softplus(-1.5).
    ep = ob.dpo_epilogue([-10.0], [-20.0], [-11.0], [-18.0], 0.5)
    assert ep["delta"][0] == 1.5 and ep["margin"] == 1.5 and ep["accuracy"] == 1.0
    assert ep["loss"] == pytest.approx(math.log1p(math.exp(-1.5)), rel=1e-15)
    assert ep["dL_dw"][0] == pytest.approx(-0.5 / (1.0 + math.exp(1.5)), rel=1e-14)


# ----------------------------------------------------------------------------- through the head
def _pair_problem(seed, cap):
    rng = _rng(seed)
    M, d, V = 14, 5, 9
    h = rng.standard_normal((M, d))
    W = rng.standard_normal((V, d)) * (1.5 if cap else 0.8)
    labels = rng.integers(0, V, size=M)
    labels[4] = -100
    labels[12:] = -100
    off = np.array([0, 3, 6, 9, 12])
    return h, W, labels, off


def _pairwise_loss(kind, h, W, labels, off, cap, params, ref=None):
    logp, _ = orc.forward(h, W, labels, cap)
    sums, n = ob.span_stats(logp, labels, off)
    means = sums / n
    if kind == "simpo":
        ep = ob.simpo_epilogue(means[0::2], means[1::2], *params)
    elif kind == "ipo":
        ep = ob.ipo_epilogue(means[0::2], means[1::2], ref[0::2], ref[1::2], *params)
    elif kind == "hinge":
        ep = ob.hinge_epilogue(sums[0::2], sums[1::2], ref[0::2], ref[1::2], *params)
    else:
        ep = ob.dpo_epilogue(sums[0::2], sums[1::2], ref[0::2], ref[1::2], *params)
    return ep, n


_FD_PARAMS = {"simpo": ((2.0, 0.3), None, 4),
              "dpo": ((0.7,), np.array([-20.0, -18.5, -17.0, -21.0]), 3),
              # IPO: reference means near the policy's, so each pair's margin is away from the
              # target 1/(2 beta) and the gradient is not degenerate.
              "ipo": ((0.8,), np.array([-2.1, -2.6, -2.4, -1.9]), 5),
              # Hinge: beta and reference sums chosen so one pair is on the sloped side and one on
              # the flat side, both far from the kink (checked below).
              "hinge": ((0.25,), np.array([-20.0, -6.0, -14.0, -10.0]), 6)}


@pytest.mark.parametrize("kind,cap", [(k, c) for k in ("simpo", "dpo", "ipo", "hinge")
                                      for c in (0.0, 2.0)])
def test_pairwise_gradients_match_central_finite_differences(kind, cap):
    params, ref, seed = _FD_PARAMS[kind]
    h, W, labels, off = _pair_problem(seed, cap)
    logp, lse = orc.forward(h, W, labels, cap)
    ep, n = _pairwise_loss(kind, h, W, labels, off, cap, params, ref)
    g = ob.pairwise_cotangent(kind, ep, n, labels, off)
    dh, dW = orc.backward(h, W, labels, lse, g, cap)
    eps = 1e-6

    def fd(arr, which):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a = arr.copy()
            a[idx] += eps
            lp = _pairwise_loss(kind, *((a, W) if which == "h" else (h, a)), labels, off, cap, params, ref)[0]["loss"]
            a[idx] -= 2 * eps
            lm = _pairwise_loss(kind, *((a, W) if which == "h" else (h, a)), labels, off, cap, params, ref)[0]["loss"]
            out[idx] = (lp - lm) / (2 * eps)
        return out

    if kind == "hinge":
        u = 1.0 - params[0] * ep["h"]
        assert np.min(np.abs(u)) > 0.05 and np.any(u > 0) and np.any(u < 0), u
    gh, gw = fd(h, "h"), fd(W, "W")
    assert np.linalg.norm(gh) > 0
    assert np.linalg.norm(dh - gh) <= 1e-6 * np.linalg.norm(gh)
    assert np.linalg.norm(dW - gw) <= 1e-6 * np.linalg.norm(gw)
    assert np.all(dh[[4, 12, 13]] == 0.0)


# ----------------------------------------------------------------------------- IPO, hinge
def test_ipo_at_target_margin_and_at_zero_margin():
    # beta = 0.5: target 1/(2 beta) = 1. Margin exactly 1 -> zero loss and zero gradient.
    ep = ob.ipo_epilogue([-1.0], [-2.0], [0.0], [0.0], 0.5)
    assert ep["h"][0] == 1.0 and ep["loss"] == 0.0 and ep["dL_dw"][0] == 0.0
    # Policy equal to the reference: h = 0, L = 1/(4 beta^2), dL/dlw = -1/beta / P.
    ep = ob.ipo_epilogue([-1.25, -3.0], [-2.0, -0.5], [-1.25, -3.0], [-2.0, -0.5], 0.25)
    assert np.all(ep["h"] == 0.0) and ep["loss"] == pytest.approx(4.0, rel=1e-15)
    assert np.allclose(ep["dL_dw"], -4.0 / 2, rtol=1e-15) and ep["accuracy"] == 0.0
    with pytest.raises(orc.OracleError):
        ob.ipo_epilogue([-1.0], [-2.0], [0.0], [0.0], 0.0)


def test_ipo_closed_form():
    # h = (-1 + 1.5) - (-3 + 2) = 1.5, beta = 2 -> target 0.25: L = 1.25^2, dL/dlw = 2.5.
    ep = ob.ipo_epilogue([-1.0], [-3.0], [-1.5], [-2.0], 2.0)
    assert ep["h"][0] == 1.5 and ep["margin"] == 1.5 and ep["accuracy"] == 1.0
    assert ep["loss"] == 1.5625 and ep["dL_dw"][0] == 2.5 and ep["dL_dr"][0] == -2.5


def test_hinge_flat_and_sloped_sides():
    # beta h >= 1: no loss, no gradient (the kink itself included).
    ep = ob.hinge_epilogue([-10.0, -10.0], [-14.0, -12.0], [0.0, 0.0], [0.0, 0.0], 0.5)
    assert list(ep["h"]) == [4.0, 2.0] and ep["loss"] == 0.0 and np.all(ep["dL_dw"] == 0.0)
    # beta h < 1: L = 1 - beta h, dL/dsw = -beta / P.
    ep = ob.hinge_epilogue([-10.0, -30.0], [-15.0, -20.0], [-1.0, 0.0], [-3.0, 0.0], 0.25)
    assert list(ep["h"]) == [3.0, -10.0]
    assert ep["loss"] == pytest.approx(((1 - 0.75) + (1 + 2.5)) / 2, rel=1e-15)
    assert np.all(ep["dL_dw"] == -0.125) and np.all(ep["dL_dr"] == 0.125)
    assert ep["accuracy"] == 0.5 and ep["margin"] == -3.5


def test_pairwise_cotangent_mean_kinds_and_sum_kinds():
    labels = np.zeros(10, dtype=np.int64)
    labels[2] = -100
    off = np.array([0, 4, 10])
    ep = ob.ipo_epilogue([-3.0], [-4.0], [0.0], [0.0], 1.0)
    g = ob.pairwise_cotangent("ipo", ep, [3, 6], labels, off)
    assert g[2] == 0.0 and np.allclose(g[[0, 1, 3]], ep["dL_dw"][0] / 3, rtol=1e-15)
    assert np.allclose(g[4:], ep["dL_dr"][0] / 6, rtol=1e-15)
    ep = ob.hinge_epilogue([-3.0], [-4.0], [0.0], [0.0], 0.5)
    g = ob.pairwise_cotangent("hinge", ep, [3, 6], labels, off)
    assert g[2] == 0.0 and np.all(g[[0, 1, 3]] == -0.5) and np.all(g[4:] == 0.5)


def test_dpo_cotangent_is_per_sequence_sum_and_simpo_per_token_mean():
    labels = np.zeros(10, dtype=np.int64)
    off = np.array([0, 4, 10])
    ep = ob.dpo_epilogue([-3.0], [-4.0], [-3.5], [-4.5], 1.0)
    g = ob.pairwise_cotangent("dpo", ep, [4, 6], labels, off)
    assert np.all(g[:4] == ep["dL_dw"][0]) and np.all(g[4:] == ep["dL_dr"][0])
    ep = ob.simpo_epilogue([-3.0], [-4.0], 1.0, 0.0)
    g = ob.pairwise_cotangent("simpo", ep, [4, 6], labels, off)
    assert np.allclose(g[:4], ep["dL_dw"][0] / 4, rtol=1e-15) and np.allclose(g[4:], ep["dL_dr"][0] / 6)


# ----------------------------------------------------------------------------- GRPO
def _grpo_inputs(seed):
    rng = _rng(seed)
    M = 20
    logp = -rng.exponential(2.0, size=M)
    old = logp + rng.normal(0, 0.3, size=M)
    ref = logp + rng.normal(0, 0.4, size=M)
    labels = rng.integers(0, 50, size=M)
    labels[[3, 17]] = -100
    labels[19] = -100
    off = np.array([0, 6, 11, 19])
    return logp, old, ref, labels, off


def test_grpo_single_sample_group_has_only_kl():
    # G = 1 => advantage 0 => no policy-gradient signal; only the KL term.
    logp, old, ref, labels, off = _grpo_inputs(1)
    adv = ob.group_advantages([0.3, 1.0, -2.0], 1)
    assert np.all(adv == 0)
    r = ob.grpo_loss(logp, old, ref, labels, off, adv, 0.2, 0.05)
    assert r["pg"] == 0.0 and r["loss"] == pytest.approx(0.05 * r["kl"], rel=1e-15)
    for s in range(3):
        ts = [t for t in range(off[s], off[s + 1]) if labels[t] != -100]
        for t in ts:
            assert r["g"][t] == pytest.approx(0.05 * (1 - math.exp(ref[t] - logp[t])) / (len(ts) * 3),
                                              rel=1e-13, abs=1e-16)


def test_grpo_no_clip_is_vanilla_pg_and_beta_zero_has_no_kl():
    logp, old, ref, labels, off = _grpo_inputs(2)
    adv = np.array([1.3, -0.7, 0.4])
    r = ob.grpo_loss(logp, old, ref, labels, off, adv, 1e9, 0.0)
    assert r["loss"] == r["pg"] and r["clip_frac"] == 0.0
    pg = []
    for s in range(3):
        ts = [t for t in range(off[s], off[s + 1]) if labels[t] != -100]
        pg.append(-np.mean([adv[s] * math.exp(logp[t] - old[t]) for t in ts]))
        for t in ts:
            assert r["g"][t] == pytest.approx(-adv[s] * math.exp(logp[t] - old[t]) / (len(ts) * 3), rel=1e-13)
    assert r["pg"] == pytest.approx(np.mean(pg), rel=1e-13)


def test_grpo_on_policy_and_at_reference():
    # logp = old => rho = 1 (inside any clip range): pg = mean(-A); logp = ref => k3 = 0, KL grad 0.
    logp, _, _, labels, off = _grpo_inputs(3)
    adv = np.array([0.5, -1.0, 2.0])
    r = ob.grpo_loss(logp, logp, logp, labels, off, adv, 0.2, 0.3)
    assert r["pg"] == pytest.approx(-np.mean(adv), rel=1e-15) and r["kl"] == 0.0
    assert r["loss"] == pytest.approx(-np.mean(adv), rel=1e-15)


def test_grpo_clipped_tokens_carry_no_pg_gradient():
    # A > 0 and rho > 1 + eps: the clipped term (1 + eps) A is the minimum -> constant in logp.
    labels = np.zeros(4, dtype=np.int64)
    logp = np.log([0.5, 0.5, 0.5, 0.5])
    old = np.log([0.25, 0.5, 0.5, 0.9])            # rho = 2, 1, 1, 0.556
    r = ob.grpo_loss(logp, old, logp, labels, [0, 4], [1.0], 0.2, 0.0)
    assert r["g"][0] == 0.0 and r["clip_frac"] == 0.25
    assert r["g"][1] == pytest.approx(-1.0 / 4, rel=1e-15)
    assert r["g"][3] == pytest.approx(-(0.5 / 0.9) / 4, rel=1e-14)   # below 1 - eps: unclipped is min
    assert r["pg"] == pytest.approx(-(1.2 + 1 + 1 + 0.5 / 0.9) / 4, rel=1e-14)


def test_grpo_gradient_matches_finite_differences_in_logp():
    logp, old, ref, labels, off = _grpo_inputs(4)
    adv = np.array([0.9, -1.1, 0.2])
    r = ob.grpo_loss(logp, old, ref, labels, off, adv, 0.25, 0.1)
    eps = 1e-7
    for t in range(len(logp)):
        a = logp.copy()
        a[t] += eps
        lp = ob.grpo_loss(a, old, ref, labels, off, adv, 0.25, 0.1)["loss"]
        a[t] -= 2 * eps
        lm = ob.grpo_loss(a, old, ref, labels, off, adv, 0.25, 0.1)["loss"]
        assert (lp - lm) / (2 * eps) == pytest.approx(r["g"][t], rel=1e-6, abs=1e-10), t


def test_group_advantages_closed_form():
    a = ob.group_advantages([1.0, 3.0, 0.0, 0.0], 2, eps=1e-300)
    assert np.allclose(a[:2], [-1.0, 1.0], rtol=1e-15)
    assert np.all(a[2:] == 0.0)                    # equal rewards: no signal
    a = ob.group_advantages([1.0, 3.0, 5.0], 3, eps=0.0)
    assert np.allclose(a, [-math.sqrt(1.5), 0.0, math.sqrt(1.5)], rtol=1e-15)
