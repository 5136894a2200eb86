"""Pins for the float64 oracle, each against something other than the oracle itself.

Closed forms, the worked ORPO pair, series expansions of log1mexp, invariances, brute force on
tiny inputs, central finite differences, and hand-packed 4-bit words. A plausible slip anywhere in
the oracle (a dropped term, a sign, an index, a transposed operand) fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import orpo_oracle as orc

LN2 = math.log(2.0)


def _rng(s=0):
    return np.random.default_rng(12345 + s)


# ----------------------------------------------------------------------------- forward
def test_zero_weights_give_minus_log_v():
    # W = 0 => every logit is 0 (softcap(0) = 0) => logp = -ln V exactly.
    V = 4096
    h = _rng().standard_normal((5, 16))
    W = np.zeros((V, 16))
    labels = np.array([0, 17, 4095, -100, 3])
    for cap in (0.0, 30.0):
        logp, lse = orc.forward(h, W, labels, cap)
        assert np.allclose(logp[[0, 1, 2, 4]], -8.317766166719343, rtol=0, atol=1e-15)
        assert logp[3] == 0.0
        assert np.allclose(lse, math.log(V), rtol=0, atol=1e-15)


def test_single_vocab_entry_has_logp_zero():
    h = _rng(1).standard_normal((4, 8))
    W = _rng(2).standard_normal((1, 8))
    logp, lse = orc.forward(h, W, np.zeros(4, dtype=np.int64), 0.0)
    assert np.all(logp == 0.0)
    assert np.allclose(lse, h @ W[0], rtol=0, atol=1e-14)


def test_identical_rows_give_minus_log_v():
    V = 37
    row = _rng(3).standard_normal(6)
    W = np.tile(row, (V, 1))
    h = _rng(4).standard_normal((3, 6))
    logp, _ = orc.forward(h, W, np.array([0, 5, 36]), 2.0)
    assert np.allclose(logp, -math.log(V), rtol=0, atol=1e-13)


@pytest.mark.parametrize("cap", [0.0, 2.0, 30.0])
def test_two_level_logits_closed_form(cap):
    # One vocab row boosted by delta, the rest zero: z_k = softcap(delta), z_j = 0.
    V, k, delta, a = 7, 3, 2.5, 1.7
    h = np.array([[a, 0.0, 0.0]] * 2)
    W = np.zeros((V, 3))
    W[k, 0] = delta / a
    zk = cap * math.tanh(delta / cap) if cap > 0 else delta
    logp, lse = orc.forward(h, W, np.array([k, 0]), cap)
    assert logp[0] == pytest.approx(-math.log(1.0 + (V - 1) * math.exp(-zk)), rel=1e-14)
    assert logp[1] == pytest.approx(-math.log(math.exp(zk) + V - 1), rel=1e-14)
    assert lse[0] == pytest.approx(math.log(math.exp(zk) + V - 1), rel=1e-14)


def test_huge_softcap_matches_no_softcap():
    h = _rng(5).standard_normal((6, 8))
    W = _rng(6).standard_normal((11, 8))
    labels = np.array([0, 1, 2, 10, -100, 5])
    a, la = orc.forward(h, W, labels, 0.0)
    b, lb = orc.forward(h, W, labels, 1e9)
    assert np.allclose(a, b, rtol=0, atol=1e-12) and np.allclose(la, lb, rtol=0, atol=1e-12)


def test_softcap_bounds_logits():
    raw = np.linspace(-500, 500, 101)
    z = orc.softcap(raw, 30.0)
    assert np.all(np.abs(z) < 30.0 + 1e-12)
    assert np.allclose(orc.softcap(np.array([1e-8]), 30.0), 1e-8, rtol=1e-12)   # slope 1 at 0
    assert orc.softcap_slope(np.array([0.0]), 30.0)[0] == 1.0


def test_forward_brute_force_tiny():
    # Independent scalar loops: dot products, max-shifted exp sums with math.fsum.
    rng = _rng(7)
    M, d, V, cap = 3, 4, 5, 2.0
    h = rng.standard_normal((M, d)) * 2
    W = rng.standard_normal((V, d))
    labels = np.array([4, 0, 2])
    logp, lse = orc.forward(h, W, labels, cap)
    for t in range(M):
        z = [cap * math.tanh(math.fsum(h[t, j] * W[v, j] for j in range(d)) / cap) for v in range(V)]
        m = max(z)
        ref_lse = m + math.log(math.fsum(math.exp(x - m) for x in z))
        assert lse[t] == pytest.approx(ref_lse, rel=1e-14)
        assert logp[t] == pytest.approx(z[labels[t]] - ref_lse, rel=1e-13, abs=1e-14)


def test_vocab_permutation_invariance():
    rng = _rng(8)
    h = rng.standard_normal((9, 6))
    W = rng.standard_normal((13, 6))
    labels = rng.integers(0, 13, size=9)
    labels[4] = -100
    perm = rng.permutation(13)
    inv = np.argsort(perm)
    labels2 = np.where(labels == -100, -100, inv[np.maximum(labels, 0)])
    a, la = orc.forward(h, W, labels, 3.0)
    b, lb = orc.forward(h, W[perm], labels2, 3.0)
    assert np.allclose(a, b, rtol=0, atol=1e-13) and np.allclose(la, lb, rtol=0, atol=1e-13)


def test_row_blocking_does_not_change_results():
    rng = _rng(9)
    h = rng.standard_normal((70, 5))
    W = rng.standard_normal((8, 5))
    labels = rng.integers(0, 8, size=70)
    a, la = orc.forward(h, W, labels, 0.0, rows=64)
    b, lb = orc.forward(h, W, labels, 0.0, rows=7)
    assert np.allclose(a, b, rtol=0, atol=1e-13) and np.allclose(la, lb, rtol=0, atol=1e-13)


def test_softmax_normalises_and_logp_nonpositive():
    rng = _rng(10)
    h = rng.standard_normal((20, 8)) * 3
    W = rng.standard_normal((50, 8))
    labels = rng.integers(0, 50, size=20)
    logp, lse = orc.forward(h, W, labels, 0.0)
    assert np.all(logp <= 0)
    z = h @ W.T
    assert np.allclose(np.exp(z - lse[:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(lse >= z.max(axis=1))


def test_bad_label_raises():
    with pytest.raises(orc.OracleError):
        orc.forward(np.ones((2, 2)), np.ones((3, 2)), np.array([0, 3]))
    with pytest.raises(orc.OracleError):
        orc.forward(np.ones((2, 2)), np.ones((3, 2)), np.array([-1, 0]))


# ----------------------------------------------------------------------------- branch means
def test_branch_means_exact_rationals():
    logp = np.array([-1.0, -2.0, -3.0, -9.0, -4.0, -5.0, -6.0, -7.0, 0.0])
    labels = np.array([1, 1, 1, -100, 1, 1, 1, -100, -100])
    ell, n = orc.branch_means(logp, labels, np.array([0, 4, 7]))
    assert list(n) == [3, 3]
    assert ell[0] == -2.0 and ell[1] == -5.0


def test_branch_order_invariance_and_errors():
    rng = _rng(11)
    logp = -rng.random(10)
    labels = np.ones(10, dtype=np.int64)
    off = np.array([0, 6, 10])
    ell, _ = orc.branch_means(logp, labels, off)
    lp2 = logp.copy()
    lp2[:6] = lp2[:6][rng.permutation(6)]
    ell2, _ = orc.branch_means(lp2, labels, off)
    assert ell[0] == ell2[0]
    with pytest.raises(orc.OracleError):
        orc.branch_means(logp, np.full(10, -100), off)            # empty branch
    with pytest.raises(orc.OracleError):
        orc.branch_means(logp, labels, np.array([0, 7, 6]))       # not monotone
    with pytest.raises(orc.OracleError):
        orc.branch_means(logp, labels, np.array([0, 4, 11]))      # past M


# ----------------------------------------------------------------------------- epilogue
def test_worked_pair_half_quarter():
    # p_w = 1/2, p_r = 1/4: odds 1 and 1/3 => log-odds ln 3, L_OR = ln(4/3), NLL = ln 2.
    ep = orc.orpo_epilogue(np.array([math.log(0.5), math.log(0.25)]), 0.1)
    assert ep["log_odds"][0] == pytest.approx(math.log(3.0), rel=1e-14)
    assert ep["or"] == pytest.approx(math.log(4.0 / 3.0), rel=1e-14)
    assert ep["or"] == pytest.approx(0.28768207245178085, rel=1e-14)
    assert ep["nll"] == pytest.approx(LN2, rel=1e-15)
    assert ep["loss"] == pytest.approx(0.7219153878051234, rel=1e-14)
    assert ep["accuracy"] == 1.0 and ep["margin"] == pytest.approx(math.log(3.0), rel=1e-14)


def test_worked_pair_gradient_closed_form():
    # sigma(ln 3) = 3/4; F(ln 1/2) = 2, F(ln 1/4) = 4/3.
    lam = 0.1
    ep = orc.orpo_epilogue(np.array([math.log(0.5), math.log(0.25)]), lam)
    assert ep["dL_dell"][0] == pytest.approx(-1.0 - lam * 0.25 * 2.0, rel=1e-14)
    assert ep["dL_dell"][1] == pytest.approx(lam * 0.25 * (4.0 / 3.0), rel=1e-14)


def test_equal_branches_give_ln2_and_lambda_zero_is_nll():
    ep = orc.orpo_epilogue(np.array([-1.3, -1.3, -0.2, -0.2]), 0.5)
    assert ep["or"] == pytest.approx(LN2, rel=1e-15)
    assert ep["margin"] == 0.0 and ep["accuracy"] == 0.0
    ell = np.array([-1.0, -2.0, -3.0, -0.5])
    ep0 = orc.orpo_epilogue(ell, 0.0)
    assert ep0["loss"] == pytest.approx(2.0, rel=1e-15)      # -mean(lw) = (1 + 3)/2
    assert np.allclose(ep0["dL_dell"], [-0.5, 0.0, -0.5, 0.0])


def test_epilogue_matches_finite_differences():
    ell = np.array([-0.9, -1.7, -2.2, -0.4, -3.0, -3.5])
    lam = 0.37
    ep = orc.orpo_epilogue(ell, lam)
    for i in range(6):
        e = np.zeros(6)
        e[i] = 1e-6
        fd = (orc.orpo_epilogue(ell + e, lam)["loss"] - orc.orpo_epilogue(ell - e, lam)["loss"]) / 2e-6
        assert fd == pytest.approx(ep["dL_dell"][i], rel=1e-7, abs=1e-10)


def test_log1mexp_series_and_naive_agreement():
    for x in (-1e-3, -1e-6, -1e-9):   # x -> 0-: log(-x) + x/2 + x^2/24 (next term x^4/2880)
        v, c = orc.log1mexp(x)
        assert not c and v == pytest.approx(math.log(-x) + x / 2 + x * x / 24, rel=1e-15, abs=1e-15)
    for x in (-20.0, -30.0, -50.0):  # x -> -inf: -e^x - e^(2x)/2
        v, _ = orc.log1mexp(x)
        assert v == pytest.approx(-math.exp(x) - math.exp(2 * x) / 2, rel=1e-12)
    for x in np.linspace(-5, -0.7, 44):
        v, _ = orc.log1mexp(float(x))
        assert v == pytest.approx(math.log(1 - math.exp(x)), rel=1e-13)


def test_log1mexp_clamp():
    v, c = orc.log1mexp(-1e-14)
    assert c and v == math.log(1e-12)
    v, c = orc.log1mexp(0.0)
    assert c and v == math.log(1e-12)
    # A clamped branch still gives a finite loss and the documented slope-1 gradient.
    ep = orc.orpo_epilogue(np.array([0.0, -1.0]), 0.1)
    assert math.isfinite(ep["loss"]) and math.isfinite(ep["dL_dell"][0])


def test_extreme_log_odds_are_stable():
    ep = orc.orpo_epilogue(np.array([-0.01, -40.0]), 1.0)      # log_odds large positive
    assert 0 <= ep["or"] < 1e-3 and math.isfinite(ep["loss"])
    ep = orc.orpo_epilogue(np.array([-40.0, -0.01]), 1.0)      # large negative
    assert ep["or"] == pytest.approx(-ep["log_odds"][0], rel=1e-6)


# ----------------------------------------------------------------------------- whole step
def test_zero_weights_tiny_shape_loss_closed_form():
    # M=256, d=256, V=4096, one pair of 128+128: every ell = -ln V, log-odds 0 => L = ln V + lam ln 2.
    M, d, V, lam = 256, 256, 4096, 0.1
    h = _rng(12).standard_normal((M, d))
    labels = _rng(13).integers(0, V, size=M)
    out = orc.head_step(h, np.zeros((V, d)), labels, np.array([0, 128, 256]), 0.0, lam, want_dW=False)
    assert out["loss"] == pytest.approx(8.387080884775337, rel=1e-14)
    assert out["loss"] == pytest.approx(math.log(V) + lam * LN2, rel=1e-14)


def test_zero_weights_gradient_closed_form():
    # W = 0: p = 1/V, sech^2 = 1, dh = 0, dW_v = sum_t g_t (1[v = y_t] - 1/V) h_t, with
    # F(-ln V) = V/(V-1), sigma(0) = 1/2.
    rng = _rng(14)
    M, d, V, lam, P = 11, 3, 6, 0.3, 2
    h = rng.standard_normal((M, d))
    labels = rng.integers(0, V, size=M)
    labels[[2, 9, 10]] = -100
    off = np.array([0, 3, 5, 7, 9])
    out = orc.head_step(h, np.zeros((V, d)), labels, off, 2.0, lam)
    F = V / (V - 1)
    g = np.zeros(M)
    for b in range(4):
        ts = [t for t in range(off[b], off[b + 1]) if labels[t] != -100]
        dl = (-1 - lam * 0.5 * F) / P if b % 2 == 0 else lam * 0.5 * F / P
        g[ts] = dl / len(ts)
    dW = np.zeros((V, d))
    for t in range(M):
        if labels[t] != -100:
            for v in range(V):
                dW[v] += g[t] * ((v == labels[t]) - 1.0 / V) * h[t]
    assert np.allclose(out["g"], g, rtol=1e-14, atol=1e-16)
    assert np.all(out["dh"] == 0.0)
    assert np.allclose(out["dW"], dW, rtol=1e-13, atol=1e-15)


def _tiny_problem(seed, cap):
    rng = _rng(100 + seed)
    M, d, V = 12, 5, 9
    h = rng.standard_normal((M, d))
    W = rng.standard_normal((V, d)) * (1.5 if cap else 0.8)
    labels = rng.integers(0, V, size=M)
    labels[6] = -100            # ignored token inside branch 2
    labels[10:] = -100          # tail padding
    off = np.array([0, 3, 5, 8, 10])
    return h, W, labels, off


@pytest.mark.parametrize("cap,lam", list(itertools.product([0.0, 2.0], [0.0, 0.1, 1.0])))
def test_gradients_match_central_finite_differences(cap, lam):
    h, W, labels, off = _tiny_problem(int(cap * 10 + lam * 7), cap)
    out = orc.head_step(h, W, labels, off, cap, lam)
    eps = 1e-6

    def fd(arr, which):
        grad = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a = arr.copy()
            a[idx] += eps
            hp, wp = (a, W) if which == "h" else (h, a)
            lp = orc.loss_value(hp, wp, labels, off, cap, lam)
            a[idx] -= 2 * eps
            hm, wm = (a, W) if which == "h" else (h, a)
            lm = orc.loss_value(hm, wm, labels, off, cap, lam)
            grad[idx] = (lp - lm) / (2 * eps)
        return grad

    gh = fd(h, "h")
    gw = fd(W, "W")
    assert np.linalg.norm(out["dh"] - gh) <= 1e-6 * np.linalg.norm(gh)
    assert np.linalg.norm(out["dW"] - gw) <= 1e-6 * np.linalg.norm(gw)
    assert np.all(out["dh"][[6, 10, 11]] == 0.0)     # ignored / padding rows get no gradient


def test_cotangent_is_linear_in_lambda():
    h, W, labels, off = _tiny_problem(50, 2.0)
    g0 = orc.head_step(h, W, labels, off, 2.0, 0.0, want_dW=False)["g"]
    g1 = orc.head_step(h, W, labels, off, 2.0, 1.0, want_dW=False)["g"]
    g3 = orc.head_step(h, W, labels, off, 2.0, 0.3, want_dW=False)["g"]
    assert np.allclose(g3, g0 + 0.3 * (g1 - g0), rtol=1e-12, atol=1e-15)


def test_backward_without_dW_matches_dh():
    h, W, labels, off = _tiny_problem(51, 0.0)
    a = orc.head_step(h, W, labels, off, 0.0, 0.1)
    b = orc.head_step(h, W, labels, off, 0.0, 0.1, want_dW=False)
    assert b["dW"] is None and np.array_equal(a["dh"], b["dh"])


# ----------------------------------------------------------------------------- 4-bit weights
def _bf16_bits(x):
    return np.array(x, dtype=np.float32).view(np.uint32) >> 16


def test_q4_dequant_hand_packed():
    # Row 0: codes 0..15 then 15..0 in groups of 8 (word 0x76543210 holds codes 0..7 LSB-first).
    words = np.array([[0x76543210, 0xFEDCBA98, 0x89ABCDEF, 0x01234567] * 2,
                      [0x11111111] * 8,
                      [0xFFFFFFFF] * 8], dtype=np.uint32)
    scale = np.array([[_bf16_bits(0.5)], [0], [0x7F7F]], dtype=np.uint16)      # 0.5, 0, bf16 max
    bias = np.array([[_bf16_bits(-1.0)], [_bf16_bits(2.5)], [0]], dtype=np.uint16)
    w = orc.dequant_q4(words, scale, bias, 64)
    codes = list(range(16)) + list(range(15, -1, -1))
    assert np.array_equal(w[0], 0.5 * np.array(codes * 2, dtype=np.float64) - 1.0)
    assert np.all(w[1] == 2.5)                                  # scale 0 => w = bias
    bf16_max = float(np.array([0x7F7F0000], dtype=np.uint32).view(np.float32)[0])
    assert np.all(w[2] == 15 * bf16_max)


def test_q4_dequant_group_boundaries():
    V, d = 2, 128
    words = np.full((V, d // 8), 0x33333333, dtype=np.uint32)                # every code = 3
    scale = np.array([[_bf16_bits(1.0), _bf16_bits(2.0)]] * V, dtype=np.uint16)
    bias = np.array([[0, _bf16_bits(-0.25)]] * V, dtype=np.uint16)
    w = orc.dequant_q4(words, scale, bias, 64)
    assert np.all(w[:, :64] == 3.0) and np.all(w[:, 64:] == 5.75)


# ----------------------------------------------------------------------------- full-scope NLL
# Training — design, §1 "The objective", sft_scope `full`: the chosen sequence's NLL is the token
# mean of -logp over its supervised prompt positions and its response; the odds ratio keeps the
# response-only means.
def _full_problem(seed, cap, prompt_ignored=False):
    rng = _rng(300 + seed)
    M, d, V = 16, 5, 9
    h = rng.standard_normal((M, d))
    W = rng.standard_normal((V, d)) * (1.5 if cap else 0.8)
    labels = rng.integers(0, V, size=M)
    labels[1] = -100            # an ignored prompt position
    labels[9] = -100            # an ignored token of the second pair's chosen response
    labels[15] = -100           # tail padding
    off = np.array([0, 3, 5, 7, 8, 11, 14])   # pair 0: prompt 3, chosen 2, rejected 2; pair 1: 1, 3, 3
    if prompt_ignored:
        labels[7] = -100        # pair 1's prompt span holds no valid token
    return h, W, labels, off


def test_full_nll_is_the_pooled_token_mean():
    # Definition check without the combine formula: -mean of logp over the union of the prompt's
    # and the chosen response's valid tokens, per pair, then the mean over pairs.
    rng = _rng(7)
    logp = -rng.exponential(2.0, size=20)
    labels = rng.integers(0, 50, size=20)
    labels[[2, 11]] = -100
    off = np.array([0, 4, 9, 12, 13, 17, 20])
    mean, n = orc.span_means_full(logp, labels, off)
    ep = orc.orpo_epilogue_full(mean, n, 0.3)
    per_pair = []
    for p in range(2):
        toks = [t for t in range(off[3 * p], off[3 * p + 2]) if labels[t] != -100]
        per_pair.append(-float(np.mean(logp[toks])))
    assert ep["nll"] == pytest.approx(np.mean(per_pair), rel=1e-14)
    # The odds-ratio side and the metrics use the response means only.
    ell = np.array([mean[1], mean[2], mean[4], mean[5]])
    ref = orc.orpo_epilogue(ell, 0.3)
    for k in ("or", "accuracy", "margin"):
        assert ep[k] == pytest.approx(ref[k], rel=1e-15, abs=1e-15)
    assert ep["loss"] == pytest.approx(ep["nll"] + 0.3 * ref["or"], rel=1e-15)


def test_full_scope_worked_values():
    # Prompt logp = ln 1/2 at three positions, chosen ln 1/4 at one, rejected ln 1/4 at two:
    # NLL = (3 ln 2 + ln 4) / 4 = 5 ln2 / 4; lw = lr => log-odds 0, L_OR = ln 2, accuracy 0.
    logp = np.log([0.5, 0.5, 0.5, 0.25, 0.25, 0.25])
    labels = np.zeros(6, dtype=np.int64)
    mean, n = orc.span_means_full(logp, labels, [0, 3, 4, 6])
    ep = orc.orpo_epilogue_full(mean, n, 0.5)
    assert ep["nll"] == pytest.approx(5 * LN2 / 4, rel=1e-15)
    assert ep["or"] == pytest.approx(LN2, rel=1e-15)
    assert ep["loss"] == pytest.approx(5 * LN2 / 4 + 0.5 * LN2, rel=1e-15)
    assert ep["accuracy"] == 0.0 and ep["margin"] == pytest.approx(0.0, abs=1e-15)
    # dL/dpm = -3/4, so every prompt token's cotangent is -1/4 (one pair).
    g = orc.token_cotangent_full(ep["dL_dmean"], n, labels, [0, 3, 4, 6])
    assert np.allclose(g[:3], -0.25, rtol=0, atol=1e-15)


def test_empty_prompt_reduces_to_response_scope():
    # With no valid prompt position the full scope is the response scope: same loss and metrics (the
    # combine's n_w lw / n_w may round differently in the last place) and the same cotangent.
    h, W, labels, off = _full_problem(1, 2.0, prompt_ignored=True)
    labels[[0, 2]] = -100                  # pair 0's prompt fully ignored as well
    full = orc.head_step_full(h, W, labels, off, 2.0, 0.2)
    # Response-scope branches chosen_0, rejected_0, chosen_1, rejected_1; pair 1's ignored prompt
    # position (off[3]) falls inside chosen_1's range and counts for nothing.
    resp = orc.head_step(h, W, labels, off[[1, 2, 3, 5, 6]], 2.0, 0.2)
    for k in ("loss", "nll", "or", "accuracy", "margin"):
        assert full[k] == pytest.approx(resp[k], rel=4e-16, abs=0), k
    assert np.array_equal(full["g"], resp["g"])
    assert np.array_equal(full["dh"], resp["dh"]) and np.array_equal(full["dW"], resp["dW"])


@pytest.mark.parametrize("cap,lam", [(0.0, 0.1), (2.0, 0.0), (2.0, 1.0)])
def test_full_scope_gradients_match_central_finite_differences(cap, lam):
    h, W, labels, off = _full_problem(int(cap * 10 + lam * 7), cap)
    out = orc.head_step_full(h, W, labels, off, cap, lam)
    eps = 1e-6

    def fd(arr, which):
        grad = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a = arr.copy()
            a[idx] += eps
            hp, wp = (a, W) if which == "h" else (h, a)
            lp = orc.loss_value_full(hp, wp, labels, off, cap, lam)
            a[idx] -= 2 * eps
            hm, wm = (a, W) if which == "h" else (h, a)
            lm = orc.loss_value_full(hm, wm, labels, off, cap, lam)
            grad[idx] = (lp - lm) / (2 * eps)
        return grad

    gh = fd(h, "h")
    gw = fd(W, "W")
    assert np.linalg.norm(out["dh"] - gh) <= 1e-6 * np.linalg.norm(gh)
    assert np.linalg.norm(out["dW"] - gw) <= 1e-6 * np.linalg.norm(gw)
    assert np.all(out["dh"][[1, 9, 15]] == 0.0)
    assert np.all(out["dh"][[0, 2, 7]] != 0.0)       # prompt positions now carry gradient


def test_full_scope_span_errors():
    logp = np.full(6, -1.0)
    labels = np.zeros(6, dtype=np.int64)
    with pytest.raises(orc.OracleError):
        orc.span_means_full(logp, labels, [0, 2, 4])          # not 3P spans
    labels[2:4] = -100
    with pytest.raises(orc.OracleError):
        orc.span_means_full(logp, labels, [0, 2, 4, 6])       # chosen response has no valid token


# ----------------------------------------------------------------------------- backward skips
# Steel flash-CCE — handoff, Glossary E: the coefficient filter drops gradient-GEMM chunks whose
# whole coefficient block is below eps.
def _filter_problem(seed, M=300, d=6, V=200, cap=2.0):
    rng = _rng(500 + seed)
    h = rng.standard_normal((M, d))
    W = rng.standard_normal((V, d)) * 2.0
    labels = rng.integers(0, V, size=M)
    labels[5] = -100
    logp, lse = orc.forward(h, W, labels, cap)
    g = rng.standard_normal(M) * 1e-2
    g[labels == -100] = 0.0
    return h, W, labels, lse, g, cap


def test_filter_eps_zero_is_the_exact_backward():
    h, W, labels, lse, g, cap = _filter_problem(1)
    dh, dW = orc.backward(h, W, labels, lse, g, cap)
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, lse, g, cap, 0.0)
    assert kh == 1.0 and kw == 1.0
    assert np.allclose(fh, dh, rtol=1e-12, atol=1e-15) and np.allclose(fw, dW, rtol=1e-12, atol=1e-15)


def test_filter_huge_eps_drops_everything():
    h, W, labels, lse, g, cap = _filter_problem(2)
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, lse, g, cap, 1e9)
    assert kh == 0.0 and kw == 0.0 and np.all(fh == 0) and np.all(fw == 0)


def test_filter_drops_exactly_the_quiet_blocks():
    # Tokens 256.. (the second 256-token block, ragged: 44 tokens) get a negligible cotangent: every
    # dh block of theirs is dropped, every other dh row is exact; dW loses exactly their terms.
    h, W, labels, lse, g, cap = _filter_problem(3)
    g[256:] *= 1e-9
    eps = 1e-8
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, lse, g, cap, eps)
    dh, _ = orc.backward(h, W, labels, lse, g, cap)
    g0 = g.copy()
    g0[256:] = 0.0
    _, dW0 = orc.backward(h, W, labels, lse, g0, cap)
    assert np.all(fh[256:] == 0) and np.allclose(fh[:256], dh[:256], rtol=1e-12, atol=1e-15)
    assert np.allclose(fw, dW0, rtol=1e-9, atol=1e-15)
    assert kh == pytest.approx(0.5) and 0 < kw < 1     # 2 of 4 token-block rows x 4 vocab slices


def test_filter_kept_fraction_is_monotone_in_eps():
    h, W, labels, lse, g, cap = _filter_problem(4)
    prev = (1.0, 1.0)
    for eps in (1e-9, 1e-7, 1e-5, 1e-4, 1e-3):
        _, _, kh, kw = orc.backward_filtered(h, W, labels, lse, g, cap, eps)
        assert kh <= prev[0] and kw <= prev[1]
        prev = (kh, kw)


def test_filter_block_geometry_differs_for_dh_and_dw():
    # Vocabulary entries 64..127 get very negative logits and no label: their coefficients are
    # negligible for every token. dh's blocks (256 tokens x 64 entries) over that slice are all
    # quiet and dropped; dW's blocks (64 tokens x 256 entries) also hold entries 0..63 and are kept.
    h, W, labels, lse, g, cap = _filter_problem(5, cap=0.0)
    W[64:128] = 0.0
    W[64:128, 0] = -1e3 / np.abs(h[:, 0]).min()        # raw <= -1000 for every token
    h[:, 0] = np.abs(h[:, 0])
    labels[(labels >= 64) & (labels < 128)] = 3
    logp, lse = orc.forward(h, W, labels, cap)
    eps = 1e-12
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, lse, g, cap, eps)
    dh, dW = orc.backward(h, W, labels, lse, g, cap)
    assert kw == 1.0 and kh == pytest.approx(3 / 4)
    assert np.allclose(fw, dW, rtol=1e-12, atol=1e-15)
    assert np.allclose(fh, dh, rtol=1e-9, atol=1e-12)  # what is dropped is negligible here too
    fh2, _, kh2, _ = orc.backward_filtered(h, W, labels, lse, g, cap, eps, k_slice=128)
    assert kh2 == 1.0                                  # a 128-wide slice is no longer quiet


def test_filter_material_drops_follow_each_gemms_blocks():
    # Cotangent 1 on tokens 0..63, 1e-6 elsewhere; eps = 1e-3 sits between the two scales.
    # dW's blocks are 64 tokens x 256 entries: only tokens 0..63 survive, so dW is exactly their
    # contribution. dh's blocks are 256 tokens x 64 entries: the first token block keeps every
    # slice that token 0..63 make loud (with the quiet tokens' small terms), the ragged second
    # block (tokens 256..299) is dropped whole.
    h, W, labels, lse, g, cap = _filter_problem(6)
    g[:] = 1e-6
    g[:64] = 1.0
    g[labels == -100] = 0.0
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, lse, g, cap, 1e-3)
    g_loud = np.where(np.arange(len(g)) < 64, g, 0.0)
    _, dW_loud = orc.backward(h, W, labels, lse, g_loud, cap)
    assert np.allclose(fw, dW_loud, rtol=1e-12, atol=1e-15)
    dh, _ = orc.backward(h, W, labels, lse, g, cap)
    assert np.all(fh[256:] == 0.0)
    # Rows 64..255 keep their (tiny) terms in the slices that stay: exact there, nonzero.
    assert np.allclose(fh[:64], dh[:64], rtol=1e-6, atol=1e-12)
    assert np.any(fh[64:256] != 0.0)


def test_filter_decides_on_the_block_maximum():
    # One loud token (cotangent 1) in a block of quiet ones: its label entry's coefficient (about
    # 1 - p) keeps that (256-token, 64-entry) block although the block's mean is far below eps.
    h, W, labels, lse, g, cap = _filter_problem(7)
    g[:] = 0.0
    g[0] = 1.0
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, lse, g, cap, 1e-3)
    dh, dW = orc.backward(h, W, labels, lse, g, cap)
    assert np.linalg.norm(fh[0] - dh[0]) <= 0.05 * np.linalg.norm(dh[0])
    assert np.linalg.norm(fw - dW) <= 0.05 * np.linalg.norm(dW)
    assert 0 < kh < 1
