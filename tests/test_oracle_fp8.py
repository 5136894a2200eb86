"""Pins of the FP8 (E4M3) quantisation oracle and of the backward with separate logit operands.

The code table is pinned to the OCP 8-bit floating-point format's defining values (largest normal
S.1111.110 = 448, smallest normal S.0001.000 = 2^-6, smallest subnormal S.0000.001 = 2^-9, NaN
S.1111.111, no infinities) and to torch's float8_e4m3fn (an independent library routine) for every
code and for rounding at and between every pair of neighbouring codes. The row scale rule is pinned
by closed forms, quantisation by the round-to-nearest error bound, and the split backward by
central finite differences of the loss taken through the logit operands.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import orpo_oracle as orc


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(values_f32):
    t = torch.from_numpy(np.asarray(values_f32, dtype=np.float32).copy()).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_defining_values_of_the_format():
    d = fp8.e4m3_decode(np.array([0x7E, 0x08, 0x07, 0x01, 0x38, 0x00, 0x80, 0xFE, 0x40, 0x3C]))
    assert d[0] == 448.0 and d[1] == 2.0 ** -6 and d[2] == 0.875 * 2.0 ** -6 and d[3] == 2.0 ** -9
    assert d[4] == 1.0 and d[5] == 0.0 and d[6] == 0.0 and math.copysign(1.0, d[6]) == -1.0
    assert d[7] == -448.0 and d[8] == 2.0 and d[9] == 1.5
    assert np.isnan(fp8.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_every_code_matches_torch_float8_e4m3fn():
    codes = np.arange(256)
    ours, ref = fp8.e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_encode_round_trips_and_matches_torch_at_and_between_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = fp8.e4m3_decode(codes)
    assert np.array_equal(fp8.e4m3_encode(vals), codes.astype(np.uint8))
    # Midpoints between neighbouring positive values (ties: even code), and points a quarter and
    # three quarters of the way, all exact in float32; then the negatives.
    pos = np.sort(np.unique(vals[(vals >= 0) & ~np.signbit(vals)]))
    lo, hi = pos[:-1], pos[1:]
    probes = np.concatenate([lo + (hi - lo) * f for f in (0.25, 0.5, 0.75)])
    probes = np.concatenate([probes, -probes])
    assert np.array_equal(fp8.e4m3_encode(probes), _torch_encode(probes))
    rng = np.random.default_rng(7)
    r = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000))).astype(np.float32)
    r = np.clip(r, -448, 448)
    assert np.array_equal(fp8.e4m3_encode(r), _torch_encode(r))


def test_ties_go_to_the_even_code():
    assert fp8.e4m3_encode(np.array([1.0625]))[0] == 0x38      # between 1.0 (0x38) and 1.125 (0x39)
    assert fp8.e4m3_encode(np.array([1.1875]))[0] == 0x3A      # between 1.125 and 1.25 (0x3A)
    assert fp8.e4m3_encode(np.array([7.5 * 2.0 ** -9]))[0] == 0x08   # onto the smallest normal
    assert fp8.e4m3_encode(np.array([0.5 * 2.0 ** -9]))[0] == 0x00
    assert fp8.e4m3_encode(np.array([-0.5 * 2.0 ** -9]))[0] == 0x80   # sign kept on a zero
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([448.5]))


def test_row_exponent_closed_forms():
    assert fp8.row_exponent(448.0) == 0
    assert fp8.row_exponent(448.5) == 1
    assert fp8.row_exponent(224.0) == -1
    assert fp8.row_exponent(224.5) == 0
    assert fp8.row_exponent(1.0) == -8            # 448 / 512 = 0.875 < 1 <= 1.75
    assert fp8.row_exponent(1.75) == -8 and fp8.row_exponent(1.78125) == -7
    assert fp8.row_exponent(0.0) == 0
    assert fp8.row_exponent(2.0 ** -133) == -127  # clamped to the smallest E8M0 exponent
    for e in range(-100, 100, 7):
        assert fp8.row_exponent(math.ldexp(448.0, e)) == e


def test_quantize_rows_error_bound_and_scale_placement():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 256)) * np.exp2(rng.integers(-20, 20, (40, 1)))
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()   # bf16 values, as h and W
    codes, exps = fp8.quantize_rows(x)
    deq = fp8.dequantize_rows(codes, exps)
    e = exps.astype(np.int64) - 127
    amax = np.abs(x).max(axis=1)
    scaled = amax * np.exp2(-e.astype(np.float64))
    assert np.all(scaled <= 448.0) and np.all(scaled > 224.0)
    # Round to nearest: half a unit in the last place, 2^-4 relative in the normal range and
    # 2^-10 2^e absolute in the subnormal range.
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.exp2(e.astype(np.float64) - 10.0)[:, None])
    assert np.all(err <= bound)
    assert np.array_equal(np.signbit(deq[x != 0]), np.signbit(x[x != 0]))


def test_quantize_rows_is_the_identity_on_representable_rows():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (12, 64)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    codes[:, 0] = 0x7E                                   # each row reaches 448 (scale exponent e)
    e = rng.integers(-30, 30, 12)
    x = fp8.dequantize_rows(codes, (e + 127).astype(np.uint8))
    q, ex = fp8.quantize_rows(x)
    assert np.array_equal(ex.astype(np.int64) - 127, e)
    assert np.array_equal(fp8.dequantize_rows(q, ex), x)
    zero_q, zero_e = fp8.quantize_rows(np.zeros((2, 8)))
    assert np.all(zero_q == 0) and np.all(zero_e == 127)


def _tiny(seed, cap):
    rng = np.random.default_rng(seed)
    M, d, V = 10, 6, 9
    h = rng.standard_normal((M, d))
    W = rng.standard_normal((V, d))
    labels = rng.integers(0, V, M)
    labels[4] = -100
    off = np.array([0, 3, 5, 8, 10])
    return h, W, labels, off


@pytest.mark.parametrize("cap", [0.0, 2.0])
def test_split_backward_matches_finite_differences_through_the_logit_operands(cap):
    h, W, labels, off = _tiny(11, cap)
    rng = np.random.default_rng(12)
    h_l = h + 0.05 * rng.standard_normal(h.shape)      # logit operands near, not equal to, h and W
    W_l = W + 0.05 * rng.standard_normal(W.shape)
    lam = 0.3
    ref = orc.head_step(h_l, W_l, labels, off, cap, lam)   # g and lse from the logit operands
    # dh with W = W_l, and dW with h = h_l, are the true gradients of the loss through (h_l, W_l).
    dh, _ = orc.backward(h, W_l, labels, ref["lse"], ref["g"], cap, logit_operands=(h_l, W_l))
    _, dW = orc.backward(h_l, W, labels, ref["lse"], ref["g"], cap, logit_operands=(h_l, W_l))
    eps = 1e-6

    def fd(arr, which):
        grad = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a = arr.copy()
            a[idx] += eps
            lp = orc.loss_value(a, W_l, labels, off, cap, lam) if which == "h" else \
                orc.loss_value(h_l, a, labels, off, cap, lam)
            a[idx] -= 2 * eps
            lm = orc.loss_value(a, W_l, labels, off, cap, lam) if which == "h" else \
                orc.loss_value(h_l, a, labels, off, cap, lam)
            grad[idx] = (lp - lm) / (2 * eps)
        return grad

    gh, gw = fd(h_l, "h"), fd(W_l, "W")
    assert np.linalg.norm(dh - gh) <= 1e-6 * np.linalg.norm(gh)
    assert np.linalg.norm(dW - gw) <= 1e-6 * np.linalg.norm(gw)
    # The gradient products take the given h and W: dh is linear in W, dW in h, at fixed logits.
    W2 = rng.standard_normal(W.shape)
    h2 = rng.standard_normal(h.shape)
    a1, b1 = orc.backward(h, W, labels, ref["lse"], ref["g"], cap, logit_operands=(h_l, W_l))
    a2, b2 = orc.backward(h2, W2, labels, ref["lse"], ref["g"], cap, logit_operands=(h_l, W_l))
    a3, b3 = orc.backward(h + h2, W + W2, labels, ref["lse"], ref["g"], cap,
                          logit_operands=(h_l, W_l))
    assert np.allclose(a1 + a2, a3, rtol=1e-12, atol=1e-14)
    assert np.allclose(b1 + b2, b3, rtol=1e-12, atol=1e-14)
    assert not np.allclose(a1, a2)


@pytest.mark.parametrize("cap", [0.0, 2.0])
def test_filtered_backward_with_logit_operands_reduces_to_its_special_cases(cap):
    h, W, labels, off = _tiny(21, cap)
    rng = np.random.default_rng(22)
    h_l = h + 0.05 * rng.standard_normal(h.shape)
    W_l = W + 0.05 * rng.standard_normal(W.shape)
    ref = orc.head_step(h_l, W_l, labels, off, cap, 0.2)
    ops = (h_l, W_l)
    dh, dW = orc.backward(h, W, labels, ref["lse"], ref["g"], cap, logit_operands=ops)
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, ref["lse"], ref["g"], cap, 0.0,
                                           tok_block=4, k_slice=2, logit_operands=ops)
    assert kh == 1.0 and kw == 1.0                      # eps = 0: the split backward itself
    assert np.allclose(fh, dh, rtol=1e-12, atol=1e-15) and np.allclose(fw, dW, rtol=1e-12, atol=1e-15)
    fh, fw, kh, kw = orc.backward_filtered(h, W, labels, ref["lse"], ref["g"], cap, 1e9,
                                           tok_block=4, k_slice=2, logit_operands=ops)
    assert kh == 0.0 and kw == 0.0 and np.all(fh == 0) and np.all(fw == 0)
    # A middle eps keeps some blocks, decided on the coefficients of the logit operands: the same
    # call without them (logits from h and W) keeps a different set here.
    eps = np.quantile(np.abs(ref["g"][ref["g"] != 0]), 0.5) * 0.05
    a = orc.backward_filtered(h, W, labels, ref["lse"], ref["g"], cap, eps, tok_block=4, k_slice=2,
                              logit_operands=ops)
    b = orc.backward_filtered(h, W, labels, ref["lse"], ref["g"], cap, eps, tok_block=4, k_slice=2)
    assert 0.0 < a[2] < 1.0
    assert not np.allclose(a[0], b[0])
