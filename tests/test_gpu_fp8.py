"""The FP8 head on the GPU (row-wise E4M3 logit operands, an opt-in approximation of the bf16 head).

Parity is against the oracle evaluating the same definition (oracle/fp8.py): the quantised codes
and row exponents bit for bit; logp, lse, the branch means and the loss terms within 1e-3 and dh,
dW within 1e-2, with the oracle quantising h and W itself and taking its logits from the
dequantised operands and its gradient products from the bf16 ones. Small ragged shapes compare
every output; the e4b shape compares sampled rows (forward) and a g-sparse backward probe. The
approximation's distance from the exact head is measured separately and only loosely bounded.
"""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from oracle import fp8
from oracle import orpo_oracle as orc
from tests.gpu_helpers import TOL_GRAD, TOL_SCALAR, assert_parity, dev, rel, say

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().numpy().astype(np.float64)


def _oracle_fp8_step(inp, want_dW=True):
    """The oracle's FP8 step: logits (forward, loss, g) from the dequantised operands, gradient
    products with the bf16 h and W."""
    cfg = inp.cfg
    h, W = _f64(inp.h), _f64(inp.w)
    hq, he = fp8.quantize_rows(h)
    wq, we = fp8.quantize_rows(W)
    h_l, W_l = fp8.dequantize_rows(hq, he), fp8.dequantize_rows(wq, we)
    ora = orc.head_step(h_l, W_l, inp.labels, inp.seg_offsets, cfg.softcap, cfg.lam, want_dW=False)
    ora["dh"], ora["dW"] = orc.backward(h, W, inp.labels, ora["lse"], ora["g"], cfg.softcap,
                                        want_dW=want_dW, logit_operands=(h_l, W_l))
    return ora


def _gpu_fp8_step(inp, want_dW=True, dh_bf16=False):
    d = dev()
    cfg = inp.cfg
    h, w = inp.h.to(d), inp.w.to(d)
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    st = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, want_dW=want_dW, fp8=True,
                    dh_bf16=dh_bf16)
    st.step()
    torch.cuda.synchronize()
    P = cfg.pairs
    o = st.out.cpu().numpy()
    return st, {
        "logp": st.logp.cpu().numpy(), "lse": st.lse.cpu().numpy(), "g": st.g.cpu().numpy(),
        "loss": o[0], "nll": o[1], "or": o[2], "accuracy": o[3], "margin": o[4],
        "lw": o[5:5 + P], "lr": o[5 + P:5 + 2 * P],
        "dh": st.dh.float().cpu().numpy(), "dW": None if st.dW is None else st.dW.cpu().numpy(),
    }


def test_quantisation_matches_the_oracle_bit_for_bit():
    rng = np.random.default_rng(5)
    R, C = 70, 264
    x = rng.standard_normal((R, C)) * np.exp2(rng.integers(-40, 40, (R, 1)))
    x[0] = 0.0                                                    # all-zero row: exponent 0
    x[1, :] = 0.0
    x[1, ::2] = -0.0                                              # signed zeros
    x[1, 5] = 3.0
    x[2, :8] = [448.0, 1.0625, 1.1875, -1.0625, 7.5 * 2.0 ** -9, 0.5 * 2.0 ** -9,
                -0.5 * 2.0 ** -9, 0.875 * 2.0 ** -6]              # amax 448: e = 0, ties on codes
    x[3] *= 2.0 ** -100                                           # exponent clamped at -127
    x[4] = x[4] * 0 + np.linspace(-1, 1, C) * 2.0 ** 100          # large row scale
    xb = torch.from_numpy(x).to(torch.bfloat16)
    ref_q, ref_e = fp8.quantize_rows(_f64(xb))
    say(f"[fp8 quant] R={R} C={C}")
    q, e = H.quantize_fp8(xb.to(dev()))
    torch.cuda.synchronize()
    q, e = q.cpu().numpy(), e.cpu().numpy()
    assert np.array_equal(e, ref_e), np.nonzero(e != ref_e)
    bad = np.argwhere(q != ref_q)
    assert bad.size == 0, (bad[:5], q[tuple(bad[0])], ref_q[tuple(bad[0])])
    # Rows longer than the kernel holds in registers (read twice), and rows of one 8-value chunk.
    for shape in ((9, 4608), (5, 8)):
        xl = torch.from_numpy(rng.standard_normal(shape) * 3.0).to(torch.bfloat16)
        rq, re_ = fp8.quantize_rows(_f64(xl))
        ql, el = H.quantize_fp8(xl.to(dev()))
        torch.cuda.synchronize()
        assert np.array_equal(el.cpu().numpy(), re_) and np.array_equal(ql.cpu().numpy(), rq), shape
    # An e4b-sized weight (262144 x 2560, entries N(0, (3 / sqrt(d))^2) as the workloads draw
    # them), exactly, in blocks.
    V, dd = 262144, 2560
    gen = torch.Generator().manual_seed(3)
    wt = (torch.randn(V, dd, generator=gen) * (3.0 / dd ** 0.5)).to(torch.bfloat16)
    wq, we = H.quantize_fp8(wt.to(dev()))
    torch.cuda.synchronize()
    wq, we = wq.cpu().numpy(), we.cpu().numpy()
    for r0 in range(0, V, 65536):
        rq, re_ = fp8.quantize_rows(_f64(wt[r0:r0 + 65536]))
        assert np.array_equal(we[r0:r0 + 65536], re_) and np.array_equal(wq[r0:r0 + 65536], rq), r0


CASES = [
    # (M, d, V, pairs, len_lo, len_hi, cap)
    (600, 256, 3000, 2, 100, 150, 30.0),      # ragged M and V, two chunks of tiles
    (512, 384, 4096, 2, 100, 128, 0.0),       # no softcap, d = 3 x 128
    (1000, 128, 5000, 3, 100, 160, 30.0),     # one K step (d = 128), ragged V
    (300, 256, 100, 1, 100, 120, 30.0),       # V below one tile: every scale read past V
]


@pytest.mark.parametrize("M,d,V,pairs,lo,hi,cap", CASES)
def test_fp8_step_parity_small(M, d, V, pairs, lo, hi, cap):
    cfg = synth.HeadConfig(0, f"fp8-M{M}-d{d}-V{V}-cap{cap}", M=M, d=d, V=V, pairs=pairs,
                           len_lo=lo, len_hi=hi, softcap=cap, lam=0.1)
    inp = synth.make_inputs(cfg, seed=11)
    say(f"[fp8 parity] {cfg.name}")
    st, gpu = _gpu_fp8_step(inp)
    ora = _oracle_fp8_step(inp)
    assert H.read_status(st.fws) == 0
    assert_parity(gpu, ora, cfg.name)


def _fp8_random_cases(n, seed, budget=4e9):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([rng.integers(16, 128), rng.integers(128, 700), rng.integers(700, 1300)]))
        d = int(rng.choice([128, 256, 384, 512]))
        V = int(rng.choice([rng.integers(2, 600), rng.integers(600, 8000), rng.integers(8000, 30000)]))
        pairs = int(rng.integers(1, 4))
        cap = float(rng.choice([0.0, 30.0]))
        if M * V * d > budget or M < 4 * pairs:
            continue
        lo = max(1, M // (4 * pairs))
        out.append((M, d, V, pairs, lo, max(lo, M // (2 * pairs) - 1), cap))
    return out


@pytest.mark.parametrize("M,d,V,pairs,lo,hi,cap", _fp8_random_cases(6, 5081))
def test_fp8_step_parity_random_shapes(M, d, V, pairs, lo, hi, cap):
    # Seeded random shapes: a handful of tokens to over a thousand, vocabularies from one tile to
    # ~30k (the backward's dh tiles split 1 to 16 ways, the forward merged either way).
    test_fp8_step_parity_small(M, d, V, pairs, lo, hi, cap)


def test_fp8_step_dh_bf16_and_tiled_backward():
    cfg = synth.HeadConfig(0, "fp8-tiled", M=1024, d=256, V=4096, pairs=2, len_lo=200, len_hi=256,
                           softcap=30.0, lam=0.1)
    inp = synth.make_inputs(cfg, seed=12)
    try:
        H.set_bwd_tiling(256, 256 * 512 * 2)           # 4 token chunks x 8 vocabulary blocks
        _, a = _gpu_fp8_step(inp)
        _, b = _gpu_fp8_step(inp, dh_bf16=True)
    finally:
        H.set_bwd_tiling(0, 0)
    ora = _oracle_fp8_step(inp)
    assert_parity(a, ora, "fp8 tiled")
    ref = torch.from_numpy(a["dh"]).to(torch.bfloat16).float().numpy()
    assert np.array_equal(b["dh"], ref)                # the fp32 sums rounded once


def test_fp8_distance_from_the_exact_head():
    # The approximation itself (not a parity gate): FP8 vs the exact bf16 head on the GPU.
    cfg = synth.HeadConfig(0, "fp8-fidelity", M=1024, d=512, V=8192, pairs=2, len_lo=200,
                           len_hi=256, softcap=30.0, lam=0.1)
    inp = synth.make_inputs(cfg, seed=13)
    d = dev()
    h, w = inp.h.to(d), inp.w.to(d)
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    ex = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam)
    ap = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, fp8=True)
    ex.step()
    ap.step()
    torch.cuda.synchronize()
    e = {k: rel(getattr(ap, k).float().cpu().numpy(), getattr(ex, k).float().cpu().numpy())
         for k in ("logp", "lse", "dh", "dW")}
    e["loss"] = abs(float(ap.out[0]) - float(ex.out[0])) / abs(float(ex.out[0]))
    say("[fp8 fidelity] " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))
    # E4M3 keeps 3 mantissa bits: per-logit errors of a few percent of the logit spread, far
    # smaller after the softmax and the branch means.
    assert e["logp"] < 5e-2 and e["lse"] < 1e-2 and e["loss"] < 1e-2
    assert e["dh"] < 5e-2 and e["dW"] < 5e-2


def test_fp8_full_size_sampled_parity():
    cfg = synth.workload("e4b-bf16-softcap30")
    say(f"[fp8 fullsize] {cfg.name} M={cfg.M} d={cfg.d} V={cfg.V}")
    inp = synth.make_inputs(cfg, seed=0, label_device="cuda")
    d = dev()
    h, w = inp.h.to(d), inp.w.to(d)
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    st = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, fp8=True)
    st.forward()
    st.loss()
    torch.cuda.synchronize()
    assert H.read_status(st.fws) == 0 and H.read_status(st.lws) == 0
    logp = st.logp.cpu().numpy().astype(np.float64)
    lse = st.lse.cpu().numpy().astype(np.float64)
    g = st.g.cpu().numpy()
    hh, W = _f64(inp.h), _f64(inp.w)
    hq, he = fp8.quantize_rows(hh)
    wq, we = fp8.quantize_rows(W)
    h_l, W_l = fp8.dequantize_rows(hq, he), fp8.dequantize_rows(wq, we)
    del wq
    rng = np.random.default_rng(0)
    off_np = inp.seg_offsets
    rows = np.unique(np.concatenate([rng.integers(off_np[b], off_np[b + 1], 2)
                                     for b in range(len(off_np) - 1)] + [[cfg.M - 1]]))
    ref_logp, ref_lse = orc.forward(h_l[rows], W_l, inp.labels[rows], cfg.softcap)
    e_logp, e_lse = rel(logp[rows], ref_logp), rel(lse[rows], ref_lse)
    say(f"[fp8 fullsize] rows={len(rows)} logp={e_logp:.2e} lse={e_lse:.2e}")
    assert e_logp <= TOL_SCALAR and e_lse <= TOL_SCALAR
    # g-sparse backward probe: the coefficients of the probed rows only.
    probe = rows[inp.labels[rows] != -100][:6]
    gs = np.zeros(cfg.M, dtype=np.float32)
    gs[probe] = g[probe]
    st.g.copy_(torch.from_numpy(gs).to(d))
    st.backward()
    torch.cuda.synchronize()
    dh = st.dh.cpu().numpy()
    _, plse = orc.forward(h_l[probe], W_l, inp.labels[probe], cfg.softcap)
    rdh, rdW = orc.backward(hh[probe], W, inp.labels[probe], plse, gs[probe].astype(np.float64),
                            cfg.softcap, logit_operands=(h_l[probe], W_l))
    others = np.setdiff1d(np.arange(cfg.M), probe)
    assert np.all(dh[others] == 0.0)
    e_dh, e_dW = rel(dh[probe], rdh), rel(st.dW.cpu().numpy(), rdW)
    say(f"[fp8 fullsize] probe={len(probe)} dh={e_dh:.2e} dW={e_dW:.2e}")
    assert e_dh <= TOL_GRAD and e_dW <= TOL_GRAD


def test_fp8_step_with_the_coefficient_filter():
    # The FP8 head with skip_eps (filter + the cold-tile skip from the FP8 forward's per-tile
    # maxima) against the oracle's filtered backward on the same quantised logits. Peaked logits
    # (std 12 under the softcap), 95 % argmax labels, eps 1e-5.
    cfg = synth.HeadConfig(0, "fp8-peaked", M=1024, d=256, V=16384, pairs=2, len_lo=200,
                           len_hi=256, softcap=30.0, lam=0.1, w_std=12.0, p_argmax=0.95)
    inp = synth.make_inputs(cfg, 0, label_device="cuda")
    d = dev()
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    eps = 1e-5
    say("[fp8 filter] peaked eps=1e-5")
    st = H.HeadStep(inp.h.to(d), inp.w.to(d), labels, off, cfg.V, cfg.softcap, cfg.lam, fp8=True,
                    skip_eps=eps)
    st.step()
    torch.cuda.synchronize()
    hh, W = _f64(inp.h), _f64(inp.w)
    hq, he = fp8.quantize_rows(hh)
    wq, we = fp8.quantize_rows(W)
    ops = (fp8.dequantize_rows(hq, he), fp8.dequantize_rows(wq, we))
    ora = orc.head_step(ops[0], ops[1], inp.labels, inp.seg_offsets, cfg.softcap, cfg.lam,
                        want_dW=False)
    assert rel(st.logp.cpu().numpy(), ora["logp"]) <= TOL_SCALAR
    fh, fw, kh, kw = orc.backward_filtered(hh, W, inp.labels, ora["lse"], ora["g"], cfg.softcap, eps,
                                           logit_operands=ops)
    e_dh, e_dW = rel(st.dh.cpu().numpy(), fh), rel(st.dW.cpu().numpy(), fw)
    say(f"[fp8 filter] kept dh {kh:.3f} dW {kw:.3f}; vs oracle filtered dh={e_dh:.2e} dW={e_dW:.2e}")
    assert kh < 0.9 and kw < 0.9                        # the filter does drop blocks here
    assert e_dh <= TOL_GRAD and e_dW <= TOL_GRAD
