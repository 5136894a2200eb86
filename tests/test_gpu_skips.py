"""GPU parity for the backward's coefficient filter (orpo_head_desc.skip_eps > 0): the HIP
backward against the oracle's filtered backward (the same block definition, in float64), plus the
exact path's invariance. The filter is an approximation; its distance from the exact backward is
reported (fidelity) and gated loosely on peaked data."""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from oracle import orpo_oracle as orc
from tests.gpu_helpers import TOL_GRAD, dev, mfma_operand_weight, oracle_weight, rel, say

pytestmark = pytest.mark.gpu


def _custom(M, d, V, cap, seed, w_std=3.0):
    rng = np.random.default_rng(seed)
    h = synth.to_bf16(rng.standard_normal((M, d)))
    w = synth.to_bf16((rng.standard_normal((V, d)) * (w_std / np.sqrt(d))).astype(np.float32))
    labels = rng.integers(0, V, size=M).astype(np.int32)
    labels[M - 3:] = -100
    labels[10] = -100
    return h, w, labels


def _gpu_bwd(h, w, labels, lse_o, g, cap, eps, scales=None, biases=None, want_dW=True):
    d = dev()
    lab = torch.from_numpy(labels).to(d)
    lse = torch.from_numpy(lse_o.astype(np.float32)).to(d)
    gg = torch.from_numpy(g.astype(np.float32)).to(d)
    dh, dW = H.head_bwd(h.to(d), w.to(d), lab, lse, gg, cap, want_dW=want_dW,
                        scales=None if scales is None else scales.to(d),
                        biases=None if biases is None else biases.to(d), skip_eps=eps)
    torch.cuda.synchronize()
    return dh.cpu().numpy(), (None if dW is None else dW.cpu().numpy())


def test_tiny_eps_is_bitwise_the_exact_backward():
    h, w, labels = _custom(700, 192, 3001, 30.0, seed=1)
    hh, W = h.float().numpy().astype(np.float64), w.float().numpy().astype(np.float64)
    _, lse = orc.forward(hh, W, labels, 30.0)
    g = np.random.default_rng(2).standard_normal(700) * 1e-3
    g[labels == -100] = 0
    a = _gpu_bwd(h, w, labels, lse, g, 30.0, 0.0)
    b = _gpu_bwd(h, w, labels, lse, g, 30.0, 1e-30)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_filter_matches_the_oracles_filtered_backward():
    # Loud cotangent on tokens 0..63 and 300..363, 1e-6 elsewhere; eps = 1e-3 between the two: the
    # quiet token block 512..699 is dropped from dh whole, dW keeps only the loud 64-token slices.
    h, w, labels = _custom(700, 192, 3001, 30.0, seed=3)
    hh, W = h.float().numpy().astype(np.float64), w.float().numpy().astype(np.float64)
    _, lse = orc.forward(hh, W, labels, 30.0)
    g = np.full(700, 1e-6)
    g[:64] = 1.0
    g[300:364] = -0.5
    g[labels == -100] = 0
    eps = 1e-3
    dh, dW = _gpu_bwd(h, w, labels, lse, g, 30.0, eps)
    fh, fw, kh, kw = orc.backward_filtered(hh, W, labels, lse, g, 30.0, eps)
    e_dh, e_dW = rel(dh, fh), rel(dW, fw)
    say(f"[filter] kept dh {kh:.3f} dW {kw:.3f}; vs oracle filtered dh={e_dh:.2e} dW={e_dW:.2e}")
    assert e_dh <= TOL_GRAD and e_dW <= TOL_GRAD
    assert np.all(dh[512:] == 0.0)                      # the dropped token block
    ex_dh, _ = orc.backward(hh, W, labels, lse, g, 30.0)
    assert np.any(ex_dh[512:697] != 0.0)                 # ... which the exact backward fills


@pytest.mark.parametrize("chunked", [False, True])
def test_filter_on_peaked_data(chunked):
    # Peaked logits (std 12 under the softcap), 95 % argmax labels, the ORPO cotangent, eps 1e-5.
    cfg = synth.HeadConfig(0, "peaked-small", M=1024, d=256, V=16384, pairs=2, len_lo=200,
                           len_hi=256, softcap=30.0, lam=0.1, w_std=12.0, p_argmax=0.95)
    inp = synth.make_inputs(cfg, 0, label_device="cuda")
    hh, W = inp.h.float().numpy().astype(np.float64), oracle_weight(inp)
    ora = orc.head_step(hh, W, inp.labels, inp.seg_offsets, cfg.softcap, cfg.lam)
    eps = 1e-5
    say(f"[case] filter peaked chunked={chunked}")
    if chunked:
        H.set_bwd_tiling(256, 256 * 2048 * 2)          # 4 token chunks x 8 vocabulary blocks
    try:
        dh, dW = _gpu_bwd(inp.h, inp.w, inp.labels, ora["lse"], ora["g"], cfg.softcap, eps)
    finally:
        H.set_bwd_tiling(0, 0)
    fh, fw, kh, kw = orc.backward_filtered(hh, W, inp.labels, ora["lse"], ora["g"], cfg.softcap, eps)
    e_dh, e_dW = rel(dh, fh), rel(dW, fw)
    f_dh, f_dW = rel(dh, ora["dh"]), rel(dW, ora["dW"])
    say(f"[filter peaked] kept dh {kh:.3f} dW {kw:.3f}; vs filtered dh={e_dh:.2e} dW={e_dW:.2e}; "
        f"fidelity vs exact dh={f_dh:.2e} dW={f_dW:.2e}")
    assert kh < 0.9 and kw < 0.9                        # the filter does drop blocks here
    assert e_dh <= TOL_GRAD and e_dW <= TOL_GRAD
    assert f_dh <= 5e-2 and f_dW <= 5e-2


def test_filter_with_4bit_weights():
    cfg = synth.HeadConfig(0, "peaked-q4", M=512, d=256, V=4096, pairs=1, len_lo=200,
                           len_hi=256, softcap=30.0, lam=0.1, q4=True, w_std=12.0, p_argmax=0.95)
    inp = synth.make_inputs(cfg, 0, label_device="cuda")
    hh, W = inp.h.float().numpy().astype(np.float64), oracle_weight(inp)
    ora = orc.head_step(hh, W, inp.labels, inp.seg_offsets, cfg.softcap, cfg.lam, want_dW=False)
    eps = 1e-5
    w = torch.from_numpy(inp.wq.view(np.int32))
    dh, _ = _gpu_bwd(inp.h, w, inp.labels, ora["lse"], ora["g"], cfg.softcap, eps,
                     scales=inp.scales, biases=inp.biases, want_dW=False)
    fh, _, kh, _ = orc.backward_filtered(hh, W, inp.labels, ora["lse"], ora["g"], cfg.softcap, eps)
    e = rel(dh, fh)
    say(f"[filter q4] kept dh {kh:.3f} vs filtered dh={e:.2e}")
    assert e <= TOL_GRAD


def test_q4_filter_running_max_odd_k_steps():
    # The 4-bit head with the filter and the cold-tile skip under a softcap of 50 (the forward's
    # running maximum with per-tile maxima) and d = 192 (three K steps, padded to four with zeros):
    # the forward at parity with the oracle on the MFMA's operands, the backward equal to the
    # filter-only result bit for bit and to the oracle's filtered backward within the gate.
    cfg = synth.HeadConfig(0, "peaked-q4-cap50-d192", M=512, d=192, V=4096, pairs=1, len_lo=200,
                           len_hi=256, softcap=50.0, lam=0.1, q4=True, w_std=12.0, p_argmax=0.95)
    inp = synth.make_inputs(cfg, 0, label_device="cuda")
    d = dev()
    hh = inp.h.float().numpy().astype(np.float64)
    Wop = mfma_operand_weight(inp)
    h, lab = inp.h.to(d), torch.from_numpy(inp.labels).to(d)
    w = torch.from_numpy(inp.wq.view(np.int32)).to(d)
    sc, bi = inp.scales.to(d), inp.biases.to(d)
    eps = 1e-5
    logp, lse, fws = H.head_fwd(h, w, lab, cfg.softcap, scales=sc, biases=bi, return_ws=True,
                                skip_eps=eps)
    torch.cuda.synchronize()
    assert H.read_status(fws) == 0
    lp_o, lse_o = orc.forward(hh, Wop, inp.labels, cfg.softcap)
    ok = inp.labels != -100
    e_lp = float(np.max(np.abs(logp.cpu().numpy()[ok] - lp_o[ok]) / (np.abs(lp_o[ok]) + 1.0)))
    e_lse = float(np.max(np.abs(lse.cpu().numpy() - lse_o) / (np.abs(lse_o) + 1.0)))
    say(f"[q4 cap50 d192] forward logp {e_lp:.2e} lse {e_lse:.2e}")
    assert e_lp <= 1e-4 and e_lse <= 1e-4
    g = np.random.default_rng(5).standard_normal(cfg.M) * 1e-2
    g[~ok] = 0
    gg = torch.from_numpy(g.astype(np.float32)).to(d)
    dh0, _ = H.head_bwd(h, w, lab, lse, gg, cfg.softcap, want_dW=False, scales=sc, biases=bi,
                        skip_eps=eps)
    dh1, _ = H.head_bwd(h, w, lab, lse, gg, cfg.softcap, want_dW=False, scales=sc, biases=bi,
                        skip_eps=eps, fwd_ws=fws)
    torch.cuda.synchronize()
    assert torch.equal(dh0, dh1)
    fh, _, kh, _ = orc.backward_filtered(hh, Wop, inp.labels, lse.cpu().numpy().astype(np.float64),
                                         g, cfg.softcap, eps)
    e = rel(dh0.cpu().numpy(), fh)
    say(f"[q4 cap50 d192] kept dh {kh:.3f}; vs filtered dh={e:.2e}")
    assert e <= TOL_GRAD


def test_filter_is_rejected_for_fp32():
    d = dev()
    h = torch.zeros(256, 64, device=d)
    w = torch.zeros(512, 64, device=d)
    lab = torch.zeros(256, dtype=torch.int32, device=d)
    z = torch.zeros(256, device=d)
    with pytest.raises(H.OrpoError):
        H.head_bwd(h, w, lab, z, z, 0.0, skip_eps=1e-5)


def test_cold_tile_skip_is_exact_for_the_filter_and_skips_tiles():
    # With the forward's workspace the backward also skips whole cold coefficient tiles; the filter
    # would drop all of their blocks, so dh and dW equal the filter-only result bit for bit. The
    # skipped tiles leave their part of the coefficient buffer untouched (a sentinel fill shows it).
    import ctypes
    d = dev()
    # 256 vocabulary tiles, so a 256-token tile's labels leave many of them label-free.
    cfg = synth.HeadConfig(0, "peaked-cold", M=1024, d=256, V=65536, pairs=2, len_lo=200,
                           len_hi=256, softcap=30.0, lam=0.1, w_std=12.0, p_argmax=0.95)
    inp = synth.make_inputs(cfg, 0, label_device="cuda")
    eps = 1e-4
    h, w = inp.h.to(d), inp.w.to(d)
    lab = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    logp, lse, fws = H.head_fwd(h, w, lab, cfg.softcap, return_ws=True, skip_eps=eps)
    _, g = H.orpo_loss(logp, lab, off, cfg.V, cfg.lam)
    desc = H.make_desc(cfg.M, cfg.d, cfg.V, h.dtype, H._w_fmt(w, None), cfg.softcap, skip_eps=eps)
    L = H.lib()
    # One backward item (the whole [1024, 65536] coefficient block in buffer 0) for both runs, so
    # that the layout read below holds and both sum dh in the same order.
    assert L.orpo_set_bwd_tiling(0, 1024 * 65536 * 2) == 0
    try:
        dh0, dW0 = H.head_bwd(h, w, lab, lse, g, cfg.softcap, skip_eps=eps)         # filter only
        nbytes = L.orpo_head_bwd_workspace_bytes(ctypes.byref(desc))
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=d)
        dh = torch.empty_like(dh0)
        dW = torch.empty_like(dW0)
        st = L.orpo_head_bwd(ctypes.byref(desc), H._ptr(h), H.Weight(w.data_ptr(), None, None),
                             H._ptr(lab), H._ptr(lse), H._ptr(g), H._ptr(dh), H._ptr(dW),
                             H._ptr(ws), nbytes, H._ptr(fws), H._stream(d))
        assert st == 0
        torch.cuda.synchronize()
    finally:
        assert L.orpo_set_bwd_tiling(0, 0) == 0
    assert torch.equal(dh, dh0) and torch.equal(dW, dW0)
    # One item here (C = 1024 tokens, BVb = 65536): buffer 0 holds its [1024, 65536] coefficients.
    coeff = ws[256:256 + 1024 * 65536 * 2].view(torch.int16).view(1024, 65536)
    untouched = (coeff == -1).view(4, 256, 256, 256).all(dim=3).all(dim=1)    # [token tile, vocab tile]
    n_cold = int(untouched.sum().item())
    say(f"[filter cold tiles] {n_cold} of {untouched.numel()} coefficient tiles skipped")
    assert n_cold > 0


def _filter_cases(n, seed, budget=4e9):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([rng.integers(16, 64), rng.integers(64, 700), rng.integers(700, 1300)]))
        d = int(rng.choice([64, 128, 192, 256, 320, 448, 512]))
        V = int(rng.choice([rng.integers(2, 600), rng.integers(600, 8000), rng.integers(8000, 30000)]))
        cap = float(rng.choice([0.0, 30.0]))
        if M * V * d > budget:
            continue
        out.append((M, d, V, cap, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("M,d,V,cap,seed", _filter_cases(8, 4049))
def test_filter_random_shapes(M, d, V, cap, seed):
    # Seeded random shapes (one to several token tiles, short and long vocabulary blocks, so the dh
    # tiles' K is split 1 to 16 ways): a cotangent loud on random 64-token blocks and 1e-6
    # elsewhere, eps = 1e-3, against the oracle's filtered backward; and eps = 1e-30 (only the
    # all-zero slices past V dropped) bitwise equal to the exact backward.
    say(f"[case] filter sweep M={M} d={d} V={V} cap={cap} seed={seed}")
    h, w, labels = _custom(M, d, V, cap, seed=seed)
    hh, W = h.float().numpy().astype(np.float64), w.float().numpy().astype(np.float64)
    _, lse = orc.forward(hh, W, labels, cap)
    rng = np.random.default_rng(seed + 1)
    g = np.full(M, 1e-6)
    for b in range(0, M, 64):
        if rng.random() < 0.4:
            g[b:b + 64] = rng.choice([-1.0, 0.5])
    g[labels == -100] = 0
    dh, dW = _gpu_bwd(h, w, labels, lse, g, cap, 1e-3)
    fh, fw, kh, kw = orc.backward_filtered(hh, W, labels, lse, g, cap, 1e-3)
    e_dh, e_dW = rel(dh, fh), rel(dW, fw)
    say(f"[filter sweep] kept dh {kh:.3f} dW {kw:.3f}; vs filtered dh={e_dh:.2e} dW={e_dW:.2e}")
    assert e_dh <= TOL_GRAD and e_dW <= TOL_GRAD
    a = _gpu_bwd(h, w, labels, lse, g, cap, 0.0)
    b = _gpu_bwd(h, w, labels, lse, g, cap, 1e-30)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
