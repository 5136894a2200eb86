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
from tests.gpu_helpers import TOL_GRAD, TOL_SCALAR, dev, oracle_weight, rel, say

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


@pytest.mark.parametrize("key", [2, 3, 4, 5, 6])
def test_full_size_sampled_parity(key):
    cfg = synth.CONFIGS[key]
    say(f"[fullsize] {cfg.name} M={cfg.M} d={cfg.d} V={cfg.V}")
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
                      want_dW=not cfg.q4, scope=cfg.scope)
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

    # Forward on sampled rows.
    rows = _sample_rows(inp)
    ref_logp, ref_lse = orc.forward(hh[rows], W, inp.labels[rows], cfg.softcap)
    e_logp, e_lse = rel(logp[rows], ref_logp), rel(lse[rows], ref_lse)
    say(f"[fullsize {cfg.name}] rows={len(rows)} logp={e_logp:.2e} lse={e_lse:.2e}")
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
    msg = f"[fullsize {cfg.name}] probe={len(probe)} dh={e_dh:.2e}"
    assert e_dh <= TOL_GRAD
    if not cfg.q4:
        e_dW = rel(step.dW.cpu().numpy(), rdW)
        msg += f" dW={e_dW:.2e}"
        assert e_dW <= TOL_GRAD
    say(msg)
