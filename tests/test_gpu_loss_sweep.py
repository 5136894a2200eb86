"""GPU: the loss kernels alone on seeded random span layouts. A synthetic float32 log-prob vector
(no head) goes through orpo_loss at both NLL scopes and through the pairwise sibling objectives,
against the oracle's float64 epilogues on the same vector: from one pair to several hundred, M up to
100000, spans from one token to hundreds, ignored tokens inside spans, padding before the first
span and after the last. Both sides read the same float32 inputs, so the gates are the float64
epilogue's own rounding (1e-9) and float32 g (1e-6)."""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from oracle import objectives as ob
from oracle import orpo_oracle as orc
from tests.gpu_helpers import dev, rel, say

pytestmark = pytest.mark.gpu


def _layout(seed, n_spans):
    """(logp, labels, offsets, M): n_spans consecutive spans after a short padded prefix, a padded
    tail, about a tenth of the tokens ignored but never a whole span."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, int(rng.choice([8, 64, 400])) + 1, size=n_spans)
    pre, post = int(rng.integers(0, 40)), int(rng.integers(0, 300))
    M = pre + int(lens.sum()) + post
    off = np.concatenate([[pre], pre + np.cumsum(lens)]).astype(np.int32)
    V = 50000
    labels = rng.integers(0, V, size=M).astype(np.int32)
    labels[:pre] = -100
    labels[off[-1]:] = -100
    for s in range(n_spans):
        a, b = off[s], off[s + 1]
        drop = rng.random(b - a) < 0.1
        drop[rng.integers(0, b - a)] = False                  # keep one valid token per span
        labels[a:b][drop] = -100
    logp = (-rng.uniform(0.05, 12.0, size=M)).astype(np.float32)
    logp[labels == -100] = 0.0                                 # as the forward leaves them
    return logp, labels, off, V


def _gpu(t):
    return torch.from_numpy(t).to(dev())


@pytest.mark.parametrize("P,seed", [(1, 1), (3, 2), (16, 3), (64, 4), (257, 5), (300, 6)])
def test_orpo_response_scope(P, seed):
    logp, labels, off, V = _layout(seed, 2 * P)
    lam = float(np.random.default_rng(seed).uniform(0.05, 1.0))
    say(f"[case] orpo response P={P} M={len(logp)} lam={lam:.3f}")
    out, g = H.orpo_loss(_gpu(logp), _gpu(labels), _gpu(off), V, lam)
    torch.cuda.synchronize()
    o, g = out.cpu().numpy(), g.cpu().numpy()
    ell, n = orc.branch_means(logp.astype(np.float64), labels, off)
    ep = orc.orpo_epilogue(ell, lam)
    for i, k in enumerate(("loss", "nll", "or", "accuracy", "margin")):
        assert abs(o[i] - ep[k]) <= 1e-9 * max(1.0, abs(ep[k])), (k, o[i], ep[k])
    assert np.allclose(o[5:5 + P], ep["lw"], rtol=1e-9, atol=1e-12)
    assert np.allclose(o[5 + P:5 + 2 * P], ep["lr"], rtol=1e-9, atol=1e-12)
    gref = orc.token_cotangent(ep["dL_dell"], n, labels, off)
    assert rel(g, gref) <= 1e-6
    assert np.all(g[labels == -100] == 0.0)


@pytest.mark.parametrize("P,seed", [(1, 11), (7, 12), (100, 13)])
def test_orpo_full_scope(P, seed):
    logp, labels, off, V = _layout(seed, 3 * P)
    say(f"[case] orpo full P={P} M={len(logp)}")
    out, g = H.orpo_loss(_gpu(logp), _gpu(labels), _gpu(off), V, 0.2, scope="full")
    torch.cuda.synchronize()
    o, g = out.cpu().numpy(), g.cpu().numpy()
    mean, n = orc.span_means_full(logp.astype(np.float64), labels, off)
    ep = orc.orpo_epilogue_full(mean, n, 0.2)
    for i, k in enumerate(("loss", "nll", "or", "accuracy", "margin")):
        assert abs(o[i] - ep[k]) <= 1e-9 * max(1.0, abs(ep[k])), (k, o[i], ep[k])
    assert np.allclose(o[5 + 2 * P:5 + 3 * P], ep["pm"], rtol=1e-9, atol=1e-12)
    assert rel(g, orc.token_cotangent_full(ep["dL_dmean"], n, labels, off)) <= 1e-6


@pytest.mark.parametrize("kind,P,seed", [("simpo", 5, 21), ("simpo", 200, 22), ("dpo", 9, 23),
                                         ("dpo", 150, 24), ("ipo", 33, 25), ("ipo", 2, 26)])
def test_pairwise_objectives(kind, P, seed):
    logp, labels, off, V = _layout(seed, 2 * P)
    rng = np.random.default_rng(seed + 100)
    sums, n = ob.span_stats(logp.astype(np.float64), labels, off)
    beta, gamma = {"simpo": (2.0, 0.3), "dpo": (0.1, 0.0), "ipo": (0.5, 0.0)}[kind]
    means = sums / n
    if kind == "simpo":
        ref = None
        ep = ob.simpo_epilogue(means[0::2], means[1::2], beta, gamma)
        vals = means
    elif kind == "dpo":
        ref = sums + rng.normal(0.0, 3.0, size=sums.shape)
        ep = ob.dpo_epilogue(sums[0::2], sums[1::2], ref[0::2], ref[1::2], beta)
        vals = sums
    else:
        ref = means + rng.normal(0.0, 0.2, size=sums.shape)
        ep = ob.ipo_epilogue(means[0::2], means[1::2], ref[0::2], ref[1::2], beta)
        vals = means
    say(f"[case] {kind} P={P} M={len(logp)}")
    out, g = H.pref_loss(kind, _gpu(logp), _gpu(labels), _gpu(off), V, beta, gamma,
                         ref_sums=None if ref is None else _gpu(ref))
    torch.cuda.synchronize()
    o, g = out.cpu().numpy(), g.cpu().numpy()
    for i, k in enumerate(("loss", "accuracy", "margin")):
        assert abs(o[i] - ep[k]) <= 1e-9 * max(1.0, abs(ep[k])), (k, o[i], ep[k])
    assert np.allclose(o[3:3 + P], vals[0::2], rtol=1e-9, atol=1e-12)
    assert np.allclose(o[3 + P:3 + 2 * P], vals[1::2], rtol=1e-9, atol=1e-12)
    assert rel(g, ob.pairwise_cotangent(kind, ep, n, labels, off)) <= 1e-6
