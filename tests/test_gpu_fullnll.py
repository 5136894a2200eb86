"""GPU parity for the full-scope NLL (orpo_loss_full: the chosen sequence's NLL over its prompt span
and its response, the odds ratio on the response means) against the float64 oracle."""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from oracle import orpo_oracle as orc
from tests.gpu_helpers import assert_parity, dev, rel, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


def _custom_full(M, d, V, cap, lam, seed, pairs=3):
    """Ragged prompt/chosen/rejected spans with a padded tail; pair 1 has an empty prompt span and
    pair 2 a prompt whose tokens are all ignored; a few other tokens are ignored too."""
    rng = np.random.default_rng(seed)
    cfg = synth.HeadConfig(0, f"full-M{M}-d{d}-V{V}-cap{cap}", M=M, d=d, V=V, pairs=pairs,
                           len_lo=1, len_hi=M, softcap=cap, lam=lam, prompt_lo=0, prompt_hi=M)
    h = synth.to_bf16(rng.standard_normal((M, d)))
    w = synth.to_bf16((rng.standard_normal((V, d)) * (3.0 / np.sqrt(d))).astype(np.float32))
    used = (M * 7) // 8
    lens = rng.integers(8, 40, size=3 * pairs).astype(np.int64)
    lens[3] = 0                                    # pair 1: no prompt span at all
    lens = np.maximum(lens, 0)
    lens = (lens * used) // lens.sum()
    lens[[1, 2, 4, 5, 7, 8]] = np.maximum(lens[[1, 2, 4, 5, 7, 8]], 3)
    off = synth.seg_offsets_from_lengths(lens)
    assert off[-1] <= M
    labels = rng.integers(0, V, size=M).astype(np.int32)
    labels[off[-1]:] = -100
    labels[off[6]:off[7]] = -100                   # pair 2: prompt tokens all ignored
    labels[off[0] + 1] = -100                      # an ignored prompt token of pair 0
    labels[off[1] + 1] = -100                      # and one inside its chosen response
    return synth.HeadInputs(cfg, seed, h, w, None, None, None, labels, off, lens)


def test_e4b_full_nll_one_pair():
    cfg = synth.reduced(synth.workload("e4b-bf16-softcap30-fullnll"), 1)
    say(f"[case] {cfg.name} M={cfg.M}")
    inp = synth.make_inputs(cfg, seed=0, label_device="cuda")
    gpu = run_gpu(inp)
    assert gpu["fwd_status"] == 0 and gpu["loss_status"] == 0
    errs = assert_parity(gpu, run_oracle(inp), cfg.name)
    assert errs["pm"] <= 1e-3


@pytest.mark.parametrize("M,d,V,cap,lam", [(700, 192, 3001, 30.0, 0.2), (400, 64, 1000, 0.0, 1.0)])
def test_full_nll_ragged(M, d, V, cap, lam):
    inp = _custom_full(M, d, V, cap, lam, seed=M + V)
    say(f"[case] {inp.cfg.name}")
    gpu = run_gpu(inp)
    assert gpu["loss_status"] == 0                 # empty / ignored prompt spans are not errors
    ora = run_oracle(inp)
    assert_parity(gpu, ora, inp.cfg.name)
    assert gpu["pm"][1] == 0.0 and gpu["pm"][2] == 0.0
    # Prompt tokens carry gradient: the g-weighted rows of dh are nonzero exactly where g is.
    p0 = slice(int(inp.seg_offsets[0]), int(inp.seg_offsets[1]))
    assert np.all((gpu["g"][p0] != 0) == (inp.labels[p0] != -100))


def test_full_scope_without_prompt_tokens_is_the_response_scope_bitwise():
    d = dev()
    inp = _custom_full(700, 192, 3001, 30.0, 0.2, seed=11)
    off3 = inp.seg_offsets
    labels = inp.labels.copy()
    for p in range(3):
        labels[off3[3 * p]:off3[3 * p + 1]] = -100            # every prompt token ignored
    lab = torch.from_numpy(labels).to(d)
    logp, lse = H.head_fwd(inp.h.to(d), inp.w.to(d), lab, 30.0)
    o3, g3 = H.orpo_loss(logp, lab, torch.from_numpy(off3).to(d), 3001, 0.2, scope="full")
    # Response scope over the same responses: each pair's (ignored) prompt lies inside the range
    # of the previous pair's rejected response, where it counts for nothing.
    off2 = np.array([off3[1], off3[2], off3[4], off3[5], off3[7], off3[8], off3[9]], dtype=np.int32)
    o2, g2 = H.orpo_loss(logp, lab, torch.from_numpy(off2).to(d), 3001, 0.2)
    torch.cuda.synchronize()
    a, b = o3.cpu().numpy(), o2.cpu().numpy()
    assert np.array_equal(a[:5 + 6], b), (a[:11], b)
    assert np.all(a[11:] == 0.0)
    assert torch.equal(g3, g2)


def test_full_scope_status_bits():
    d = dev()
    inp = _custom_full(400, 64, 1000, 0.0, 0.1, seed=5)
    off = inp.seg_offsets
    labels = inp.labels.copy()
    labels[off[1]:off[2]] = -100                   # pair 0's chosen response empty: a data error
    lab = torch.from_numpy(labels).to(d)
    logp, _ = H.head_fwd(inp.h.to(d), inp.w.to(d), lab, 0.0)
    out, g, lws = H.orpo_loss(logp, lab, torch.from_numpy(off).to(d), 1000, 0.1, return_ws=True,
                              scope="full")
    assert H.read_status(lws) & 2 and np.isnan(out[0].item())
    bad = off.copy()
    bad[2], bad[3] = bad[3], bad[2]
    out, g, lws = H.orpo_loss(logp, lab, torch.from_numpy(bad).to(d), 1000, 0.1, return_ws=True,
                              scope="full")
    assert H.read_status(lws) & 4 and torch.isnan(g).all().item()


def test_full_scope_epilogue_on_gpu_logp():
    # The f64 loss kernel against the oracle's f64 epilogue on the same (GPU) logp vector.
    d = dev()
    inp = _custom_full(700, 192, 3001, 30.0, 0.2, seed=21)
    lab = torch.from_numpy(inp.labels).to(d)
    logp, _ = H.head_fwd(inp.h.to(d), inp.w.to(d), lab, 30.0)
    out, g = H.orpo_loss(logp, lab, torch.from_numpy(inp.seg_offsets).to(d), 3001, 0.2, scope="full")
    lv = logp.cpu().numpy().astype(np.float64)
    mean, n = orc.span_means_full(lv, inp.labels, inp.seg_offsets)
    ep = orc.orpo_epilogue_full(mean, n, 0.2)
    gref = orc.token_cotangent_full(ep["dL_dmean"], n, inp.labels, inp.seg_offsets)
    o = out.cpu().numpy()
    for i, k in enumerate(("loss", "nll", "or", "accuracy", "margin")):
        assert abs(o[i] - ep[k]) <= 1e-12 * max(1.0, abs(ep[k])), k
    assert np.allclose(o[11:14], ep["pm"], rtol=1e-12, atol=1e-15)
    assert rel(g.cpu().numpy(), gref) < 1e-6
