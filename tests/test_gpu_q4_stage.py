"""GPU: the 4-bit head staged as bf16 rows (orpo_q4_stage) and the bf16 kernels run on them.

  * the staged rows against the values the kernels multiply, computed on the host from the packed
    words (fp32 scale * q + bias, rounded once to bf16), bit for bit: on ragged shapes, and on
    sampled rows of the full MiniCPM-shape and e4b-shape heads;
  * the staged step (forward, loss, dh) against the 4-bit kernels' step on the same inputs: both
    multiply the same operand values in the same order, so every output is identical;
  * the staged step against the float64 oracle, with the gates of the 4-bit parity tests.
"""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from tests.gpu_helpers import (assert_parity, dev, gpu_weights, mfma_operand_weight, run_gpu,
                               run_oracle, say)
from tests.test_gpu_parity import RAGGED_Q4, _custom

pytestmark = pytest.mark.gpu


def _staged(inp):
    w, sc, bi = gpu_weights(inp, dev())
    out = H.q4_stage(w, sc, bi)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M,d,V,cap,pad", RAGGED_Q4)
def test_staged_rows_are_the_mfma_operand(M, d, V, cap, pad):
    inp = _custom(M, d, V, "bf16", cap, 0.1, seed=M + d + 1, q4=True, pad=pad)
    say(f"[case] stage rows V={V} d={d}")
    got = _staged(inp).float().cpu().numpy()
    want = mfma_operand_weight(inp).astype(np.float32)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", ["q4g64-minicpm-shape-softcap30", "q4g64-e4b-shape-softcap30"])
def test_staged_rows_full_size_sampled(name):
    cfg = synth.workload(name)
    say(f"[case] stage rows {cfg.name} V={cfg.V} d={cfg.d}")
    inp = synth.make_inputs(cfg, seed=0, label_device="cuda")
    got = _staged(inp)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, cfg.V, size=48), [0, cfg.V - 1]]))
    sel = got[torch.from_numpy(rows).to(got.device)].float().cpu().numpy()
    np.testing.assert_array_equal(sel, mfma_operand_weight(inp, rows).astype(np.float32))


@pytest.mark.parametrize("M,d,V,cap,pad", RAGGED_Q4)
def test_staged_step_matches_the_4bit_step(M, d, V, cap, pad):
    inp = _custom(M, d, V, "bf16", cap, 0.1, seed=M + d, q4=True, pad=pad)
    say(f"[case] staged vs 4-bit kernels {inp.cfg.name}")
    fused = run_gpu(inp)
    staged = run_gpu(inp, q4_stage=True)
    for k in ("logp", "lse", "g", "dh"):
        np.testing.assert_array_equal(staged[k], fused[k], err_msg=k)
    for k in ("loss", "nll", "or"):
        assert staged[k] == fused[k], k
    assert staged["fwd_status"] == 0 and staged["loss_status"] == 0
    assert_parity(staged, run_oracle(inp), inp.cfg.name + "-q4-staged")


def test_staged_head_step_matches_the_4bit_head_step():
    # HeadStep(q4_stage=True), as bench.py --q4-stage runs it, at the MiniCPM shape with one pair.
    cfg = synth.reduced(synth.workload("q4g64-minicpm-shape-softcap30"), 1)
    say(f"[case] HeadStep staged {cfg.name} M={cfg.M}")
    inp = synth.make_inputs(cfg, seed=0, label_device="cuda")
    d = dev()
    h = inp.h.to(d)
    w, sc, bi = gpu_weights(inp, d)
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    res = []
    for stage in (False, True):
        s = H.HeadStep(h, w, labels, off, cfg.V, cfg.softcap, cfg.lam, scales=sc, biases=bi,
                       want_dW=False, q4_stage=stage)
        s.step()
        s.step()   # a second step re-stages W into the same buffer
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (s.logp, s.lse, s.out, s.g, s.dh)])
    for a, b in zip(*res):
        assert torch.equal(a, b)
