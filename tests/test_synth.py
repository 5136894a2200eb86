"""The seeded generator: packing, padding, label mix, determinism and the 4-bit encoding."""
import numpy as np
import torch

from lm_head_cross_amd import synth
from oracle import orpo_oracle as orc


def test_tiny_config_layout_and_determinism():
    a = synth.make_inputs(synth.workload("tiny-f32"), seed=0)
    b = synth.make_inputs(synth.workload("tiny-f32"), seed=0)
    assert list(a.seg_offsets) == [0, 128, 256]
    assert a.h.dtype == torch.float32 and a.w.dtype == torch.float32
    assert torch.equal(a.h, b.h) and torch.equal(a.w, b.w) and np.array_equal(a.labels, b.labels)
    rms = a.h.double().pow(2).mean(dim=1).sqrt()
    assert torch.allclose(rms, torch.ones_like(rms), atol=1e-5)
    assert a.labels.min() >= 0 and a.labels.max() < 4096


def test_packing_padding_and_peaked_labels():
    cfg = synth.reduced(synth.workload("minicpm-like-bf16"), pairs=2).replace(V=2048, d=128)
    x = synth.make_inputs(cfg, seed=1)
    off = x.seg_offsets
    assert off[0] == 0 and np.all(np.diff(off) >= 1) and off[-1] <= cfg.M
    lens = np.diff(off)
    assert np.all((lens >= cfg.len_lo) & (lens <= cfg.len_hi))
    assert np.all(x.labels[off[-1]:] == synth.IGNORE_INDEX)
    valid = x.labels[:off[-1]]
    logits = x.h[:off[-1]].float() @ x.w.float().T
    frac_argmax = float(np.mean(valid == torch.argmax(logits, dim=1).numpy()))
    assert 0.6 < frac_argmax < 0.8


def test_lengths_are_scaled_when_they_overflow():
    rng = np.random.default_rng(0)
    lens = synth.draw_lengths(rng, 8, 100, 100, 500)
    assert lens.sum() <= 500 and np.all(lens == 62)


def test_q4_encoding_roundtrip_error_is_half_a_step():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((16, 128)) * 0.1).astype(np.float32)
    packed, scale, bias = synth.encode_q4(w, 64)
    deq = orc.dequant_q4(packed, synth.bf16_bits(scale), synth.bf16_bits(bias), 64)
    step = np.repeat(scale.float().numpy(), 64, axis=1)
    lo = np.repeat(bias.float().numpy(), 64, axis=1)
    # Codes saturate at 15; away from the clamp, the error is at most half a step (plus bf16 slack).
    inside = (w - lo) <= 15 * step
    err = np.abs(deq - w)
    assert np.all(err[inside] <= 0.5 * step[inside] * (1 + 1e-2) + 1e-7)


def test_prompt_spans_layout():
    # The full-NLL workload: per pair (prompt, chosen, rejected), prompt lengths in their range (up to
    # the packing scale), responses in theirs, all within M; the response-scope draws are unchanged
    # by the prompt option (same seed, same response lengths before any packing scale).
    cfg = synth.reduced(synth.workload("e4b-bf16-softcap30-fullnll"), 3).replace(d=256, V=4096)   # layout only: small head
    inp = synth.make_inputs(cfg, seed=2)
    assert cfg.scope == "full" and cfg.spans_per_pair == 3
    off = inp.seg_offsets
    assert off.shape == (3 * 3 + 1,) and off[0] == 0 and off[-1] <= cfg.M
    assert np.all(np.diff(off) >= 1)
    lens = np.diff(off)
    assert np.all((lens[0::3] >= 1) & (lens[0::3] <= cfg.prompt_hi))
    base = synth.make_inputs(cfg.replace(prompt_lo=0, prompt_hi=0), seed=2)
    assert base.seg_offsets.shape == (2 * 3 + 1,)
    resp = np.stack([lens[1::3], lens[2::3]], axis=1).reshape(-1)
    assert np.array_equal(resp, np.diff(base.seg_offsets))
