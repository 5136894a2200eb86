"""GPU parity: the HIP head (through the C ABI) against the float64 oracle, element by element, on
the same seeded inputs. Sizes are ones the oracle finishes in seconds but that still span several
256-wide tiles and ragged tails in M and V; the full-size configurations are covered by
test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth
from oracle import orpo_oracle as orc
from tests.gpu_helpers import (TOL_GRAD, assert_parity, dev, rel, run_gpu, run_oracle, say)

pytestmark = pytest.mark.gpu


def _check_config(cfg, seed=0):
    say(f"[case] {cfg.name} M={cfg.M} d={cfg.d} V={cfg.V} cap={cfg.softcap} seed={seed}")
    inp = synth.make_inputs(cfg, seed=seed, label_device="cuda")
    gpu = run_gpu(inp)
    assert gpu["fwd_status"] == 0 and gpu["loss_status"] == 0
    ora = run_oracle(inp)
    return assert_parity(gpu, ora, cfg.name)


def test_tiny_f32_full():
    errs = _check_config(synth.workload("tiny-f32"))
    # fp32 operands: far inside the gates.
    assert errs["logp"] < 1e-5 and errs["dh"] < 1e-4 and errs["dW"] < 1e-4


def test_minicpm_shape_one_pair():
    _check_config(synth.reduced(synth.workload("minicpm-like-bf16"), 1))


def test_e4b_shape_one_pair():
    _check_config(synth.reduced(synth.workload("e4b-bf16-softcap30"), 1))


def test_q4_head_one_pair():
    _check_config(synth.reduced(synth.workload("q4g64-minicpm-shape-softcap30"), 1))


def test_q4_head_e4b_shape_one_pair():
    # The 4-bit head at the e4b shape (d = 2560, V = 262144), one pair against the full oracle.
    _check_config(synth.reduced(synth.workload("q4g64-e4b-shape-softcap30"), 1))


def test_12b_shape_short_pair():
    cfg = synth.workload("12b-like-bf16-softcap30").replace(pairs=1, M=512, len_lo=200, len_hi=256, name="12b-like-short")
    _check_config(cfg)


# ------------------------------------------------------------------------------------------
# Hand-built shapes: ragged M and V, ignored tokens inside branches, padding, softcap on/off,
# and the backward's token-chunk x vocabulary-block loop forced to several iterations.
# ------------------------------------------------------------------------------------------
def _custom(M, d, V, dtype, cap, lam, seed, pairs=2, q4=False, pad=True):
    """Seeded inputs of an arbitrary shape: ragged branches over the first 7/8 of M (all of M with
    pad=False, so the last token tile can hold a single valid token), the rest padding, and one
    ignored token inside every branch of 3 or more tokens."""
    rng = np.random.default_rng(seed)
    cfg = synth.HeadConfig(0, f"custom-M{M}-d{d}-V{V}-{dtype}-cap{cap}{'' if pad else '-nopad'}",
                           M=M, d=d, V=V, pairs=pairs, len_lo=1, len_hi=M, softcap=cap, lam=lam,
                           dtype=dtype, q4=q4)
    h64 = rng.standard_normal((M, d))
    w32 = (rng.standard_normal((V, d)) * (3.0 / np.sqrt(d))).astype(np.float32)
    if dtype == "f32":
        h, w = torch.from_numpy(h64.astype(np.float32)), torch.from_numpy(w32)
    else:
        h, w = synth.to_bf16(h64), synth.to_bf16(w32)
    # Branch lengths: ragged, leaving a padded tail.
    used = max(2 * pairs, (M * 7) // 8) if pad else M
    cuts = np.sort(rng.choice(np.arange(1, used), size=2 * pairs - 1, replace=False))
    off = np.concatenate([[0], cuts, [used]]).astype(np.int32)
    labels = rng.integers(0, V, size=M).astype(np.int32)
    labels[used:] = -100
    # Ignore a few tokens inside branches, but never a whole branch.
    for b in range(2 * pairs):
        if off[b + 1] - off[b] >= 3:
            labels[off[b] + 1] = -100
    wq = scales = biases = None
    if q4:
        wq, scales, biases = synth.encode_q4(w32, 64)
        w = None
    return synth.HeadInputs(cfg, seed, h, w, wq, scales, biases, labels, off, np.diff(off))


CUSTOM = [
    (300, 64, 1000, "bf16", 0.0, 0.1),
    (513, 128, 257, "bf16", 30.0, 0.5),
    (37, 192, 7, "bf16", 5.0, 1.0),
    (260, 256, 2000, "f32", 2.0, 0.1),
    (700, 320, 3001, "bf16", 30.0, 0.2),
    # Softcaps above the fixed-reference range: the forward keeps a running maximum.
    (300, 128, 1000, "bf16", 50.0, 0.1),
    (700, 320, 3001, "bf16", 200.0, 0.2),
]


@pytest.mark.parametrize("M,d,V,dtype,cap,lam", CUSTOM)
def test_ragged_shapes(M, d, V, dtype, cap, lam):
    inp = _custom(M, d, V, dtype, cap, lam, seed=M + V)
    say(f"[case] {inp.cfg.name}")
    assert_parity(run_gpu(inp), run_oracle(inp), inp.cfg.name)


# Every position inside a branch (no padding): the last token tile holds exactly one valid token
# (M = 257, 513) and the last vocabulary tile one row (V = 257), so a tail-tile error is a whole
# token's or a whole dW row's and the per-token / per-row gates see it undiluted.
ONE_IN_TAIL = [
    (257, 64, 257, "bf16", 30.0, 0.1),
    (513, 128, 1000, "bf16", 0.0, 0.1),
    (257, 128, 257, "f32", 0.0, 0.5),
    (513, 192, 257, "bf16", 50.0, 0.1),
]


@pytest.mark.parametrize("M,d,V,dtype,cap,lam", ONE_IN_TAIL)
def test_one_token_and_one_row_tails(M, d, V, dtype, cap, lam):
    inp = _custom(M, d, V, dtype, cap, lam, seed=3 * M + V, pad=False)
    say(f"[case] {inp.cfg.name}")
    assert inp.labels[-1] != -100
    assert_parity(run_gpu(inp), run_oracle(inp), inp.cfg.name)


# A handful of tokens over a wide vocabulary: one token tile spread over 79 vocabulary splits (the
# merge's one-wave-per-token path, most of its waves past M), and the backward's single dh tile
# split 16 ways over two vocabulary blocks, the second 3617 rows wide (splits of 3 or 4 K steps).
FEW_TOKENS = [
    (5, 128, 20001, "bf16", 30.0, 0.1),
    (2, 64, 20001, "f32", 0.0, 0.1),
]


@pytest.mark.parametrize("M,d,V,dtype,cap,lam", FEW_TOKENS)
def test_few_tokens_wide_vocabulary(M, d, V, dtype, cap, lam):
    inp = _custom(M, d, V, dtype, cap, lam, seed=7 * M + V, pairs=1)
    say(f"[case] {inp.cfg.name}")
    assert_parity(run_gpu(inp), run_oracle(inp), inp.cfg.name)


def test_ignored_rows_with_huge_logits_no_softcap():
    # Without a softcap, padding and ignored tokens whose raw logits exceed the float range of
    # e^raw must still get zero coefficients: dh rows exactly zero, dW finite and at parity.
    inp = _custom(300, 128, 1000, "bf16", 0.0, 0.1, seed=12)
    ign = np.nonzero(inp.labels == -100)[0]
    inp.h[ign] = inp.h[ign] * 40.0             # raw logits of std ~120 on these rows
    say(f"[case] ignored rows with logits up to {float((inp.h[ign].float() @ inp.w.float().T).max()):.0f}")
    gpu = run_gpu(inp)
    assert np.isfinite(gpu["dW"]).all() and np.isfinite(gpu["dh"]).all()
    assert np.all(gpu["dh"][ign] == 0.0)
    assert_parity(gpu, run_oracle(inp), "huge-ignored-logits")


# The 4-bit head: K steps of 64 codes, an odd count (d = 64, 192, 320) adding a step of zeros per
# tile; a one-token tail (pad False); softcaps 0, 30 and 50 (the running maximum).
RAGGED_Q4 = [
    (300, 128, 1000, 30.0, True),
    (257, 64, 257, 30.0, False),
    (513, 192, 1000, 50.0, True),
    (300, 320, 3001, 0.0, True),
]


@pytest.mark.parametrize("M,d,V,cap,pad", RAGGED_Q4)
def test_ragged_q4(M, d, V, cap, pad):
    inp = _custom(M, d, V, "bf16", cap, 0.1, seed=9 if (M, d) == (300, 128) else M + d, q4=True,
                  pad=pad)
    say(f"[case] {inp.cfg.name} q4")
    assert_parity(run_gpu(inp), run_oracle(inp), inp.cfg.name + "-q4")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_chunk_and_block_loop(dtype):
    # C = 256 tokens and a 512-wide vocabulary block: 3 chunks x 3 blocks.
    inp = _custom(600, 128, 1500, dtype, 30.0, 0.1, seed=77)
    esize = 4 if dtype == "f32" else 2
    say(f"[case] chunk/block loop {dtype}")
    H.set_bwd_tiling(256, 256 * 512 * esize)
    try:
        gpu = run_gpu(inp)
    finally:
        H.set_bwd_tiling(0, 0)
    assert_parity(gpu, run_oracle(inp), "chunked-" + dtype)


def test_zero_weights_closed_form():
    inp = _custom(300, 64, 4096, "bf16", 0.0, 0.1, seed=3)
    inp.w.zero_()
    gpu = run_gpu(inp)
    valid = inp.labels != -100
    assert np.allclose(gpu["logp"][valid], -np.log(4096.0), rtol=0, atol=2e-6)
    assert np.all(gpu["logp"][~valid] == 0)
    assert np.all(gpu["dh"] == 0)


def test_deterministic_bitwise():
    inp = synth.make_inputs(synth.reduced(synth.workload("minicpm-like-bf16"), 1), seed=4, label_device="cuda")
    a = run_gpu(inp)
    b = run_gpu(inp)
    for k in ("logp", "lse", "g", "dh", "dW"):
        assert np.array_equal(a[k], b[k]), k
    assert a["loss"] == b["loss"]


def test_dw_accumulate_adds():
    inp = _custom(300, 128, 1000, "bf16", 0.0, 0.1, seed=5)
    d = dev()
    h, w = inp.h.to(d), inp.w.to(d)
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    logp, lse = H.head_fwd(h, w, labels, 0.0)
    _, g = H.orpo_loss(logp, labels, off, 1000, 0.1)
    _, dW1 = H.head_bwd(h, w, labels, lse, g, 0.0)
    dW2 = dW1.clone()
    H.head_bwd(h, w, labels, lse, g, 0.0, dW=dW2, accumulate=True)
    torch.cuda.synchronize()
    assert rel(dW2.cpu().numpy(), 2 * dW1.cpu().numpy()) < 1e-6


def test_status_bits_and_nan_outputs():
    d = dev()
    inp = _custom(300, 64, 1000, "bf16", 0.0, 0.1, seed=6)
    labels = inp.labels.copy()
    labels[0] = 5000                      # out of range: flagged, treated as ignored
    lab = torch.from_numpy(labels).to(d)
    h, w = inp.h.to(d), inp.w.to(d)
    logp, lse, ws = H.head_fwd(h, w, lab, 0.0, return_ws=True)
    assert H.read_status(ws) & 1
    assert logp[0].item() == 0.0
    # Empty branch: every token of branch 1 ignored.
    labels2 = inp.labels.copy()
    labels2[inp.seg_offsets[1]:inp.seg_offsets[2]] = -100
    lab2 = torch.from_numpy(labels2).to(d)
    logp2, _ = H.head_fwd(h, w, lab2, 0.0)
    out, g, lws = H.orpo_loss(logp2, lab2, torch.from_numpy(inp.seg_offsets).to(d), 1000, 0.1,
                              return_ws=True)
    assert H.read_status(lws) & 2
    assert np.isnan(out[0].item())
    # Non-monotone offsets.
    bad = inp.seg_offsets.copy()
    bad[1], bad[2] = bad[2], bad[1]
    out, g, lws = H.orpo_loss(logp, lab, torch.from_numpy(bad).to(d), 1000, 0.1, return_ws=True)
    assert H.read_status(lws) & 4
    assert np.isnan(out[0].item()) and torch.isnan(g).all().item()
    # The loss epilogue on the GPU's own logp vector matches the oracle's epilogue on it.
    out, g = H.orpo_loss(logp, lab, torch.from_numpy(inp.seg_offsets).to(d), 1000, 0.1)
    lv = logp.cpu().numpy().astype(np.float64)
    lab_ok = np.where((labels >= 0) & (labels < 1000), labels, -100)
    ell, n = orc.branch_means(lv, lab_ok, inp.seg_offsets)
    ep = orc.orpo_epilogue(ell, 0.1)
    gref = orc.token_cotangent(ep["dL_dell"], n, lab_ok, inp.seg_offsets)
    o = out.cpu().numpy()
    assert abs(o[0] - ep["loss"]) <= 1e-12 * abs(ep["loss"]) + 1e-13
    assert rel(g.cpu().numpy(), gref) < 1e-6


@pytest.mark.parametrize("case", ["one-block", "chunks-blocks", "q4-chunks-blocks", "filter"])
def test_dh_bf16_is_the_fp32_dh_rounded_once(case):
    # ORPO_DH_BF16: the same fp32 sums over vocabulary blocks (kept in an fp32 accumulator across
    # them), rounded to bf16 once, so it equals the fp32 output rounded to nearest even, bit for
    # bit; dW is unaffected. Checked on one block, on 3 token chunks x 3 vocabulary blocks, with a
    # 4-bit head, and under the coefficient filter.
    q4 = case.startswith("q4")
    inp = _custom(600, 128, 1500, "bf16", 30.0, 0.1, seed=78, q4=q4)
    say(f"[case] dh bf16 {case}")
    d = dev()
    h = inp.h.to(d)
    if q4:
        w = torch.from_numpy(inp.wq.view(np.int32)).to(d)
        sc, bi = inp.scales.to(d), inp.biases.to(d)
    else:
        w, sc, bi = inp.w.to(d), None, None
    labels = torch.from_numpy(inp.labels).to(d)
    off = torch.from_numpy(inp.seg_offsets).to(d)
    eps = 1e-6 if case == "filter" else 0.0
    logp, lse, fws = H.head_fwd(h, w, labels, 30.0, scales=sc, biases=bi, return_ws=True,
                                skip_eps=eps)
    _, g = H.orpo_loss(logp, labels, off, 1500, 0.1)
    if case != "one-block":
        H.set_bwd_tiling(256, 256 * 512 * 2)
    try:
        kw = dict(want_dW=not q4, scales=sc, biases=bi, skip_eps=eps, fwd_ws=fws if eps else None)
        dh32, dW32 = H.head_bwd(h, w, labels, lse, g, 30.0, **kw)
        dh16, dW16 = H.head_bwd(h, w, labels, lse, g, 30.0, dh_bf16=True, **kw)
        torch.cuda.synchronize()
    finally:
        H.set_bwd_tiling(0, 0)
    assert dh16.dtype == torch.bfloat16
    assert torch.equal(dh16, dh32.to(torch.bfloat16))
    if not q4:
        assert torch.equal(dW16, dW32)
    if case == "chunks-blocks":   # and against the oracle, to the gradient gate
        ora = run_oracle(inp)
        e = rel(dh16.float().cpu().numpy(), ora["dh"])
        say(f"[dh bf16] rel {e:.2e}")
        assert e <= TOL_GRAD


@pytest.mark.parametrize("cap", [40.0, 50.0, 1024.0])
def test_softcap_with_saturated_logits(cap):
    # Every raw logit hugely negative, so every z sits at the lower end -cap: at 40 the edge of the
    # fixed softmax reference (terms e^(z - cap) ~ e^-80, still normal floats), above it the running
    # maximum. All logits then tie: logp = -ln V exactly (up to rounding), lse = -cap + ln V, and
    # sech^2 underflows so dh and dW vanish. The oracle agrees.
    inp = _custom(300, 64, 1000, "bf16", cap, 0.1, seed=11)
    inp.h.copy_(torch.ones_like(inp.h))
    inp.w.copy_(torch.full_like(inp.w, -2.0 * cap))      # raw = -128 cap for every (token, vocab)
    say(f"[case] softcap {cap}, saturated logits")
    gpu = run_gpu(inp)
    valid = inp.labels != -100
    assert gpu["fwd_status"] == 0
    # z and lse are fp32 values of magnitude ~cap: allow 16 units in the last place of cap.
    atol = 1e-5 + 16.0 * cap * 2.0 ** -24
    assert np.allclose(gpu["logp"][valid], -np.log(1000.0), rtol=0, atol=atol)
    assert np.allclose(gpu["lse"][valid], -cap + np.log(1000.0), rtol=0, atol=atol)
    assert np.all(gpu["dh"] == 0) and np.all(gpu["dW"] == 0)
    ora = run_oracle(inp)
    assert np.max(np.abs(gpu["logp"] - ora["logp"])) <= atol


def test_empty_batch_zeroes_dW():
    # M = 0: nothing to compute; dW (overwritten by default) is set to zero, or left as it is when
    # accumulating.
    d = dev()
    h = torch.empty(0, 128, dtype=torch.bfloat16, device=d)
    w = torch.randn(300, 128, device=d).to(torch.bfloat16)
    labels = torch.empty(0, dtype=torch.int32, device=d)
    lse = torch.empty(0, dtype=torch.float32, device=d)
    dW = torch.full((300, 128), 7.0, device=d)
    H.head_bwd(h, w, labels, lse, lse, 30.0, dW=dW, accumulate=True)
    torch.cuda.synchronize()
    assert bool((dW == 7.0).all())
    H.head_bwd(h, w, labels, lse, lse, 30.0, dW=dW)
    torch.cuda.synchronize()
    assert bool((dW == 0.0).all())


def test_orpo_check_reports_data_errors():
    d = dev()
    inp = _custom(300, 64, 1000, "bf16", 0.0, 0.1, seed=13)
    h, w = inp.h.to(d), inp.w.to(d)
    lab = torch.from_numpy(inp.labels).to(d)
    _, _, ws = H.head_fwd(h, w, lab, 0.0, return_ws=True)
    assert H.check(ws)
    bad = inp.labels.copy()
    bad[3] = 1000                          # == V: out of range
    _, _, ws = H.head_fwd(h, w, torch.from_numpy(bad).to(d), 0.0, return_ws=True)
    assert not H.check(ws) and H.read_status(ws) == 1


def test_head_step_dh_bf16_matches_rounded_fp32():
    inp = _custom(600, 128, 1500, "bf16", 30.0, 0.1, seed=79)
    say("[case] HeadStep dh bf16")
    d = dev()
    args = (inp.h.to(d), inp.w.to(d), torch.from_numpy(inp.labels).to(d),
            torch.from_numpy(inp.seg_offsets).to(d), 1500, 30.0, 0.1)
    s32, s16 = H.HeadStep(*args), H.HeadStep(*args, dh_bf16=True)
    s32.step()
    s16.step()
    torch.cuda.synchronize()
    assert s16.dh.dtype == torch.bfloat16
    assert torch.equal(s16.dh, s32.dh.to(torch.bfloat16)) and torch.equal(s16.dW, s32.dW)
