"""The binding refuses mismatched shapes before anything reaches the library (CPU only: no launch).

Every check runs before the tensors' device is looked at, so CPU tensors reach it; a call whose
shapes are right then fails on the device check instead, which shows that the shape check is what
stopped the wrong ones."""
import pytest
import torch

from lm_head_cross_amd import head as H

M, D, V = 40, 128, 300
BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def t(*shape, dtype=BF):
    return torch.zeros(*shape, dtype=dtype)


def _raises_shape(fn, what):
    with pytest.raises(H.OrpoError) as e:
        fn()
    assert "shape" in str(e.value) and what in str(e.value), str(e.value)


def _raises_device(fn):
    with pytest.raises(H.OrpoError) as e:
        fn()
    assert "GPU" in str(e.value), str(e.value)


def test_head_fwd_shapes():
    _raises_device(lambda: H.head_fwd(t(M, D), t(V, D), t(M, dtype=I32)))
    _raises_shape(lambda: H.head_fwd(t(M, D), t(V, D + 64), t(M, dtype=I32)), "w")
    _raises_shape(lambda: H.head_fwd(t(M, D), t(V, D), t(M + 1, dtype=I32)), "labels")
    with pytest.raises(H.OrpoError):
        H.head_fwd(t(M * D), t(V, D), t(M, dtype=I32))                      # h not 2-D


def test_q4_shapes():
    wq, sc, bi = t(V, D // 8, dtype=I32), t(V, D // 64), t(V, D // 64)
    _raises_device(lambda: H.head_fwd(t(M, D), wq, t(M, dtype=I32), scales=sc, biases=bi))
    _raises_shape(lambda: H.head_fwd(t(M, D), t(V, D // 4, dtype=I32), t(M, dtype=I32),
                                     scales=sc, biases=bi), "w")
    _raises_shape(lambda: H.head_fwd(t(M, D), wq, t(M, dtype=I32), scales=t(V - 1, D // 64),
                                     biases=bi), "scales")
    _raises_shape(lambda: H.head_fwd(t(M, D), wq, t(M, dtype=I32), scales=sc,
                                     biases=t(V, D // 32)), "biases")
    with pytest.raises(H.OrpoError, match="frozen"):
        H.head_bwd(t(M, D), wq, t(M, dtype=I32), t(M, dtype=F32), t(M, dtype=F32), 30.0,
                   scales=sc, biases=bi)


def test_q4_stage_shapes():
    wq, sc, bi = t(V, D // 8, dtype=I32), t(V, D // 64), t(V, D // 64)
    _raises_device(lambda: H.q4_stage(wq, sc, bi))
    _raises_device(lambda: H.q4_stage(wq, sc, bi, out=t(V, D)))
    _raises_shape(lambda: H.q4_stage(wq, t(V, D // 32), bi), "scales")
    _raises_shape(lambda: H.q4_stage(wq, sc, t(V + 1, D // 64)), "biases")
    _raises_shape(lambda: H.q4_stage(wq, sc, bi, out=t(V, D + 64)), "out")
    with pytest.raises(H.OrpoError, match="bfloat16"):
        H.q4_stage(wq, sc, bi, out=t(V, D, dtype=F32))
    with pytest.raises(H.OrpoError):
        H.q4_stage(t(V * D // 8, dtype=I32), sc, bi)                       # words not 2-D


def test_head_bwd_shapes():
    h, w, lab = t(M, D), t(V, D), t(M, dtype=I32)
    lse, g = t(M, dtype=F32), t(M, dtype=F32)
    _raises_device(lambda: H.head_bwd(h, w, lab, lse, g, 30.0))
    _raises_shape(lambda: H.head_bwd(h, w, lab, t(M - 1, dtype=F32), g, 30.0), "lse")
    _raises_shape(lambda: H.head_bwd(h, w, lab, lse, t(M + 1, dtype=F32), 30.0), "g")
    _raises_shape(lambda: H.head_bwd(h, w, lab, lse, g, 30.0, dW=t(V, D + 1, dtype=F32)), "dW")
    _raises_shape(lambda: H.head_bwd(h, w, lab, lse, g, 30.0, dW=t(V + 1, D, dtype=F32)), "dW")


def test_loss_shapes():
    logp, lab = t(M, dtype=F32), t(M, dtype=I32)
    _raises_device(lambda: H.orpo_loss(logp, lab, t(5, dtype=I32), V, 0.1))
    _raises_shape(lambda: H.orpo_loss(logp, t(M - 1, dtype=I32), t(5, dtype=I32), V, 0.1), "labels")
    _raises_shape(lambda: H.orpo_loss(logp, lab, t(4, dtype=I32), V, 0.1), "seg_offsets")
    _raises_shape(lambda: H.orpo_loss(logp, lab, t(5, dtype=I32), V, 0.1, scope="full"), "seg_offsets")
    _raises_shape(lambda: H.orpo_loss(logp, lab, t(1, dtype=I32), V, 0.1), "seg_offsets")
    _raises_device(lambda: H.orpo_loss(logp, lab, t(7, dtype=I32), V, 0.1, scope="full"))


def test_objective_shapes():
    logp, lab, off = t(M, dtype=F32), t(M, dtype=I32), t(5, dtype=I32)
    _raises_device(lambda: H.pref_loss("dpo", logp, lab, off, V, 0.1, ref_sums=t(4, dtype=torch.float64)))
    _raises_shape(lambda: H.pref_loss("dpo", logp, lab, off, V, 0.1,
                                      ref_sums=t(3, dtype=torch.float64)), "ref_sums")
    with pytest.raises(H.OrpoError, match="unknown"):
        H.pref_loss("orpo", logp, lab, off, V, 0.1)
    S = 4
    _raises_device(lambda: H.grpo_loss(logp, logp, logp, t(S, dtype=F32), lab, off, V, 0.2, 0.04))
    _raises_shape(lambda: H.grpo_loss(logp, t(M + 1, dtype=F32), logp, t(S, dtype=F32), lab, off,
                                      V, 0.2, 0.04), "old_logp")
    _raises_shape(lambda: H.grpo_loss(logp, logp, logp, t(S + 1, dtype=F32), lab, off, V, 0.2,
                                      0.04), "advantages")


def test_fp8_shapes():
    hq, he = t(M, D, dtype=torch.uint8), t(M, dtype=torch.uint8)
    wq, we = t(V, D, dtype=torch.uint8), t(V, dtype=torch.uint8)
    lab = t(M, dtype=I32)
    _raises_device(lambda: H.head_fwd_fp8(hq, he, wq, we, lab))
    _raises_shape(lambda: H.head_fwd_fp8(hq, t(M + 1, dtype=torch.uint8), wq, we, lab), "h_exp")
    _raises_shape(lambda: H.head_fwd_fp8(hq, he, wq, t(V - 1, dtype=torch.uint8), lab), "w_exp")
    _raises_shape(lambda: H.head_fwd_fp8(hq, he, t(V, D + 8, dtype=torch.uint8), we, lab), "wq")
    _raises_shape(lambda: H.head_fwd_fp8(hq, he, wq, we, t(M - 1, dtype=I32)), "labels")


def test_head_step_checks():
    h, w, lab, off = t(M, D), t(V, D), t(M, dtype=I32), t(5, dtype=I32)
    _raises_device(lambda: H.HeadStep(h, w, lab, off, V, 30.0, 0.1))
    with pytest.raises(H.OrpoError, match="vocabulary rows"):
        H.HeadStep(h, w, lab, off, V + 1, 30.0, 0.1)
    _raises_shape(lambda: H.HeadStep(h, w, lab, t(6, dtype=I32), V, 30.0, 0.1), "seg_offsets")
    _raises_shape(lambda: H.HeadStep(h, w, lab, off, V, 30.0, 0.1, objective="dpo",
                                     obj={"beta": 0.1, "ref_sums": t(5, dtype=torch.float64)}),
                  "ref_sums")
    with pytest.raises(H.OrpoError, match="ref_sums"):
        H.HeadStep(h, w, lab, off, V, 30.0, 0.1, objective="dpo", obj={"beta": 0.1})
    with pytest.raises(H.OrpoError, match="q4_stage"):                    # a bf16 head has no words
        H.HeadStep(h, w, lab, off, V, 30.0, 0.1, q4_stage=True)
    wq, sc, bi = t(V, D // 8, dtype=I32), t(V, D // 64), t(V, D // 64)
    _raises_device(lambda: H.HeadStep(h, wq, lab, off, V, 30.0, 0.1, scales=sc, biases=bi,
                                      want_dW=False, q4_stage=True))
    g_obj = {"clip_eps": 0.2, "beta": 0.04, "old_logp": t(M, dtype=F32), "ref_logp": t(M, dtype=F32),
             "advantages": t(4, dtype=F32)}
    _raises_device(lambda: H.HeadStep(h, w, lab, off, V, 30.0, 0.1, objective="grpo", obj=g_obj))
    bad = dict(g_obj, advantages=t(3, dtype=F32))
    _raises_shape(lambda: H.HeadStep(h, w, lab, off, V, 30.0, 0.1, objective="grpo", obj=bad),
                  "advantages")
