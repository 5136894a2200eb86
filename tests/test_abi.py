"""The C-ABI library without a GPU: it loads, exports every symbol include/orpo_head.h declares,
and rejects bad arguments on the host before anything is enqueued (no kernel is launched)."""
import ctypes
import os
import re

import pytest

from lm_head_cross_amd import head as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EINVAL, EUNSUP, ENOWS = -1, -2, -3


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "orpo_head.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(orpo_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = H.lib()
    syms = declared_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(L, s), s


def _desc(M=512, d=256, V=4096, h=H.ORPO_BF16, w=H.ORPO_BF16, cap=0.0, flags=0):
    return H.Desc(M, d, V, h, w, cap, -100, flags, 0.0)


def _cd(a, b):
    return -(-a // b)


def _dh_part_bytes(C, d, BVb, f32=False):
    """The backward's split-K dh partials, as its sizing rule states it: with K steps of 32 (fp32)
    or 64 elements, a dh tile (K = the vocabulary block BVb) is split when its K steps reach 1.5
    times the average K steps per CU (256) of a launch, into S = min(ceil(steps / average),
    256 // dh tiles, 16, steps // 4) ranges (none when S < 2). The average is taken over one item's
    dh, dW and coefficient tiles (mixed launches) and over its dh and dW tiles (the last launch);
    the partials take the larger S * C * d fp32, rounded up to 256 bytes."""
    kbk = 32 if f32 else 64
    n_jt, n_tt, n_vt = _cd(d, 256), _cd(C, 256), _cd(BVb, 256)
    nk, n_dh = _cd(BVb, kbk), n_tt * n_jt
    gemm = n_dh * nk + n_vt * n_jt * _cd(C, kbk)

    def split(work):
        per_cu = _cd(work, 256)
        if 2 * nk < 3 * per_cu:
            return 1
        S = min(_cd(nk, per_cu), 256 // n_dh, 16, nk // 4)
        return S if S >= 2 else 1
    S = max(split(gemm + n_tt * n_vt * _cd(d, kbk)), split(gemm))
    return _cd(S * C * d * 4, 256) * 256 if S >= 2 else 0


def test_workspace_sizes():
    L = H.lib()
    d = _desc(M=8192, d=2560, V=262144)
    fws = L.orpo_head_fwd_workspace_bytes(ctypes.byref(d))
    bws = L.orpo_head_bwd_workspace_bytes(ctypes.byref(d))
    assert fws == 256 + 8 * 8192 * 8           # 8 vocabulary splits of 128 tiles, float2 each
    assert bws == 256 + 2 * 8192 * 16384 * 2   # two 256 MiB bf16 coefficient tiles
    # The backward workspace does not grow with M past one chunk.
    d2 = _desc(M=32768, d=2560, V=262144)
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(d2)) == bws
    assert L.orpo_loss_workspace_bytes(100, 4) == 256 + 512
    assert L.orpo_loss_workspace_bytes(100, 0) == 0
    assert L.orpo_head_fwd_workspace_bytes(ctypes.byref(_desc(d=100))) == 0
    # Default block rule: the 256 MiB budget, and no wider than max(16384, V/8 rounded up to 256)
    # nor than V. (M, V) -> BVb:
    for M, V, bv in ((8192, 73448, 16384), (4096, 73448, 16384), (2048, 150000, 18944),
                     (8192, 1 << 20, 16384), (2048, 1 << 20, 65536), (8192, 4096, 4096)):
        dv = _desc(M=M, d=1536, V=V)
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(dv)) == (256 + 2 * M * bv * 2 +
                                                                    _dh_part_bytes(M, 1536, bv)), (M, V)
    # fp32 coefficients: the budget binds first.
    df = _desc(M=8192, d=256, V=262144, h=H.ORPO_F32, w=H.ORPO_F32)
    parts = _dh_part_bytes(8192, 256, 8192, f32=True)
    assert parts == 4 * 8192 * 256 * 4        # 32 dh tiles of 256 K steps: the last launch's 4 splits
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(df)) == 256 + 2 * 8192 * 8192 * 4 + parts
    # The e4b head at a small M: 40 dh tiles of 512 steps against ~240 per CU in the mixed
    # launches (3 splits) and ~160 in the last (4 splits).
    ds = _desc(M=1024, d=2560, V=262144)
    assert _dh_part_bytes(1024, 2560, 32768) == 4 * 1024 * 2560 * 4
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(ds)) == (256 + 2 * 1024 * 32768 * 2 +
                                                                4 * 1024 * 2560 * 4)
    # At M = 8192 nothing splits.
    assert _dh_part_bytes(8192, 2560, 16384) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), EUNSUP),                    # d not a multiple of 64
    (dict(h=H.ORPO_F32, w=H.ORPO_BF16), EUNSUP),
    (dict(h=H.ORPO_F32, w=H.ORPO_Q4G64), EUNSUP),
    (dict(h=7), EINVAL),
    (dict(M=-1), EINVAL),
    (dict(V=0), EINVAL),
    (dict(flags=8), EINVAL),
    (dict(flags=4), EINVAL),
    (dict(cap=float("nan")), EINVAL),
    (dict(cap=1024.5), EUNSUP),               # beyond the softcap range evaluated to fp32 accuracy
])
def test_fwd_rejects_bad_descriptors(kw, code):
    L = H.lib()
    d = _desc(**kw)
    w = H.Weight(16, None, None)
    assert L.orpo_head_fwd(ctypes.byref(d), 16, w, 16, 16, 16, 4096, 1 << 30, None) == code


def test_fwd_rejects_bad_weights_and_workspace():
    L = H.lib()
    d = _desc()
    assert L.orpo_head_fwd(ctypes.byref(d), 16, H.Weight(None, None, None), 16, 16, 16, 4096, 1 << 30, None) == EINVAL
    assert L.orpo_head_fwd(ctypes.byref(d), 16, H.Weight(16, 16, None), 16, 16, 16, 4096, 1 << 30, None) == EINVAL
    q = _desc(w=H.ORPO_Q4G64)
    assert L.orpo_head_fwd(ctypes.byref(q), 16, H.Weight(16, None, None), 16, 16, 16, 4096, 1 << 30, None) == EINVAL
    assert L.orpo_head_fwd(ctypes.byref(d), 16, H.Weight(16, None, None), 16, 16, 16, None, 1 << 30, None) == ENOWS
    assert L.orpo_head_fwd(ctypes.byref(d), 16, H.Weight(16, None, None), 16, 16, 16, 4096, 255, None) == ENOWS
    assert L.orpo_head_fwd(ctypes.byref(d), 16, H.Weight(16, None, None), 16, 16, 16, 4100, 1 << 30, None) == ENOWS
    assert L.orpo_head_fwd(ctypes.byref(d), None, H.Weight(16, None, None), 16, 16, 16, 4096, 1 << 30, None) == EINVAL


def test_bwd_rejects_dW_for_quantised_head():
    L = H.lib()
    q = _desc(w=H.ORPO_Q4G64)
    st = L.orpo_head_bwd(ctypes.byref(q), 16, H.Weight(16, 16, 16), 16, 16, 16, 16, 16, 4096, 1 << 30, None, None)
    assert st == EUNSUP


def test_loss_rejects_bad_arguments():
    L = H.lib()
    assert L.orpo_loss(10, 0, 16, 16, 16, 100, -100, 0.1, 16, 16, 4096, 4096, None) == EINVAL
    assert L.orpo_loss(-1, 1, 16, 16, 16, 100, -100, 0.1, 16, 16, 4096, 4096, None) == EINVAL
    assert L.orpo_loss(10, 1, None, 16, 16, 100, -100, 0.1, 16, 16, 4096, 4096, None) == EINVAL
    assert L.orpo_loss(10, 1, 16, 16, 16, 100, -100, float("nan"), 16, 16, 4096, 4096, None) == EINVAL
    assert L.orpo_loss(10, 1, 16, 16, 16, 100, -100, 0.1, 16, 16, 4096, 16, None) == ENOWS


def test_bwd_tiling_knob_validates_and_resizes():
    L = H.lib()
    assert L.orpo_set_bwd_tiling(100, 0) == EINVAL
    d = _desc(M=4096, d=256, V=4096)
    try:
        assert L.orpo_set_bwd_tiling(512, 512 * 1024 * 2) == 0
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(d)) == (256 + 2 * 512 * 1024 * 2 +
                                                                   _dh_part_bytes(512, 256, 1024))
    finally:
        assert L.orpo_set_bwd_tiling(0, 0) == 0
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(d)) == (256 + 2 * 4096 * 4096 * 2 +
                                                               _dh_part_bytes(4096, 256, 4096))


def test_filter_k_step_limit_reported_by_workspace_size_and_entry_point():
    L = H.lib()
    ws = (ctypes.c_char * 512)()
    base = ctypes.addressof(ws) + (-ctypes.addressof(ws)) % 256
    big = H.Desc(256, 256, 1 << 20, H.ORPO_BF16, H.ORPO_BF16, 30.0, -100, 0, 1e-5)
    exact = H.Desc(256, 256, 1 << 20, H.ORPO_BF16, H.ORPO_BF16, 30.0, -100, 0, 0.0)
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(big)) > 0
    try:
        assert L.orpo_set_bwd_tiling(256, 256 * 524288 * 2) == 0           # 8192 slices of 64: the limit
        fl = 524288 // 64 * 4 + 524288 // 256 * 4 * 2                       # dh and dW block flags
        parts = _dh_part_bytes(256, 256, 524288)
        assert parts == 16 * 256 * 256 * 4                                 # one dh tile, 8192 steps
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(big)) == (256 + 2 * 256 * 524288 * 2 +
                                                                     2 * fl + parts)
        assert L.orpo_set_bwd_tiling(256, 256 * (524288 + 256) * 2) == 0   # one slice more
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(big)) == 0
        w = H.Weight(16, None, None)
        st = L.orpo_head_bwd(ctypes.byref(big), 16, w, 16, 16, 16, 16, None, base, 256, None, None)
        assert st == EUNSUP                                                # before the workspace check
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(exact)) > 0   # no limit without the filter
    finally:
        assert L.orpo_set_bwd_tiling(0, 0) == 0


def test_bwd_tiling_bounds_keep_workspace_sizes_from_wrapping():
    L = H.lib()
    assert L.orpo_set_bwd_tiling((1 << 31) + 256, 0) == EINVAL
    assert L.orpo_set_bwd_tiling(0, (1 << 40) + 1) == EINVAL
    big = _desc(M=(1 << 31) - 1, d=1 << 20, V=(1 << 31) - 1, flags=2)   # bf16 dh: the fp32 chunk accumulator
    try:
        # Every backward loader addresses at most 2^31 bytes through one descriptor: with rows of
        # d = 2^20 bf16 (2 MiB) a token chunk and a vocabulary block hold at most 1024 rows,
        # whatever the knob asks for.
        assert L.orpo_set_bwd_tiling(1 << 31, 1 << 40) == 0
        # C = 1024 tokens, BVb = 1024 entries: 2 tiles of 1024 x 1024 bf16 + the fp32 [C, d] accumulator.
        expect = 256 + 2 * 1024 * 1024 * 2 + 1024 * (1 << 20) * 4
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(big)) == expect
        assert L.orpo_set_bwd_tiling(256, 1 << 40) == 0
        # C = 256 tokens, BVb = 1024 entries (the row cap, below the budget's 2^31).
        expect = 256 + 2 * 256 * 1024 * 2 + 256 * (1 << 20) * 4
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(big)) == expect
    finally:
        assert L.orpo_set_bwd_tiling(0, 0) == 0


def test_status_strings():
    L = H.lib()
    assert L.orpo_status_string(0) == b"ok"
    assert b"workspace" in L.orpo_status_string(ENOWS)
    assert b"data error" in L.orpo_status_string(-5)
    # orpo_check validates its workspace pointer before touching the stream.
    assert L.orpo_check(None, None) == EINVAL


def test_objective_entry_points_reject_bad_arguments():
    L = H.lib()
    assert L.orpo_objective_workspace_bytes(100, 8) == 256 + 512
    assert L.orpo_objective_workspace_bytes(100, 0) == 0
    ws = 1 << 20
    # kind, M, P, off, logp, labels, V, ignore, beta, gamma, ref, out, g, ws, bytes, stream
    for kind in (0, 5):
        assert L.orpo_pref_loss(kind, 10, 1, 16, 16, 16, 100, -100, 0.1, 0.0, 16, 16, 16, ws, 4096, None) == EINVAL
    for beta in (0.0, -0.5):   # IPO's target margin 1/(2 beta) needs beta > 0
        assert L.orpo_pref_loss(3, 10, 1, 16, 16, 16, 100, -100, beta, 0.0, None, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_pref_loss(4, 10, 1, 16, 16, 16, 100, -100, 0.1, 0.0, None, 16, 16, ws, 16, None) == ENOWS
    assert L.orpo_pref_loss(2, 10, 1, 16, 16, 16, 100, -100, 0.1, 0.0, None, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_pref_loss(1, 10, 0, 16, 16, 16, 100, -100, 0.1, 0.0, None, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_pref_loss(1, 10, 1, 16, 16, 16, 100, -100, float("nan"), 0.0, None, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_pref_loss(1, 10, 1, 16, 16, 16, 100, -100, 0.1, 0.0, None, 16, 16, ws, 16, None) == ENOWS
    # M, S, off, logp, old, ref, adv, labels, V, ignore, eps, beta, out, g, ws, bytes, stream
    assert L.orpo_grpo_loss(10, 0, 16, 16, 16, 16, 16, 16, 100, -100, 0.2, 0.1, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_grpo_loss(10, 1, 16, 16, 16, 16, None, 16, 100, -100, 0.2, 0.1, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_grpo_loss(10, 1, 16, 16, None, 16, 16, 16, 100, -100, 0.2, 0.1, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_grpo_loss(10, 1, 16, 16, 16, 16, 16, 16, 100, -100, -1.0, 0.1, 16, 16, ws, 4096, None) == EINVAL
    assert L.orpo_grpo_loss(10, 1, 16, 16, 16, 16, 16, 16, 100, -100, 0.2, 0.1, 16, 16, ws, 16, None) == ENOWS


def test_skip_eps_validation_and_workspaces():
    L = H.lib()
    d = _desc(M=8192, d=2560, V=262144)
    fws0 = L.orpo_head_fwd_workspace_bytes(ctypes.byref(d))
    bws0 = L.orpo_head_bwd_workspace_bytes(ctypes.byref(d))
    d.skip_eps = 1e-5
    # Forward: + the per-tile, per-wave logit maxima [32 token tiles][1024 vocabulary tiles][8].
    assert L.orpo_head_fwd_workspace_bytes(ctypes.byref(d)) == fws0 + 32 * 1024 * 8 * 4
    # Backward: + two sets of filter flags, dh [32][256][4] and dW [64][128][2] bytes.
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(d)) == bws0 + 2 * (32 * 256 * 4 + 64 * 128 * 2)
    for bad in (-1e-5, float("inf"), float("nan")):
        d.skip_eps = bad
        assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(d)) == 0
    f32 = _desc(h=H.ORPO_F32, w=H.ORPO_F32)
    f32.skip_eps = 1e-5
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(f32)) == 0     # unsupported for fp32
    st = L.orpo_head_bwd(ctypes.byref(f32), 16, H.Weight(16, None, None), 16, 16, 16, 16, 16, 16,
                         1 << 30, None, None)
    assert st == EUNSUP


def test_dh_bf16_flag_workspace_and_formats():
    L = H.lib()
    d = _desc(M=8192, d=2560, V=262144)
    base = L.orpo_head_bwd_workspace_bytes(ctypes.byref(d))
    d.flags = H.ORPO_DH_BF16
    # Several vocabulary blocks: + the chunk's fp32 dh accumulator [C, d].
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(d)) == base + 8192 * 2560 * 4
    one = _desc(M=1024, d=256, V=4096)
    b1 = L.orpo_head_bwd_workspace_bytes(ctypes.byref(one))
    one.flags = H.ORPO_DH_BF16
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(one)) == b1     # one block: no accumulator
    f32 = _desc(h=H.ORPO_F32, w=H.ORPO_F32, flags=H.ORPO_DH_BF16)
    assert L.orpo_head_bwd_workspace_bytes(ctypes.byref(f32)) == 0      # unsupported for fp32
    st = L.orpo_head_bwd(ctypes.byref(f32), 16, H.Weight(16, None, None), 16, 16, 16, 16, 16, 16,
                         1 << 30, None, None)
    assert st == EUNSUP


def test_binding_rejects_wrong_dtypes_before_any_launch():
    # The kernels read raw memory: a wrong element type must be refused, not reinterpreted.
    import torch
    h = torch.zeros(4, 64, dtype=torch.float16)
    w = torch.zeros(8, 64, dtype=torch.float16)
    lab = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(H.OrpoError, match="h must be"):
        H.head_fwd(h, w, lab.int())
    with pytest.raises(H.OrpoError, match="labels must be int32"):
        H.head_fwd(h.bfloat16(), w.bfloat16(), lab)
    with pytest.raises(H.OrpoError, match="w must be bfloat16"):
        H.head_fwd(h.bfloat16(), w.float(), lab.int())
    with pytest.raises(H.OrpoError, match="seg_offsets must be int32"):
        H.orpo_loss(torch.zeros(4), lab.int(), torch.zeros(3, dtype=torch.int64), 8, 0.1)
    with pytest.raises(H.OrpoError, match="g must be float32"):
        H.head_bwd(h.bfloat16(), w.bfloat16(), lab.int(), torch.zeros(4), torch.zeros(4).double())
    with pytest.raises(H.OrpoError, match="ref_sums must be float64"):
        H.pref_loss("dpo", torch.zeros(4), lab.int(), torch.zeros(3, dtype=torch.int32), 8, 0.1,
                    ref_sums=torch.zeros(2))
    with pytest.raises(H.OrpoError, match="scales must be bfloat16"):
        H.head_fwd(h.bfloat16(), torch.zeros(8, 8, dtype=torch.int32), lab.int(),
                   scales=torch.zeros(8, 1), biases=torch.zeros(8, 1, dtype=torch.bfloat16))
    # Right dtypes on the CPU: refused for placement, still before anything is launched.
    with pytest.raises(H.OrpoError, match="on a GPU"):
        H.head_fwd(h.bfloat16(), w.bfloat16(), lab.int())
    with pytest.raises(H.OrpoError, match="multiple of 128"):
        H.HeadStep(h.bfloat16(), w.bfloat16(), lab.int(), torch.zeros(3, dtype=torch.int32), 8, 0.0,
                   0.1, fp8=True)
    with pytest.raises(H.OrpoError, match="approximates a bf16 head"):
        H.HeadStep(h.float(), w.float(), lab.int(), torch.zeros(3, dtype=torch.int32), 8, 0.0, 0.1,
                   fp8=True)
    with pytest.raises(H.OrpoError, match="unknown objective"):
        H.HeadStep(h.bfloat16(), w.bfloat16(), lab.int(), torch.zeros(3, dtype=torch.int32), 8, 0.0,
                   0.1, objective="kto")


def test_fp8_entry_points_validate_before_any_launch():
    L = H.lib()
    ws = (ctypes.c_char * 1024)()
    base = ctypes.addressof(ws) + (-ctypes.addressof(ws)) % 256
    q8 = H.Fp8Operands(4096, 4096, 4096, 4096)
    d = _desc(M=512, d=256, V=4096, cap=30.0)
    fws = L.orpo_head_fwd_workspace_bytes(ctypes.byref(d))
    assert fws > 256
    # Valid request, one byte of workspace short: ENOWS (nothing launched).
    assert L.orpo_head_fwd_fp8(ctypes.byref(d), ctypes.byref(q8), 16, 16, 16, base, fws - 1, None) == ENOWS
    assert L.orpo_head_fwd_fp8(ctypes.byref(d), None, 16, 16, 16, base, 1 << 30, None) == EINVAL
    assert L.orpo_head_fwd_fp8(ctypes.byref(d), ctypes.byref(H.Fp8Operands(4096, None, 4096, 4096)),
                               16, 16, 16, base, 1 << 30, None) == EINVAL
    d64 = _desc(M=512, d=192, V=4096)                       # d not a multiple of 128
    assert L.orpo_head_fwd_fp8(ctypes.byref(d64), ctypes.byref(q8), 16, 16, 16, base, 1 << 30, None) == EUNSUP
    f32 = _desc(h=H.ORPO_F32, w=H.ORPO_F32)                 # the FP8 head approximates a bf16 head
    assert L.orpo_head_fwd_fp8(ctypes.byref(f32), ctypes.byref(q8), 16, 16, 16, base, 1 << 30, None) == EUNSUP
    # A softcap above 40 (running maximum) with the coefficient filter's tile maxima: refused.
    big = H.Desc(512, 256, 4096, H.ORPO_BF16, H.ORPO_BF16, 50.0, -100, 0, 1e-5)
    assert L.orpo_head_fwd_fp8(ctypes.byref(big), ctypes.byref(q8), 16, 16, 16, base, 1 << 30, None) == EUNSUP
    assert L.orpo_head_bwd_fp8(ctypes.byref(big), ctypes.byref(q8), 16, H.Weight(16, None, None), 16,
                               16, 16, 16, 16, base, 1 << 30, None, None) == EUNSUP
    bws = L.orpo_head_bwd_workspace_bytes(ctypes.byref(d))
    w = H.Weight(16, None, None)
    assert L.orpo_head_bwd_fp8(ctypes.byref(d), ctypes.byref(q8), 16, w, 16, 16, 16, 16, 16, base,
                               bws - 1, None, None) == ENOWS
    assert L.orpo_head_bwd_fp8(ctypes.byref(d64), ctypes.byref(q8), 16, w, 16, 16, 16, 16, 16, base,
                               1 << 30, None, None) == EUNSUP
    assert L.orpo_head_bwd_fp8(ctypes.byref(d), None, 16, w, 16, 16, 16, 16, 16, base, 1 << 30,
                               None, None) == EINVAL
    # Quantisation: shape and alignment checks.
    assert L.orpo_quantize_fp8(4096, 4, 12, 4096, 4096, None) == EINVAL      # cols % 8
    assert L.orpo_quantize_fp8(4096, -1, 64, 4096, 4096, None) == EINVAL
    assert L.orpo_quantize_fp8(4104, 4, 64, 4096, 4096, None) == EINVAL      # x not 16-byte aligned
    assert L.orpo_quantize_fp8(4096, 4, 64, 4100, 4096, None) == EINVAL      # q not 8-byte aligned
    assert L.orpo_quantize_fp8(None, 4, 64, 4096, 4096, None) == EINVAL
    assert L.orpo_quantize_fp8(None, 0, 64, None, None, None) == 0           # nothing to do
    # 4-bit staging: sizes, nulls and alignment are refused before any launch.
    q4 = H.Weight(4096, 8192, 8192)
    assert L.orpo_q4_stage(q4, 4, 96, 4096, None) == EINVAL                   # d % 64
    assert L.orpo_q4_stage(q4, 0, 64, 4096, None) == EINVAL                   # V = 0
    assert L.orpo_q4_stage(q4, 4, 64, None, None) == EINVAL                   # no output
    assert L.orpo_q4_stage(H.Weight(4096, None, 8192), 4, 64, 4096, None) == EINVAL
    assert L.orpo_q4_stage(H.Weight(4098, 8192, 8192), 4, 64, 4096, None) == EINVAL  # words not 4-byte aligned
    assert L.orpo_q4_stage(H.Weight(4096, 8193, 8192), 4, 64, 4096, None) == EINVAL  # scales not 2-byte aligned
    assert L.orpo_q4_stage(q4, 4, 64, 4104, None) == EINVAL                   # output not 16-byte aligned
