"""Python binding of the C ABI in include/orpo_head.h (argument marshalling only).

Every step of the head runs in the HIP library `liborpo_head.so`; this module checks tensor
placement and dtypes, allocates outputs and workspaces through PyTorch (device memory and the
current stream are PyTorch's), and calls the library with ctypes. There is no fallback: if the
library is missing or the tensors are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

ORPO_F32, ORPO_BF16, ORPO_Q4G64 = 0, 1, 2
ORPO_DW_ACCUMULATE = 1
ORPO_DH_BF16 = 2
STATUS_BITS = {1: "bad label", 2: "empty branch", 4: "bad segment offsets"}
IGNORE_INDEX = -100

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liborpo_head.so")


class OrpoError(RuntimeError):
    pass


class Desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("d", ctypes.c_int64), ("V", ctypes.c_int64),
                ("h_fmt", ctypes.c_int32), ("w_fmt", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("ignore_index", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("skip_eps", ctypes.c_float)]


class Weight(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class Fp8Operands(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_void_p), ("h_exp", ctypes.c_void_p), ("wq", ctypes.c_void_p),
                ("w_exp", ctypes.c_void_p)]


_P = ctypes.c_void_p
_SIGS = {
    "orpo_head_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Desc)]),
    "orpo_head_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Desc)]),
    "orpo_loss_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32]),
    "orpo_head_fwd": (ctypes.c_int, [ctypes.POINTER(Desc), _P, Weight, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "orpo_head_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(Desc), _P, Weight, _P, _P, _P, _P]),
    "orpo_loss": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, ctypes.c_int64,
                                 ctypes.c_int32, ctypes.c_double, _P, _P, _P, ctypes.c_size_t, _P]),
    "orpo_loss_full": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.c_double, _P, _P, _P, ctypes.c_size_t,
                                      _P]),
    "orpo_objective_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32]),
    "orpo_pref_loss": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P, _P,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                                      ctypes.c_double, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "orpo_grpo_loss": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                                      ctypes.c_double, _P, _P, _P, ctypes.c_size_t, _P]),
    "orpo_head_bwd": (ctypes.c_int, [ctypes.POINTER(Desc), _P, Weight, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P, _P]),
    "orpo_quantize_fp8": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P]),
    "orpo_q4_stage": (ctypes.c_int, [Weight, ctypes.c_int64, ctypes.c_int64, _P, _P]),
    "orpo_head_fwd_fp8": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Fp8Operands), _P, _P,
                                         _P, _P, ctypes.c_size_t, _P]),
    "orpo_head_bwd_fp8": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Fp8Operands), _P,
                                         Weight, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "orpo_read_status": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_uint32), _P]),
    "orpo_check": (ctypes.c_int, [_P, _P]),
    "orpo_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "orpo_last_hip_error": (ctypes.c_int32, []),
    "orpo_set_bwd_tiling": (ctypes.c_int, [ctypes.c_int64, ctypes.c_size_t]),
    "orpo_trace_enable": (ctypes.c_int, [ctypes.c_int32]),
    "orpo_trace_collect": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    "orpo_trace_reset": (ctypes.c_int, []),
}
KERNEL_KINDS = {0: "fwd", 1: "merge", 2: "loss", 3: "coeff", 4: "dhdw", 5: "bwd", 6: "quant",
                7: "stage", 8: "dhsum"}
_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (built in-tree by lm_head_cross_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OrpoError(f"{LIB_PATH} is not built; run `python -m lm_head_cross_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(st: int, what: str):
    if st != 0:
        msg = lib().orpo_status_string(st).decode()
        raise OrpoError(f"{what}: {msg} (status {st}, hip error {lib().orpo_last_hip_error()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise OrpoError("tensors must be contiguous and on a GPU")
        if dev is not None and t.device != dev:
            raise OrpoError(f"tensors on different devices ({dev} and {t.device})")
        dev = t.device


def _need_dtype(what: str, t, *dtypes):
    """Raise unless `t` (None allowed) has one of `dtypes`: the kernels read raw memory, so a wrong
    element type would be reinterpreted, not converted."""
    if t is not None and t.dtype not in dtypes:
        names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise OrpoError(f"{what} must be {names}, got {str(t.dtype).replace('torch.', '')}")


def _head_dtypes(h, w, labels, scales=None, biases=None):
    _need_dtype("h", h, torch.bfloat16, torch.float32)
    _need_dtype("labels", labels, torch.int32)
    if scales is not None or biases is not None:
        _need_dtype("w (packed 4-bit words)", w, torch.int32)
        _need_dtype("scales", scales, torch.bfloat16)
        _need_dtype("biases", biases, torch.bfloat16)
        if h.dtype != torch.bfloat16:
            raise OrpoError("a 4-bit head needs bfloat16 h")
    else:
        _need_dtype("w", w, h.dtype)


def _need_shape(what: str, t, shape):
    """Raise unless `t` (None allowed) has exactly `shape`: the kernels index raw memory with the
    sizes derived from h and w, so a mismatch would read or write out of bounds."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise OrpoError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _head_shapes(h, w, labels, scales=None, biases=None):
    """(M, d, V) of a head call, after checking every operand's shape against them."""
    if h.dim() != 2:
        raise OrpoError(f"h must be [M, d], got shape {tuple(h.shape)}")
    M, d = h.shape
    if w.dim() != 2:
        raise OrpoError(f"w must be 2-D, got shape {tuple(w.shape)}")
    V = w.shape[0]
    if scales is not None or biases is not None:
        if d % 64:
            raise OrpoError(f"a 4-bit head needs d a multiple of 64 (d = {d})")
        _need_shape("w (packed 4-bit words)", w, (V, d // 8))
        _need_shape("scales", scales, (V, d // 64))
        _need_shape("biases", biases, (V, d // 64))
    else:
        _need_shape("w", w, (V, d))
    _need_shape("labels", labels, (M,))
    return M, d, V


def _need_offsets(seg_offsets, spans: int) -> int:
    """Number of groups (pairs, or completions for spans = 1) described by seg_offsets."""
    if seg_offsets.dim() != 1 or seg_offsets.shape[0] < spans + 1 or (seg_offsets.shape[0] - 1) % spans:
        raise OrpoError(f"seg_offsets must be 1-D with {spans} * n + 1 entries (n >= 1), "
                        f"got shape {tuple(seg_offsets.shape)}")
    return (seg_offsets.shape[0] - 1) // spans


def make_desc(M, d, V, h_dtype, w_fmt, softcap, ignore_index=IGNORE_INDEX, flags=0,
              skip_eps=0.0) -> Desc:
    if h_dtype not in (torch.float32, torch.bfloat16):
        raise OrpoError(f"h must be bfloat16 or float32, got {h_dtype}")
    h_fmt = ORPO_F32 if h_dtype == torch.float32 else ORPO_BF16
    return Desc(M, d, V, h_fmt, w_fmt, float(softcap), ignore_index, flags, float(skip_eps))


def _w_fmt(w, scales):
    if scales is not None:
        return ORPO_Q4G64
    return ORPO_F32 if w.dtype == torch.float32 else ORPO_BF16


def _workspace(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def _need_fwd_ws(fwd_ws, desc):
    """The backward reads the forward workspace's per-tile maxima (skip_eps > 0) at an offset the
    descriptor fixes: the tensor must be the uint8 workspace of a forward with the same sizes."""
    if fwd_ws is None:
        return
    _need_dtype("fwd_ws", fwd_ws, torch.uint8)
    need = lib().orpo_head_fwd_workspace_bytes(ctypes.byref(desc))
    if fwd_ws.dim() != 1 or fwd_ws.numel() < need:
        raise OrpoError(f"fwd_ws must be a forward workspace of at least {need} bytes, "
                        f"got shape {tuple(fwd_ws.shape)}")


def set_bwd_tiling(chunk_tokens: int = 0, coeff_bytes: int = 0):
    """Token chunk and coefficient-tile budget of the backward (0 restores the defaults)."""
    _check(lib().orpo_set_bwd_tiling(chunk_tokens, coeff_bytes), "orpo_set_bwd_tiling")


def read_status(ws: torch.Tensor) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().orpo_read_status(_ptr(ws), ctypes.byref(v), _stream(ws.device)), "orpo_read_status")
    return int(v.value)


ORPO_EDATA = -5


def check(ws: torch.Tensor) -> bool:
    """orpo_check: True when the workspace's status word holds no data-error bit (waits for the
    stream); False when the device reported one (read_status gives the bits)."""
    st = lib().orpo_check(_ptr(ws), _stream(ws.device))
    if st == ORPO_EDATA:
        return False
    _check(st, "orpo_check")
    return True


def head_fwd(h, w, labels, softcap=0.0, ignore_index=IGNORE_INDEX, scales=None, biases=None,
             return_ws=False, skip_eps=0.0):
    """logp[M], lse[M] (float32). `w` is W[V,d] (f32/bf16) or the packed q4 words [V,d/8] (int32).
    skip_eps > 0 also records the per-tile logit maxima the backward's cold-tile skip reads."""
    _head_dtypes(h, w, labels, scales, biases)
    M, d, V = _head_shapes(h, w, labels, scales, biases)
    _need_gpu(h, w, labels, scales, biases)
    desc = make_desc(M, d, V, h.dtype, _w_fmt(w, scales), softcap, ignore_index, skip_eps=skip_eps)
    L = lib()
    ws = _workspace(L.orpo_head_fwd_workspace_bytes(ctypes.byref(desc)), h.device)
    logp = torch.empty(M, dtype=torch.float32, device=h.device)
    lse = torch.empty(M, dtype=torch.float32, device=h.device)
    wt = Weight(w.data_ptr(), None if scales is None else scales.data_ptr(),
                None if biases is None else biases.data_ptr())
    _check(L.orpo_head_fwd(ctypes.byref(desc), _ptr(h), wt, _ptr(labels), _ptr(logp), _ptr(lse),
                           _ptr(ws), ws.numel(), _stream(h.device)), "orpo_head_fwd")
    return (logp, lse, ws) if return_ws else (logp, lse)


def head_fwd_noalloc(h, w, labels, logp, lse, softcap=0.0, ignore_index=IGNORE_INDEX, scales=None,
                     biases=None):
    """orpo_head_fwd_noalloc: logp[M] and lse[M] written into the caller's float32 tensors, the
    workspace taken from the library's own device array (nothing allocated, here or in the call)."""
    _head_dtypes(h, w, labels, scales, biases)
    _need_dtype("logp", logp, torch.float32)
    _need_dtype("lse", lse, torch.float32)
    M, d, V = _head_shapes(h, w, labels, scales, biases)
    _need_shape("logp", logp, (M,))
    _need_shape("lse", lse, (M,))
    _need_gpu(h, w, labels, scales, biases, logp, lse)
    desc = make_desc(M, d, V, h.dtype, _w_fmt(w, scales), softcap, ignore_index)
    wt = Weight(w.data_ptr(), None if scales is None else scales.data_ptr(),
                None if biases is None else biases.data_ptr())
    _check(lib().orpo_head_fwd_noalloc(ctypes.byref(desc), _ptr(h), wt, _ptr(labels), _ptr(logp),
                                       _ptr(lse), _stream(h.device)), "orpo_head_fwd_noalloc")
    return logp, lse


SCOPES = {"response": 2, "full": 3}   # spans per pair in seg_offsets


def orpo_loss(logp, labels, seg_offsets, V, lam, ignore_index=IGNORE_INDEX, return_ws=False,
              scope="response"):
    """out (float64) and g[M] (float32). scope "response": seg_offsets [2P+1] = (chosen, rejected)
    per pair, out = [loss, nll, or, accuracy, margin, lw[P], lr[P]]; scope "full": seg_offsets
    [3P+1] = (prompt, chosen, rejected) per pair, the NLL over prompt + chosen, out adds pm[P]."""
    _need_dtype("logp", logp, torch.float32)
    _need_dtype("labels", labels, torch.int32)
    _need_dtype("seg_offsets", seg_offsets, torch.int32)
    S = SCOPES[scope]
    if logp.dim() != 1:
        raise OrpoError(f"logp must be [M], got shape {tuple(logp.shape)}")
    M = logp.shape[0]
    _need_shape("labels", labels, (M,))
    P = _need_offsets(seg_offsets, S)
    _need_gpu(logp, labels, seg_offsets)
    L = lib()
    ws = _workspace(L.orpo_loss_workspace_bytes(M, P), logp.device)
    out = torch.empty(5 + (S if S == 3 else 2) * P, dtype=torch.float64, device=logp.device)
    g = torch.empty(M, dtype=torch.float32, device=logp.device)
    fn = L.orpo_loss_full if S == 3 else L.orpo_loss
    _check(fn(M, P, _ptr(seg_offsets), _ptr(logp), _ptr(labels), V, ignore_index, float(lam),
              _ptr(out), _ptr(g), _ptr(ws), ws.numel(), _stream(logp.device)), "orpo_loss")
    return (out, g, ws) if return_ws else (out, g)


def head_bwd(h, w, labels, lse, g, softcap=0.0, want_dW=True, ignore_index=IGNORE_INDEX,
             scales=None, biases=None, dW=None, accumulate=False, skip_eps=0.0, fwd_ws=None,
             dh_bf16=False):
    """dh[M,d] and dW[V,d] (float32; dW None when want_dW is False; dh bfloat16 with dh_bf16, the
    same fp32 sums rounded once). skip_eps > 0 turns on the coefficient filter (an approximation;
    see orpo_head_desc.skip_eps); fwd_ws, the forward's workspace (head_fwd(..., skip_eps=...,
    return_ws=True)), adds its exact cold-tile skip."""
    _head_dtypes(h, w, labels, scales, biases)
    _need_dtype("lse", lse, torch.float32)
    _need_dtype("g", g, torch.float32)
    _need_dtype("dW", dW, torch.float32)
    M, d, V = _head_shapes(h, w, labels, scales, biases)
    _need_shape("lse", lse, (M,))
    _need_shape("g", g, (M,))
    _need_shape("dW", dW, (V, d))
    if scales is not None and (want_dW or dW is not None):
        raise OrpoError("a 4-bit head is frozen: it has no dW (pass want_dW=False)")
    _need_gpu(h, w, labels, lse, g, scales, biases, dW, fwd_ws)
    flags = (ORPO_DW_ACCUMULATE if accumulate else 0) | (ORPO_DH_BF16 if dh_bf16 else 0)
    desc = make_desc(M, d, V, h.dtype, _w_fmt(w, scales), softcap, ignore_index, flags, skip_eps)
    L = lib()
    _need_fwd_ws(fwd_ws, desc)
    ws = _workspace(L.orpo_head_bwd_workspace_bytes(ctypes.byref(desc)), h.device)
    dh = torch.empty(M, d, dtype=torch.bfloat16 if dh_bf16 else torch.float32, device=h.device)
    if want_dW and dW is None:
        dW = torch.empty(V, d, dtype=torch.float32, device=h.device)
    if not want_dW:
        dW = None
    wt = Weight(w.data_ptr(), None if scales is None else scales.data_ptr(),
                None if biases is None else biases.data_ptr())
    _check(L.orpo_head_bwd(ctypes.byref(desc), _ptr(h), wt, _ptr(labels), _ptr(lse), _ptr(g),
                           _ptr(dh), _ptr(dW), _ptr(ws), ws.numel(), _ptr(fwd_ws), _stream(h.device)),
           "orpo_head_bwd")
    return dh, dW


def q4_stage(w, scales, biases, out=None):
    """The 4-bit head (packed words [V, d/8] int32, bf16 scales and biases [V, d/64]) dequantised
    to bf16 rows [V, d] (orpo_q4_stage): the operand values the 4-bit kernels stage per tile."""
    _need_dtype("w", w, torch.int32)
    _need_dtype("scales", scales, torch.bfloat16)
    _need_dtype("biases", biases, torch.bfloat16)
    _need_dtype("out", out, torch.bfloat16)
    if w.dim() != 2:
        raise OrpoError("w must be the packed words [V, d/8]")
    V, d = w.shape[0], w.shape[1] * 8
    _need_shape("scales", scales, (V, d // 64))
    _need_shape("biases", biases, (V, d // 64))
    _need_shape("out", out, (V, d))
    _need_gpu(w, scales, biases, out)
    if out is None:
        out = torch.empty(V, d, dtype=torch.bfloat16, device=w.device)
    _check(lib().orpo_q4_stage(Weight(w.data_ptr(), scales.data_ptr(), biases.data_ptr()), V, d,
                               _ptr(out), _stream(w.device)), "orpo_q4_stage")
    return out


# ------------------------------------------------------------------------------------------------
# The FP8 head: row-wise E4M3 logit operands (an opt-in approximation of the bf16 head)
# ------------------------------------------------------------------------------------------------
def quantize_fp8(x, q=None, exps=None):
    """E4M3 codes [R, C] (uint8) and E8M0 row exponents [R] (uint8) of a bf16 matrix x [R, C]."""
    _need_dtype("x", x, torch.bfloat16)
    _need_dtype("q", q, torch.uint8)
    _need_dtype("exps", exps, torch.uint8)
    _need_gpu(x, q, exps)
    R, C = x.shape
    if q is None:
        q = torch.empty(R, C, dtype=torch.uint8, device=x.device)
    if exps is None:
        exps = torch.empty(R, dtype=torch.uint8, device=x.device)
    if q.shape != x.shape or exps.shape != (R,):
        raise OrpoError("q must have the shape of x and exps one entry per row")
    _check(lib().orpo_quantize_fp8(_ptr(x), R, C, _ptr(q), _ptr(exps), _stream(x.device)),
           "orpo_quantize_fp8")
    return q, exps


def _fp8_operands(hq, h_exp, wq, w_exp):
    for name, t in (("hq", hq), ("h_exp", h_exp), ("wq", wq), ("w_exp", w_exp)):
        _need_dtype(name, t, torch.uint8)
    if hq.dim() != 2 or wq.dim() != 2:
        raise OrpoError("hq and wq must be 2-D")
    _need_shape("h_exp", h_exp, (hq.shape[0],))
    _need_shape("w_exp", w_exp, (wq.shape[0],))
    _need_shape("wq", wq, (wq.shape[0], hq.shape[1]))
    return Fp8Operands(hq.data_ptr(), h_exp.data_ptr(), wq.data_ptr(), w_exp.data_ptr())


def head_fwd_fp8(hq, h_exp, wq, w_exp, labels, softcap=0.0, ignore_index=IGNORE_INDEX,
                 return_ws=False, skip_eps=0.0):
    """logp[M], lse[M] of the FP8 head: logits from the quantised operands (quantize_fp8)."""
    _need_dtype("labels", labels, torch.int32)
    q8 = _fp8_operands(hq, h_exp, wq, w_exp)
    M, d = hq.shape
    V = wq.shape[0]
    _need_shape("labels", labels, (M,))
    _need_gpu(hq, h_exp, wq, w_exp, labels)
    desc = make_desc(M, d, V, torch.bfloat16, ORPO_BF16, softcap, ignore_index, skip_eps=skip_eps)
    L = lib()
    ws = _workspace(L.orpo_head_fwd_workspace_bytes(ctypes.byref(desc)), hq.device)
    logp = torch.empty(M, dtype=torch.float32, device=hq.device)
    lse = torch.empty(M, dtype=torch.float32, device=hq.device)
    _check(L.orpo_head_fwd_fp8(ctypes.byref(desc), ctypes.byref(q8), _ptr(labels), _ptr(logp),
                               _ptr(lse), _ptr(ws), ws.numel(), _stream(hq.device)), "orpo_head_fwd_fp8")
    return (logp, lse, ws) if return_ws else (logp, lse)


def head_bwd_fp8(hq, h_exp, wq, w_exp, h, w, labels, lse, g, softcap=0.0, want_dW=True,
                 ignore_index=IGNORE_INDEX, dW=None, accumulate=False, skip_eps=0.0, fwd_ws=None,
                 dh_bf16=False):
    """dh, dW of the FP8 head: coefficients from the quantised logits, products with bf16 h, W."""
    _head_dtypes(h, w, labels)
    _need_dtype("h", h, torch.bfloat16)
    _need_dtype("lse", lse, torch.float32)
    _need_dtype("g", g, torch.float32)
    _need_dtype("dW", dW, torch.float32)
    q8 = _fp8_operands(hq, h_exp, wq, w_exp)
    M, d, V = _head_shapes(h, w, labels)
    if hq.shape != (M, d) or wq.shape != (V, d):
        raise OrpoError("FP8 operands must have the shapes of h and w")
    _need_shape("lse", lse, (M,))
    _need_shape("g", g, (M,))
    _need_shape("dW", dW, (V, d))
    _need_gpu(hq, h_exp, wq, w_exp, h, w, labels, lse, g, dW, fwd_ws)
    flags = (ORPO_DW_ACCUMULATE if accumulate else 0) | (ORPO_DH_BF16 if dh_bf16 else 0)
    desc = make_desc(M, d, V, h.dtype, ORPO_BF16, softcap, ignore_index, flags, skip_eps)
    L = lib()
    _need_fwd_ws(fwd_ws, desc)
    ws = _workspace(L.orpo_head_bwd_workspace_bytes(ctypes.byref(desc)), h.device)
    dh = torch.empty(M, d, dtype=torch.bfloat16 if dh_bf16 else torch.float32, device=h.device)
    if want_dW and dW is None:
        dW = torch.empty(V, d, dtype=torch.float32, device=h.device)
    if not want_dW:
        dW = None
    _check(L.orpo_head_bwd_fp8(ctypes.byref(desc), ctypes.byref(q8), _ptr(h), Weight(w.data_ptr()),
                               _ptr(labels), _ptr(lse), _ptr(g), _ptr(dh), _ptr(dW), _ptr(ws),
                               ws.numel(), _ptr(fwd_ws), _stream(h.device)), "orpo_head_bwd_fp8")
    return dh, dW


# ------------------------------------------------------------------------------------------------
# Tracing (HIP event pairs recorded by the library around each of its launches)
# ------------------------------------------------------------------------------------------------
def trace_enable(max_launches: int):
    _check(lib().orpo_trace_enable(int(max_launches)), "orpo_trace_enable")


def trace_reset():
    _check(lib().orpo_trace_reset(), "orpo_trace_reset")


def trace_collect() -> dict:
    """{kind: (launches, total_ms, algorithmic_flops)} for the launches recorded since the reset."""
    res = {}
    for k, name in KERNEL_KINDS.items():
        n, ms, fl = ctypes.c_int64(0), ctypes.c_double(0), ctypes.c_double(0)
        _check(lib().orpo_trace_collect(k, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl)),
               "orpo_trace_collect")
        res[name] = (int(n.value), float(ms.value), float(fl.value))
    return res


# ------------------------------------------------------------------------------------------------
# A preallocated head step: fwd -> loss -> bwd with every buffer and workspace allocated once.
# ------------------------------------------------------------------------------------------------
PREF_KINDS = {"simpo": 1, "dpo": 2, "ipo": 3, "hinge": 4}


def pref_loss(kind, logp, labels, seg_offsets, V, beta, gamma=0.0, ref_sums=None,
              ignore_index=IGNORE_INDEX, return_ws=False):
    """SimPO ("simpo": mean log-probs, margin gamma), DPO ("dpo": sequence sums against the cached
    reference sums ref_sums [2P] float64), IPO ("ipo": means, optional reference means) or hinge
    ("hinge": sums, optional reference sums) over chosen/rejected spans seg_offsets [2P+1].
    Returns out (float64 [3 + 2P]: loss, accuracy, margin, chosen values, rejected values), g."""
    _need_dtype("logp", logp, torch.float32)
    _need_dtype("labels", labels, torch.int32)
    _need_dtype("seg_offsets", seg_offsets, torch.int32)
    _need_dtype("ref_sums", ref_sums, torch.float64)
    if logp.dim() != 1:
        raise OrpoError(f"logp must be [M], got shape {tuple(logp.shape)}")
    M = logp.shape[0]
    _need_shape("labels", labels, (M,))
    P = _need_offsets(seg_offsets, 2)
    _need_shape("ref_sums", ref_sums, (2 * P,))
    if kind not in PREF_KINDS:
        raise OrpoError(f"unknown preference objective {kind!r}")
    _need_gpu(logp, labels, seg_offsets, ref_sums)
    L = lib()
    ws = _workspace(L.orpo_objective_workspace_bytes(M, 2 * P), logp.device)
    out = torch.empty(3 + 2 * P, dtype=torch.float64, device=logp.device)
    g = torch.empty(M, dtype=torch.float32, device=logp.device)
    _check(L.orpo_pref_loss(PREF_KINDS[kind], M, P, _ptr(seg_offsets), _ptr(logp), _ptr(labels), V,
                            ignore_index, float(beta), float(gamma), _ptr(ref_sums), _ptr(out),
                            _ptr(g), _ptr(ws), ws.numel(), _stream(logp.device)), "orpo_pref_loss")
    return (out, g, ws) if return_ws else (out, g)


def grpo_loss(logp, old_logp, ref_logp, advantages, labels, seg_offsets, V, clip_eps, beta,
              ignore_index=IGNORE_INDEX, return_ws=False):
    """GRPO's clipped policy gradient + beta * k3 KL over completions seg_offsets [S+1] with one
    advantage each. Returns out (float64 [4]: loss, pg, kl, clip fraction), g."""
    for name, t in (("logp", logp), ("old_logp", old_logp), ("ref_logp", ref_logp),
                    ("advantages", advantages)):
        _need_dtype(name, t, torch.float32)
    _need_dtype("labels", labels, torch.int32)
    _need_dtype("seg_offsets", seg_offsets, torch.int32)
    if logp.dim() != 1:
        raise OrpoError(f"logp must be [M], got shape {tuple(logp.shape)}")
    M = logp.shape[0]
    for name, t in (("old_logp", old_logp), ("ref_logp", ref_logp), ("labels", labels)):
        _need_shape(name, t, (M,))
    S = _need_offsets(seg_offsets, 1)
    _need_shape("advantages", advantages, (S,))
    _need_gpu(logp, old_logp, ref_logp, advantages, labels, seg_offsets)
    L = lib()
    ws = _workspace(L.orpo_objective_workspace_bytes(M, S), logp.device)
    out = torch.empty(4, dtype=torch.float64, device=logp.device)
    g = torch.empty(M, dtype=torch.float32, device=logp.device)
    _check(L.orpo_grpo_loss(M, S, _ptr(seg_offsets), _ptr(logp), _ptr(old_logp), _ptr(ref_logp),
                            _ptr(advantages), _ptr(labels), V, ignore_index, float(clip_eps),
                            float(beta), _ptr(out), _ptr(g), _ptr(ws), ws.numel(),
                            _stream(logp.device)), "orpo_grpo_loss")
    return (out, g, ws) if return_ws else (out, g)


class HeadStep:
    def __init__(self, h, w, labels, seg_offsets, V, softcap, lam, scales=None, biases=None,
                 want_dW=True, ignore_index=IGNORE_INDEX, scope="response", objective="orpo",
                 obj=None, skip_eps=0.0, dh_bf16=False, fp8=False, q4_stage=False):
        """One head step: forward -> loss -> backward on preallocated buffers.

        objective "orpo" (lam, scope "response" | "full"), or a sibling on the same forward and
        backward, with its parameters and inputs in `obj`: "simpo" {beta, gamma}, "dpo" {beta,
        ref_sums [2P] float64}, "ipo" / "hinge" {beta, optional ref_sums}, "grpo" {clip_eps,
        beta, old_logp [M], ref_logp [M], advantages [S] float32, seg_offsets are then [S+1]
        completions}. dh_bf16: dh as bfloat16 (the fp32 sums rounded once). fp8: the FP8 head (an
        approximation): each step quantises h and W to row-wise E4M3 (part of the step) and takes
        the logits from them; the gradient products keep the bf16 h and W. q4_stage (a 4-bit
        head): each step first dequantises W once into a bf16 copy (orpo_q4_stage, part of the
        step, 2 V d bytes more memory) and runs the bf16 kernels on it, with the operand values
        the 4-bit kernels would stage tile by tile."""
        if objective != "orpo" and objective != "grpo" and objective not in PREF_KINDS:
            raise OrpoError(f"unknown objective {objective!r}")
        o = dict(obj or {})
        _head_dtypes(h, w, labels, scales, biases)
        if fp8:
            if h.dtype != torch.bfloat16 or w.dtype != torch.bfloat16 or scales is not None:
                raise OrpoError("the FP8 head approximates a bf16 head")
            if h.shape[1] % 128:
                raise OrpoError(f"the FP8 head needs d a multiple of 128 (d = {h.shape[1]})")
        _need_dtype("seg_offsets", seg_offsets, torch.int32)
        _need_dtype("ref_sums", o.get("ref_sums"), torch.float64)
        for k in ("old_logp", "ref_logp", "advantages"):
            _need_dtype(k, o.get(k), torch.float32)
        M, d, Vw = _head_shapes(h, w, labels, scales, biases)
        if V != Vw:
            raise OrpoError(f"V = {V} but the head has {Vw} vocabulary rows")
        if scales is not None and want_dW:
            raise OrpoError("a 4-bit head is frozen: it has no dW (pass want_dW=False)")
        if q4_stage and (scales is None or fp8):
            raise OrpoError("q4_stage stages a 4-bit head (scales and biases given, not fp8)")
        S = SCOPES[scope] if objective == "orpo" else (1 if objective == "grpo" else 2)
        P = _need_offsets(seg_offsets, S)
        if objective in ("dpo", "ipo", "hinge"):
            _need_shape("ref_sums", o.get("ref_sums"), (2 * P,))
        if objective == "grpo":
            for k in ("old_logp", "ref_logp"):
                if o.get(k) is None:
                    raise OrpoError(f"grpo needs obj[{k!r}]")
                _need_shape(k, o[k], (M,))
            if o.get("advantages") is None:
                raise OrpoError("grpo needs obj['advantages']")
            _need_shape("advantages", o["advantages"], (P,))
        if objective == "dpo" and o.get("ref_sums") is None:
            raise OrpoError("dpo needs obj['ref_sums']")
        _need_gpu(h, w, labels, seg_offsets, scales, biases,
                  *(o.get(k) for k in ("ref_sums", "old_logp", "ref_logp", "advantages")))
        self.h, self.w, self.labels, self.off = h, w, labels, seg_offsets
        self.scales, self.biases = scales, biases
        self.M, self.d = M, d
        self.V, self.softcap, self.lam, self.ignore = V, float(softcap), float(lam), ignore_index
        self.objective, self.obj = objective, dict(obj or {})
        self.S = S
        self.P = P
        dev = h.device
        self.q4_stage = bool(q4_stage)
        self.desc = make_desc(self.M, self.d, V, h.dtype,
                              ORPO_BF16 if self.q4_stage else _w_fmt(w, scales), softcap,
                              ignore_index, flags=ORPO_DH_BF16 if dh_bf16 else 0, skip_eps=skip_eps)
        L = lib()
        self.fws = _workspace(L.orpo_head_fwd_workspace_bytes(ctypes.byref(self.desc)), dev)
        self.bws = _workspace(L.orpo_head_bwd_workspace_bytes(ctypes.byref(self.desc)), dev)
        self.lws = _workspace(L.orpo_loss_workspace_bytes(self.M, self.P) if objective == "orpo"
                              else L.orpo_objective_workspace_bytes(self.M, self.S * self.P), dev)
        self.logp = torch.empty(self.M, dtype=torch.float32, device=dev)
        self.lse = torch.empty(self.M, dtype=torch.float32, device=dev)
        n_out = {"orpo": 5 + (3 if self.S == 3 else 2) * self.P, "grpo": 4}.get(objective, 3 + 2 * self.P)
        self.out = torch.empty(n_out, dtype=torch.float64, device=dev)
        self.g = torch.empty(self.M, dtype=torch.float32, device=dev)
        self.dh = torch.empty(self.M, self.d, dtype=torch.bfloat16 if dh_bf16 else torch.float32,
                              device=dev)
        self.dW = torch.empty(V, self.d, dtype=torch.float32, device=dev) if want_dW else None
        self.wt = Weight(w.data_ptr(), None if scales is None else scales.data_ptr(),
                         None if biases is None else biases.data_ptr())
        if self.q4_stage:
            self.wq4 = self.wt
            self.w16 = torch.empty(V, self.d, dtype=torch.bfloat16, device=dev)
            self.wt = Weight(self.w16.data_ptr(), None, None)
        self.fp8 = bool(fp8)
        if self.fp8:
            self.hq = torch.empty(self.M, self.d, dtype=torch.uint8, device=dev)
            self.h_exp = torch.empty(self.M, dtype=torch.uint8, device=dev)
            self.wq = torch.empty(V, self.d, dtype=torch.uint8, device=dev)
            self.w_exp = torch.empty(V, dtype=torch.uint8, device=dev)
            self.q8 = Fp8Operands(self.hq.data_ptr(), self.h_exp.data_ptr(), self.wq.data_ptr(),
                                  self.w_exp.data_ptr())
        self.stream = None

    def _s(self):
        return _stream(self.h.device)

    def forward(self):
        if self.q4_stage:
            _check(lib().orpo_q4_stage(self.wq4, self.V, self.d, _ptr(self.w16), self._s()),
                   "orpo_q4_stage")
        if self.fp8:
            L = lib()
            _check(L.orpo_quantize_fp8(_ptr(self.h), self.M, self.d, _ptr(self.hq), _ptr(self.h_exp),
                                       self._s()), "orpo_quantize_fp8")
            _check(L.orpo_quantize_fp8(_ptr(self.w), self.V, self.d, _ptr(self.wq), _ptr(self.w_exp),
                                       self._s()), "orpo_quantize_fp8")
            _check(L.orpo_head_fwd_fp8(ctypes.byref(self.desc), ctypes.byref(self.q8),
                                       _ptr(self.labels), _ptr(self.logp), _ptr(self.lse),
                                       _ptr(self.fws), self.fws.numel(), self._s()),
                   "orpo_head_fwd_fp8")
            return
        _check(lib().orpo_head_fwd(ctypes.byref(self.desc), _ptr(self.h), self.wt, _ptr(self.labels),
                                   _ptr(self.logp), _ptr(self.lse), _ptr(self.fws), self.fws.numel(),
                                   self._s()), "orpo_head_fwd")

    def loss(self):
        o = self.obj
        if self.objective in PREF_KINDS:
            _check(lib().orpo_pref_loss(PREF_KINDS[self.objective], self.M, self.P, _ptr(self.off),
                                        _ptr(self.logp), _ptr(self.labels), self.V, self.ignore,
                                        float(o["beta"]), float(o.get("gamma", 0.0)),
                                        _ptr(o.get("ref_sums")), _ptr(self.out), _ptr(self.g),
                                        _ptr(self.lws), self.lws.numel(), self._s()), "orpo_pref_loss")
            return
        if self.objective == "grpo":
            _check(lib().orpo_grpo_loss(self.M, self.P, _ptr(self.off), _ptr(self.logp),
                                        _ptr(o["old_logp"]), _ptr(o["ref_logp"]),
                                        _ptr(o["advantages"]), _ptr(self.labels), self.V,
                                        self.ignore, float(o["clip_eps"]), float(o["beta"]),
                                        _ptr(self.out), _ptr(self.g), _ptr(self.lws),
                                        self.lws.numel(), self._s()), "orpo_grpo_loss")
            return
        fn = lib().orpo_loss_full if self.S == 3 else lib().orpo_loss
        _check(fn(self.M, self.P, _ptr(self.off), _ptr(self.logp), _ptr(self.labels), self.V,
                  self.ignore, self.lam, _ptr(self.out), _ptr(self.g), _ptr(self.lws),
                  self.lws.numel(), self._s()), "orpo_loss")

    def backward(self):
        if self.fp8:
            _check(lib().orpo_head_bwd_fp8(ctypes.byref(self.desc), ctypes.byref(self.q8),
                                           _ptr(self.h), self.wt, _ptr(self.labels), _ptr(self.lse),
                                           _ptr(self.g), _ptr(self.dh), _ptr(self.dW),
                                           _ptr(self.bws), self.bws.numel(), _ptr(self.fws),
                                           self._s()), "orpo_head_bwd_fp8")
            return
        _check(lib().orpo_head_bwd(ctypes.byref(self.desc), _ptr(self.h), self.wt, _ptr(self.labels),
                                   _ptr(self.lse), _ptr(self.g), _ptr(self.dh), _ptr(self.dW),
                                   _ptr(self.bws), self.bws.numel(), _ptr(self.fws), self._s()),
               "orpo_head_bwd")

    def step(self):
        self.forward()
        self.loss()
        self.backward()

    def workspace_bytes(self) -> int:
        n = self.fws.numel() + self.bws.numel() + self.lws.numel()
        if self.fp8:
            n += self.hq.numel() + self.h_exp.numel() + self.wq.numel() + self.w_exp.numel()
        if self.q4_stage:
            n += self.w16.numel() * 2
        return n
