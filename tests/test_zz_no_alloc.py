"""The allocation-free forward (orpo_head_fwd_noalloc, through the C ABI) against orpo_head_fwd:
bit for bit, on two calls in a row, the second with a smaller input (the shared device array keeps
the first call's contents), plus the refusal of a call whose workspace exceeds the array."""
import ctypes

import numpy as np
import pytest
import torch

from lm_head_cross_amd import head as H
from lm_head_cross_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(M, d, V, cap, seed):
    rng = np.random.default_rng(seed)
    h = synth.to_bf16(rng.standard_normal((M, d)))
    w = synth.to_bf16((rng.standard_normal((V, d)) * (3.0 / np.sqrt(d))).astype(np.float32))
    labels = rng.integers(0, V, size=M).astype(np.int32)
    labels[::7] = -100
    return h, w, labels


@pytest.mark.parametrize("cap", [30.0, 0.0])
def test_noalloc_forward_matches_allocating_forward(cap):
    d = torch.device("cuda:0")
    # The second call is smaller than the first in M and V: what it reads must be what it wrote.
    for M, dd, V in ((3000, 256, 20000), (700, 256, 5000)):
        print(f"[case] noalloc M={M} d={dd} V={V} cap={cap}", flush=True)
        h, w, labels = _inputs(M, dd, V, cap, seed=M + V)
        h, w, lab = h.to(d), w.to(d), torch.from_numpy(labels).to(d)
        ref_logp, ref_lse = H.head_fwd(h, w, lab, cap)
        logp = torch.full((M,), float("nan"), device=d)
        lse = torch.full((M,), float("nan"), device=d)
        H.head_fwd_noalloc(h, w, lab, logp, lse, cap)
        torch.cuda.synchronize()
        assert torch.equal(logp, ref_logp) and torch.equal(lse, ref_lse)


def test_noalloc_forward_4bit_head():
    # The 4-bit head through the same entry point, two calls in a row (the second smaller).
    d = torch.device("cuda:0")
    for M, dd, V in ((1100, 192, 3001), (300, 128, 1000)):
        print(f"[case] noalloc q4 M={M} d={dd} V={V}", flush=True)
        rng = np.random.default_rng(M)
        h = synth.to_bf16(rng.standard_normal((M, dd))).to(d)
        w32 = (rng.standard_normal((V, dd)) * (3.0 / np.sqrt(dd))).astype(np.float32)
        wq, sc, bi = synth.encode_q4(w32, 64)
        w = torch.from_numpy(wq.view(np.int32)).to(d)
        sc, bi = sc.to(d), bi.to(d)
        labels = rng.integers(0, V, size=M).astype(np.int32)
        labels[::5] = -100
        lab = torch.from_numpy(labels).to(d)
        ref_logp, ref_lse = H.head_fwd(h, w, lab, 30.0, scales=sc, biases=bi)
        logp = torch.full((M,), float("nan"), device=d)
        lse = torch.full((M,), float("nan"), device=d)
        H.head_fwd_noalloc(h, w, lab, logp, lse, 30.0, scales=sc, biases=bi)
        torch.cuda.synchronize()
        assert torch.equal(logp, ref_logp) and torch.equal(lse, ref_lse)


def test_noalloc_refuses_a_call_beyond_its_array():
    # M = 2^20 tokens needs 8 MiB of partials: refused before anything is enqueued.
    L = H.lib()
    desc = H.make_desc(1 << 20, 256, 4096, torch.bfloat16, H.ORPO_BF16, 30.0)
    assert L.orpo_head_fwd_workspace_bytes(ctypes.byref(desc)) > (4 << 20)
    st = L.orpo_head_fwd_noalloc(ctypes.byref(desc), 16, H.Weight(16, None, None), 16, 16, 16, None)
    assert st == -3
