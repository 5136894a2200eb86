"""Memory: at the e4b head shape the step allocates nothing beyond its outputs and workspaces, the
backward workspace does not grow with M past one token chunk, and nothing of size M x V appears."""
import pytest
import torch

from lm_head_cross_amd import head as H
from tests.gpu_helpers import dev, say

pytestmark = pytest.mark.gpu

MiB = 1 << 20


def test_peak_memory_flat_in_M():
    d = dev()
    D, V = 2560, 262144
    g = torch.Generator(device=d)
    g.manual_seed(0)
    W = (torch.randn(V, D, device=d, generator=g) * (3.0 / D ** 0.5)).to(torch.bfloat16)
    rows = []
    for M in (1024, 2048, 4096, 8192, 16384, 32768):
        h = torch.randn(M, D, device=d, generator=g).to(torch.bfloat16)
        labels = torch.randint(0, V, (M,), device=d, generator=g, dtype=torch.int32)
        off = torch.tensor([0, M // 2, M], dtype=torch.int32, device=d)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        step = H.HeadStep(h, W, labels, off, V, 30.0, 0.1)
        step.step()
        torch.cuda.synchronize()
        extra = torch.cuda.max_memory_allocated() - base
        outputs = 3 * 4 * M + 4 * M * D + 4 * V * D + 8 * (5 + 2)     # logp, lse, g, dh, dW, out
        ws_bwd, ws_fwd = step.bws.numel(), step.fws.numel()
        expected = outputs + ws_bwd + ws_fwd + step.lws.numel()
        say(f"[memory] M={M}: extra {extra / MiB:.1f} MiB = outputs {outputs / MiB:.1f} + "
            f"bwd ws {ws_bwd / MiB:.1f} + fwd ws {ws_fwd / MiB:.2f} (expected {expected / MiB:.1f})")
        # Everything allocated during the step is accounted for (allocator rounding aside) ...
        assert expected <= extra <= expected + 8 * MiB
        # ... and the only large scratch is the fixed coefficient budget (two 256 MiB tiles), not an
        # M x V buffer (bf16 [M, V] would be 0.5-16 GiB here).
        assert ws_bwd <= 2 * 256 * MiB + 256 and ws_fwd <= 8 * max(M, 512 * 256) + 512
        rows.append((M, ws_bwd, ws_fwd))
        del step, h, labels, off
        torch.cuda.empty_cache()
    # The backward workspace is constant once M reaches one token chunk (8192).
    assert rows[3][1] == rows[4][1] == rows[5][1]
    # The forward partials ([NBLK, M] with NBLK * (M / 256) ~ 256 workgroups) stay ~1 MiB here and
    # grow at most linearly with M (like lse).
    assert rows[4][2] <= 2 * rows[3][2] and rows[5][2] <= 2 * rows[4][2]
