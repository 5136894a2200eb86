"""GPU parity on seeded random shapes: token counts from a handful to over a thousand, hidden sizes
64-512, vocabularies from a few rows to tens of thousands, bf16 / fp32 / 4-bit heads, softcap off,
30 (fixed reference) and 50 (running maximum), with and without padding. Together they reach the
paths that fixed shapes pin one at a time: one and many vocabulary splits (both merges), split and
unsplit dh tiles with ragged K ranges, several backward items, and tail tiles of every width."""
import numpy as np
import pytest

from tests.gpu_helpers import assert_parity, run_gpu, run_oracle, say
from tests.test_gpu_parity import _custom

pytestmark = pytest.mark.gpu


def _cases(n, seed, budget=6e9):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([rng.integers(2, 64), rng.integers(64, 700), rng.integers(700, 1300)]))
        d = int(rng.choice([64, 128, 192, 256, 320, 448, 512]))
        V = int(rng.choice([rng.integers(1, 600), rng.integers(600, 8000), rng.integers(8000, 40000)]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        q4 = dtype == "bf16" and rng.random() < 0.3
        cap = float(rng.choice([0.0, 30.0, 50.0]))
        pairs = int(max(1, min(4, M // 2)))
        pad = bool(rng.random() < 0.7)
        if M * V * d > budget:
            continue
        out.append((M, d, V, dtype, q4, cap, pairs, pad, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("M,d,V,dtype,q4,cap,pairs,pad,seed", _cases(30, 2027))
def test_random_shape_parity(M, d, V, dtype, q4, cap, pairs, pad, seed):
    inp = _custom(M, d, V, dtype, cap, 0.1, seed=seed, pairs=pairs, q4=q4, pad=pad)
    say(f"[case] {inp.cfg.name} q4={q4} pairs={pairs} seed={seed}")
    assert_parity(run_gpu(inp), run_oracle(inp), inp.cfg.name)
