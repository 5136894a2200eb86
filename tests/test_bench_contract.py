"""bench.py's host-side contract without a GPU: the multi-GPU refusal, the GPU requirement, and
the CPU-baseline leg (the oracle timed on a bounded sample) for every objective and weight format."""
import os
import subprocess
import sys

import pytest

from lm_head_cross_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_no_gpu_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1 and "needs a GPU" in r.stderr and r.stdout == ""


def test_tokens_option_scales_the_workload():
    sys.path.insert(0, ROOT)
    import bench
    cfg = bench.workload_for("e4b-bf16-softcap30", 512)
    assert (cfg.M, cfg.pairs, cfg.d, cfg.V) == (512, 1, 2560, 262144)
    assert cfg.name == "e4b-bf16-softcap30-M512"
    assert bench.workload_for("e4b-bf16-softcap30", 2048).pairs == 4
    assert bench.workload_for("3") == synth.workload(3)
    # The two branches of the one pair are drawn from [192, 320] and shrink to fit in 512 tokens.
    lens = synth.draw_lengths(synth._streams(cfg.key, 0)[0], 2, cfg.len_lo, cfg.len_hi, cfg.M)
    assert lens.sum() <= 512 and (lens >= 1).all()
    with pytest.raises(ValueError):
        bench.workload_for("e4b-bf16-softcap30", -1)


@pytest.mark.parametrize("objective,q4,full", [("orpo", False, False), ("orpo", True, False),
                                               ("orpo", False, True), ("simpo", False, False),
                                               ("dpo", False, False), ("ipo", False, False),
                                               ("hinge", False, False), ("grpo", False, False),
                                               ("orpo", None, False)])
def test_cpu_baseline_leg(objective, q4, full):
    # q4 None: the bf16 head with a frozen weight (bench.py --no-dw), dh only.
    want_dw = q4 is False
    q4 = bool(q4)
    sys.path.insert(0, ROOT)
    import bench
    cfg = synth.HeadConfig(0, "cpu-leg", M=256, d=128, V=1024, pairs=1, len_lo=100, len_hi=120,
                           softcap=30.0, lam=0.1, q4=q4, prompt_lo=20 if full else 0,
                           prompt_hi=30 if full else 0)
    inp = synth.make_inputs(cfg, seed=1)
    out = bench.cpu_baseline(inp, 96, objective, want_dw)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "first 96 tokens" in out["sample"] and objective in out["sample"]
    assert ("+ dW" in out["sample"]) == want_dw
