"""Seeded synthetic inputs for the ORPO head (shared by the tests, the bench and the oracle runs).

This module only *draws* inputs: hidden states, head weights (dense or 4-bit group-encoded), branch
lengths and labels. It holds none of the head's arithmetic (no softcap, no log-sum-exp, no loss, no
dequantisation). The one matmul here is the plain ``h @ W.T`` used to pick "peaked" labels
(argmax of the raw logits for 70% of the tokens), done by a library primitive.

Workload recipe (restating the pages' workloads in synthetic form; the real e4b / MiniCPM heads and
teacher-forced hiddens the pages measure on are not available, and these distributions stand in):
  * h    : N(0,1) per element, each row divided by its RMS, then rounded to bf16 (fp32 for the tiny
           fp32 workload).
  * W    : N(0,1) * 3/sqrt(d), rounded to bf16 (fp32 for the tiny workload), so logit std is ~3.
  * q4   : W encoded per 64-wide group along d: bias = bf16(min), scale = bf16((max-min)/15),
           q = clamp(rint((w - bias)/scale), 0, 15), 8 codes per uint32, LSB-first along d.
  * labels: with prob. 0.7 the argmax of the raw logits h.W^T (lowest index on ties; for the q4
           workload taken on the unquantised weights), else uniform on [0, V); padding = -100.
  * lengths: every branch length drawn independently, uniform on [lo, hi] (inclusive); if the sum
           exceeds M every length is scaled by M/sum (floor, at least 1). Branches are packed
           chosen_0, rejected_0, chosen_1, ... from position 0; positions after the last branch
           are padding.
Seeds: numpy SeedSequence(1000*k + s).spawn(5) -> [lengths, h, W, label-coin, label-uniform].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class HeadConfig:
    key: int
    name: str
    M: int
    d: int
    V: int
    pairs: int
    len_lo: int
    len_hi: int
    softcap: float
    lam: float
    dtype: str = "bf16"      # "f32" or "bf16" (h and W)
    q4: bool = False         # W as 4-bit group-encoded (group 64 along d)
    prompt_lo: int = 0       # prompt span lengths U[prompt_lo, prompt_hi] per pair; prompt_hi = 0:
    prompt_hi: int = 0       # no prompt spans (response-scope NLL)
    w_std: float = 3.0       # W entries N(0, (w_std / sqrt(d))^2): logit standard deviation ~ w_std
    p_argmax: float = 0.7    # share of labels that are the row's argmax (the rest uniform)

    @property
    def scope(self) -> str:
        """NLL scope of the workload: "full" (prompt + chosen) when it has prompt spans."""
        return "full" if self.prompt_hi > 0 else "response"

    @property
    def spans_per_pair(self) -> int:
        return 3 if self.prompt_hi > 0 else 2

    def replace(self, **kw) -> "HeadConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: HeadConfig(1, "tiny-f32", M=256, d=256, V=4096, pairs=1, len_lo=128, len_hi=128,
                  softcap=0.0, lam=0.1, dtype="f32"),
    2: HeadConfig(2, "minicpm-like-bf16", M=4096, d=1536, V=73448, pairs=8, len_lo=128, len_hi=384,
                  softcap=0.0, lam=0.1),
    3: HeadConfig(3, "e4b-bf16-softcap30", M=8192, d=2560, V=262144, pairs=16, len_lo=192, len_hi=320,
                  softcap=30.0, lam=0.1),
    4: HeadConfig(4, "q4g64-minicpm-shape-softcap30", M=8192, d=1536, V=73448, pairs=16, len_lo=128,
                  len_hi=384, softcap=30.0, lam=0.1, q4=True),
    5: HeadConfig(5, "12b-like-bf16-softcap30", M=32768, d=3840, V=262144, pairs=32, len_lo=256,
                  len_hi=768, softcap=30.0, lam=0.2),
    # The e4b head on peaked, teacher-forced-like logits (logit std 12 under the softcap, 95 % of
    # labels the argmax): the data the backward's coefficient filter is meant for.
    7: HeadConfig(7, "e4b-bf16-softcap30-peaked", M=8192, d=2560, V=262144, pairs=16, len_lo=192,
                  len_hi=320, softcap=30.0, lam=0.1, w_std=12.0, p_argmax=0.95),
    # The 4-bit head at the e4b shape (d = 2560, V = 262144): the shape of the pages' own quantised
    # head; lengths, softcap and lambda as the 4-bit workload at the MiniCPM shape. dh only.
    8: HeadConfig(8, "q4g64-e4b-shape-softcap30", M=8192, d=2560, V=262144, pairs=16, len_lo=128,
                  len_hi=384, softcap=30.0, lam=0.1, q4=True),
    # The e4b head with the full-scope NLL: each pair's chosen sequence also carries its prompt span.
    6: HeadConfig(6, "e4b-bf16-softcap30-fullnll", M=8192, d=2560, V=262144, pairs=16, len_lo=144,
                  len_hi=240, softcap=30.0, lam=0.1, prompt_lo=64, prompt_hi=128),
}


WORKLOADS = {cfg.name: cfg for cfg in CONFIGS.values()}   # the same workloads, by name


def workload(name_or_key) -> HeadConfig:
    """A workload by its name (e.g. "e4b-bf16-softcap30") or its integer seed key."""
    if isinstance(name_or_key, int) or str(name_or_key).isdigit():
        return CONFIGS[int(name_or_key)]
    return WORKLOADS[name_or_key]


def reduced(cfg: HeadConfig, pairs: int = 1) -> HeadConfig:
    """Same d, V, softcap and distributions with only `pairs` pairs; M = the largest packing."""
    return cfg.replace(pairs=pairs, M=pairs * (2 * cfg.len_hi + cfg.prompt_hi),
                       name=cfg.name + f"-{pairs}pair")


def _streams(key: int, seed: int):
    ss = np.random.SeedSequence(1000 * key + seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]


def draw_lengths(rng: np.random.Generator, n_branches: int, lo: int, hi: int, M: int) -> np.ndarray:
    lens = rng.integers(lo, hi + 1, size=n_branches).astype(np.int64)
    tot = int(lens.sum())
    if tot > M:
        lens = np.maximum(1, (lens * M) // tot)
    return lens


def seg_offsets_from_lengths(lens: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lens) + 1, dtype=np.int32)
    off[1:] = np.cumsum(lens)
    return off


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """Round-to-nearest-even to bf16 (torch's conversion)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def encode_q4(w: np.ndarray, group: int = 64):
    """Affine 4-bit encoding per `group` columns: returns (packed uint32 [V, d/8], scale bf16, bias bf16)."""
    V, d = w.shape
    assert d % group == 0 and group % 8 == 0
    g = w.reshape(V, d // group, group).astype(np.float32)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    scale_t = to_bf16((hi - lo) / 15.0)
    bias_t = to_bf16(lo)
    scale = scale_t.float().numpy()
    bias = bias_t.float().numpy()
    safe = np.where(scale == 0, 1.0, scale)
    q = np.rint((g - bias[:, :, None]) / safe[:, :, None])
    q = np.where(scale[:, :, None] == 0, 0, np.clip(q, 0, 15)).astype(np.uint32).reshape(V, d)
    q = q.reshape(V, d // 8, 8)
    shifts = (np.arange(8, dtype=np.uint32) * 4)[None, None, :]
    packed = np.bitwise_or.reduce(q << shifts, axis=2).astype(np.uint32)
    return packed, scale_t, bias_t


def argmax_labels(h: torch.Tensor, w: torch.Tensor, device: str, rows: int = 1024) -> np.ndarray:
    """argmax_v (h . W_v) per row in fp32 (first index on ties), in row chunks on `device`."""
    out = np.empty(h.shape[0], dtype=np.int64)
    wd = w.to(device=device, dtype=torch.float32)
    prev = None
    if device.startswith("cuda"):
        prev = torch.backends.cuda.matmul.allow_tf32
        torch.backends.cuda.matmul.allow_tf32 = False
    try:
        for r0 in range(0, h.shape[0], rows):
            hd = h[r0:r0 + rows].to(device=device, dtype=torch.float32)
            out[r0:r0 + rows] = torch.argmax(hd @ wd.T, dim=1).cpu().numpy()
    finally:
        if prev is not None:
            torch.backends.cuda.matmul.allow_tf32 = prev
    del wd
    return out


@dataclasses.dataclass
class HeadInputs:
    cfg: HeadConfig
    seed: int
    h: torch.Tensor                 # [M, d] float32 or bfloat16 (CPU)
    w: torch.Tensor | None          # [V, d] float32 or bfloat16 (CPU); None for q4
    wq: np.ndarray | None           # [V, d/8] uint32 (q4 only)
    scales: torch.Tensor | None     # [V, d/64] bfloat16 (q4 only)
    biases: torch.Tensor | None     # [V, d/64] bfloat16 (q4 only)
    labels: np.ndarray              # [M] int32, -100 for padding
    seg_offsets: np.ndarray         # [2P+1] int32 ([3P+1] with prompt spans)
    lengths: np.ndarray             # [2P] int64 ([3P])

    @property
    def n_valid(self) -> int:
        return int((self.labels != IGNORE_INDEX).sum())


def make_inputs(cfg: HeadConfig, seed: int = 0, label_device: str = "cpu") -> HeadInputs:
    r_len, r_h, r_w, r_coin, r_uni = _streams(cfg.key, seed)
    M, d, V = cfg.M, cfg.d, cfg.V
    lens = draw_lengths(r_len, 2 * cfg.pairs, cfg.len_lo, cfg.len_hi, M)
    if cfg.prompt_hi > 0:
        # Spans per pair: prompt, chosen, rejected (prompt lengths drawn after the responses', so a
        # workload without prompts draws exactly what it did before prompts existed).
        resp = lens
        prompts = r_len.integers(cfg.prompt_lo, cfg.prompt_hi + 1, size=cfg.pairs).astype(np.int64)
        lens = np.stack([prompts, resp[0::2], resp[1::2]], axis=1).reshape(-1)
        tot = int(lens.sum())
        if tot > M:
            lens = np.maximum(1, (lens * M) // tot)
    off = seg_offsets_from_lengths(lens)

    h64 = r_h.standard_normal((M, d))
    h64 /= np.sqrt(np.mean(h64 * h64, axis=1, keepdims=True))
    w32 = r_w.standard_normal((V, d), dtype=np.float32) * np.float32(cfg.w_std / math.sqrt(d))
    if cfg.dtype == "f32":
        h = torch.from_numpy(h64.astype(np.float32))
        w = torch.from_numpy(w32)
    else:
        h = to_bf16(h64)
        w = to_bf16(w32)
    del h64

    coin = r_coin.random(M)
    uni = r_uni.integers(0, V, size=M)
    arg = argmax_labels(h, torch.from_numpy(w32) if cfg.q4 else w, label_device)
    labels = np.where(coin < cfg.p_argmax, arg, uni).astype(np.int32)
    labels[int(off[-1]):] = IGNORE_INDEX

    wq = scales = biases = None
    if cfg.q4:
        wq, scales, biases = encode_q4(w32, 64)
        w = None
    del w32
    return HeadInputs(cfg, seed, h, w, wq, scales, biases, labels, off, lens)
