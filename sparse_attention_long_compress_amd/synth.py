"""Seeded synthetic inputs for the NSA forward/backward workloads.

This module only draws random numbers and shapes them; it contains none of the
attention arithmetic.  Tests, the smoke check and the benchmark all take their
inputs from here, and both the HIP library and the CPU oracle consume exactly
the same values (bf16 inputs are rounded once, round-to-nearest-even, and the
oracle reads those rounded values widened to float64).

Recipe (numpy ``default_rng(seed)``; draw order q, k, v, gate logits, dO, all
float32 standard normal):
  * gates = sigmoid(logits) in float32, layout [B, T, Hq, 3] = (cmp, sel, win);
  * ``qk_norm``: every (token, head) vector of q and k is rescaled to L2 norm
    sqrt(D) (QK-norm-like); v is left N(0, 1);
  * ``planted_sigma``: after the draws above, one offset c ~ N(0, sigma^2 I) per
    (batch, 64-token block, KV head) is drawn and added to every key of that
    block, which spreads the block-importance scores so that most top-k
    decisions have a clear margin.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

try:  # torch is plumbing only (device memory); numpy does the drawing
    import torch
except Exception:  # pragma: no cover
    torch = None


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    top_k: int = 16
    window: int = 512
    block: int = 64
    dtype: str = "bf16"  # "bf16" or "fp32"
    qk_norm: bool = False
    seed: int = 1000
    gate_override: tuple | None = None  # force (g_cmp, g_sel, g_win) values; None = drawn
    flags: tuple = field(default_factory=tuple)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the study's configuration (block 64, top-k 16, window
# 512 at sequence 8192), plus the tiny fp32 case and the 32k long-context case.
WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", 1, 1024, 4, 1, 64, top_k=4, window=128,
                          dtype="fp32", seed=1000),
    "340m-gqa4": Workload("340m-gqa4", 1, 8192, 16, 4, 64, seed=1001),
    "1b3-gqa4": Workload("1b3-gqa4", 4, 8192, 16, 4, 128, qk_norm=True, seed=1002),
    "mqa-ablation": Workload("mqa-ablation", 4, 8192, 16, 1, 128, seed=1003),
    "32k-fwd-bwd": Workload("32k-fwd-bwd", 1, 32768, 16, 4, 128, seed=1004),
}


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def draw(wl: Workload, *, planted_sigma: float = 0.0, with_dout: bool = False,
         seq_len: int | None = None, prefix: int | None = None):
    """Draw float32 numpy inputs for ``wl`` (optionally with a shorter sequence).

    ``seq_len`` draws a different, shorter workload; ``prefix`` draws the full
    workload and keeps its first ``prefix`` positions (a causal slice of it).
    Returns dict(q, k, v, gates[, dout]) of float32 arrays in the layouts
    q/dout [B,T,Hq,D], k/v [B,T,Hkv,D], gates [B,T,Hq,3]."""
    if prefix is not None:
        full = draw(wl, planted_sigma=planted_sigma, with_dout=with_dout)
        return {k: np.ascontiguousarray(v[:, :prefix]) for k, v in full.items()}
    T = seq_len if seq_len is not None else wl.seq_len
    B, Hq, Hkv, D = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    rng = np.random.default_rng(wl.seed)
    q = rng.standard_normal((B, T, Hq, D), dtype=np.float32)
    k = rng.standard_normal((B, T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, T, Hkv, D), dtype=np.float32)
    logits = rng.standard_normal((B, T, Hq, 3), dtype=np.float32)
    dout = rng.standard_normal((B, T, Hq, D), dtype=np.float32) if with_dout else None
    if wl.qk_norm:
        for x in (q, k):
            n = np.sqrt((x.astype(np.float64) ** 2).sum(-1, keepdims=True))
            x *= (np.sqrt(D) / n).astype(np.float32)
    if planted_sigma > 0.0:
        nb = -(-T // wl.block)
        off = rng.standard_normal((B, nb, Hkv, D), dtype=np.float32) * np.float32(planted_sigma)
        k += np.repeat(off, wl.block, axis=1)[:, :T]
    gates = _sigmoid(logits)
    if wl.gate_override is not None:
        gates[...] = np.asarray(wl.gate_override, dtype=np.float32)
    out = {"q": q, "k": k, "v": v, "gates": gates}
    if with_dout:
        out["dout"] = dout
    return out


def to_dtype(arrs: dict, dtype: str) -> dict:
    """Round every float array once to the workload dtype (bf16: RNE via torch).
    Returns torch CPU tensors."""
    assert torch is not None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {name: torch.from_numpy(np.ascontiguousarray(a)).to(tdt) for name, a in arrs.items()}


def as_f64(t) -> np.ndarray:
    """Exact widening of a (CPU or device) torch tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
