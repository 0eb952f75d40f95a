"""Shared helpers for the GPU parity tests: run the HIP library and the oracle
on the same seeded inputs and compare them at the stated tolerances.

Tolerances (from the target statement of the method): bf16 inputs with fp32
accumulation -> max-abs 2e-2 and mean-abs 2e-3; fp32 inputs -> max-abs 1e-4.
Selected block indices must match exactly wherever the oracle's gap between
the m-th and (m+1)-th candidate score exceeds 1e-3; elsewhere the GPU's set
must be a valid top-m within that tolerance."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_attention_long_compress_amd as nsa
from sparse_attention_long_compress_amd.synth import Workload, as_f64, draw, to_dtype

GAP_TOL = 1e-3


def tol(dtype: str):
    return (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-4)


def device_inputs(wl: Workload, *, seq_len=None, planted_sigma=0.0, with_dout=False, q_scale=1.0,
                  prefix=None):
    arrs = draw(wl, planted_sigma=planted_sigma, with_dout=with_dout, seq_len=seq_len,
                prefix=prefix)
    if q_scale != 1.0:
        arrs["q"] = arrs["q"] * np.float32(q_scale)
    cpu = to_dtype(arrs, wl.dtype)
    dev = {k: v.to("cuda") for k, v in cpu.items()}
    f64 = {k: as_f64(v) for k, v in cpu.items()}
    return dev, f64


def oracle_forward(wl: Workload, f64, *, rows=None, indices=None, want_scores=False):
    return oracle.forward(f64["q"], f64["k"], f64["v"], f64["gates"], top_k=wl.top_k,
                          window=wl.window, scale=wl.scale, rows=rows, indices=indices,
                          want_scores=want_scores)


def assert_close(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx_tol, mean_tol = tol(dtype)
    assert err.max() <= mx_tol, f"{what}: max-abs {err.max():.3e} > {mx_tol}"
    assert err.mean() <= mean_tol, f"{what}: mean-abs {err.mean():.3e} > {mean_tol}"


def check_indices(gpu_idx, ora, top_k, rows=None, scores=None):
    """Bit-exact on decisive rows, set-valid elsewhere.  Returns the boolean
    [B, Hkv, T'] mask of rows whose index sets agree exactly."""
    gi = np.asarray(gpu_idx)
    oi = np.asarray(ora["indices"])
    gap = np.asarray(ora["gap"])
    if rows is not None:
        gi, oi, gap = gi[:, :, rows], oi[:, :, rows], gap[:, :, rows]
    agree = np.all(gi == oi, axis=-1)
    decisive = gap > GAP_TOL
    bad = decisive & ~agree
    assert not bad.any(), f"{bad.sum()} decisive rows differ, e.g. {np.argwhere(bad)[:5]}"
    # structural validity of every GPU row: ascending, -1 padded, forced blocks present
    B, Hkv, Tn, K = gi.shape
    tpos = np.asarray(rows) if rows is not None else np.arange(Tn)
    for b, g, ti in np.argwhere(~agree):
        t = int(tpos[ti])
        row = [int(x) for x in gi[b, g, ti] if x >= 0]
        own = t // 64
        assert row == sorted(set(row)), row
        assert 0 in row and own in row, (t, row)
        m = top_k - (1 if own == 0 else 2)
        free = [j for j in row if j not in (0, own)]
        assert len(free) == min(m, max(own - 1, 0)), (t, row)
        assert all(1 <= j < own for j in free), (t, row)
        if scores is not None:
            S = scores[b, g, t]
            cands = np.arange(1, own)
            order = np.sort(S[cands])[::-1]
            s_m, s_m1 = order[m - 1], order[m]
            for j in cands:
                if j in free:
                    assert S[j] >= s_m - GAP_TOL, (t, j)
                else:
                    assert S[j] <= s_m1 + GAP_TOL, (t, j)
    return agree


def rows_mask_from_groups(agree, Hq):
    """[B, Hkv, T'] -> [B, T', Hq] boolean mask for per-head outputs."""
    B, Hkv, Tn = agree.shape
    G = Hq // Hkv
    return np.repeat(np.transpose(agree, (0, 2, 1)), G, axis=2)


def gpu_forward(wl: Workload, dev, **kw):
    return nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                       window=wl.window, scale=wl.scale, **kw)


def to_np(t):
    return as_f64(t)
