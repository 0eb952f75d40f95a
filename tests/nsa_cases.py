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


def check_indices(gpu_idx, ora, top_k, rows=None, scores=None, tpos=None):
    """Bit-exact on decisive rows, set-valid elsewhere.  Returns the boolean
    [B, Hkv, T'] mask of rows whose index sets agree exactly.

    Set validity of a row that differs from the oracle's (a near-tie, the
    reading of the target statement's gap rule): ascending, -1 padded, the
    forced blocks 0 and own present, the right number of free picks, all
    earlier than the own block; with the oracle's scores S given, every chosen
    free block has S >= S_(m) - 1e-3 and every unchosen candidate has
    S <= S_(m+1) + 1e-3, where S_(m) is the oracle's m-th largest candidate
    score.

    ``rows`` selects query positions of [B, Hkv, T, ...] tables; ``tpos``
    instead gives the query position of each entry of the third axis directly
    (the tables are then already that size)."""
    gi = np.asarray(gpu_idx)
    oi = np.asarray(ora["indices"])
    gap = np.asarray(ora["gap"])
    Sc = None if scores is None else np.asarray(scores)
    if rows is not None:
        gi, oi, gap = gi[:, :, rows], oi[:, :, rows], gap[:, :, rows]
        if Sc is not None:
            Sc = Sc[:, :, rows]
    agree = np.all(gi == oi, axis=-1)
    decisive = gap > GAP_TOL
    bad = decisive & ~agree
    assert not bad.any(), f"{bad.sum()} decisive rows differ, e.g. {np.argwhere(bad)[:5]}"
    B, Hkv, Tn, K = gi.shape
    if tpos is None:
        tpos = np.asarray(rows) if rows is not None else np.arange(Tn)
    tpos = np.asarray(tpos)
    dif = np.argwhere(~agree)
    if len(dif) == 0:
        return agree
    R = gi[dif[:, 0], dif[:, 1], dif[:, 2]].astype(np.int64)       # [n, K]
    t = tpos[dif[:, 2]].astype(np.int64)
    own = t // 64
    valid = R >= 0
    # -1 padding only at the end, strictly ascending entries before it
    nv = valid.sum(1)
    assert np.all(valid == (np.arange(K)[None, :] < nv[:, None])), "padding not at the end"
    asc = np.where(valid[:, 1:], R[:, 1:] > R[:, :-1], True)
    assert np.all(asc), "entries not strictly ascending"
    has0 = np.any(R == 0, axis=1)
    hasown = np.any(R == own[:, None], axis=1)
    assert np.all(has0 & hasown), "forced blocks missing"
    free = valid & (R != 0) & (R != own[:, None])
    m = top_k - np.where(own == 0, 1, 2)
    nfree = free.sum(1)
    assert np.all(nfree == np.minimum(m, np.maximum(own - 1, 0))), "wrong number of free picks"
    assert np.all(np.where(free, (R >= 1) & (R < own[:, None]), True)), "free pick out of range"
    if Sc is not None:
        nb = Sc.shape[-1]
        for n, (b, g, ti) in enumerate(dif):
            o = int(own[n])
            mm = int(m[n])
            if o - 1 <= mm:
                continue  # every candidate taken: nothing to rank
            S = Sc[b, g, ti]
            cand = np.arange(1, o)
            chosen = np.zeros(nb, dtype=bool)
            chosen[R[n][free[n]]] = True
            order = np.sort(S[cand])[::-1]
            s_m, s_m1 = order[mm - 1], order[mm]
            c = chosen[cand]
            assert np.all(S[cand][c] >= s_m - GAP_TOL), (int(t[n]), "chosen below the m-th score")
            assert np.all(S[cand][~c] <= s_m1 + GAP_TOL), (int(t[n]), "unchosen above the (m+1)-th score")
    return agree


def gpu_forward(wl: Workload, dev, **kw):
    return nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                       window=wl.window, scale=wl.scale, **kw)


def to_np(t):
    return as_f64(t)
