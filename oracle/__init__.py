"""fp64 CPU oracle for the NSA forward pass and the selection-branch gradient.

TEST INFRASTRUCTURE ONLY.  This package is the independent reference that the
HIP library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it.  It shares no code with
the HIP library (``sparse_attention_long_compress_amd``) and imports nothing
from it; the product path never calls it.

The arithmetic lives in ``nsa_oracle.c`` (plain C, double precision, OpenMP
across independent rows).  This module only builds that file with gcc, loads it
with ctypes and marshals numpy arrays.  Every function takes and returns
float64 arrays; bf16 inputs are widened to float64 exactly by the caller.

Parity-pin status (what pins each function; see tests/test_oracle_pins.py):
  pool              constant block, arithmetic-progression closed form
  forward/o_cmp     constant keys (uniform weights, closed form), torch fp64
                    SDPA over avg-pooled keys with a block-causal mask
  forward/indices   all-ties closed form, brute-force subset enumeration,
                    numpy stable argsort, the sparsity arithmetic of the
                    "Sparsity is Cool" Key claims (tests/golden)
  forward/o_sel     full causal attention when top-k covers all blocks (torch
                    SDPA), explicit-mask SDPA given the index table
  forward/lse_cmp   torch logsumexp over avg-pooled keys with the block-causal
                    mask; constant keys give tau q.c + log n_c (closed form)
  forward/lse_sel   torch logsumexp of causal attention (full coverage) and of
                    the explicit mask given the index table
  forward/o_win     W >= T full causal, W = 1 returns v_t, banded-mask SDPA
  forward/lse_win   torch logsumexp over the band; W >= T gives the causal
                    log-sum-exp, W = 1 gives tau q_t.k_t (closed forms)
  forward/out       zero gates, unit gates, linearity, shift invariances
  select_bwd        central finite differences, torch autograd of causal and
                    masked SDPA
  decode            the forward restricted to the last row of each prefix (its
                    definition); pinned by an explicit per-query enumeration of
                    the compressed, selected and window key sets in the tests;
                    its importance scores are those of forward/indices
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile nsa_oracle.c into libnsa_oracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-std=c99", "-Wall", "-shared", "-fPIC",
             _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
        ):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        ci = ctypes.c_int
        lib.nsa_oracle_pool.argtypes = [ci, ci, ci, ci, ci, dp, dp]
        lib.nsa_oracle_pool.restype = ci
        lib.nsa_oracle_forward.argtypes = (
            [ci] * 8 + [ctypes.c_double] + [dp] * 4 + [dp] * 7 + [ip, ci, dp, dp, ip, ci, ci]
        )
        lib.nsa_oracle_forward.restype = ci
        lib.nsa_oracle_select_bwd.argtypes = (
            [ci] * 7 + [ctypes.c_double] + [dp] * 4 + [ip, dp, dp, dp, dp, ci]
        )
        lib.nsa_oracle_select_bwd.restype = ci
        lib.nsa_oracle_backward.argtypes = (
            [ci] * 8 + [ctypes.c_double] + [dp] * 4 + [ip, dp, dp, dp, dp, dp, ci]
        )
        lib.nsa_oracle_backward.restype = ci
        _lib = lib
    return _lib


def _dptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def default_threads() -> int:
    return int(os.environ.get("NSA_ORACLE_THREADS", "0")) or (os.cpu_count() or 1)


def pool(x, blk: int = 64):
    """Mean-pool [B,T,H,D] over non-overlapping complete blocks -> [B,T//blk,H,D]."""
    x = _f64(x)
    B, T, H, D = x.shape
    out = np.zeros((B, T // blk, H, D), dtype=np.float64)
    rc = _load().nsa_oracle_pool(B, T, H, D, blk, _dptr(x), _dptr(out))
    if rc != 0:
        raise ValueError(f"nsa_oracle_pool failed: {rc}")
    return out


def forward(q, k, v, gates, *, top_k: int, window: int, blk: int = 64, scale: float | None = None,
            indices=None, want_scores: bool = False, rows=None, threads: int | None = None):
    """Full NSA forward.  Returns a dict of float64/int32 numpy arrays:
    out, o_cmp, o_sel, o_win [B,T,Hq,D]; lse_sel, lse_win, lse_cmp [B,Hq,T] (lse_cmp
    is -inf where no compressed block is visible); indices [B,Hkv,T,top_k];
    gap [B,Hkv,T]; scores [B,Hkv,T,nblk] (when want_scores).

    ``indices`` (optional, int32) freezes the selection to a table the oracle
    produced earlier instead of running the top-k step.  ``rows`` (optional)
    restricts the computation to those query positions; other rows stay 0."""
    q, k, v, gates = _f64(q), _f64(k), _f64(v), _f64(gates)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nblk = -(-T // blk)
    res = {
        "out": np.zeros((B, T, Hq, D)),
        "o_cmp": np.zeros((B, T, Hq, D)),
        "o_sel": np.zeros((B, T, Hq, D)),
        "o_win": np.zeros((B, T, Hq, D)),
        "lse_sel": np.zeros((B, Hq, T)),
        "lse_win": np.zeros((B, Hq, T)),
        "lse_cmp": np.zeros((B, Hq, T)),
        "gap": np.zeros((B, Hkv, T)),
    }
    if indices is not None:
        idx = np.ascontiguousarray(np.asarray(indices, dtype=np.int32)).copy()
        assert idx.shape == (B, Hkv, T, top_k)
    else:
        idx = np.zeros((B, Hkv, T, top_k), dtype=np.int32)
    res["indices"] = idx
    scores = np.zeros((B, Hkv, T, nblk)) if want_scores else None
    rows_a = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    rc = _load().nsa_oracle_forward(
        B, T, Hq, Hkv, D, blk, top_k, window, float(scale),
        _dptr(q), _dptr(k), _dptr(v), _dptr(gates),
        _dptr(res["out"]), _dptr(res["o_cmp"]), _dptr(res["o_sel"]), _dptr(res["o_win"]),
        _dptr(res["lse_sel"]), _dptr(res["lse_win"]), _dptr(res["lse_cmp"]),
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        1 if indices is not None else 0, _dptr(scores), _dptr(res["gap"]),
        rows_a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if rows_a is not None
        else ctypes.POINTER(ctypes.c_int32)(), 0 if rows_a is None else len(rows_a),
        threads if threads is not None else default_threads())
    if rc != 0:
        raise ValueError(f"nsa_oracle_forward failed: {rc}")
    if want_scores:
        res["scores"] = scores
    return res


def select_bwd(q, k, v, gates, indices, dout, *, top_k: int, blk: int = 64,
               scale: float | None = None, threads: int | None = None):
    """Gradient of the selection branch (indices and gates frozen).
    Returns (dq [B,T,Hq,D], dk [B,T,Hkv,D], dv [B,T,Hkv,D]) in float64."""
    q, k, v, gates, dout = _f64(q), _f64(k), _f64(v), _f64(gates), _f64(dout)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    idx = np.ascontiguousarray(np.asarray(indices, dtype=np.int32))
    assert idx.shape == (B, Hkv, T, top_k)
    dq = np.zeros((B, T, Hq, D))
    dk = np.zeros((B, T, Hkv, D))
    dv = np.zeros((B, T, Hkv, D))
    rc = _load().nsa_oracle_select_bwd(
        B, T, Hq, Hkv, D, blk, top_k, float(scale),
        _dptr(q), _dptr(k), _dptr(v), _dptr(gates),
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _dptr(dout),
        _dptr(dq), _dptr(dk), _dptr(dv),
        threads if threads is not None else default_threads())
    if rc != 0:
        raise ValueError(f"nsa_oracle_select_bwd failed: {rc}")
    return dq, dk, dv


def backward(q, k, v, gates, indices, dout, *, top_k: int, window: int, blk: int = 64,
             scale: float | None = None, threads: int | None = None):
    """Gradient of the whole NSA output (all three branches and the gates;
    the selection frozen to ``indices``).  Returns (dq [B,T,Hq,D], dk, dv
    [B,T,Hkv,D], dgates [B,T,Hq,3]) in float64."""
    q, k, v, gates, dout = _f64(q), _f64(k), _f64(v), _f64(gates), _f64(dout)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    idx = np.ascontiguousarray(np.asarray(indices, dtype=np.int32))
    assert idx.shape == (B, Hkv, T, top_k)
    dq = np.zeros((B, T, Hq, D))
    dk = np.zeros((B, T, Hkv, D))
    dv = np.zeros((B, T, Hkv, D))
    dg = np.zeros((B, T, Hq, 3))
    rc = _load().nsa_oracle_backward(
        B, T, Hq, Hkv, D, blk, top_k, window, float(scale),
        _dptr(q), _dptr(k), _dptr(v), _dptr(gates),
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _dptr(dout),
        _dptr(dq), _dptr(dk), _dptr(dv), _dptr(dg),
        threads if threads is not None else default_threads())
    if rc != 0:
        raise ValueError(f"nsa_oracle_backward failed: {rc}")
    return dq, dk, dv, dg


def decode(q, k_cache, v_cache, gates, seq_lens, *, top_k: int, window: int, blk: int = 64,
           scale: float | None = None, indices=None, threads: int | None = None):
    """One decode step ("DeepSeek's Native Sparse Attention", How Does NSA Work?,
    for a single query): sequence b of length L = seq_lens[b] has its query at
    t = L - 1, and its output is the prefill output of row t over the first L
    positions.  q [B,Hq,D], k_cache/v_cache [B,Lmax,Hkv,D], gates [B,Hq,3].
    ``indices`` (optional int32 [B,Hkv,top_k]) freezes the selection.
    Returns out, o_cmp, o_sel, o_win [B,Hq,D], indices [B,Hkv,top_k], the
    k-th vs (k+1)-th importance gap [B,Hkv] and the block importance scores
    [B,Hkv,ceil(Lmax/blk)] of each sequence's query row (0 past its complete
    blocks)."""
    q, kc, vc, gates = _f64(q), _f64(k_cache), _f64(v_cache), _f64(gates)
    B, Hq, D = q.shape
    Hkv = kc.shape[2]
    res = {n: np.zeros((B, Hq, D)) for n in ("out", "o_cmp", "o_sel", "o_win")}
    res["indices"] = np.zeros((B, Hkv, top_k), dtype=np.int32)
    res["gap"] = np.zeros((B, Hkv))
    res["scores"] = np.zeros((B, Hkv, -(-kc.shape[1] // blk)))
    for b in range(B):
        L = int(seq_lens[b])
        t = L - 1
        qf = np.zeros((1, L, Hq, D))
        qf[0, t] = q[b]
        gf = np.zeros((1, L, Hq, 3))
        gf[0, t] = gates[b]
        idx = None
        if indices is not None:
            idx = np.zeros((1, Hkv, L, top_k), dtype=np.int32)
            idx[0, :, t] = np.asarray(indices)[b]
        r = forward(qf, kc[b:b + 1, :L], vc[b:b + 1, :L], gf, top_k=top_k, window=window,
                    blk=blk, scale=scale, indices=idx, rows=[t], want_scores=True,
                    threads=threads)
        for n in ("out", "o_cmp", "o_sel", "o_win"):
            res[n][b] = r[n][0, t]
        res["indices"][b] = r["indices"][0, :, t]
        res["gap"][b] = r["gap"][0, :, t]
        sc = r["scores"][0, :, t]
        res["scores"][b, :, :sc.shape[-1]] = sc
    return res
