"""GPU parity of the selection-branch backward (two-pass, atomic-free) against
the fp64 oracle.  The selection is frozen to the oracle's own index table on
both sides (the library takes it through NSA_INDICES_IN), so the saved
log-sum-exp and selection output that the backward consumes match the
oracle's selection exactly.

Tolerances: the pages give none for gradients.  Reading used here: the
forward's bounds scaled by the gradient's root-mean-square magnitude --
max-abs <= 2e-2 * max(1, rms_ref) and mean-abs <= 2e-3 * max(1, rms_ref) for
bf16, 1e-4 * max(1, rms_ref) for fp32 -- with one addition for bf16: each
product in a gradient sum has operands that carry up to four bf16 unit
roundoffs (2^-8 each) of relative error -- P rounded for the MFMA and
normalised by the saved log-sum-exp (itself a sum of bf16-rounded
probabilities), dS = P (dP - Delta) rounded, g_sel dO rounded -- so an element
may also be off by 2^-6 of its own magnitude (elements are as large as their
own terms make them: the first keys, which few queries share, get gradients
~50x the rms).  dk and dv of one key sum the terms of all G query heads of its
group: with rounding errors of independent sign, their spread grows as the
square root of the number of terms, so for G > 4 (more heads per key than the
GQA-4 workloads the bound was set on) the max-abs allowance is scaled by
sqrt(G / 4).  Each case prints its measured errors."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_compress_amd as nsa
from sparse_attention_long_compress_amd.synth import WORKLOADS
from tests.nsa_cases import device_inputs, oracle_forward, to_np

pytestmark = pytest.mark.gpu


REL_BF16 = 2.0 ** -6


def grad_close(got, ref, dtype, what, heads_per_key=1):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    rms = max(1.0, float(np.sqrt((ref ** 2).mean())))
    err = np.abs(got - ref)
    mx, mean = (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-4)
    mx *= np.sqrt(max(1.0, heads_per_key / 4.0))
    rel = REL_BF16 if dtype == "bf16" else 0.0
    excess = float((err - rel * np.abs(ref)).max())
    print(f"{what}: max|ref| {np.abs(ref).max():.3g} rms_ref {np.sqrt((ref ** 2).mean()):.3g} "
          f"max-abs {err.max():.3e} mean-abs {err.mean():.3e} "
          f"max(|err| - {rel:.3g}|ref|) {excess:.3e} bound {mx * rms:.1e}", flush=True)
    assert excess <= mx * rms, f"{what}: max(|err| - {rel}|ref|) {excess:.3e} > {mx * rms:.3e}"
    assert err.mean() <= mean * rms, f"{what}: mean-abs {err.mean():.3e} > {mean * rms:.3e}"


def run_both(wl, T, planted=0.0, prefix=False):
    if prefix:
        dev, f64 = device_inputs(wl, prefix=T, with_dout=True)
        wl = wl.with_(seq_len=T)
    else:
        dev, f64 = device_inputs(wl, seq_len=T, planted_sigma=planted, with_dout=True)
    ora = oracle_forward(wl, f64)
    idx = torch.from_numpy(ora["indices"]).to("cuda")
    fwd = nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                      window=wl.window, scale=wl.scale, indices=idx, want_lse=True,
                      want_o_sel=True)
    dq, dk, dv = nsa.select_bwd(dev["q"], dev["k"], dev["v"], dev["gates"], idx, fwd["lse_sel"],
                                fwd["o_sel"], dev["dout"], top_k=wl.top_k, scale=wl.scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.select_bwd(f64["q"], f64["k"], f64["v"], f64["gates"], ora["indices"],
                                   f64["dout"], top_k=wl.top_k, scale=wl.scale)
    return (dq, dk, dv), (rq, rk, rv), dev, idx, fwd


CASES = [
    ("tiny-fp32", 512, {}),
    ("340m-gqa4", 1024, {}),
    ("340m-gqa4", 2048, {}),
    ("1b3-gqa4", 1024, {"batch": 1}),
    ("mqa-ablation", 512, {"batch": 1}),
    ("340m-gqa4", 512, {"n_q_heads": 4, "n_kv_heads": 4}),                # G = 1
    ("1b3-gqa4", 512, {"batch": 2, "n_q_heads": 8, "n_kv_heads": 4}),     # G = 2
    ("1b3-gqa4", 512, {"batch": 1, "n_q_heads": 16, "n_kv_heads": 2}),    # G = 8
    ("340m-gqa4", 640, {"top_k": 3}),
]


@pytest.mark.parametrize("name,T,over", CASES)
def test_select_bwd_matches_oracle(name, T, over):
    wl = WORKLOADS[name].with_(**over)
    print("case", name, T, over, flush=True)
    got, ref, *_ = run_both(wl, T)
    G = wl.n_q_heads // wl.n_kv_heads
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        grad_close(to_np(g_), r_, wl.dtype, nm, heads_per_key=1 if nm == "dq" else G)


def test_select_bwd_full_size_340m():
    # the launch the bench times: 340M shapes at T = 8192, every element
    wl = WORKLOADS["340m-gqa4"]
    print("case 340m-gqa4 full size", flush=True)
    got, ref, *_ = run_both(wl, wl.seq_len)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        grad_close(to_np(g_), r_, wl.dtype, nm + "@8192")


def test_select_bwd_longest_sequence():
    # the longest sequence the library accepts (65536 positions, 1024 key
    # blocks) on the bench's backward kernels (bf16, head_dim 64, four query
    # heads per KV group), one KV group so that the oracle's scatter (one
    # thread per batch and group) finishes in about a minute; every element
    wl = WORKLOADS["340m-gqa4"].with_(n_q_heads=4, n_kv_heads=1)
    print("case 340m-gqa4 65536 Hq 4 Hkv 1", flush=True)
    got, ref, *_ = run_both(wl, 65536)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        grad_close(to_np(g_), r_, wl.dtype, nm + "@65536")


def test_select_bwd_is_bitwise_reproducible():
    wl = WORKLOADS["340m-gqa4"]
    got, _, dev, idx, fwd = run_both(wl, 1024)
    again = nsa.select_bwd(dev["q"], dev["k"], dev["v"], dev["gates"], idx, fwd["lse_sel"],
                           fwd["o_sel"], dev["dout"], top_k=wl.top_k, scale=wl.scale)
    torch.cuda.synchronize()
    for a, b in zip(got, again):
        assert torch.equal(a, b)


def test_select_bwd_32k_on_a_2048_slice():
    # Long-context workload (B1 T32768 Hq16 Hkv4 D128): by causality the first
    # 2048 positions' selections, softmax and dq are those of the 2048-token
    # prefix, which the oracle computes in full; dk/dv of the prefix run are
    # checked in the same call.
    wl = WORKLOADS["32k-fwd-bwd"]
    dev, _ = device_inputs(wl, with_dout=True)
    fwd = nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                      window=wl.window, scale=wl.scale, want_indices=True, want_lse=True,
                      want_o_sel=True)
    dq, dk, dv = nsa.select_bwd(dev["q"], dev["k"], dev["v"], dev["gates"], fwd["indices"],
                                fwd["lse_sel"], fwd["o_sel"], dev["dout"], top_k=wl.top_k,
                                scale=wl.scale)
    torch.cuda.synchronize()
    got_pre, ref_pre, _, idx_pre, _ = run_both(wl, 2048, prefix=True)
    # the 2048-prefix run reproduces the first 2048 dq rows of the full run
    # (same kernels, same tiles) wherever the two index tables agree
    same_idx = (fwd["indices"][:, :, :2048] == idx_pre).all(-1).cpu()
    rows = same_idx.permute(0, 2, 1).repeat_interleave(wl.n_q_heads // wl.n_kv_heads, dim=2)
    assert rows.float().mean() > 0.9
    d_full = dq[:, :2048].float().cpu()[rows]
    d_pre = got_pre[0].float().cpu()[rows]
    assert torch.equal(d_full, d_pre)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got_pre, ref_pre):
        grad_close(to_np(g_), r_, wl.dtype, nm + "@2048")


SINGLE_CASES = [
    ("340m-gqa4", 1024, {}),
    ("1b3-gqa4", 1024, {"batch": 1}),
    ("340m-gqa4", 512, {"n_q_heads": 4, "n_kv_heads": 4}),                # G = 1
    ("1b3-gqa4", 512, {"batch": 1, "n_q_heads": 16, "n_kv_heads": 2}),    # G = 8
    ("340m-gqa4", 640, {"top_k": 3}),
]


@pytest.mark.parametrize("name,T,over", SINGLE_CASES)
def test_single_pass_atomic_backward_matches_oracle(name, T, over):
    # the one-pass alternative (dk / dv by fp32 atomics) at the same bounds
    wl = WORKLOADS[name].with_(**over)
    print("case", name, T, over, flush=True)
    _, ref, dev, idx, fwd = run_both(wl, T)
    got = nsa.select_bwd_single(dev["q"], dev["k"], dev["v"], dev["gates"], idx, fwd["lse_sel"],
                                fwd["o_sel"], dev["dout"], top_k=wl.top_k, scale=wl.scale)
    torch.cuda.synchronize()
    G = wl.n_q_heads // wl.n_kv_heads
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        grad_close(to_np(g_), r_, wl.dtype, nm, heads_per_key=1 if nm == "dq" else G)
