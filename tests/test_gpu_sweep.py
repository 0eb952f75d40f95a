"""GPU parity over a seeded sweep of shapes inside the library's envelope:
random batch, sequence length, heads per KV group, head dim, dtype, top-k and
window, each forward compared with the fp64 oracle row by row, the selection
backward on half of the shapes and the full backward (all branches and the
gates) on the other half with the oracle's gradients, the skip flags on a
third of them, logits 40 times larger (the exact-maximum path) on a quarter;
and a seeded sweep of decode steps (caches of random lengths, skip flags).  The shapes are drawn once
from a fixed seed, so the set is the same on every run."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_compress_amd as nsa
from sparse_attention_long_compress_amd.synth import Workload
from tests.nsa_cases import (assert_close, check_indices, device_inputs, gpu_forward,
                             oracle_forward, to_np)
from tests.test_gpu_backward import grad_close, run_both
from tests.test_gpu_full_backward import check_full
from tests.test_gpu_forward import LSE_TOL, _skip_flag_case
from tests.test_gpu_decode import run_case as decode_case

pytestmark = pytest.mark.gpu


def _draw_cases(seed=20261203):
    # every (heads per group, head dim / dtype) pair twice, the rest drawn
    rng = np.random.default_rng(seed)
    cases = []
    for rep in range(2):
        for g in (1, 2, 4, 8, 16):
            for d, dtype in ((64, "bf16"), (128, "bf16"), (64, "fp32")):
                hkv = int(rng.integers(1, max(1, 16 // g) + 1))
                T = 64 * int(rng.integers(1, 33))           # 64 .. 2048
                cases.append(dict(batch=int(rng.integers(1, 3)), seq_len=T, n_q_heads=g * hkv,
                                  n_kv_heads=hkv, head_dim=d, top_k=int(rng.integers(2, 33)),
                                  window=int(rng.choice([1, 63, 64, 100, 500, 512, 777, 1024, 4096])),
                                  dtype=dtype, qk_norm=bool(d == 128 and rng.random() < 0.5),
                                  seed=5000 + len(cases), planted=float(rng.choice([0.0, 1.0]))))
    return cases


def _draw_long_packed_cases(seed=20261205):
    # four heads per KV group at head_dim 64 in bf16 (the packed selection
    # kernel) at lengths where its walk spans several 48-block item tables
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(6):
        hkv = int(rng.integers(1, 5))
        cases.append(dict(batch=int(rng.integers(1, 3)), seq_len=64 * int(rng.integers(49, 257)),
                          n_q_heads=4 * hkv, n_kv_heads=hkv, head_dim=64,
                          top_k=int(rng.integers(2, 33)),
                          window=int(rng.choice([1, 64, 500, 512, 777, 1024, 2048])), dtype="bf16",
                          qk_norm=False, seed=7000 + i, planted=float(rng.choice([0.0, 1.0]))))
    return cases


BASE = _draw_cases()
LONG = _draw_long_packed_cases()
CASES = BASE + LONG


def _wl(c):
    return Workload("sweep", c["batch"], c["seq_len"], c["n_q_heads"], c["n_kv_heads"], c["head_dim"],
                    top_k=c["top_k"], window=c["window"], dtype=c["dtype"], qk_norm=c["qk_norm"],
                    seed=c["seed"])


@pytest.mark.parametrize("c", CASES, ids=[f"s{c['seed']}" for c in CASES])
def test_forward_sweep(c):
    wl = _wl(c)
    print("case", c, flush=True)
    dev, f64 = device_inputs(wl, seq_len=c["seq_len"], planted_sigma=c["planted"])
    res = gpu_forward(wl, dev, want_indices=True, want_lse=True, want_o_sel=True)
    torch.cuda.synchronize()
    ora = oracle_forward(wl, f64, want_scores=True)
    gi = res["indices"].cpu().numpy()
    agree = check_indices(gi, ora, wl.top_k, scores=ora["scores"])
    print("index agreement", agree.mean(), flush=True)
    if not agree.all():
        ora = oracle_forward(wl, f64, indices=gi)
    assert_close(to_np(res["out"]), ora["out"], wl.dtype, "out")
    assert_close(to_np(res["o_sel"]), ora["o_sel"], wl.dtype, "o_sel")
    err = np.abs(res["lse_sel"].cpu().double().numpy() - ora["lse_sel"])
    assert err.max() < LSE_TOL[wl.dtype], err.max()


# the selection backward on every other short shape of the sweep
@pytest.mark.parametrize("c", BASE[::2], ids=[f"s{c['seed']}" for c in BASE[::2]])
def test_select_bwd_sweep(c):
    wl = _wl(c)
    print("case", c, flush=True)
    got, ref, *_ = run_both(wl, c["seq_len"], planted=c["planted"])
    G = wl.n_q_heads // wl.n_kv_heads
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        grad_close(to_np(g_), r_, wl.dtype, nm, heads_per_key=1 if nm == "dq" else G)


# the full backward (all branches, gate gradients) on the remaining short shapes and two long ones
@pytest.mark.parametrize("c", BASE[1::2] + LONG[1:4:2], ids=[f"s{c['seed']}" for c in BASE[1::2] + LONG[1:4:2]])
def test_full_backward_sweep(c):
    wl = _wl(c)
    print("case", c, flush=True)
    check_full(wl, c["seq_len"])


FLAG_SETS = [nsa.SKIP_CMP_OUT, nsa.SKIP_SEL, nsa.SKIP_WIN, nsa.SKIP_CMP_OUT | nsa.SKIP_SEL,
             nsa.SKIP_CMP_OUT | nsa.SKIP_WIN, nsa.SKIP_SEL | nsa.SKIP_WIN]


# skip flags (a skipped branch equals a zero gate) on every third shape
@pytest.mark.parametrize("c", CASES[::3], ids=[f"s{c['seed']}" for c in CASES[::3]])
def test_skip_flags_sweep(c):
    wl = _wl(c)
    flag = FLAG_SETS[c["seed"] % len(FLAG_SETS)]
    print("case", c, "flags", flag, flush=True)
    dev, f64 = device_inputs(wl, seq_len=c["seq_len"], planted_sigma=c["planted"])
    _skip_flag_case(wl, dev, f64, flag)


def _draw_decode_cases(seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for g in (1, 2, 4, 8, 16):
        for d, dtype in ((64, "bf16"), (128, "bf16"), (64, "fp32")):
            hkv = int(rng.integers(1, max(1, 16 // g) + 1))
            B = int(rng.integers(1, 5))
            lmax = 64 * int(rng.integers(1, 65))           # 64 .. 4096
            lens = sorted(int(x) for x in rng.integers(1, lmax + 1, B))
            lens[-1] = lmax
            flags = int(rng.choice([0, 0, 0] + FLAG_SETS[:4]))
            cases.append(dict(batch=B, seq_len=lmax, lens=lens, n_q_heads=g * hkv, n_kv_heads=hkv,
                              head_dim=d, top_k=int(rng.integers(2, 33)),
                              window=int(rng.choice([1, 63, 64, 100, 500, 512, 777, 1024, 4096])),
                              dtype=dtype, qk_norm=bool(d == 128 and rng.random() < 0.5),
                              seed=6000 + len(cases), flags=flags))
    return cases


DECODE_CASES = _draw_decode_cases()


@pytest.mark.parametrize("c", DECODE_CASES, ids=[f"d{c['seed']}" for c in DECODE_CASES])
def test_decode_sweep(c):
    wl = _wl(c)
    decode_case(wl, c["batch"], c["seq_len"], c["lens"], seed=c["seed"], flags=c["flags"])


# logits large enough that the fixed Cauchy-Schwarz reference is too loose (the
# exact-maximum path), every fourth shape: every saved tensor of the training
# forward against the oracle on the oracle's index table
@pytest.mark.parametrize("c", CASES[::4], ids=[f"s{c['seed']}" for c in CASES[::4]])
def test_large_logits_sweep(c):
    wl = _wl(c)
    print("case", c, "q x 40", flush=True)
    dev, f64 = device_inputs(wl, seq_len=c["seq_len"], planted_sigma=1.0, q_scale=40.0)
    ora = oracle_forward(wl, f64)
    idx = torch.from_numpy(ora["indices"]).to("cuda")
    sv = nsa.forward_train(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                           window=wl.window, scale=wl.scale, indices=idx)
    torch.cuda.synchronize()
    for nm in ("out", "o_sel", "o_win", "o_cmp"):
        assert_close(to_np(sv[nm]), ora[nm], wl.dtype, nm)
    for nm in ("lse_sel", "lse_win"):
        got = sv[nm].cpu().double().numpy()
        fin = np.isfinite(ora[nm])
        np.testing.assert_array_equal(np.isfinite(got), fin)
        rel = np.abs(got[fin] - ora[nm][fin]) / np.maximum(1.0, np.abs(ora[nm][fin]))
        print(nm, "max rel", rel.max(), flush=True)
        assert rel.max() < 2e-3, (nm, rel.max())
