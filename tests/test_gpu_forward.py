"""GPU parity of the NSA forward (HIP library through the C ABI) against the
fp64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_compress_amd as nsa
from sparse_attention_long_compress_amd.synth import WORKLOADS, Workload
from tests.nsa_cases import (assert_close, check_indices, device_inputs, gpu_forward,
                             oracle_forward, to_np)

# Saved log-sum-exp of the selection softmax.  The library normalises with the
# sum of the bf16-rounded probabilities it feeds to the PV product (so that the
# output is an exact weighted average of those weights); each term carries a
# relative rounding error <= 2^-8 (bf16 unit roundoff), so the sum is off by
# <= 2^-8 relative and lse by <= ln(1 + 2^-8) ~ 3.90e-3, plus fp32 summation
# error far below that.  fp32 inputs keep fp32 probabilities.
LSE_TOL = {"bf16": 4e-3, "fp32": 1e-5}

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ pool (K1)
@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
def test_pool_integer_inputs_bit_exact(dtype, D):
    # integers in [-8, 8]: the fp32 block sum is exact and /64 is exact
    g = torch.Generator().manual_seed(D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.randint(-8, 9, (2, 256, 3, D), generator=g).to(tdt)
    v = torch.randint(-8, 9, (2, 256, 3, D), generator=g).to(tdt)
    kc, vc = nsa.pool(k.cuda(), v.cuda())
    want_k = oracle.pool(k.double().numpy())
    want_v = oracle.pool(v.double().numpy())
    np.testing.assert_array_equal(to_np(kc), torch.from_numpy(want_k).to(tdt).double().numpy())
    np.testing.assert_array_equal(to_np(vc), torch.from_numpy(want_v).to(tdt).double().numpy())


def test_pool_normal_inputs_one_rounding():
    wl = WORKLOADS["340m-gqa4"]
    dev, f64 = device_inputs(wl, seq_len=1024)
    kc, _ = nsa.pool(dev["k"], dev["v"])
    want = torch.from_numpy(oracle.pool(f64["k"]))
    got = kc.double().cpu()
    # the fp32 sum of 64 bf16 values can sit on the other side of a rounding
    # boundary from the exact mean: allow one bf16 ulp there, exact elsewhere
    ulp = torch.finfo(torch.bfloat16).eps * want.abs().clamp_min(1e-30)
    err = (got - want.to(torch.bfloat16).double()).abs()
    assert (err <= ulp * 1.01).all()
    assert (err == 0).float().mean() > 0.99


# ---------------------------------------------------- compress + select (K1+K2)
@pytest.mark.parametrize("name,T,planted", [
    ("340m-gqa4", 2048, 1.0), ("1b3-gqa4", 1024, 1.0), ("mqa-ablation", 1024, 1.0),
    ("tiny-fp32", 1024, 0.0), ("340m-gqa4", 4096, 0.0)])
def test_compress_select_matches_oracle(name, T, planted):
    wl = WORKLOADS[name].with_(batch=1)
    _print("case", name, T, planted)
    dev, f64 = device_inputs(wl, seq_len=T, planted_sigma=planted)
    o_cmp, idx = nsa.compress_select(dev["q"], dev["k"], dev["v"], top_k=wl.top_k, scale=wl.scale)
    torch.cuda.synchronize()
    ora = oracle_forward(wl, f64, want_scores=True)
    assert_close(to_np(o_cmp), ora["o_cmp"], wl.dtype, "o_cmp")
    agree = check_indices(idx.cpu().numpy(), ora, wl.top_k, scores=ora["scores"])
    _print("index agreement", agree.mean(), "decisive", (ora["gap"] > 1e-3).mean())
    if planted > 0 or wl.dtype == "fp32":
        assert agree.mean() > 0.97


# ------------------------------------------------------------- full forward
CASES = [
    # name, T, planted sigma, extra workload overrides
    ("tiny-fp32", 1024, 0.0, {}),
    ("340m-gqa4", 2048, 1.0, {}),
    ("1b3-gqa4", 1024, 1.0, {}),
    ("mqa-ablation", 1024, 1.0, {"batch": 1}),
    ("340m-gqa4", 1024, 1.0, {"n_q_heads": 4, "n_kv_heads": 4}),      # G = 1
    ("340m-gqa4", 1024, 1.0, {"n_q_heads": 8, "n_kv_heads": 4}),      # G = 2
    ("1b3-gqa4", 1024, 1.0, {"n_q_heads": 16, "n_kv_heads": 2, "batch": 1}),  # G = 8
    ("1b3-gqa4", 512, 0.0, {"batch": 2, "top_k": 2, "window": 1}),
    ("340m-gqa4", 640, 1.0, {"top_k": 3, "window": 1000}),
    ("tiny-fp32", 256, 0.0, {"n_q_heads": 16, "n_kv_heads": 1}),
    # four heads per group at head_dim 64 take the packed-selection kernel: three
    # batch entries (12 KV groups, an ungrouped workgroup order) and a ragged tile
    ("340m-gqa4", 1024, 1.0, {"batch": 3}),
    # a window range beyond 32 blocks falls back to the general kernel
    ("340m-gqa4", 2048, 1.0, {"window": 2048}),
    # packed-selection kernel edge cases: only the forced blocks and a one-key
    # window; a single block; top-k covering every block (all blocks are items)
    ("340m-gqa4", 512, 0.0, {"top_k": 2, "window": 1}),
    ("340m-gqa4", 64, 0.0, {"batch": 2}),
    ("340m-gqa4", 1024, 0.0, {"top_k": 32, "window": 64}),
    # a window that is not a whole number of blocks: the column groups' windows
    # start in different blocks, and the register range starts at the earliest
    ("340m-gqa4", 1024, 1.0, {"window": 500}),
    # the packed kernel's longest sequence: 256 key blocks, so its item masks and
    # per-block tables are at their largest and a tile walks five table chunks
    ("340m-gqa4", 16384, 1.0, {}),
    # the longest sequence the library accepts: 1024 key blocks (the general
    # kernel; the compressed branch stages 16 chunks of pooled keys)
    ("340m-gqa4", 65536, 1.0, {"n_q_heads": 4, "n_kv_heads": 1}),
]


@pytest.mark.skip(reason="fp32 with head_dim 128 is outside the envelope: its selection/window "
                         "kernel spilled to scratch and took a memory fault whose cause was not "
                         "found; the library now returns NSA_ERR_UNSUPPORTED for it")
def test_forward_fp32_head_dim_128():
    wl = WORKLOADS["tiny-fp32"].with_(n_q_heads=16, n_kv_heads=1, head_dim=128)
    dev, f64 = device_inputs(wl, seq_len=256)
    gpu_forward(wl, dev)


def test_fp32_head_dim_128_is_rejected():
    wl = WORKLOADS["tiny-fp32"].with_(head_dim=128)
    dev, _ = device_inputs(wl, seq_len=128)
    with pytest.raises(nsa.NsaError, match="UNSUPPORTED"):
        gpu_forward(wl, dev)


@pytest.mark.parametrize("name,T,planted,over", CASES)
def test_forward_matches_oracle(name, T, planted, over):
    wl = WORKLOADS[name].with_(**over)
    _print("case", name, T, planted, over)
    dev, f64 = device_inputs(wl, seq_len=T, planted_sigma=planted)
    res = gpu_forward(wl, dev, want_indices=True, want_lse=True, want_o_sel=True)
    torch.cuda.synchronize()
    ora = oracle_forward(wl, f64, want_scores=True)
    gi = res["indices"].cpu().numpy()
    agree = check_indices(gi, ora, wl.top_k, scores=ora["scores"])
    _print("index agreement", agree.mean(), "decisive", (ora["gap"] > 1e-3).mean())
    # every row, against the oracle on the GPU's index table (near-tie reading)
    if not agree.all():
        ora = oracle_forward(wl, f64, indices=gi)
    assert_close(to_np(res["out"]), ora["out"], wl.dtype, "out")
    assert_close(to_np(res["o_sel"]), ora["o_sel"], wl.dtype, "o_sel")
    err = np.abs(res["lse_sel"].cpu().double().numpy() - ora["lse_sel"])
    assert err.max() < LSE_TOL[wl.dtype], err.max()


def test_forward_with_oracle_indices_every_row():
    # The oracle's own table fed to the library (NSA_INDICES_IN): every row compares.
    wl = WORKLOADS["340m-gqa4"]
    dev, f64 = device_inputs(wl, seq_len=2048)
    ora = oracle_forward(wl, f64)
    idx = torch.from_numpy(ora["indices"]).to("cuda")
    res = gpu_forward(wl, dev, indices=idx, want_lse=True, want_o_sel=True)
    torch.cuda.synchronize()
    assert_close(to_np(res["out"]), ora["out"], "bf16", "out")
    assert_close(to_np(res["o_sel"]), ora["o_sel"], "bf16", "o_sel")
    assert np.abs(res["lse_sel"].cpu().double().numpy() - ora["lse_sel"]).max() < LSE_TOL[wl.dtype]
    assert torch.equal(idx.cpu(), torch.from_numpy(ora["indices"]))  # input left untouched


def _skip_flag_case(wl, dev, f64, flag):
    """GPU output with a skip flag against the oracle run on the gates with the
    skipped branches' gates zeroed ("a zero gate removes its branch"); where the
    selection branch contributes, the oracle takes the GPU's own index table
    (near-ties may pick either valid set)."""
    zero = [i for i, f in ((0, nsa.SKIP_CMP_OUT), (1, nsa.SKIP_SEL), (2, nsa.SKIP_WIN)) if flag & f]
    sel_used = not (flag & nsa.SKIP_SEL)
    res = gpu_forward(wl, dev, flags=flag, want_indices=sel_used)
    torch.cuda.synchronize()
    gz = f64["gates"].copy()
    gz[..., zero] = 0.0
    idx = res["indices"].cpu().numpy() if sel_used else None
    ora = oracle.forward(f64["q"], f64["k"], f64["v"], gz, top_k=wl.top_k, window=wl.window,
                         scale=wl.scale, indices=idx)
    assert_close(to_np(res["out"]), ora["out"], wl.dtype, f"out (flags {flag})")


@pytest.mark.parametrize("flag", [nsa.SKIP_CMP_OUT, nsa.SKIP_SEL, nsa.SKIP_WIN,
                                  nsa.SKIP_CMP_OUT | nsa.SKIP_SEL])
def test_skip_flags_match_oracle_with_zero_gates(flag):
    wl = WORKLOADS["340m-gqa4"]
    _print("case skip flag", flag)
    dev, f64 = device_inputs(wl, seq_len=2048)
    _skip_flag_case(wl, dev, f64, flag)


def test_mqa_ablation_runs_match_oracle():
    # The MQA ablation at its full size (B4 T8192 Hq16 Hkv1 D128): all branches,
    # compression output pruned (g_cmp = 0), window only (g_cmp = g_sel = 0).
    wl = WORKLOADS["mqa-ablation"]
    dev, f64 = device_inputs(wl)
    for flag in (0, nsa.SKIP_CMP_OUT, nsa.SKIP_CMP_OUT | nsa.SKIP_SEL):
        _print("case mqa ablation flags", flag)
        _skip_flag_case(wl, dev, f64, flag)


def test_window_only_matches_oracle():
    wl = WORKLOADS["mqa-ablation"].with_(batch=1, gate_override=(0.0, 0.0, 0.7))
    dev, f64 = device_inputs(wl, seq_len=1024)
    res = gpu_forward(wl, dev, flags=nsa.SKIP_CMP_OUT | nsa.SKIP_SEL)
    torch.cuda.synchronize()
    ora = oracle_forward(wl, f64)
    assert_close(to_np(res["out"]), ora["out"], "bf16", "out")


def test_large_logits_take_the_exact_maximum_path():
    # q scaled x40: the logit bound minus the forced maximum exceeds the fixed
    # reference window, so the kernel computes exact maxima of both branches.
    # At T = 2048 (32 blocks, top-k 16) window blocks that no row of a column
    # group selected exist, so the window's own reference is exercised; every
    # saved tensor of both branches is compared.
    wl = WORKLOADS["340m-gqa4"]
    dev, f64 = device_inputs(wl, seq_len=2048, planted_sigma=1.0, q_scale=40.0)
    ora = oracle_forward(wl, f64)
    idx = torch.from_numpy(ora["indices"]).to("cuda")
    sv = nsa.forward_train(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                           window=wl.window, scale=wl.scale, indices=idx)
    torch.cuda.synchronize()
    for nm in ("out", "o_sel", "o_win", "o_cmp"):
        assert_close(to_np(sv[nm]), ora[nm], "bf16", nm)
    for nm in ("lse_sel", "lse_win"):
        got = sv[nm].cpu().double().numpy()
        rel = np.abs(got - ora[nm]) / np.maximum(1.0, np.abs(ora[nm]))
        _print(nm, "max rel", rel.max())
        assert rel.max() < 2e-3, (nm, rel.max())


def test_large_logits_window_only_matches_oracle():
    # the exact-maximum path with the selection skipped (window reference only)
    wl = WORKLOADS["340m-gqa4"]
    dev, f64 = device_inputs(wl, seq_len=1024, planted_sigma=1.0, q_scale=40.0)
    _skip_flag_case(wl, dev, f64, nsa.SKIP_CMP_OUT | nsa.SKIP_SEL)


# ------------------------------------------------ full-size workloads, every row
@pytest.mark.parametrize("name", ["340m-gqa4", "1b3-gqa4", "mqa-ablation", "32k-fwd-bwd"])
def test_full_size_workloads_every_row(name):
    # Every row of the workload at its full size.  Indices: bit-exact where the
    # oracle's gap is decisive, a valid top-m of the oracle's scores elsewhere.
    # Outputs: every row against the oracle run on the GPU's own index table
    # (the near-tie reading), so rows whose index sets differ are compared too.
    wl = WORKLOADS[name]
    _print("case full-size", name)
    dev, f64 = device_inputs(wl)
    res = gpu_forward(wl, dev, want_indices=True, want_lse=True, want_o_sel=True)
    torch.cuda.synchronize()
    gi = res["indices"].cpu().numpy()
    ora = oracle_forward(wl, f64, want_scores=True)
    agree = check_indices(gi, ora, wl.top_k, scores=ora["scores"])
    decisive = ora["gap"] > 1e-3
    _print(f"{name}: index sets equal on {agree.mean():.4f} of rows; decisive rows "
           f"{decisive.mean():.4f}, all of them equal; rows compared 1.0000")
    del ora
    ora = oracle_forward(wl, f64, indices=gi)
    assert_close(to_np(res["out"]), ora["out"], wl.dtype, "out")
    assert_close(to_np(res["o_sel"]), ora["o_sel"], wl.dtype, "o_sel")
    err = np.abs(res["lse_sel"].cpu().double().numpy() - ora["lse_sel"])
    assert err.max() < LSE_TOL[wl.dtype], err.max()
    del dev
    torch.cuda.empty_cache()
