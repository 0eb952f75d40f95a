"""GPU parity of the training forward's saved tensors and of the gradient of
the whole NSA output (all three branches and the gates) against the fp64
oracle.  The selection is frozen to the oracle's own index table on both
sides (INDICES_IN), so every saved tensor the backward consumes is the one
the oracle's selection defines.

Tolerances: the forward outputs use the forward bounds (bf16 max-abs 2e-2,
mean-abs 2e-3; fp32 1e-4) and the log-sum-exps the forward's LSE bound; dq,
dk, dv use the bounds of the selection-backward tests and the reading stated
there.  The gate gradients are dgates_b = dO . o_b (the chain rule of
out = sum_b g_b o_b) over the forward's saved outputs, so the GPU's differ from
the oracle's by dO . (o_b,GPU - o_b,oracle) -- the forward's own output error
(checked above) carried through a head_dim-long dot product -- plus the
rounding of the fp32 sum to the output dtype: the test checks that
decomposition element by element, and the mean-abs bound on the whole."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_compress_amd as nsa
from sparse_attention_long_compress_amd.synth import WORKLOADS
from tests.nsa_cases import assert_close, device_inputs, oracle_forward, to_np
from tests.test_gpu_backward import grad_close

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 4e-3, "fp32": 1e-5}


def run_full(wl, T):
    dev, f64 = device_inputs(wl, seq_len=T, with_dout=True)
    ora = oracle_forward(wl, f64)
    idx = torch.from_numpy(ora["indices"]).to("cuda")
    sv = nsa.forward_train(dev["q"], dev["k"], dev["v"], dev["gates"], top_k=wl.top_k,
                           window=wl.window, scale=wl.scale, indices=idx)
    got = nsa.backward(dev["q"], dev["k"], dev["v"], dev["gates"], sv, dev["dout"],
                       top_k=wl.top_k, window=wl.window, scale=wl.scale)
    torch.cuda.synchronize()
    ref = oracle.backward(f64["q"], f64["k"], f64["v"], f64["gates"], ora["indices"], f64["dout"],
                          top_k=wl.top_k, window=wl.window, scale=wl.scale)
    return sv, got, ora, ref, dev, f64


def dgates_close(got, ref, dout, o_gpu, o_ora, dtype):
    got = np.asarray(got, np.float64)
    prop = np.stack([(dout * (og - oo)).sum(-1) for og, oo in zip(o_gpu, o_ora)], -1)
    rms = max(1.0, float(np.sqrt((ref ** 2).mean())))
    err = np.abs(got - ref)
    resid = np.abs(got - ref - prop)
    unit = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    mean = 2e-3 if dtype == "bf16" else 1e-4
    print(f"dgates: max|ref| {np.abs(ref).max():.3g} rms_ref {np.sqrt((ref ** 2).mean()):.3g} "
          f"max-abs {err.max():.3e} mean-abs {err.mean():.3e} forward-propagated max "
          f"{np.abs(prop).max():.3e} residual max {resid.max():.3e}", flush=True)
    assert np.all(np.isfinite(got))
    bound = unit * np.abs(ref) + 1e-4 * rms
    assert np.all(resid <= bound), f"dgates: residual {(resid - bound).max():.3e} over its bound"
    assert err.mean() <= mean * rms, f"dgates: mean-abs {err.mean():.3e} > {mean * rms:.3e}"


CASES = [
    ("tiny-fp32", 512, {}),
    ("340m-gqa4", 1024, {}),
    ("340m-gqa4", 2048, {}),
    ("1b3-gqa4", 1024, {"batch": 1}),
    ("mqa-ablation", 512, {"batch": 1}),
    ("340m-gqa4", 512, {"n_q_heads": 4, "n_kv_heads": 4}),                # G = 1
    ("1b3-gqa4", 512, {"batch": 2, "n_q_heads": 8, "n_kv_heads": 4}),     # G = 2
    ("1b3-gqa4", 512, {"batch": 1, "n_q_heads": 16, "n_kv_heads": 2}),    # G = 8
    ("340m-gqa4", 640, {"top_k": 3, "window": 100}),
    ("340m-gqa4", 4160, {"window": 64}),    # more than 64 pooled keys: two pooled-key blocks
]


def check_full(wl, T):
    """Saved tensors, dq / dk / dv and the gate gradients of one workload against the oracle."""
    sv, got, ora, ref, _, f64 = run_full(wl, T)
    for nm in ("o_sel", "o_win", "o_cmp"):
        assert_close(to_np(sv[nm]), ora[nm], wl.dtype, nm)
    for nm in ("lse_sel", "lse_win"):
        err = np.abs(sv[nm].cpu().double().numpy() - ora[nm]).max()
        assert err < LSE_TOL[wl.dtype], (nm, err)
    lc = sv["lse_cmp"].cpu().double().numpy()
    fin = np.isfinite(ora["lse_cmp"])
    np.testing.assert_array_equal(np.isfinite(lc), fin)
    assert np.abs(lc[fin] - ora["lse_cmp"][fin]).max() < LSE_TOL[wl.dtype]
    G = wl.n_q_heads // wl.n_kv_heads
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        grad_close(to_np(g_), r_, wl.dtype, nm, heads_per_key=1 if nm == "dq" else G)
    branches = ("o_cmp", "o_sel", "o_win")
    dgates_close(to_np(got[3]), ref[3], f64["dout"], [to_np(sv[n]) for n in branches],
                 [ora[n] for n in branches], wl.dtype)


@pytest.mark.parametrize("name,T,over", CASES)
def test_full_backward_matches_oracle(name, T, over):
    wl = WORKLOADS[name].with_(**over)
    print("case", name, T, over, flush=True)
    check_full(wl, T)


def test_full_backward_is_bitwise_reproducible():
    wl = WORKLOADS["340m-gqa4"]
    sv, got, _, _, dev, _ = run_full(wl, 1024)
    again = nsa.backward(dev["q"], dev["k"], dev["v"], dev["gates"], sv, dev["dout"],
                         top_k=wl.top_k, window=wl.window, scale=wl.scale)
    torch.cuda.synchronize()
    for a, b in zip(got, again):
        assert torch.equal(a, b)


def test_train_forward_out_equals_forward():
    wl = WORKLOADS["340m-gqa4"]
    dev, _ = device_inputs(wl, seq_len=2048)
    kw = dict(top_k=wl.top_k, window=wl.window, scale=wl.scale)
    a = nsa.forward(dev["q"], dev["k"], dev["v"], dev["gates"], want_indices=True, want_lse=True,
                    want_o_sel=True, **kw)
    b = nsa.forward_train(dev["q"], dev["k"], dev["v"], dev["gates"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(a["out"], b["out"])
    assert torch.equal(a["indices"], b["indices"])
    assert torch.equal(a["lse_sel"], b["lse_sel"])
    assert torch.equal(a["o_sel"], b["o_sel"])
