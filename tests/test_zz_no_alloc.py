"""nsa_forward_noalloc (the forward over the library's fixed per-GPU scratch
array, for callers that cannot allocate) against nsa_forward with a caller
workspace: same kernels, so every output must be bit-for-bit equal.  Two calls
in a row, the second on a smaller input, so the second runs over the first
one's leftover scratch contents; also with the selection fed in."""
import numpy as np
import pytest
import torch

import sparse_attention_long_compress_amd as nsa
from sparse_attention_long_compress_amd.synth import WORKLOADS
from tests.nsa_cases import device_inputs, gpu_forward

pytestmark = pytest.mark.gpu


def _noalloc(wl, dev, indices=None):
    q = dev["q"]
    B, T, Hq, _ = q.shape
    Hkv = dev["k"].shape[2]
    out = torch.empty_like(q)
    idx = indices if indices is not None else torch.empty((B, Hkv, T, wl.top_k), dtype=torch.int32,
                                                          device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    o_sel = torch.empty_like(q)
    nsa.forward_noalloc(q, dev["k"], dev["v"], dev["gates"], top_k=wl.top_k, window=wl.window,
                        scale=wl.scale, indices=indices, out=out,
                        indices_out=None if indices is not None else idx, lse_sel=lse, o_sel=o_sel)
    return {"out": out, "indices": idx, "lse_sel": lse, "o_sel": o_sel}


def test_noalloc_equals_forward_on_two_calls_second_smaller():
    wl = WORKLOADS["340m-gqa4"]
    for T in (8192, 1024):
        print("case noalloc T", T, flush=True)
        dev, _ = device_inputs(wl, seq_len=T)
        ref = gpu_forward(wl, dev, want_indices=True, want_lse=True, want_o_sel=True)
        got = _noalloc(wl, dev)
        torch.cuda.synchronize()
        for n in ("out", "indices", "lse_sel", "o_sel"):
            assert torch.equal(got[n], ref[n]), (T, n)
        assert np.isfinite(got["out"].float().cpu().numpy()).all()


def test_noalloc_with_indices_in_and_other_shapes():
    # the selection fed in (INDICES_IN), then a head_dim-128 shape (the general
    # selection/window kernel) that still fits the scratch array
    wl = WORKLOADS["340m-gqa4"]
    dev, _ = device_inputs(wl, seq_len=2048)
    ref = gpu_forward(wl, dev, want_indices=True, want_lse=True, want_o_sel=True)
    got = _noalloc(wl, dev, indices=ref["indices"])
    torch.cuda.synchronize()
    for n in ("out", "lse_sel", "o_sel"):
        assert torch.equal(got[n], ref[n]), n
    wl = WORKLOADS["1b3-gqa4"].with_(batch=1)
    dev, _ = device_inputs(wl, seq_len=2048)
    ref = gpu_forward(wl, dev, want_indices=True, want_lse=True, want_o_sel=True)
    got = _noalloc(wl, dev)
    torch.cuda.synchronize()
    for n in ("out", "indices", "lse_sel", "o_sel"):
        assert torch.equal(got[n], ref[n]), n


def test_noalloc_rejects_a_workspace_beyond_the_scratch_array():
    wl = WORKLOADS["1b3-gqa4"]  # B4 T8192 D128: about 210 MiB of workspace
    dev, _ = device_inputs(wl.with_(batch=4), seq_len=8192)
    with pytest.raises(nsa.NsaError, match="WORKSPACE"):
        _noalloc(wl, dev)


def test_noalloc_equals_forward_over_the_shape_sweep():
    # the sweep's shapes whose workspace fits the scratch array, one after the
    # other (each call runs over the previous one's leftover scratch contents)
    from tests.test_gpu_sweep import BASE, _wl
    n = 0
    for c in BASE:
        wl = _wl(c)
        dev, _ = device_inputs(wl, seq_len=c["seq_len"], planted_sigma=c["planted"])
        p = nsa.params_for(dev["q"], dev["k"], top_k=wl.top_k, window=wl.window, scale=wl.scale)
        if nsa.workspace_size(p) > nsa.NOALLOC_SCRATCH_BYTES:
            continue
        print("case noalloc", c, flush=True)
        ref = gpu_forward(wl, dev, want_indices=True, want_lse=True, want_o_sel=True)
        got = _noalloc(wl, dev)
        torch.cuda.synchronize()
        for nm in ("out", "indices", "lse_sel", "o_sel"):
            assert torch.equal(got[nm], ref[nm]), (c["seed"], nm)
        n += 1
    assert n >= 20, n
