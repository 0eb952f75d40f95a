"""Pins for the fp64 oracle: each test checks the oracle against something other
than itself -- a closed form, an invariant, a library routine in a special case,
brute-force enumeration, or the sparsity arithmetic the pages print.

Sources cited:
  [SIC] "Sparsity is Cool: Reverse-Engineering MoBA and NSA" (wiki summary), Method / Key claims
  [DSA] "DeepSeek's Native Sparse Attention" (newsletter), How Does NSA Work? bullets
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(B, T, Hq, Hkv, D, seed=0, gates=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    g = rng.uniform(0.05, 0.95, (B, T, Hq, 3)) if gates is None else np.broadcast_to(
        np.asarray(gates, dtype=np.float64), (B, T, Hq, 3)).copy()
    return q, k, v, g


def heads_first(x, Hq):
    """[B,T,H,D] -> [B,Hq,T,D], expanding KV heads to their query heads."""
    t = torch.from_numpy(np.ascontiguousarray(x)).permute(0, 2, 1, 3)
    H = t.shape[1]
    if H != Hq:
        t = t.repeat_interleave(Hq // H, dim=1)
    return t.contiguous()


def sdpa(q, k, v, mask, scale):
    """torch fp64 SDPA; q/k/v [B,T,*,D] numpy; mask [B,Hq,T,S] or [T,S] bool."""
    Hq = q.shape[2]
    qt, kt, vt = heads_first(q, Hq), heads_first(k, Hq), heads_first(v, Hq)
    m = torch.from_numpy(np.ascontiguousarray(mask))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def sdpa_lse(q, k, mask, scale):
    Hq = q.shape[2]
    qt, kt = heads_first(q, Hq), heads_first(k, Hq)
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~torch.from_numpy(np.ascontiguousarray(mask)), float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()  # [B,Hq,T]


def causal_mask(T):
    return np.tril(np.ones((T, T), dtype=bool))


# ----------------------------------------------------------------------------- pool
def test_pool_constant_block_returns_constant():
    # A mean-pool of a constant is that constant ([SIC] Method: mean-pooling).
    x = np.full((2, 192, 3, 5), 0.0)
    x += np.arange(3)[None, None, :, None] * 1.25 - 0.5
    out = oracle.pool(x, 64)
    assert out.shape == (2, 3, 3, 5)
    np.testing.assert_array_equal(out, np.broadcast_to(x[:, :3], out.shape))


def test_pool_arithmetic_progression_closed_form():
    # x_t = t: the mean over block j is 64 j + 31.5 (non-overlapping, stride 64);
    # a trailing partial block is not pooled.
    T = 64 * 5 + 17
    x = np.broadcast_to(np.arange(T, dtype=np.float64)[None, :, None, None], (1, T, 2, 3)).copy()
    x[:, :, 1, :] *= -2.0
    out = oracle.pool(x, 64)
    assert out.shape == (1, 5, 2, 3)
    want = 64.0 * np.arange(5) + 31.5
    np.testing.assert_array_equal(out[0, :, 0, 0], want)
    np.testing.assert_array_equal(out[0, :, 1, 2], -2.0 * want)


# ---------------------------------------------------------------- compressed branch
def test_cmp_constant_keys_uniform_weights():
    # With every key of a KV head equal, all compressed logits of a query tie, so
    # the weights are uniform over the n_c(t) = floor((t+1)/64) visible blocks and
    # o_cmp is the plain mean of V over positions [0, 64 n_c); o_cmp = 0 when no
    # block is complete yet.
    B, T, Hq, Hkv, D = 1, 320, 4, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=1)
    k[:] = np.random.default_rng(2).standard_normal((1, 1, Hkv, D))
    r = oracle.forward(q, k, v, g, top_k=3, window=16)
    G = Hq // Hkv
    for t in [0, 62, 63, 64, 127, 128, 200, 319]:
        nc = (t + 1) // 64
        for h in range(Hq):
            want = v[0, : 64 * nc, h // G].mean(0) if nc else np.zeros(D)
            np.testing.assert_allclose(r["o_cmp"][0, t, h], want, rtol=0, atol=1e-12)


def test_cmp_matches_sdpa_over_library_avgpool():
    # Library pin: torch avg_pool1d builds the block means; torch SDPA with the
    # block-causal visibility mask (block j visible iff 64(j+1)-1 <= t).
    B, T, Hq, Hkv, D = 2, 384, 4, 2, 16
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=3)
    r = oracle.forward(q, k, v, g, top_k=3, window=32)
    kt = torch.from_numpy(k).permute(0, 2, 3, 1).reshape(B * Hkv, D, T)
    vt = torch.from_numpy(v).permute(0, 2, 3, 1).reshape(B * Hkv, D, T)
    kc = F.avg_pool1d(kt, 64, 64).reshape(B, Hkv, D, -1).permute(0, 3, 1, 2).numpy()
    vc = F.avg_pool1d(vt, 64, 64).reshape(B, Hkv, D, -1).permute(0, 3, 1, 2).numpy()
    nc = T // 64
    vis = (np.arange(nc)[None, :] * 64 + 63) <= np.arange(T)[:, None]  # [T, nc]
    want = sdpa(q, kc, vc, vis, 1.0 / np.sqrt(D))
    rows = np.arange(T) >= 63
    np.testing.assert_allclose(r["o_cmp"][:, rows], want[:, rows], rtol=0, atol=1e-12)
    assert np.all(r["o_cmp"][:, ~rows] == 0.0)


def test_cmp_lse_matches_logsumexp_over_library_avgpool():
    # The compressed branch's log-sum-exp: torch logsumexp of the scaled logits
    # over avg_pool1d block means with the block-causal mask (block j visible
    # iff 64(j+1)-1 <= t); -inf before the first block completes (t < 63).
    B, T, Hq, Hkv, D = 2, 384, 4, 2, 16
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=31)
    r = oracle.forward(q, k, v, g, top_k=3, window=32)
    kt = torch.from_numpy(k).permute(0, 2, 3, 1).reshape(B * Hkv, D, T)
    kc = F.avg_pool1d(kt, 64, 64).reshape(B, Hkv, D, -1).permute(0, 3, 1, 2).numpy()
    nc = T // 64
    vis = (np.arange(nc)[None, :] * 64 + 63) <= np.arange(T)[:, None]  # [T, nc]
    want = sdpa_lse(q, kc, vis, 1.0 / np.sqrt(D))
    rows = np.arange(T) >= 63
    np.testing.assert_allclose(r["lse_cmp"][:, :, rows], want[:, :, rows], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(r["lse_cmp"][:, :, ~rows]))


def test_cmp_lse_constant_keys_closed_form():
    # Every key of a KV head equal to c: each visible block mean is c, so the
    # log-sum-exp is tau q.c + log n_c(t) exactly (up to rounding).
    B, T, Hq, Hkv, D = 1, 320, 4, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=32)
    c = np.random.default_rng(33).standard_normal((Hkv, D))
    k[:] = c[None, None]
    r = oracle.forward(q, k, v, g, top_k=3, window=16)
    G, tau = Hq // Hkv, 1.0 / np.sqrt(D)
    for t in [63, 64, 127, 128, 250, 319]:
        nc = (t + 1) // 64
        for h in range(Hq):
            want = tau * q[0, t, h] @ c[h // G] + np.log(nc)
            assert abs(r["lse_cmp"][0, h, t] - want) < 1e-12


# ------------------------------------------------------------------ importance + top-k
def test_scores_are_group_summed_softmax_probabilities():
    # The block importance is the compressed-branch attention probability summed
    # over the query heads of a KV group ([DSA] SELECTION: reuse of the
    # compression scores).  Library pin via torch.softmax.
    B, T, Hq, Hkv, D = 1, 448, 6, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=4)
    r = oracle.forward(q, k, v, g, top_k=3, window=8, want_scores=True)
    kc = k[:, : (T // 64) * 64].reshape(B, T // 64, 64, Hkv, D).mean(2)
    G = Hq // Hkv
    for t in [63, 100, 255, 447]:
        nc = (t + 1) // 64
        for gg in range(Hkv):
            tot = torch.zeros(nc, dtype=torch.float64)
            for h in range(gg * G, (gg + 1) * G):
                logit = torch.from_numpy(kc[0, :nc, gg] @ q[0, t, h]) / np.sqrt(D)
                tot += torch.softmax(logit, 0)
            np.testing.assert_allclose(r["scores"][0, gg, t, :nc], tot.numpy(), atol=1e-13)
            assert np.all(r["scores"][0, gg, t, nc:] == 0.0)


def test_topk_all_ties_takes_lowest_indices():
    # K = 0 makes every compressed logit 0, so all candidate scores tie and the
    # lower-index rule gives I = {0, 1, ..., m, own} (k counts the forced blocks).
    B, T, Hq, Hkv, D, topk = 1, 640, 2, 1, 4, 4
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=5)
    k[:] = 0.0
    r = oracle.forward(q, k, v, g, top_k=topk, window=4)
    idx = r["indices"][0, 0]
    for t in range(T):
        own = t // 64
        if own == 0:
            want = [0]
        elif own - 1 <= topk - 2:
            want = list(range(own + 1))
        else:
            want = [0] + list(range(1, topk - 1)) + [own]
        want = sorted(want) + [-1] * (topk - len(want))
        assert list(idx[t]) == want, (t, list(idx[t]), want)


def _bruteforce_select(S, own, topk):
    forced = [0] if own == 0 else [0, own]
    m = topk - len(forced)
    cands = list(range(1, own))
    if len(cands) <= m:
        chosen = cands
    else:
        best, best_set = None, None
        for sub in itertools.combinations(cands, m):  # ascending tuples
            val = sum(S[j] for j in sub)
            # max total score; among equal totals the lexicographically smallest
            if best is None or val > best or (val == best and list(sub) < best_set):
                best, best_set = val, list(sub)
        chosen = best_set
    out = sorted(forced + chosen)
    return out + [-1] * (topk - len(out))


@pytest.mark.parametrize("topk", [3, 4, 5])
def test_topk_matches_bruteforce_subset_enumeration(topk):
    B, T, Hq, Hkv, D = 1, 512, 4, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=6 + topk)
    # one exact tie between two candidates in group 0, to exercise tie-breaking
    k[0, 64 * 3: 64 * 4, 0] = k[0, 64 * 5: 64 * 6, 0]
    r = oracle.forward(q, k, v, g, top_k=topk, window=8, want_scores=True)
    for gg in range(Hkv):
        for t in range(0, T, 7):
            want = _bruteforce_select(r["scores"][0, gg, t], t // 64, topk)
            assert list(r["indices"][0, gg, t]) == want


def test_topk_matches_numpy_stable_argsort():
    B, T, Hq, Hkv, D, topk = 1, 1536, 4, 1, 16, 6
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=11)
    r = oracle.forward(q, k, v, g, top_k=topk, window=8, want_scores=True)
    for t in range(0, T, 5):
        own = t // 64
        S = r["scores"][0, 0, t]
        cand = np.arange(1, own)
        m = topk - (1 if own == 0 else 2)
        if len(cand) <= m:
            chosen = list(cand)
        else:
            order = np.argsort(-S[cand], kind="stable")
            chosen = list(cand[order[:m]])
            gap = S[cand[order[m - 1]]] - S[cand[order[m]]]
            np.testing.assert_allclose(r["gap"][0, 0, t], gap, rtol=0, atol=0)
        if len(cand) <= m:
            # every candidate is taken (exactly m of them at own = 5): no
            # competing block, so the selection is decisive
            assert r["gap"][0, 0, t] == np.inf
        want = sorted(([0] if own == 0 else [0, own]) + chosen)
        got = [int(x) for x in r["indices"][0, 0, t] if x >= 0]
        assert got == want


def test_sparsity_arithmetic_from_the_pages():
    # [SIC] Method: block 64 / top-k 16 / window 512 at sequence 8192 has the same
    # ~81% sparsity as MoBA 512 / top-3: 1 - (16*64 + 512)/8192 = 0.8125.  This
    # holds only if k counts the forced blocks: the last query attends exactly 16
    # blocks of 64 plus a 512-token window.
    fx = json.load(open(os.path.join(GOLDEN, "sparsity_nsa_vs_moba.json")))
    T, blk, topk, W = fx["seq_len"], fx["block"], fx["top_k"], fx["window"]
    q, k, v, g = rand_inputs(1, T, 1, 1, 2, seed=12)
    r = oracle.forward(q, k, v, g, top_k=topk, window=W)
    t = T - 1
    nsel = int((r["indices"][0, 0, t] >= 0).sum())
    n_keys = nsel * blk + min(W, t + 1)
    assert nsel == topk
    assert n_keys == fx["attended_keys"]
    assert round(100 * (1 - n_keys / T)) == fx["sparsity_percent_rounded"]
    # MoBA at the same setting: block 512, top-3
    assert 1 - fx["moba_block"] * fx["moba_top_k"] / T == pytest.approx(1 - n_keys / T)


# ----------------------------------------------------------------- selection branch
@pytest.mark.parametrize("T,topk", [(256, 4), (1024, 16), (200, 4)])
def test_selection_full_coverage_is_causal_attention(T, topk):
    # When top-k covers every causal block (T <= 64 k) the selection branch is
    # plain causal attention ([SIC] Key claims: short sequences degenerate to
    # dense attention).  Library pin: torch SDPA, causal.
    B, Hq, Hkv, D = 1, 4, 2, 16
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=13)
    r = oracle.forward(q, k, v, g, top_k=topk, window=8)
    want = sdpa(q, k, v, causal_mask(T), 1.0 / np.sqrt(D))
    np.testing.assert_allclose(r["o_sel"], want, rtol=0, atol=1e-12)
    lse = sdpa_lse(q, k, causal_mask(T), 1.0 / np.sqrt(D))
    np.testing.assert_allclose(r["lse_sel"], lse, rtol=0, atol=1e-12)


def test_selection_matches_masked_sdpa_given_indices():
    B, T, Hq, Hkv, D, topk = 2, 640, 4, 2, 8, 4
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=14)
    r = oracle.forward(q, k, v, g, top_k=topk, window=8)
    G = Hq // Hkv
    mask = np.zeros((B, Hq, T, T), dtype=bool)
    blk_of = np.arange(T) // 64
    for b in range(B):
        for h in range(Hq):
            for t in range(T):
                sel = r["indices"][b, h // G, t]
                mask[b, h, t] = np.isin(blk_of, sel[sel >= 0]) & (np.arange(T) <= t)
    want = sdpa(q, k, v, mask, 1.0 / np.sqrt(D))
    np.testing.assert_allclose(r["o_sel"], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse_sel"], sdpa_lse(q, k, mask, 1.0 / np.sqrt(D)), atol=1e-12)


# -------------------------------------------------------------------- window branch
def test_window_at_least_T_is_causal_attention():
    B, T, Hq, Hkv, D = 1, 300, 4, 1, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=15)
    r = oracle.forward(q, k, v, g, top_k=2, window=T)
    np.testing.assert_allclose(r["o_win"], sdpa(q, k, v, causal_mask(T), 1 / np.sqrt(D)),
                               rtol=0, atol=1e-12)


def test_window_one_returns_own_value():
    B, T, Hq, Hkv, D = 1, 130, 4, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=16)
    r = oracle.forward(q, k, v, g, top_k=2, window=1)
    np.testing.assert_array_equal(r["o_win"], np.repeat(v, 2, axis=2))


def test_window_matches_banded_sdpa():
    # [DSA] SLIDING WINDOW; reading: W keys including the query, t-W < s <= t.
    B, T, Hq, Hkv, D, W = 1, 400, 2, 1, 8, 37
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=17)
    r = oracle.forward(q, k, v, g, top_k=2, window=W)
    s, t = np.meshgrid(np.arange(T), np.arange(T))
    band = (s <= t) & (s > t - W)
    np.testing.assert_allclose(r["o_win"], sdpa(q, k, v, band, 1 / np.sqrt(D)), rtol=0, atol=1e-12)


def test_window_lse_matches_banded_logsumexp():
    # lse_win against torch logsumexp over the band t-W < s <= t, and the two
    # closed forms: W >= T gives the causal log-sum-exp, W = 1 gives tau q_t.k_t.
    B, T, Hq, Hkv, D, W = 1, 400, 4, 2, 8, 37
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=34)
    tau = 1.0 / np.sqrt(D)
    s, t = np.meshgrid(np.arange(T), np.arange(T))
    band = (s <= t) & (s > t - W)
    r = oracle.forward(q, k, v, g, top_k=2, window=W)
    np.testing.assert_allclose(r["lse_win"], sdpa_lse(q, k, band, tau), rtol=0, atol=1e-12)
    r = oracle.forward(q, k, v, g, top_k=2, window=T + 5)
    np.testing.assert_allclose(r["lse_win"], sdpa_lse(q, k, causal_mask(T), tau), rtol=0, atol=1e-12)
    r = oracle.forward(q, k, v, g, top_k=2, window=1)
    own = tau * np.einsum("bthd,bthd->bht", q, np.repeat(k, Hq // Hkv, axis=2))
    np.testing.assert_allclose(r["lse_win"], own, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------- combine
def test_zero_and_unit_gates_isolate_branches():
    B, T, Hq, Hkv, D = 1, 256, 4, 2, 8
    q, k, v, _ = rand_inputs(B, T, Hq, Hkv, D, seed=18)
    base = oracle.forward(q, k, v, np.full((B, T, Hq, 3), 0.5), top_k=3, window=20)
    for i, name in enumerate(["o_cmp", "o_sel", "o_win"]):
        g = np.zeros((B, T, Hq, 3))
        g[..., i] = 1.0
        r = oracle.forward(q, k, v, g, top_k=3, window=20)
        np.testing.assert_array_equal(r["out"], base[name])
    r0 = oracle.forward(q, k, v, np.zeros((B, T, Hq, 3)), top_k=3, window=20)
    assert np.all(r0["out"] == 0.0)


def test_output_is_linear_in_gates():
    B, T, Hq, Hkv, D = 1, 256, 4, 2, 8
    q, k, v, g1 = rand_inputs(B, T, Hq, Hkv, D, seed=19)
    g2 = np.random.default_rng(20).uniform(0, 1, g1.shape)
    r1 = oracle.forward(q, k, v, g1, top_k=3, window=20)
    r2 = oracle.forward(q, k, v, g2, top_k=3, window=20)
    r12 = oracle.forward(q, k, v, g1 + g2, top_k=3, window=20)
    np.testing.assert_allclose(r12["out"], r1["out"] + r2["out"], atol=1e-12)
    np.testing.assert_array_equal(r1["indices"], r12["indices"])


# ------------------------------------------------------------------- whole-op invariants
def test_key_shift_invariance():
    # Adding one constant vector per KV head to every key shifts each query's
    # logits by a constant, which every softmax ignores: indices and outputs stay.
    B, T, Hq, Hkv, D = 1, 512, 4, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=21)
    c = np.random.default_rng(22).standard_normal((1, 1, Hkv, D))
    r1 = oracle.forward(q, k, v, g, top_k=4, window=40)
    r2 = oracle.forward(q, k + c, v, g, top_k=4, window=40)
    np.testing.assert_array_equal(r1["indices"][r1["gap"] > 1e-9], r2["indices"][r1["gap"] > 1e-9])
    same = np.all(r1["indices"] == r2["indices"], axis=-1)  # [B,Hkv,T]
    rows = np.repeat(same.transpose(0, 2, 1), Hq // Hkv, axis=2)  # [B,T,Hq]
    np.testing.assert_allclose(r2["out"][rows], r1["out"][rows], atol=1e-10)
    assert same.mean() > 0.99


def test_value_shift_moves_output_by_gate_sum():
    B, T, Hq, Hkv, D = 1, 300, 4, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=23)
    c = np.random.default_rng(24).standard_normal(D)
    r1 = oracle.forward(q, k, v, g, top_k=3, window=30)
    r2 = oracle.forward(q, k, v + c, g, top_k=3, window=30)
    vis = ((np.arange(T) + 1) // 64 > 0).astype(np.float64)[None, :, None]
    w = g[..., 0] * vis + g[..., 1] + g[..., 2]
    np.testing.assert_allclose(r2["out"] - r1["out"], w[..., None] * c, atol=1e-12)


def test_head_permutation_within_group():
    B, T, Hq, Hkv, D = 1, 400, 4, 1, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=25)
    perm = [2, 0, 3, 1]
    r1 = oracle.forward(q, k, v, g, top_k=4, window=30)
    r2 = oracle.forward(q[:, :, perm], k, v, g[:, :, perm], top_k=4, window=30)
    np.testing.assert_array_equal(r1["indices"], r2["indices"])
    np.testing.assert_allclose(r2["out"], r1["out"][:, :, perm], atol=1e-13)


def test_batch_entries_are_independent():
    T, Hq, Hkv, D = 256, 2, 1, 8
    q, k, v, g = rand_inputs(2, T, Hq, Hkv, D, seed=26)
    r = oracle.forward(q, k, v, g, top_k=3, window=17)
    r1 = oracle.forward(q[1:], k[1:], v[1:], g[1:], top_k=3, window=17)
    np.testing.assert_array_equal(r["out"][1:], r1["out"])
    np.testing.assert_array_equal(r["indices"][1:], r1["indices"])


# ------------------------------------------------------------------ selection gradient
def _loss_and_grads_torch(q, k, v, g, mask, dout, scale):
    """Library pin: autograd of torch fp64 SDPA with an explicit mask, times g_sel."""
    Hq = q.shape[2]
    G = Hq // k.shape[2]
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    qh = qt.permute(0, 2, 1, 3)
    kh = kt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vh = vt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=torch.from_numpy(mask), scale=scale)
    o = o.permute(0, 2, 1, 3) * torch.from_numpy(g[..., 1:2])
    (o * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_select_bwd_full_coverage_matches_autograd_of_causal_attention():
    B, T, Hq, Hkv, D, topk = 1, 192, 4, 2, 8, 4
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=27)
    dout = np.random.default_rng(28).standard_normal(q.shape)
    r = oracle.forward(q, k, v, g, top_k=topk, window=8)
    dq, dk, dv = oracle.select_bwd(q, k, v, g, r["indices"], dout, top_k=topk)
    want = _loss_and_grads_torch(q, k, v, g, causal_mask(T), dout, 1 / np.sqrt(D))
    for got, ref in zip((dq, dk, dv), want):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


def test_select_bwd_matches_autograd_of_masked_attention():
    B, T, Hq, Hkv, D, topk = 1, 512, 4, 2, 8, 3
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=29)
    dout = np.random.default_rng(30).standard_normal(q.shape)
    r = oracle.forward(q, k, v, g, top_k=topk, window=8)
    G = Hq // Hkv
    mask = np.zeros((B, Hq, T, T), dtype=bool)
    blk_of = np.arange(T) // 64
    for h in range(Hq):
        for t in range(T):
            sel = r["indices"][0, h // G, t]
            mask[0, h, t] = np.isin(blk_of, sel[sel >= 0]) & (np.arange(T) <= t)
    dq, dk, dv = oracle.select_bwd(q, k, v, g, r["indices"], dout, top_k=topk)
    want = _loss_and_grads_torch(q, k, v, g, mask, dout, 1 / np.sqrt(D))
    for got, ref in zip((dq, dk, dv), want):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


def test_select_bwd_central_finite_differences():
    # d/dx of L = sum(dout * g_sel * o_sel) with the selection frozen.
    B, T, Hq, Hkv, D, topk = 1, 160, 2, 1, 4, 2
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=31)
    dout = np.random.default_rng(32).standard_normal(q.shape)
    r = oracle.forward(q, k, v, g, top_k=topk, window=4)
    idx = r["indices"]
    dq, dk, dv = oracle.select_bwd(q, k, v, g, idx, dout, top_k=topk)

    def loss(qq, kk, vv):
        o = oracle.forward(qq, kk, vv, g, top_k=topk, window=4, indices=idx)["o_sel"]
        return float((dout * g[..., 1:2] * o).sum())

    rng = np.random.default_rng(33)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[pos] += h
            am[pos] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = ap, am
            fd = (loss(**{"qq": args_p["q"], "kk": args_p["k"], "vv": args_p["v"]})
                  - loss(**{"qq": args_m["q"], "kk": args_m["k"], "vv": args_m["v"]})) / (2 * h)
            assert abs(fd - grad[pos]) < 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_row_subset_matches_full_run():
    # Restricting the oracle to some query positions changes nothing for them.
    B, T, Hq, Hkv, D = 1, 700, 4, 2, 8
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=34)
    full = oracle.forward(q, k, v, g, top_k=4, window=50)
    rows = [0, 63, 64, 333, 699]
    sub = oracle.forward(q, k, v, g, top_k=4, window=50, rows=rows)
    for name in ("out", "o_cmp", "o_sel", "o_win"):
        np.testing.assert_array_equal(sub[name][:, rows], full[name][:, rows])
    np.testing.assert_array_equal(sub["indices"][:, :, rows], full["indices"][:, :, rows])
    np.testing.assert_array_equal(sub["lse_sel"][:, :, rows], full["lse_sel"][:, :, rows])


# ------------------------------------------------------------------ full gradient
def test_backward_central_finite_differences():
    # d/dx of L = sum(dout * out) over all three branches and the gates, with the
    # selection frozen; window 40 cuts blocks, top_k 2 leaves block 1 unselected
    # for the last block's queries.
    B, T, Hq, Hkv, D, topk, W = 1, 192, 2, 1, 4, 2, 40
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=41)
    dout = np.random.default_rng(42).standard_normal(q.shape)
    idx = oracle.forward(q, k, v, g, top_k=topk, window=W)["indices"]
    dq, dk, dv, dg = oracle.backward(q, k, v, g, idx, dout, top_k=topk, window=W)

    def loss(**kw):
        a = {"q": q, "k": k, "v": v, "gates": g}
        a.update(kw)
        o = oracle.forward(a["q"], a["k"], a["v"], a["gates"], top_k=topk, window=W, indices=idx)
        return float((dout * o["out"]).sum())

    rng = np.random.default_rng(43)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("gates", g, dg)):
        for _ in range(8):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[pos] += h
            am[pos] -= h
            fd = (loss(**{name: ap}) - loss(**{name: am})) / (2 * h)
            assert abs(fd - grad[pos]) < 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def _nsa_loss_torch(q, k, v, g, idx, dout, topk, W, scale, blk=64):
    """Library pin: the three branches written with torch fp64 ops (avg_pool1d
    for the compression, explicit boolean masks), differentiated by autograd."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    gt = torch.from_numpy(g).requires_grad_(True)
    qh = qt.permute(0, 2, 1, 3)                                        # [B,Hq,T,D]
    kh = kt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vh = vt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    t_ = np.arange(T)
    blk_of = t_ // blk
    # selection and window masks
    msel = np.zeros((B, Hq, T, T), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for t in range(T):
                sel = idx[b, h // G, t]
                msel[b, h, t] = np.isin(blk_of, sel[sel >= 0]) & (t_ <= t)
    mwin = (t_[None, :] <= t_[:, None]) & (t_[None, :] > t_[:, None] - W)
    o_sel = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=torch.from_numpy(msel), scale=scale)
    o_win = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=torch.from_numpy(mwin), scale=scale)
    # compression: pooled keys over complete blocks, visible when 64 (j + 1) - 1 <= t
    nc = T // blk
    kc = F.avg_pool1d(kh.reshape(-1, T, D).transpose(1, 2), blk, blk).transpose(1, 2).reshape(B, Hq, nc, D)
    vc = F.avg_pool1d(vh.reshape(-1, T, D).transpose(1, 2), blk, blk).transpose(1, 2).reshape(B, Hq, nc, D)
    rows = np.arange(blk - 1, T)                                       # rows with a visible block
    mcmp = (blk * (np.arange(nc)[None, :] + 1) - 1) <= rows[:, None]
    o_rows = F.scaled_dot_product_attention(qh[:, :, rows], kc, vc, attn_mask=torch.from_numpy(mcmp),
                                            scale=scale)
    o_cmp = torch.zeros_like(o_sel)
    o_cmp = o_cmp.index_copy(2, torch.from_numpy(rows), o_rows)
    gh = gt.permute(0, 2, 1, 3)                                        # [B,Hq,T,3]
    out = gh[..., 0:1] * o_cmp + gh[..., 1:2] * o_sel + gh[..., 2:3] * o_win
    (out.permute(0, 2, 1, 3) * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), gt.grad.numpy()


def test_backward_matches_autograd_of_torch_branches():
    B, T, Hq, Hkv, D, topk, W = 2, 320, 4, 2, 8, 3, 100
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=44)
    dout = np.random.default_rng(45).standard_normal(q.shape)
    idx = oracle.forward(q, k, v, g, top_k=topk, window=W)["indices"]
    got = oracle.backward(q, k, v, g, idx, dout, top_k=topk, window=W)
    want = _nsa_loss_torch(q, k, v, g, idx, dout, topk, W, 1 / np.sqrt(D))
    for name, a, b_ in zip(("dq", "dk", "dv", "dgates"), got, want):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-11, err_msg=name)


def test_backward_selection_part_equals_select_bwd():
    # with the compression and window gates at zero only the selection gradient remains
    B, T, Hq, Hkv, D, topk = 1, 256, 4, 2, 8, 3
    q, k, v, g = rand_inputs(B, T, Hq, Hkv, D, seed=46)
    g[..., 0] = 0.0
    g[..., 2] = 0.0
    dout = np.random.default_rng(47).standard_normal(q.shape)
    idx = oracle.forward(q, k, v, g, top_k=topk, window=30)["indices"]
    dq, dk, dv, _ = oracle.backward(q, k, v, g, idx, dout, top_k=topk, window=30)
    rq, rk, rv = oracle.select_bwd(q, k, v, g, idx, dout, top_k=topk)
    for a, b_ in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- decode step
def _decode_by_enumeration(q, K, V, gates, L, top_k, W, blk=64):
    """One query at t = L - 1 written out from the method's statement: mean of
    each complete block, softmax over the blocks complete at t, importance
    summed over the group's heads, blocks 0 and t // blk forced, the rest by
    (importance desc, index asc), one softmax over the selected tokens s <= t,
    one over t - W < s <= t, outputs mixed by the gates.  Also returns the
    importance of every complete block (0 past them) and the gap between the
    m-th and (m+1)-th candidate (inf when every candidate is taken)."""
    Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    tau = 1.0 / np.sqrt(D)
    t = L - 1
    own, nc = t // blk, L // blk
    out = np.zeros((Hq, D))
    chosen_all = []
    scores = np.zeros((Hkv, -(-L // blk)))
    gaps = np.full(Hkv, np.inf)
    for g in range(Hkv):
        heads = range(g * G, (g + 1) * G)
        Kc = [K[j * blk:(j + 1) * blk, g].mean(0) for j in range(nc)]
        Vc = [V[j * blk:(j + 1) * blk, g].mean(0) for j in range(nc)]
        p_cmp = {}
        for h in heads:
            if nc == 0:
                p_cmp[h] = np.zeros(0)
                continue
            z = np.array([tau * q[h] @ Kc[j] for j in range(nc)])
            e = np.exp(z - z.max())
            p_cmp[h] = e / e.sum()
        for j in range(nc):
            scores[g, j] = sum(p_cmp[h][j] for h in heads)
        forced = [0] if own == 0 else [0, own]
        cands = list(range(1, own))
        m = top_k - len(forced)
        if len(cands) <= m:
            pick = cands
        else:
            imp = {j: sum(p_cmp[h][j] for h in heads) for j in cands}
            ranked = sorted(cands, key=lambda j: (-imp[j], j))
            pick = ranked[:m]
            gaps[g] = imp[ranked[m - 1]] - imp[ranked[m]]
        chosen = sorted(forced + pick)
        chosen_all.append(chosen + [-1] * (top_k - len(chosen)))
        sel_keys = [s for j in chosen for s in range(j * blk, (j + 1) * blk) if s <= t]
        win_keys = list(range(max(0, t - W + 1), t + 1))
        for h in heads:
            def attend(keys):
                z = np.array([tau * q[h] @ K[s, g] for s in keys])
                e = np.exp(z - z.max())
                return (e / e.sum()) @ np.array([V[s, g] for s in keys])
            o_cmp = sum(p_cmp[h][j] * Vc[j] for j in range(nc)) if nc else np.zeros(D)
            out[h] = gates[h, 0] * o_cmp + gates[h, 1] * attend(sel_keys) + gates[h, 2] * attend(win_keys)
    return out, np.array(chosen_all), scores, gaps


def test_decode_matches_per_query_enumeration():
    rng = np.random.default_rng(7)
    B, Lmax, Hq, Hkv, D, top_k, W = 7, 768, 4, 2, 8, 3, 40
    lens = [1, 63, 64, 128, 150, 700, 768]
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Lmax, Hkv, D))
    vc = rng.standard_normal((B, Lmax, Hkv, D))
    gates = rng.random((B, Hq, 3))
    got = oracle.decode(q, kc, vc, gates, lens, top_k=top_k, window=W)
    for b, L in enumerate(lens):
        ref, idx, sc, gp = _decode_by_enumeration(q[b], kc[b, :L], vc[b, :L], gates[b], L, top_k, W)
        np.testing.assert_allclose(got["out"][b], ref, atol=1e-12, rtol=1e-10)
        assert np.array_equal(got["indices"][b], idx), (L, got["indices"][b], idx)
        # the importance the selection ranks, and the gap the GPU tests use
        # to tell decisive rows from near-ties
        np.testing.assert_allclose(got["scores"][b, :, :sc.shape[1]], sc, atol=1e-13, rtol=0)
        assert np.all(got["scores"][b, :, sc.shape[1]:] == 0.0)
        np.testing.assert_allclose(got["gap"][b], gp, atol=1e-13, rtol=0)


def test_decode_is_independent_of_cache_past_the_length():
    # positions >= L must not influence the step
    rng = np.random.default_rng(8)
    B, Lmax, Hq, Hkv, D = 2, 256, 4, 1, 8
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Lmax, Hkv, D))
    vc = rng.standard_normal((B, Lmax, Hkv, D))
    gates = rng.random((B, Hq, 3))
    a = oracle.decode(q, kc, vc, gates, [100, 200], top_k=3, window=30)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, 100:] = 1e3
    vc2[1, 200:] = -1e3
    b = oracle.decode(q, kc2, vc2, gates, [100, 200], top_k=3, window=30)
    assert np.array_equal(a["out"], b["out"])
