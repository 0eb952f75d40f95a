"""The index checker the GPU parity tests rely on, exercised on the CPU with
the oracle's own tables: it accepts the oracle's selection and a swap across a
near-tie, and rejects a swap on a decisive row, a swap that skips a better
block, a missing forced block and bad ordering (the gap rule of the target
statement: exact where the m-th vs (m+1)-th gap exceeds 1e-3, a valid top-m
within 1e-3 elsewhere)."""
import numpy as np
import pytest

import oracle
from tests.nsa_cases import check_indices

TOPK = 4


@pytest.fixture(scope="module")
def ora():
    rng = np.random.default_rng(5)
    B, T, Hq, Hkv, D = 1, 1024, 4, 1, 16
    q = rng.standard_normal((B, T, Hq, D)) * 0.3
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    g = np.full((B, T, Hq, 3), 0.5)
    return oracle.forward(q, k, v, g, top_k=TOPK, window=64, want_scores=True)


def _row(ora, decisive):
    gap = ora["gap"][0, 0]
    t = np.arange(gap.size)
    ok = (t // 64 >= 8) & ((gap > 1e-2) if decisive else (gap < 1e-3))
    assert ok.any()
    return int(t[ok][0])


def _swap(ora, t, pick_rank):
    """Replace the lowest-ranked free pick of row t by the candidate ranked
    pick_rank (0-based, over blocks 1..own-1 sorted by score)."""
    idx = ora["indices"].copy()
    S = ora["scores"][0, 0, t]
    own = t // 64
    cand = np.arange(1, own)
    order = cand[np.lexsort((cand, -S[cand]))]
    m = TOPK - 2
    row = [x for x in idx[0, 0, t] if x >= 0]
    row.remove(int(order[m - 1]))
    row.append(int(order[pick_rank]))
    idx[0, 0, t] = sorted(row) + [-1] * (TOPK - len(row))
    return idx


def test_accepts_the_oracles_own_table(ora):
    agree = check_indices(ora["indices"], ora, TOPK, scores=ora["scores"])
    assert agree.all()


def test_accepts_a_swap_across_a_near_tie(ora):
    t = _row(ora, decisive=False)
    idx = _swap(ora, t, TOPK - 2)  # the (m+1)-th candidate for the m-th
    agree = check_indices(idx, ora, TOPK, scores=ora["scores"])
    assert not agree[0, 0, t] and agree.sum() == agree.size - 1


def test_rejects_a_swap_on_a_decisive_row(ora):
    t = _row(ora, decisive=True)
    with pytest.raises(AssertionError, match="decisive"):
        check_indices(_swap(ora, t, TOPK - 2), ora, TOPK, scores=ora["scores"])


def test_rejects_a_pick_far_below_the_cut(ora):
    gap = ora["gap"][0, 0]
    t = _row(ora, decisive=False)
    own = t // 64
    S = ora["scores"][0, 0, t]
    cand = np.arange(1, own)
    order = np.sort(S[cand])[::-1]
    far = [r for r in range(TOPK - 1, own - 1) if order[TOPK - 3] - order[r] > 2e-3]
    assert far, gap[t]
    with pytest.raises(AssertionError):
        check_indices(_swap(ora, t, far[0]), ora, TOPK, scores=ora["scores"])


def test_rejects_structural_errors(ora):
    t = _row(ora, decisive=False)
    bad = ora["indices"].copy()
    bad[0, 0, t] = bad[0, 0, t][::-1]  # descending
    with pytest.raises(AssertionError):
        check_indices(bad, ora, TOPK)
    bad = ora["indices"].copy()
    row = [x for x in bad[0, 0, t] if x >= 0]
    own = t // 64
    row = [x for x in row if x != own] + [own - 1 if own - 1 not in row else own - 2]
    bad[0, 0, t] = sorted(row)
    with pytest.raises(AssertionError):
        check_indices(bad, ora, TOPK)
