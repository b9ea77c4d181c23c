"""Pins for the oracle's mask generality (CPU only).

After the a2a exchange the sequence metadata, the mask and the attention math
are those of cp_size = 1, so every mask type and window size stays valid
("[PyTorch] Extend no-load-balance CP to the a2a comm type", PR body). The
oracle's reading: a real query at position p attends the real tokens of its
document at positions [p - left, p + right], -1 meaning unbounded.

Pinned against things other than the oracle: torch CPU float64
scaled_dot_product_attention (and its autograd) per document, unmasked and
with a boolean band mask built from positions here; a pure-Python brute
force on a padded two-document layout; closed forms (a one-key window, K = 0
giving the mean of V over the window and LSE = log of its size, pair counts
of a sliding window); the union of ranks equals cp_size 1 under a window;
window sizes at or past the document length equal no bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

DCS, NLB = O.DUAL_CHUNK_SWAP, O.NO_LOAD_BALANCE

WINDOWS = [(-1, -1), (3, 0), (2, 1), (0, 2), (-1, 3), (5, -1), (0, 0)]


def _inputs(T, H, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, D)) for _ in range(4)]   # q, k, v, do


def _band(L, window):
    """bool [L, L]: key position j allowed for query position i."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    ok = np.ones((L, L), dtype=bool)
    if window[0] >= 0:
        ok &= j >= i - window[0]
    if window[1] >= 0:
        ok &= j <= i + window[1]
    return ok


@pytest.mark.parametrize("window", WINDOWS)
def test_cp1_matches_torch_sdpa_with_band_mask(window):
    # cp_size 1, whole documents without padding: per document, the library's
    # attention with an explicit boolean mask (or none for (-1, -1)).
    cu = [0, 9, 9, 40, 57]
    T = cu[-1]
    q, k, v, do = _inputs(T, 2, 8, 21)
    idx = np.arange(T)
    o, lse = O.attention_fwd(q, k, v, idx, cu, cu, T, window=window)
    dq, dk, dv = O.attention_bwd(q, k, v, do, idx, cu, cu, T, window=window)
    for d in range(len(cu) - 1):
        a, b = cu[d], cu[d + 1]
        if b == a:
            continue
        tq, tk, tv = (torch.tensor(x[a:b].transpose(1, 0, 2), requires_grad=True)
                      for x in (q, k, v))
        mask = None if window == (-1, -1) else torch.tensor(_band(b - a, window))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
        np.testing.assert_allclose(o[a:b], ref.detach().numpy().transpose(1, 0, 2),
                                   rtol=1e-10, atol=1e-12)
        ref.backward(torch.tensor(do[a:b].transpose(1, 0, 2)))
        np.testing.assert_allclose(dq[a:b], tq.grad.numpy().transpose(1, 0, 2), rtol=1e-9,
                                   atol=1e-11)
        np.testing.assert_allclose(dk[a:b], tk.grad.numpy().transpose(1, 0, 2), rtol=1e-9,
                                   atol=1e-11)
        np.testing.assert_allclose(dv[a:b], tv.grad.numpy().transpose(1, 0, 2), rtol=1e-9,
                                   atol=1e-11)
        # LSE against the masked scores written out with a library logsumexp
        s = np.einsum("ihd,jhd->hij", q[a:b], k[a:b]) / math.sqrt(8)
        s = np.where(_band(b - a, window)[None], s, -np.inf)
        np.testing.assert_allclose(lse[:, a:b], torch.logsumexp(torch.tensor(s), -1).numpy(),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [(2, 1), (-1, -1), (1, 0)])
def test_brute_force_padded_rank_share(window):
    # two padded documents, DUAL_CHUNK_SWAP cp 2 rank 1: every output row by
    # scanning all T keys with the conditions written out one by one
    cu, cup, T, cp = [0, 5, 12], [0, 8, 16], 16, 2
    q, k, v, do = _inputs(T, 1, 3, 4)
    idx = O.partition_index(cup, T, cp, 1, DCS)
    o, lse = O.attention_fwd(q[idx], k, v, idx, cu, cup, T, window=window)
    sc = 1.0 / math.sqrt(3)
    for m, g in enumerate(idx):
        d = 0 if g < 8 else 1
        start, real = cup[d], cu[d + 1] - cu[d]
        if g - start >= real:
            assert lse[0, m] == -np.inf and np.all(o[m] == 0)
            continue
        keys = []
        for j in range(T):
            if not (start <= j < start + real):
                continue
            if window[0] >= 0 and j < g - window[0]:
                continue
            if window[1] >= 0 and j > g + window[1]:
                continue
            keys.append(j)
        s = [sc * sum(q[g, 0, x] * k[j, 0, x] for x in range(3)) for j in keys]
        mx = max(s)
        tot = sum(math.exp(x - mx) for x in s)
        assert math.isclose(lse[0, m], mx + math.log(tot), abs_tol=1e-12)
        for x in range(3):
            ref = sum(math.exp(sv - mx) / tot * v[j, 0, x] for sv, j in zip(s, keys))
            assert math.isclose(o[m, 0, x], ref, abs_tol=1e-12)


def test_one_key_window_closed_form():
    # window (0, 0): each real row attends only itself -> O = V_g,
    # LSE = scale <q_g, k_g>, dQ = dK = 0, dV_g = dO_g; padding rows 0
    cu, cup, T = [0, 5, 12], [0, 8, 16], 16
    q, k, v, do = _inputs(T, 2, 4, 6)
    idx = np.arange(T)
    o, lse = O.attention_fwd(q, k, v, idx, cu, cup, T, window=(0, 0))
    dq, dk, dv = O.attention_bwd(q, k, v, do, idx, cu, cup, T, window=(0, 0))
    _, _, valid = O.token_table(cu, cup, T)
    np.testing.assert_allclose(o[valid], v[valid], atol=1e-14)
    np.testing.assert_allclose(lse.T[valid], 0.5 * np.einsum("thd,thd->th", q, k)[valid],
                               atol=1e-13)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    np.testing.assert_allclose(dv[valid], do[valid], atol=1e-14)
    assert np.all(dv[~valid] == 0) and np.all(o[~valid] == 0)


@pytest.mark.parametrize("window", WINDOWS)
def test_zero_keys_give_window_mean(window):
    # K = 0: every allowed score is 0, so O is the mean of V over the window
    # and LSE = log of the window's size, clipped to the document's real rows
    cu, cup, T = [0, 7, 20], [0, 9, 24], 24
    q, _, v, _ = _inputs(T, 1, 4, 8)
    k = np.zeros_like(q)
    idx = np.arange(T)
    o, lse = O.attention_fwd(q, k, v, idx, cu, cup, T, window=window)
    for g in range(T):
        d = 0 if g < 9 else 1
        a, L = cup[d], cu[d + 1] - cu[d]
        p = g - a
        if p >= L:
            continue
        lo = 0 if window[0] < 0 else max(0, p - window[0])
        hi = L - 1 if window[1] < 0 else min(L - 1, p + window[1])
        assert math.isclose(lse[0, g], math.log(hi - lo + 1), abs_tol=1e-13)
        np.testing.assert_allclose(o[g, 0], v[a + lo:a + hi + 1, 0].mean(axis=0), atol=1e-13)


def test_sliding_window_pair_counts():
    # one document of L tokens, causal window (w, 0): sum over p of min(p, w) + 1
    # = (w+1)(w+2)/2 + (L-w-1)(w+1) for L > w; no bound: L(L+1)/2; (-1, -1): L^2
    L, w = 50, 7
    cu = [0, L]
    idx = np.arange(L)
    assert O.causal_pairs(cu, cu, L, idx, window=(w, 0)) == \
        (w + 1) * (w + 2) // 2 + (L - w - 1) * (w + 1)
    assert O.causal_pairs(cu, cu, L, idx) == L * (L + 1) // 2
    assert O.causal_pairs(cu, cu, L, idx, window=(-1, -1)) == L * L
    # touched keys under a window: exactly the keys some local query reaches
    t = O.touched_keys(cu, cu, L, [30, 31], window=(3, 1))
    assert np.flatnonzero(t).tolist() == list(range(27, 33))


@pytest.mark.parametrize("window", [(-1, -1), (6, 0), (3, 2)])
@pytest.mark.parametrize("strategy", [DCS, NLB])
def test_union_of_ranks_equals_cp1_under_window(window, strategy):
    cu, cup, T, cp = ([0, 5, 5, 16], [0, 8, 8, 24], 24, 2) if strategy == DCS else \
        ([0, 5, 13], [0, 7, 15], 18, 3)
    q, k, v, do = _inputs(T, 2, 4, 12)
    all_idx = np.arange(T)
    o1, l1 = O.attention_fwd(q, k, v, all_idx, cu, cup, T, window=window)
    dq1, dk1, dv1 = O.attention_bwd(q, k, v, do, all_idx, cu, cup, T, window=window)
    o_u = np.zeros_like(o1)
    dq_u = np.zeros_like(dq1)
    dk_u = np.zeros_like(dk1)
    dv_u = np.zeros_like(dv1)
    for r in range(cp):
        idx, o, lse, dq, dk, dv = O.rank_share(q, k, v, do, cu, cup, T, cp, r, strategy,
                                               window=window)
        o_u[idx] = o
        dq_u[idx] = dq
        dk_u += dk
        dv_u += dv
    np.testing.assert_allclose(o_u, o1, atol=1e-12)
    np.testing.assert_allclose(dq_u, dq1, atol=1e-12)
    np.testing.assert_allclose(dk_u, dk1, atol=1e-12)
    np.testing.assert_allclose(dv_u, dv1, atol=1e-12)
    # per document: sum of dK is 0 (shift invariance), sum of dV is sum of dO
    _, _, valid = O.token_table(cu, cup, T)
    for d in range(len(cup) - 1):
        a, b = cup[d], cup[d + 1]
        if b > a:
            assert np.abs(dk1[a:b].sum(axis=0)).max() < 1e-12
            np.testing.assert_allclose(dv1[a:b].sum(axis=0),
                                       do[a:b][valid[a:b]].sum(axis=0), atol=1e-12)


def test_window_past_document_is_unbounded():
    cu, cup, T = [0, 7, 20], [0, 9, 24], 24
    q, k, v, do = _inputs(T, 1, 4, 3)
    idx = np.arange(T)
    for wide, open_ in (((13, 0), (-1, 0)), ((-1, 13), (-1, -1)), ((40, 40), (-1, -1))):
        a = O.attention_fwd(q, k, v, idx, cu, cup, T, window=wide)
        b = O.attention_fwd(q, k, v, idx, cu, cup, T, window=open_)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
