"""Pins for the oracle's attention forward/backward (CPU only).

The pages print no attention values, so these pin the oracle to things other
than itself: a pure-Python brute force on tiny inputs, a library routine on
the special case cp_size=1 with whole documents (torch CPU float64
scaled_dot_product_attention and its autograd), closed forms, central finite
differences, and the invariants named for the method: the union of all ranks
equals the cp_size=1 result, softmax rows sum to 1, padding contributes
nothing.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

DCS, NLB = O.DUAL_CHUNK_SWAP, O.NO_LOAD_BALANCE


def _layout(kind):
    """(cu_seqlens, cu_seqlens_padded, T, cp, strategy) small layouts with padding."""
    if kind == "dcs_pad":
        return [0, 5, 5, 16], [0, 8, 8, 24], 24, 2, DCS          # doc1 empty, pads in doc0/doc2
    if kind == "nlb_pad":
        return [0, 5, 13], [0, 7, 15], 18, 3, NLB               # doc paddings + a tail of 3
    if kind == "dcs_nopad":
        return [0, 8, 24], [0, 8, 24], 24, 2, DCS
    if kind == "nlb_nopad":
        return [0, 7, 20], [0, 7, 20], 20, 4, NLB
    raise KeyError(kind)


def _inputs(T, H, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, D)) for _ in range(4)]   # q, k, v, do


# ---------------------------------------------------------------- brute force

def _brute_fwd_row(qrow, k, v, g, cu, cup, scale):
    """Pure-Python: scan all keys, apply doc/valid/causal conditions directly."""
    d = None
    for i in range(len(cup) - 1):
        if cup[i] <= g < cup[i + 1]:
            d = i
    if d is None or g - cup[d] >= cu[d + 1] - cu[d]:
        return None
    s = []
    for j in range(k.shape[0]):
        if cup[d] <= j <= g:
            s.append((j, scale * sum(qrow[x] * k[j][x] for x in range(len(qrow)))))
    mx = max(val for _, val in s)
    tot = sum(math.exp(val - mx) for _, val in s)
    out = [0.0] * v.shape[1]
    for j, val in s:
        p = math.exp(val - mx) / tot
        for x in range(v.shape[1]):
            out[x] += p * v[j][x]
    return out, mx + math.log(tot)


@pytest.mark.parametrize("kind", ["dcs_pad", "nlb_pad", "dcs_nopad", "nlb_nopad"])
def test_fwd_matches_brute_force(kind):
    cu, cup, T, cp, strat = _layout(kind)
    H, D = 2, 3
    q, k, v, _ = _inputs(T, H, D, 1)
    scale = 1 / math.sqrt(D)
    for r in range(cp):
        idx = O.partition_index(cup, T, cp, r, strat)
        o, lse = O.attention_fwd(q[idx], k, v, idx, cu, cup, T)
        for m, g in enumerate(idx):
            for h in range(H):
                ref = _brute_fwd_row(q[g, h], k[:, h], v[:, h], int(g), cu, cup, scale)
                if ref is None:
                    assert np.all(o[m, h] == 0) and lse[h, m] == -np.inf
                else:
                    np.testing.assert_allclose(o[m, h], ref[0], rtol=1e-12, atol=1e-12)
                    assert abs(lse[h, m] - ref[1]) < 1e-12


# ---------------------------------------------------------------- library routine

def _per_doc_sdpa(q, k, v, cu, scale=None):
    """cp_size=1, no padding: per-document torch SDPA (causal), float64."""
    outs = []
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        if b == a:
            continue
        qt = torch.from_numpy(q[a:b]).permute(1, 0, 2)
        kt = torch.from_numpy(k[a:b]).permute(1, 0, 2)
        vt = torch.from_numpy(v[a:b]).permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                             scale=scale)
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


def test_fwd_cp1_matches_torch_sdpa():
    cu = [0, 37, 128, 129, 300]
    T = cu[-1]
    q, k, v, _ = _inputs(T, 3, 16, 2)
    idx = O.partition_index(cu, T, 1, 0, NLB)
    o, _ = O.attention_fwd(q[idx], k, v, idx, cu, cu, T)
    np.testing.assert_allclose(o, _per_doc_sdpa(q, k, v, cu), rtol=1e-10, atol=1e-12)


def test_bwd_cp1_matches_torch_autograd():
    cu = [0, 17, 60, 61, 90]
    T = cu[-1]
    q, k, v, do = _inputs(T, 2, 8, 3)
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    outs = []
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        o = torch.nn.functional.scaled_dot_product_attention(
            tq[a:b].permute(1, 0, 2), tk[a:b].permute(1, 0, 2), tv[a:b].permute(1, 0, 2),
            is_causal=True)
        outs.append(o.permute(1, 0, 2))
    (torch.cat(outs) * torch.from_numpy(do)).sum().backward()
    idx = np.arange(T)
    dq, dk, dv = O.attention_bwd(q, k, v, do, idx, cu, cu, T)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("kind", ["dcs_pad", "nlb_pad"])
def test_fwd_closed_forms(kind):
    cu, cup, T, cp, strat = _layout(kind)
    H, D = 2, 4
    q, k, v, _ = _inputs(T, H, D, 4)
    doc, pos, valid = O.token_table(cu, cup, T)
    for r in range(cp):
        idx = O.partition_index(cup, T, cp, r, strat)
        # K = 0: uniform weights over the allowed keys [doc start, g].
        o, lse = O.attention_fwd(q[idx], np.zeros_like(k), v, idx, cu, cup, T)
        for m, g in enumerate(idx):
            if not valid[g]:
                continue
            a = cup[doc[g]]
            np.testing.assert_allclose(o[m], v[a:g + 1].mean(axis=0), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[:, m], math.log(g - a + 1), rtol=1e-13)
        # Constant V rows: O equals the constant on real rows.
        c = np.broadcast_to(np.arange(1, D + 1, dtype=np.float64), (T, H, D)).copy()
        o, _ = O.attention_fwd(q[idx], k, c, idx, cu, cup, T)
        for m, g in enumerate(idx):
            if valid[g]:
                np.testing.assert_allclose(o[m], c[0], rtol=1e-13)


@pytest.mark.parametrize("kind", ["dcs_pad", "nlb_pad", "dcs_nopad"])
def test_softmax_rows_sum_to_one(kind):
    # One-hot V rows make O the probability row itself.
    cu, cup, T, cp, strat = _layout(kind)
    q, k, _, _ = _inputs(T, 1, 4, 5)
    onehot = np.eye(T)[:, None, :]
    doc, pos, valid = O.token_table(cu, cup, T)
    for r in range(cp):
        idx = O.partition_index(cup, T, cp, r, strat)
        p, _ = O.attention_fwd(q[idx], k, onehot, idx, cu, cup, T, scale=0.5)
        for m, g in enumerate(idx):
            row = p[m, 0]
            if not valid[g]:
                assert np.all(row == 0)
                continue
            a = cup[doc[g]]
            assert abs(row.sum() - 1) < 1e-12
            assert np.all(row >= 0)
            allowed = np.zeros(T, bool)
            allowed[a:g + 1] = True
            assert np.all(row[~allowed] == 0) and np.all(row[allowed] > 0)


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("kind", ["dcs_pad", "nlb_pad"])
def test_bwd_finite_differences(kind):
    cu, cup, T, cp, strat = _layout(kind)
    H, D = 1, 3
    q, k, v, do = _inputs(T, H, D, 6)
    eps = 1e-6
    for r in range(cp):
        idx = O.partition_index(cup, T, cp, r, strat)
        ql, dol = q[idx], do[idx]

        def loss(ql_, k_, v_):
            o, _ = O.attention_fwd(ql_, k_, v_, idx, cu, cup, T)
            return float((o * dol).sum())

        dq, dk, dv = O.attention_bwd(ql, k, v, dol, idx, cu, cup, T)
        for name, arr, grad in (("q", ql, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(arr)
            for pos_ in np.ndindex(arr.shape):
                ap, am = arr.copy(), arr.copy()
                ap[pos_] += eps
                am[pos_] -= eps
                args_p = {"q": (ap, k, v), "k": (ql, ap, v), "v": (ql, k, ap)}[name]
                args_m = {"q": (am, k, v), "k": (ql, am, v), "v": (ql, k, am)}[name]
                num[pos_] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("kind", ["dcs_pad", "nlb_pad"])
def test_bwd_invariants(kind):
    cu, cup, T, cp, strat = _layout(kind)
    H, D = 2, 4
    q, k, v, do = _inputs(T, H, D, 7)
    doc, pos, valid = O.token_table(cu, cup, T)
    for r in range(cp):
        idx = O.partition_index(cup, T, cp, r, strat)
        dq, dk, dv = O.attention_bwd(q[idx], k, v, do[idx], idx, cu, cup, T)
        # Constant V: the output does not depend on Q or K.
        vc = np.ones_like(v) * 0.7
        dq0, dk0, _ = O.attention_bwd(q[idx], k, vc, do[idx], idx, cu, cup, T)
        assert np.abs(dq0).max() < 1e-12 and np.abs(dk0).max() < 1e-12
        for i in range(len(cu) - 1):
            a, b = cup[i], cup[i + 1]
            # Shifting all keys of a document leaves softmax rows unchanged.
            np.testing.assert_allclose(dk[a:b].sum(axis=0), 0, atol=1e-12)
            # Softmax rows sum to 1, so dV summed over a doc is the doc's dO sum.
            local_rows = [m for m, g in enumerate(idx) if valid[g] and doc[g] == i]
            exp = do[idx][local_rows].sum(axis=0) if local_rows else 0
            np.testing.assert_allclose(dv[a:b].sum(axis=0), exp, atol=1e-12)
        # Keys no local query attends get no gradient.
        touched = O.touched_keys(cu, cup, T, idx)
        assert np.all(dk[~touched] == 0) and np.all(dv[~touched] == 0)


@pytest.mark.parametrize("kind", ["dcs_pad", "nlb_pad", "dcs_nopad", "nlb_nopad"])
def test_union_of_ranks_equals_cp1(kind):
    cu, cup, T, cp, strat = _layout(kind)
    H, D = 2, 4
    q, k, v, do = _inputs(T, H, D, 8)
    ref_idx = np.arange(T)
    o1, lse1 = O.attention_fwd(q, k, v, ref_idx, cu, cup, T)
    dq1, dk1, dv1 = O.attention_bwd(q, k, v, do, ref_idx, cu, cup, T)
    o_u = np.zeros_like(o1)
    lse_u = np.full_like(lse1, np.nan)
    dq_u = np.zeros_like(dq1)
    dk_u = np.zeros_like(dk1)
    dv_u = np.zeros_like(dv1)
    for r in range(cp):
        idx, o, lse, dq, dk, dv = O.rank_share(q, k, v, do, cu, cup, T, cp, r, strat)
        o_u[idx] = o
        lse_u[:, idx] = lse
        dq_u[idx] = dq
        dk_u += dk
        dv_u += dv
    for a, b in ((o_u, o1), (dq_u, dq1), (dk_u, dk1), (dv_u, dv1)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isinf(lse_u), np.isinf(lse1))
    fin = np.isfinite(lse1)
    np.testing.assert_allclose(lse_u[fin], lse1[fin], rtol=1e-13)


@pytest.mark.parametrize("kind", ["dcs_pad", "nlb_pad"])
def test_padding_poison_contributes_nothing(kind):
    cu, cup, T, cp, strat = _layout(kind)
    H, D = 2, 4
    q, k, v, do = _inputs(T, H, D, 9)
    _, _, valid = O.token_table(cu, cup, T)
    poisoned = [x.copy() for x in (q, k, v, do)]
    for x in poisoned:
        x[~valid] = np.nan
    for r in range(cp):
        clean = O.rank_share(q, k, v, do, cu, cup, T, cp, r, strat)
        dirty = O.rank_share(*poisoned, cu, cup, T, cp, r, strat)
        idx = clean[0]
        for a, b in zip(clean[1:], dirty[1:]):
            assert np.array_equal(a, b)       # bit-identical, no NaN anywhere
        pad_local = ~valid[idx]
        assert np.all(clean[1][pad_local] == 0) and np.all(clean[3][pad_local] == 0)
        assert np.all(np.isneginf(clean[2][:, pad_local]))
        assert np.all(clean[4][~valid] == 0) and np.all(clean[5][~valid] == 0)
