"""Pins for the oracle's P2P (ring) step definitions (CPU only).

Under P2P context parallelism ("[PyTorch][Attention] THD P2P context-parallel
regression ...", "Describe the bug") a rank's attention runs in steps, one per
peer's K/V. The step functions are pinned to things other than themselves:
the merged steps equal the already-pinned whole-key-set attention (forward
and backward, every rank, both strategies, with padding); restricting to all
keys is the plain attention exactly; a single allowed key gives the closed
form O = V_j, LSE = s_j; the log-sum-exp merge has closed forms on equal and
empty parts; and a pure-Python brute force on a tiny case.
"""
import math

import numpy as np
import pytest

import oracle as O

DCS, NLB = O.DUAL_CHUNK_SWAP, O.NO_LOAD_BALANCE

LAYOUTS = {
    "dcs_pad": ([0, 5, 5, 16], [0, 8, 8, 24], 24, 2, DCS),
    "dcs_cp3": ([0, 10, 27, 28], [0, 12, 30, 36], 36, 3, DCS),
    "nlb_pad": ([0, 5, 13], [0, 7, 15], 18, 3, NLB),
    "nlb_nopad": ([0, 7, 20], [0, 7, 20], 20, 4, NLB),
}


def _inputs(T, H, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, D)) for _ in range(4)]   # q, k, v, do


def _delta(o, do):
    return np.einsum("nhd,nhd->hn", o, do)


@pytest.mark.parametrize("name", sorted(LAYOUTS))
def test_merged_steps_equal_whole_key_set(name):
    cu, cup, T, cp, strat = LAYOUTS[name]
    for r in range(cp):
        O.check_layout(cu, cup, T, cp, r, strat)
    q, k, v, do = _inputs(T, 2, 8, 11)
    owner = O.owner_ranks(cup, T, cp, strat)
    assert np.all(owner >= 0)
    for r in range(cp):
        idx = O.partition_index(cup, T, cp, r, strat)
        ql, dol = q[idx], do[idx]
        o_ref, lse_ref = O.attention_fwd(ql, k, v, idx, cu, cup, T)
        dq_ref, dk_ref, dv_ref = O.attention_bwd(ql, k, v, dol, idx, cu, cup, T)
        parts = []
        for i in range(cp):
            src = O.p2p_source(r, i, cp)
            parts.append(O.attention_fwd_keys(ql, k, v, idx, cu, cup, T, owner == src))
        o, lse = O.lse_merge(parts)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.allclose(lse[fin], lse_ref[fin], atol=1e-12, rtol=0)
        assert np.allclose(o, o_ref, atol=1e-12, rtol=0)
        delta = _delta(o_ref, dol)
        dq = np.zeros_like(dq_ref)
        dk = np.zeros_like(dk_ref)
        dv = np.zeros_like(dv_ref)
        for i in range(cp):
            src = O.p2p_source(r, i, cp)
            a, b, c = O.attention_bwd_keys(ql, k, v, dol, idx, cu, cup, T, owner == src,
                                           lse_ref, delta)
            # a step's key gradients live only on the rows its source rank holds
            assert np.all(b[owner != src] == 0) and np.all(c[owner != src] == 0)
            dq += a
            dk += b
            dv += c
        assert np.allclose(dq, dq_ref, atol=1e-12, rtol=0)
        assert np.allclose(dk, dk_ref, atol=1e-12, rtol=0)
        assert np.allclose(dv, dv_ref, atol=1e-12, rtol=0)


def test_all_keys_is_plain_attention():
    cu, cup, T, cp, strat = LAYOUTS["dcs_pad"]
    q, k, v, do = _inputs(T, 2, 8, 3)
    idx = O.partition_index(cup, T, cp, 1, strat)
    o_ref, lse_ref = O.attention_fwd(q[idx], k, v, idx, cu, cup, T)
    o, lse = O.attention_fwd_keys(q[idx], k, v, idx, cu, cup, T, np.ones(T, dtype=bool))
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)


def test_single_key_closed_form():
    # one document of 6 real rows, cp 1; only key 2 allowed: rows g >= 2 see
    # exactly that key (O = V_2, LSE = scale <q, k_2>), rows g < 2 see none.
    cu = cup = [0, 6]
    T = 6
    q, k, v, do = _inputs(T, 1, 4, 5)
    idx = np.arange(T)
    ok = np.zeros(T, dtype=bool)
    ok[2] = True
    o, lse = O.attention_fwd_keys(q, k, v, idx, cu, cup, T, ok)
    for g in range(T):
        if g < 2:
            assert lse[0, g] == -np.inf and np.all(o[g] == 0)
        else:
            assert np.allclose(o[g, 0], v[2, 0], atol=1e-14)
            assert math.isclose(lse[0, g], 0.5 * float(q[g, 0] @ k[2, 0]), abs_tol=1e-14)


def test_ring_order():
    # step 0 is the rank's own K/V; each later step takes the previous rank's
    assert [O.p2p_source(2, i, 4) for i in range(4)] == [2, 1, 0, 3]
    assert [O.p2p_source(0, i, 2) for i in range(2)] == [0, 1]


def test_lse_merge_closed_forms():
    rng = np.random.default_rng(7)
    o1 = rng.standard_normal((5, 2, 3))
    l1 = rng.standard_normal((2, 5))
    empty = (np.zeros_like(o1), np.full_like(l1, -np.inf))
    o, lse = O.lse_merge([(o1, l1), empty])
    assert np.allclose(o, o1, atol=1e-15) and np.allclose(lse, l1, atol=1e-15)
    o, lse = O.lse_merge([(o1, l1), (o1, l1)])
    assert np.allclose(o, o1, atol=1e-14) and np.allclose(lse, l1 + math.log(2.0), atol=1e-14)
    o, lse = O.lse_merge([empty, empty])
    assert np.all(o == 0) and np.all(lse == -np.inf)
    # weights exp(L1)/(exp(L1)+exp(L2)) written out for one element
    o2 = rng.standard_normal((5, 2, 3))
    l2 = rng.standard_normal((2, 5))
    o, lse = O.lse_merge([(o1, l1), (o2, l2)])
    w1 = math.exp(l1[1, 3]) / (math.exp(l1[1, 3]) + math.exp(l2[1, 3]))
    assert math.isclose(o[3, 1, 2], w1 * o1[3, 1, 2] + (1 - w1) * o2[3, 1, 2], abs_tol=1e-14)
    assert math.isclose(lse[1, 3], math.log(math.exp(l1[1, 3]) + math.exp(l2[1, 3])),
                        abs_tol=1e-14)


def test_step_brute_force_tiny():
    # one document of 8 rows, cp 2 DUAL_CHUNK_SWAP: chunks of 2; rank 1 holds
    # rows {2, 3, 4, 5}, rank 0 {0, 1, 6, 7}. Rank 1's step against rank 0's
    # keys, written out with Python loops.
    cu = cup = [0, 8]
    T, cp = 8, 2
    q, k, v, do = _inputs(T, 1, 3, 9)
    idx = O.partition_index(cup, T, cp, 1, DCS)
    assert idx.tolist() == [2, 3, 4, 5]
    owner = O.owner_ranks(cup, T, cp, DCS)
    o, lse = O.attention_fwd_keys(q[idx], k, v, idx, cu, cup, T, owner == 0)
    sc = 1.0 / math.sqrt(3)
    for m, g in enumerate(idx):
        keys = [j for j in range(T) if owner[j] == 0 and j <= g]
        s = [sc * sum(q[g, 0, x] * k[j, 0, x] for x in range(3)) for j in keys]
        mx = max(s)
        tot = sum(math.exp(x - mx) for x in s)
        assert math.isclose(lse[0, m], mx + math.log(tot), abs_tol=1e-12)
        for x in range(3):
            ref = sum(math.exp(sv - mx) / tot * v[j, 0, x] for sv, j in zip(s, keys))
            assert math.isclose(o[m, 0, x], ref, abs_tol=1e-12)
