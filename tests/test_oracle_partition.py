"""Pins for the oracle's metadata functions (CPU only).

The pages print no partition tables, so the partition is pinned by the
hand-worked fixtures in tests/golden/, by brute force, and by the invariants
the pages imply: every token lands on exactly one rank, NO_LOAD_BALANCE is
one contiguous physical range per rank, and DUAL_CHUNK_SWAP balances causal
work across ranks (it is the load-balanced strategy; "Why" of the all-gather
CP page).
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _expected(e):
    if isinstance(e, str) and e.startswith("range:"):
        _, a, b = e.split(":")
        return list(range(int(a), int(b)))
    return list(e)


@pytest.mark.parametrize("case", _load("partition_examples.json")["cases"], ids=lambda c: c["name"])
def test_partition_hand_examples(case):
    got = O.partition_index(case["cu_seqlens_padded"], case["T"], case["cp_size"], case["rank"],
                            case["strategy"])
    assert got.tolist() == _expected(case["expected"])


def _random_layout(rng, strategy, cp, n_docs, pad_tail=0):
    mult = 2 * cp if strategy == O.DUAL_CHUNK_SWAP else 1
    lengths = rng.integers(0, 40, size=n_docs)
    padded = ((lengths + mult - 1) // mult) * mult
    extra = rng.integers(0, 2, size=n_docs) * mult       # some docs get extra padding
    padded = padded + extra
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cup = np.concatenate([[0], np.cumsum(padded)])
    T = int(cup[-1])
    if strategy == O.NO_LOAD_BALANCE:
        T = ((T + pad_tail + cp - 1) // cp) * cp
    return cu, cup, T


@pytest.mark.parametrize("strategy", [O.DUAL_CHUNK_SWAP, O.NO_LOAD_BALANCE])
@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_partition_is_permutation(strategy, cp):
    rng = np.random.default_rng(cp * 7 + len(strategy))
    for trial in range(20):
        cu, cup, T = _random_layout(rng, strategy, cp, int(rng.integers(1, 9)), pad_tail=5)
        O.check_layout(cu, cup, T, cp, 0, strategy)
        allrows = np.concatenate([O.partition_index(cup, T, cp, r, strategy) for r in range(cp)])
        assert len(allrows) == T
        assert sorted(allrows.tolist()) == list(range(T))
        for r in range(cp):
            assert len(O.partition_index(cup, T, cp, r, strategy)) == T // cp


def test_nlb_is_contiguous_and_rank_ordered():
    rng = np.random.default_rng(3)
    for _ in range(20):
        cp = int(rng.integers(1, 6))
        cu, cup, T = _random_layout(rng, O.NO_LOAD_BALANCE, cp, 5, pad_tail=3)
        prev_end = 0
        for r in range(cp):
            idx = O.partition_index(cup, T, cp, r, O.NO_LOAD_BALANCE)
            assert idx[0] == prev_end
            assert np.all(np.diff(idx) == 1)
            prev_end = idx[-1] + 1


@pytest.mark.parametrize("cp", [2, 3, 4, 8])
def test_dcs_balances_causal_work(cp):
    # Unpadded documents: every rank must get the same number of causal pairs.
    # A chunk pairing other than (r, 2cp-1-r) (e.g. (r, r+cp)) breaks this.
    rng = np.random.default_rng(cp)
    for _ in range(10):
        lengths = rng.integers(1, 20, size=int(rng.integers(1, 6))) * 2 * cp
        cu = np.concatenate([[0], np.cumsum(lengths)])
        T = int(cu[-1])
        pairs = [O.causal_pairs(cu, cu, T, O.partition_index(cu, T, cp, r, O.DUAL_CHUNK_SWAP))
                 for r in range(cp)]
        assert len(set(pairs)) == 1, pairs
        assert sum(pairs) == sum(int(L) * (int(L) + 1) // 2 for L in lengths)


def test_dcs_local_order_doc_major_and_ascending_in_doc():
    cup = [0, 16, 24]
    idx = O.partition_index(cup, 24, 2, 0, O.DUAL_CHUNK_SWAP)
    # doc 0: chunks 0 and 3 of size 4; doc 1: chunks 0 and 3 of size 2
    assert idx.tolist() == [0, 1, 2, 3, 12, 13, 14, 15, 16, 17, 22, 23]


def test_token_table_brute_force():
    cu = [0, 3, 3, 10]
    cup = [0, 4, 8, 12]
    doc, pos, valid = O.token_table(cu, cup, 14)
    exp_doc, exp_pos, exp_valid = [], [], []
    for t in range(14):
        d = -1
        for i in range(3):
            if cup[i] <= t < cup[i + 1]:
                d = i
        exp_doc.append(d)
        exp_pos.append(t - cup[d] if d >= 0 else 0)
        exp_valid.append(d >= 0 and (t - cup[d]) < (cu[d + 1] - cu[d]))
    assert doc.tolist() == exp_doc
    assert pos.tolist() == exp_pos
    assert valid.tolist() == exp_valid


@pytest.mark.parametrize("case", _load("metadata_examples.json")["padding"], ids=lambda c: c["name"])
def test_padding_detected_by_value(case):
    cu = np.array(case["cu_seqlens"], dtype=np.int32)
    cup = np.array(case["cu_seqlens_padded"], dtype=np.int32)   # a separate object
    assert cu is not cup
    assert O.padding_present(cu, cup, case["T"]) is case["padding"]


@pytest.mark.parametrize("case", _load("metadata_examples.json")["pairs"], ids=lambda c: c["name"])
def test_pair_counts(case):
    idx = O.partition_index(case["cu_seqlens_padded"], case["T"], case["cp_size"], case["rank"],
                            case["strategy"])
    assert O.causal_pairs(case["cu_seqlens"], case["cu_seqlens_padded"], case["T"], idx) == case["pairs"]


@pytest.mark.parametrize("strategy", [O.DUAL_CHUNK_SWAP, O.NO_LOAD_BALANCE])
def test_local_valid_lengths_brute_force(strategy):
    rng = np.random.default_rng(11)
    for _ in range(10):
        cp = int(rng.integers(1, 5))
        cu, cup, T = _random_layout(rng, strategy, cp, 4, pad_tail=2)
        total = np.zeros(len(cu) - 1, dtype=np.int64)
        for r in range(cp):
            got = O.local_valid_lengths(cu, cup, T, cp, r, strategy)
            idx = O.partition_index(cup, T, cp, r, strategy)
            exp = np.zeros(len(cu) - 1, dtype=np.int64)
            for g in idx:
                for i in range(len(cu) - 1):
                    if cup[i] <= g < cup[i] + (cu[i + 1] - cu[i]):
                        exp[i] += 1
            assert got.tolist() == exp.tolist()
            total += got
        assert total.tolist() == np.diff(cu).tolist()


def test_check_layout_rejects():
    ok = ([0, 8], [0, 8], 8)
    O.check_layout(*ok, 2, 1, O.DUAL_CHUNK_SWAP)
    with pytest.raises(ValueError):
        O.check_layout([0, 6], [0, 6], 6, 2, 0, O.DUAL_CHUNK_SWAP)      # 6 % 4 != 0
    with pytest.raises(ValueError):
        O.check_layout([0, 8], [0, 8], 8, 2, 2, O.DUAL_CHUNK_SWAP)      # rank >= cp
    with pytest.raises(ValueError):
        O.check_layout([0, 9], [0, 8], 8, 2, 0, O.NO_LOAD_BALANCE)      # actual > padded
    with pytest.raises(ValueError):
        O.check_layout([0, 7], [0, 7], 7, 2, 0, O.NO_LOAD_BALANCE)      # T % cp
    with pytest.raises(ValueError):
        O.check_layout([0, 8], [0, 8], 12, 2, 0, O.DUAL_CHUNK_SWAP)     # tail under DCS
    O.check_layout([0, 6], [0, 6], 6, 2, 0, O.NO_LOAD_BALANCE)          # NLB: only the total


def test_workload_generators_match_recorded_layouts():
    w = W.WORKLOADS
    assert list(w["dcs_8k"].lengths) == [1781, 1398, 1172, 739, 807, 329, 390, 1564]
    assert list(w["dcs_8k"].padded) == [1784, 1400, 1172, 740, 808, 332, 392, 1564]
    assert w["dcs_8k"].T == 8192
    assert len(w["nlb_32k"].lengths) == 25 and w["nlb_32k"].T == 32768
    assert w["nlb_32k"].lengths[:3] == (1244, 961, 2081) and w["nlb_32k"].lengths[-1] == 181
    assert w["pad_131k"].T == 131680
    assert sum(w["pad_131k"].padded) - sum(w["pad_131k"].lengths) == 443
    for name in W.ORDER:
        x = w[name]
        O.check_layout(x.cu_seqlens(), x.cu_seqlens_padded(), x.T, x.cp_size, x.rank, x.strategy)
    # value-equal clones are separate arrays with equal values
    x = w["nlb_32k"]
    a, b = x.cu_seqlens(), x.cu_seqlens_padded()
    assert a is not b and np.array_equal(a, b)
    assert not O.padding_present(a, b, x.T)
    assert O.padding_present(w["pad_131k"].cu_seqlens(), w["pad_131k"].cu_seqlens_padded(),
                             w["pad_131k"].T)


def test_recorded_pair_counts_of_named_ranks():
    # Per-head causal pairs of the measured rank share; these feed the FLOP count.
    exp = {"dcs_8k": 2608720, "nlb_32k": 6156937, "pad_131k": 22487238}
    for name, pairs in exp.items():
        x = W.WORKLOADS[name]
        idx = O.partition_index(x.cu_seqlens_padded(), x.T, x.cp_size, x.rank, x.strategy)
        assert O.causal_pairs(x.cu_seqlens(), x.cu_seqlens_padded(), x.T, idx) == pairs
