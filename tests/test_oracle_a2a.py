"""Pins for the oracle's all-to-all layout functions (CPU only).

"[PyTorch] Extend no-load-balance CP to the a2a comm type" (body and diagram)
fixes what the exchange must produce: after the forward exchange every rank
holds the whole sequence, in global order, for its own head slice only; after
the return exchange every rank holds its own token shard with all heads. The
pages print no example values, so the pack is pinned by a hand-worked case
and the exchange by exactly those two properties, checked against plain
slices of the global tensor (not against the pack formula), for both
strategies, with padding, a buffer tail, a cp_size that does not divide
2 * cp_size-sized chunks, and cp_size = 1.
"""
import numpy as np
import pytest

import oracle as O


def test_pack_hand_example():
    # 3 tokens x 4 heads x 1, value 10*token + head; cp_size = 2.
    x = np.array([[[10 * m + h] for h in range(4)] for m in range(3)])
    want = np.array([
        [[[0], [1]], [[10], [11]], [[20], [21]]],     # block 0: heads 0, 1
        [[[2], [3]], [[12], [13]], [[22], [23]]],     # block 1: heads 2, 3
    ])
    got = O.a2a_pack(x, 2)
    assert got.shape == (2, 3, 2, 1)
    assert np.array_equal(got, want)
    assert np.array_equal(O.a2a_unpack(want), x)


def test_pack_cp1_is_identity_and_rejects_bad_heads():
    x = np.random.default_rng(0).standard_normal((5, 3, 2))
    assert np.array_equal(O.a2a_pack(x, 1)[0], x)
    with pytest.raises(ValueError):
        O.a2a_pack(x, 2)


LAYOUTS = [
    # name, cu_seqlens_padded, T, cp, strategy
    ("bshd_one_doc_dcs", [0, 64], 64, 4, O.DUAL_CHUNK_SWAP),
    ("bshd_one_doc_flat", [0, 64], 64, 4, O.NO_LOAD_BALANCE),
    ("thd_docs_dcs", [0, 16, 48, 56, 96], 96, 4, O.DUAL_CHUNK_SWAP),
    ("thd_docs_flat_tail", [0, 13, 40, 41], 48, 4, O.NO_LOAD_BALANCE),
    # divisible by cp_size but not by 2 * cp_size (only the flat path allows it)
    ("flat_odd_chunks", [0, 9, 21], 21, 3, O.NO_LOAD_BALANCE),
    ("cp1", [0, 8, 20], 20, 1, O.DUAL_CHUNK_SWAP),
]


@pytest.mark.parametrize("name,cup,T,cp,strategy", LAYOUTS, ids=[l[0] for l in LAYOUTS])
def test_exchange_gives_global_head_slice(name, cup, T, cp, strategy):
    H, D = 2 * cp, 3
    x = np.random.default_rng(T * 7 + cp).standard_normal((T, H, D))
    shards = [x[O.partition_index(cup, T, cp, r, strategy)] for r in range(cp)]
    full = O.a2a_before_attn(shards, cup, T, cp, strategy)
    hl = H // cp
    for r in range(cp):
        assert full[r].shape == (T, hl, D)
        assert np.array_equal(full[r], x[:, r * hl:(r + 1) * hl]), f"rank {r}"


@pytest.mark.parametrize("name,cup,T,cp,strategy", LAYOUTS, ids=[l[0] for l in LAYOUTS])
def test_return_exchange_gives_local_shard(name, cup, T, cp, strategy):
    H, D = 3 * cp, 2
    y = np.random.default_rng(T * 11 + cp).standard_normal((T, H, D))
    hl = H // cp
    back = O.a2a_after_attn([y[:, r * hl:(r + 1) * hl] for r in range(cp)], cup, T, cp, strategy)
    for r in range(cp):
        idx = O.partition_index(cup, T, cp, r, strategy)
        assert np.array_equal(back[r], y[idx]), f"rank {r}"


def test_dcs_rank_major_order_differs_from_global():
    # The reorder is real work under DUAL_CHUNK_SWAP: without it rank 0 would
    # see rank-major rows, which are not in global order.
    cup, T, cp = [0, 64], 64, 4
    x = np.arange(T, dtype=np.float64).reshape(T, 1, 1).repeat(cp, axis=1)
    shards = [x[O.partition_index(cup, T, cp, r, O.DUAL_CHUNK_SWAP)] for r in range(cp)]
    rank_major = np.concatenate([O.a2a_pack(s, cp)[0] for s in shards], axis=0)
    assert not np.array_equal(rank_major[:, 0, 0], np.arange(T))
    assert np.array_equal(O.a2a_before_attn(shards, cup, T, cp)[0][:, 0, 0], np.arange(T))
