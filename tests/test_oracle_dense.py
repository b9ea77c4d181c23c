"""Pins for the oracle's dense-layout definitions (CPU only).

Flat a2a is tested over bshd, sbhd and THD ("[PyTorch] Extend no-load-balance
CP to the a2a comm type", PR body). The oracle defines a dense batch's rank
share directly: each batch element is a sequence of S tokens, sharded along S.
Pinned against: hand examples of the sequence shard; torch float64 batched
SDPA at cp_size 1 (a library routine that handles the batch itself); the
union of ranks equals cp_size 1; and the two THD views the library relies on
(bshd = B documents, sbhd = one document with B*H heads) give the same
numbers through the THD definitions.
"""
import numpy as np
import pytest
import torch

import oracle as O

DCS, NLB = O.DUAL_CHUNK_SWAP, O.NO_LOAD_BALANCE


def _dense(layout, B, S, H, D, seed):
    rng = np.random.default_rng(seed)
    shape = (B, S, H, D) if layout == "bshd" else (S, B, H, D)
    return [rng.standard_normal(shape) for _ in range(4)]


def test_sequence_shard_examples():
    assert O.sequence_shard(8, 2, 1, DCS).tolist() == [2, 3, 4, 5]
    assert O.sequence_shard(8, 2, 0, DCS).tolist() == [0, 1, 6, 7]
    assert O.sequence_shard(12, 4, 2, NLB).tolist() == [6, 7, 8]
    # divisible by cp_size but not by 2*cp_size: allowed for NO_LOAD_BALANCE only
    assert O.sequence_shard(6, 2, 1, NLB).tolist() == [3, 4, 5]
    with pytest.raises(ValueError):
        O.sequence_shard(6, 2, 1, DCS)
    for strat, S, cp in ((DCS, 24, 3), (NLB, 21, 3)):
        allpos = np.concatenate([O.sequence_shard(S, cp, r, strat) for r in range(cp)])
        assert sorted(allpos.tolist()) == list(range(S))


@pytest.mark.parametrize("layout", ["bshd", "sbhd"])
def test_cp1_matches_batched_torch_sdpa(layout):
    B, S, H, D = 3, 20, 2, 8
    q, k, v, do = _dense(layout, B, S, H, D, 1)
    pos, o, lse, dq, dk, dv = O.dense_rank_share(q, k, v, do, layout, 1, 0, NLB)
    assert pos.tolist() == list(range(S))
    to_bhsd = (0, 2, 1, 3) if layout == "bshd" else (1, 2, 0, 3)
    tq, tk, tv = (torch.tensor(x.transpose(to_bhsd), requires_grad=True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref.detach().numpy().transpose(0, 2, 1, 3), atol=1e-12)
    ref.backward(torch.tensor(do.transpose(to_bhsd)))
    np.testing.assert_allclose(dq, tq.grad.numpy().transpose(0, 2, 1, 3), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy().transpose(0, 2, 1, 3), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy().transpose(0, 2, 1, 3), atol=1e-11)


@pytest.mark.parametrize("layout", ["bshd", "sbhd"])
@pytest.mark.parametrize("strategy,S,cp", [(DCS, 24, 3), (NLB, 21, 3), (NLB, 6, 2)])
def test_union_of_ranks_equals_cp1(layout, strategy, S, cp):
    B, H, D = 2, 2, 4
    q, k, v, do = _dense(layout, B, S, H, D, 2)
    _, o1, l1, dq1, dk1, dv1 = O.dense_rank_share(q, k, v, do, layout, 1, 0, NLB)
    o_u = np.zeros_like(o1)
    dq_u = np.zeros_like(dq1)
    dk_u = np.zeros_like(dk1)
    dv_u = np.zeros_like(dv1)
    for r in range(cp):
        pos, o, lse, dq, dk, dv = O.dense_rank_share(q, k, v, do, layout, cp, r, strategy)
        o_u[:, pos] = o
        dq_u[:, pos] = dq
        dk_u += dk
        dv_u += dv
    for a, b in ((o_u, o1), (dq_u, dq1), (dk_u, dk1), (dv_u, dv1)):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("window", [(-1, 0), (-1, -1), (3, 1)])
def test_sbhd_is_one_document_with_batch_times_heads(window):
    # the THD definition on the view [S, B*H, D] with cu_seqlens [0, S]
    B, S, H, D, cp = 3, 16, 2, 4, 2
    q, k, v, do = _dense("sbhd", B, S, H, D, 3)
    view = [x.reshape(S, B * H, D) for x in (q, k, v, do)]
    for strategy in (DCS, NLB):
        for r in range(cp):
            pos, o, lse, dq, dk, dv = O.dense_rank_share(q, k, v, do, "sbhd", cp, r, strategy,
                                                         window=window)
            idx, o2, l2, dq2, dk2, dv2 = O.rank_share(*view, [0, S], [0, S], S, cp, r, strategy,
                                                      window=window)
            assert idx.tolist() == pos.tolist()
            n = len(pos)
            np.testing.assert_allclose(o2.reshape(n, B, H, D).transpose(1, 0, 2, 3), o,
                                       atol=1e-13)
            np.testing.assert_allclose(l2.reshape(B, H, n), lse, atol=1e-13)
            np.testing.assert_allclose(dq2.reshape(n, B, H, D).transpose(1, 0, 2, 3), dq,
                                       atol=1e-13)
            np.testing.assert_allclose(dk2.reshape(S, B, H, D).transpose(1, 0, 2, 3), dk,
                                       atol=1e-13)
            np.testing.assert_allclose(dv2.reshape(S, B, H, D).transpose(1, 0, 2, 3), dv,
                                       atol=1e-13)


def test_bshd_is_documents_under_dual_chunk_swap():
    # the THD definition on the view [B*S, H, D] with B documents of S tokens;
    # under DUAL_CHUNK_SWAP its partition is every sequence's shard, doc-major
    B, S, H, D, cp = 3, 16, 2, 4, 2
    q, k, v, do = _dense("bshd", B, S, H, D, 4)
    view = [x.reshape(B * S, H, D) for x in (q, k, v, do)]
    cu = list(range(0, (B + 1) * S, S))
    for r in range(cp):
        pos, o, lse, dq, dk, dv = O.dense_rank_share(q, k, v, do, "bshd", cp, r, DCS)
        idx, o2, l2, dq2, dk2, dv2 = O.rank_share(*view, cu, cu, B * S, cp, r, DCS)
        n = len(pos)
        assert idx.tolist() == [b * S + p for b in range(B) for p in pos.tolist()]
        np.testing.assert_allclose(o2.reshape(B, n, H, D), o, atol=1e-13)
        np.testing.assert_allclose(dq2.reshape(B, n, H, D), dq, atol=1e-13)
        np.testing.assert_allclose(dk2.reshape(B, S, H, D), dk, atol=1e-13)
        np.testing.assert_allclose(dv2.reshape(B, S, H, D), dv, atol=1e-13)
        np.testing.assert_allclose(l2.transpose(1, 0).reshape(B, n, H).transpose(0, 2, 1), lse,
                                   atol=1e-13)
    # under NO_LOAD_BALANCE the THD partition of the packed rows is not the
    # per-sequence shard once B > 1
    idx = O.partition_index(cu, B * S, cp, 0, NLB)
    assert idx.tolist() != [b * S + p for b in range(B)
                            for p in O.sequence_shard(S, cp, 0, NLB).tolist()]
