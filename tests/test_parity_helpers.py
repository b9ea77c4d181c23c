"""The chunked driver of the oracle (used by the whole-tensor GPU checks at
full size) computes the oracle's own results: chunks of local rows evaluated
separately, then assembled and summed, equal one call over all rows."""
import numpy as np
import pytest

import workloads as W
from _parity import f64, oracle_share, oracle_share_chunked


@pytest.mark.parametrize("lengths,padded,T,cp,rank,strategy,window", [
    ((37, 91), (37, 91), 128, 2, 1, "no_load_balance", (-1, 0)),
    ((100, 0, 250, 37), (104, 0, 256, 40), 400, 2, 0, "dual_chunk_swap", (-1, 0)),
    ((100, 0, 250, 37), (104, 0, 256, 40), 400, 2, 1, "dual_chunk_swap", (16, 3)),
    ((300, 77), (300, 80), 384, 3, 2, "no_load_balance", (-1, -1)),
    ((700,), (700,), 700, 1, 0, "no_load_balance", (-1, 0)),
])
def test_chunked_equals_one_call(lengths, padded, T, cp, rank, strategy, window):
    w = W.custom("chk", lengths, padded, T, 2, 64, cp, rank, strategy, number=7)
    t64 = f64(W.bf16_tensors(w))
    ref = oracle_share(w, rank, t64, window=window)
    for chunk, heads in ((64, None), (17, slice(1, 2))):
        got = oracle_share_chunked(w, rank, t64, heads=heads, chunk_rows=chunk, workers=3,
                                   window=window)
        hs = slice(None) if heads is None else heads
        assert np.array_equal(got["idx"], ref["idx"])
        for n in ("o", "dq", "dk", "dv"):
            np.testing.assert_allclose(got[n], ref[n][:, hs], rtol=0, atol=1e-12, err_msg=n)
        np.testing.assert_array_equal(np.isneginf(got["lse"]), np.isneginf(ref["lse"][hs]))
        fin = np.isfinite(ref["lse"][hs])
        np.testing.assert_allclose(got["lse"][fin], ref["lse"][hs][fin], rtol=0, atol=1e-12)


def test_stair_inputs_and_oracle_lse_at_large_scores():
    """workloads.stair_bf16 is deterministic and stepped as documented, and the
    oracle's LSE stays exact where it reaches ~75 (raw exponentials near e^75):
    rows of a two-document layout against scipy's logsumexp over the row's own
    scores."""
    from scipy.special import logsumexp

    w = W.custom("stair_chk", [700, 300], [704, 304], None, 1, 64, 1, 0, "no_load_balance",
                 number=8)
    a, b = W.stair_bf16(w, step_keys=64), W.stair_bf16(w, step_keys=64)
    for n in ("q", "k", "v", "do"):
        assert a[n].shape == (w.T, w.H, w.D)
        assert bool((a[n] == b[n]).all()) and bool(a[n].float().isfinite().all())
    t64 = f64(a)
    cup = w.cu_seqlens_padded()
    # K's mean over head dims rises by one step every 64 keys of a document
    km = t64["k"][:, 0].mean(axis=1)
    steps = km[cup[0]:cup[0] + 640:64]
    assert np.all(np.diff(steps) > 0)
    ref = oracle_share(w, 0, t64)
    q, k = t64["q"][:, 0], t64["k"][:, 0]
    for doc in (0, 1):
        start, end = int(cup[doc]), int(cup[doc] + w.lengths[doc])
        for g in (start, start + 63, start + 64, end - 2, end - 1):
            s = k[start:g + 1] @ q[g] / np.sqrt(w.D)
            assert abs(ref["lse"][0, g] - logsumexp(s)) <= 1e-9 * max(1.0, abs(logsumexp(s)))
    assert ref["lse"][0, int(w.lengths[0]) - 1] > 70.0  # the large-score regime
