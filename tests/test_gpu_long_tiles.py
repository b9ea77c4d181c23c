"""GPU parity of the large tiles of long-walk plans.

A rank's forward and dQ walk, per query tile, every key its rows attend, and
its dK/dV walk, per key tile, every local query that attends it ("[PyTorch]
Add no-load-balance THD all-gather CP", "Why": the rank's attention steps
over the gathered K/V). Where the average local query walks 4096 keys or
more (all-gather plans), the plan uses query tiles of 256 rows and key tiles
of 256 keys (eight waves of 32 each) instead of 128, so every staged tile
serves twice the rows; at head dim 128 the forward also reads V transposed
(a pre-pass writes V^T, with the keys no local query attends set to 0). This checks those plans against the fp64 oracle
element by element over the whole share: one long document with a ragged end
and a buffer tail (head dim 128), a padded DUAL_CHUNK_SWAP pair of documents
on both ranks (head dim 64, where half of the 8 dK/dV waves stage the query
blocks), key bands with a right bound and the whole document, forced and
automatic split walks against the unsplit plan, rank-major against global
K/V (bit-identical but for dQ's rounding), and NaN in every padding row of Q/K/V/dO changing no
output bit. Bar: max-abs 2e-2, relative-L2 5e-3.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W
from _parity import assert_close, assert_lse, err, f64, oracle_share_chunked, run_share

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


DOC = W.custom("long_doc_d128", [8700], [8704], 8800, 2, 128, 1, 0, "no_load_balance")
DCS = W.custom("long_dcs_pad_d64", [17000, 299], [17000, 304], None, 2, 64, 2, 0,
               "dual_chunk_swap")
DCS128 = W.custom("long_dcs_pad_d128", [12000, 299], [12000, 304], None, 2, 128, 2, 0,
                  "dual_chunk_swap")


def _check(got, ref, tag):
    assert_close(got["o"], ref["o"], tag + " O")
    assert_lse(got["lse"], ref["lse"], tag + " LSE")
    for n in ("dq", "dk", "dv"):
        assert_close(got[n], ref[n], f"{tag} {n}")


def test_long_doc_whole_share():
    t = W.bf16_tensors(DOC)
    ref = oracle_share_chunked(DOC, 0, f64(t))
    whole = None
    for parts in (1, 3, 0):
        _say("long tiles", DOC.name, "max_key_splits", parts)
        got = run_share(DOC, 0, t, max_key_splits=parts)
        info = got["plan"].info
        assert info.fwd_tile_rows == 256 and info.bwd_tile_keys == 256
        if parts == 1:
            assert info.n_split_tiles == 0
            whole = got
        else:
            assert info.n_split_tiles > 0
        _check(got, ref, f"{DOC.name} parts<={parts}")
        # split against whole: the same sums in another order
        assert np.abs(got["o"] - whole["o"]).max() <= 2 ** -6
        for n in ("dq", "dk", "dv"):
            _, rel = err(got[n], whole[n])
            assert rel <= 1e-3, (n, rel)


@pytest.mark.parametrize("rank", [0, 1])
def test_long_dcs_both_ranks(rank):
    t = W.bf16_tensors(DCS)
    _say("long tiles", DCS.name, "rank", rank)
    got = run_share(DCS, rank, t)
    assert got["plan"].info.fwd_tile_rows == 256 and got["plan"].info.bwd_tile_keys == 256
    ref = oracle_share_chunked(DCS, rank, f64(t))
    _check(got, ref, f"{DCS.name} r{rank}")


@pytest.mark.parametrize("window", [(3000, 2500), (-1, -1)])
def test_long_doc_bands(window):
    t = W.bf16_tensors(DOC)
    _say("long tiles", DOC.name, "window", window)
    got = run_share(DOC, 0, t, window=window)
    assert got["plan"].info.fwd_tile_rows == 256
    ref = oracle_share_chunked(DOC, 0, f64(t), window=window)
    _check(got, ref, f"{DOC.name} {window}")


def test_long_rank_major_matches_global():
    # O, LSE, dK and dV keep every bit across the two K/V layouts. dQ differs by
    # rounding only: over global-order K/V the 8-wave dQ kernel starts its dP
    # accumulators at -delta, over the rank-major map it subtracts delta per
    # element (the start at -delta spills there), so dP - delta can differ in
    # its last fp32 bit and flip the bf16 rounding of a dS element.
    t = W.bf16_tensors(DCS)
    _say("long tiles rank-major", DCS.name)
    g = run_share(DCS, 1, t)
    m = run_share(DCS, 1, t, kv_layout="rank_major")
    assert m["plan"].info.fwd_tile_rows == 256
    perm = m["perm"]
    for n in ("o", "lse"):
        assert np.array_equal(m[n], g[n]), n
    for n in ("dk", "dv"):
        assert np.array_equal(m[n], g[n][perm]), n
    scale = float(np.abs(g["dq"]).max())
    assert np.abs(m["dq"] - g["dq"]).max() <= 2e-4 * scale
    _, rel = err(m["dq"], g["dq"])
    assert rel <= 1e-4, rel


def test_short_walks_keep_128_row_tiles():
    # the same long document cut into 16 documents: walks of ~270 keys
    w = W.custom("cut_doc", [544] * 16, [544] * 16, None, 2, 128, 1, 0, "no_load_balance")
    plan = thd.Plan(w.cu_seqlens(), w.cu_seqlens_padded(), w.T, 1, 0, w.strategy, w.H, w.D,
                    upload=False)
    assert plan.info.fwd_tile_rows == 128 and plan.info.bwd_tile_keys == 128
    plan.close()


def test_long_dcs_d128_rank_major():
    # head dim 128: the transposed-V forward, its pre-pass reading K/V through
    # the rank-major map and zeroing the keys rank 1 does not attend
    t = W.bf16_tensors(DCS128)
    _say("long tiles", DCS128.name, "rank 1 rank-major")
    m = run_share(DCS128, 1, t, kv_layout="rank_major")
    assert m["plan"].info.fwd_tile_rows == 256 and m["plan"].info.n_zero_ranges > 0
    ref = oracle_share_chunked(DCS128, 1, f64(t))
    perm = m["perm"]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    got = dict(m, dk=m["dk"][inv], dv=m["dv"][inv])
    _check(got, ref, f"{DCS128.name} r1 rank-major")


def test_long_padding_poison():
    # NaN in every padding row (and the buffer tail) of Q, K, V and dO: the
    # outputs keep every bit
    cu, cup = DOC.cu_seqlens(), DOC.cu_seqlens_padded()
    _, _, valid = O.token_table(cu, cup, DOC.T)
    assert (~valid).sum() == 4 + 96
    t = W.bf16_tensors(DOC)
    bad = {n: x.clone() for n, x in t.items()}
    for x in bad.values():
        x[torch.from_numpy(~valid)] = float("nan")
    _say("long tiles poison", DOC.name)
    clean = run_share(DOC, 0, t)
    dirty = run_share(DOC, 0, bad)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(clean[n], dirty[n]), n
