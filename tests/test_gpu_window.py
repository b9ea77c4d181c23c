"""GPU parity of the attention kernels under masks other than causal.

After the a2a exchange every mask type and window size stays valid ("[PyTorch]
Extend no-load-balance CP to the a2a comm type", PR body). The plan's window
(left, right) lets a real query at document position p attend the real keys
at [p - left, p + right] (-1: no bound). Outputs are compared with the fp64
oracle under the same window: element by element on small layouts (every
rank, windows that cut tiles anywhere, the whole document, a one-key band),
and on sampled rows plus invariants at full size on the flat (post-a2a)
share. Bar as everywhere: max-abs 2e-2, relative-L2 5e-3 per tensor;
padding rows and keys no local query reaches exactly 0.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W
from _parity import assert_close, assert_lse, err, f64, oracle_share, run_share

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = [
    W.custom("win_flat_d128", [1500], [1500], None, 2, 128, 1, 0, "no_load_balance"),
    W.custom("win_flat_pad_d64", [300, 0, 901, 77], [310, 4, 901, 90], 1320, 2, 64, 1, 0,
             "no_load_balance"),
    W.custom("win_dcs_pad_d128", [200, 1, 513, 77], [208, 8, 520, 80], None, 2, 128, 2, 0,
             "dual_chunk_swap"),
    W.custom("win_nlb_tail_d128", [250, 5, 900, 333], [256, 5, 900, 340], 1548, 2, 128, 3, 0,
             "no_load_balance"),
    W.custom("win_dcs_cp4_d64", [129, 3, 700, 64], [136, 8, 704, 64], None, 2, 64, 4, 0,
             "dual_chunk_swap"),
]
WINDOWS = [(-1, -1), (64, 0), (100, 37), (0, 0), (7, 300), (200, -1)]


@pytest.mark.parametrize("window", WINDOWS, ids=lambda x: f"w{x[0]}_{x[1]}")
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_window_elementwise_all_ranks(w, window):
    t = W.bf16_tensors(w)
    t64 = f64(t)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    _, _, valid = O.token_table(cu, cup, w.T)
    nan = torch.full((w.T, w.H, w.D), float("nan"))
    for r in range(w.cp_size):
        _say("window", w.name, window, "rank", r)
        got = run_share(w, r, t, window=window, dk_init=nan, dv_init=nan)
        ref = oracle_share(w, r, t64, window=window)
        tag = f"{w.name} {window} r{r}"
        idx = ref["idx"]
        assert got["plan"].info.causal_pairs == O.causal_pairs(cu, cup, w.T, idx, window=window)
        assert_close(got["o"], ref["o"], tag + " O")
        assert_lse(got["lse"], ref["lse"], tag + " LSE")
        for n in ("dq", "dk", "dv"):
            assert np.all(np.isfinite(got[n])), tag + " " + n
            assert_close(got[n], ref[n], f"{tag} {n}")
        pad_local = ~valid[idx]
        assert np.all(got["o"][pad_local] == 0) and np.all(got["dq"][pad_local] == 0)
        untouched = ~O.touched_keys(cu, cup, w.T, idx, window=window)
        assert np.all(got["dk"][untouched] == 0) and np.all(got["dv"][untouched] == 0)


@pytest.mark.parametrize("window", [(64, 0), (-1, -1)], ids=lambda x: f"w{x[0]}_{x[1]}")
def test_window_rank_major_bit_identical(window):
    w = SMALL[2]
    t = W.bf16_tensors(w)
    for r in range(w.cp_size):
        g = run_share(w, r, t, window=window)
        m = run_share(w, r, t, window=window, kv_layout="rank_major")
        perm = m["perm"]
        for n in ("o", "lse", "dq"):
            assert np.array_equal(m[n], g[n]), n
        for n in ("dk", "dv"):
            assert np.array_equal(m[n], g[n][perm]), n


def test_causal_window_equals_default():
    # a left bound at or past every document is no bound: bit-identical
    w = SMALL[3]
    t = W.bf16_tensors(w)
    a = run_share(w, 1, t)
    b = run_share(w, 1, t, window=(w.T, 0))
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


def _window_samples(w, window, rng, n_rows=64, n_keys=12, max_attending=2500):
    """Local rows to check one by one, and key rows whose attending local rows
    are few enough to compute all of them (those rows are added)."""
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    idx = O.partition_index(cup, w.T, w.cp_size, w.rank, w.strategy)
    doc, pos, valid = O.token_table(cu, cup, w.T)
    rows = set(rng.choice(len(idx), size=min(n_rows, len(idx)), replace=False).tolist())
    rows |= {0, len(idx) - 1}
    real = np.flatnonzero(valid[idx])
    g = idx[real]
    d = doc[g]
    a = np.asarray(cup)[d]
    e = a + (np.asarray(cu)[d + 1] - np.asarray(cu)[d])
    lo = np.where(window[0] < 0, a, np.maximum(a, g - window[0]))
    hi = np.where(window[1] < 0, e - 1, np.minimum(e - 1, g + window[1]))
    touched = np.flatnonzero(O.touched_keys(cu, cup, w.T, idx, window=window))
    keys = []
    for j in rng.choice(touched, size=min(200, len(touched)), replace=False):
        att = real[(lo <= j) & (hi >= j)]
        if 0 < len(att) <= max_attending:
            keys.append(int(j))
            rows |= set(att.tolist())
            if len(keys) == n_keys:
                break
    return sorted(rows), sorted(keys)


@pytest.mark.parametrize("name,window", [("flat_75k", (1024, 0)), ("flat_75k", (300, 200)),
                                         ("flat_75k", (-1, -1)), ("dcs_8k", (256, 0)),
                                         ("pad_131k", (-1, -1))],
                         ids=lambda x: str(x))
def test_window_full_size(name, window):
    w = W.WORKLOADS[name]
    _say("window full-size", name, window)
    t = W.bf16_tensors(w)
    nan = torch.full((w.T, w.H, w.D), float("nan"))
    got = run_share(w, w.rank, t, window=window, dk_init=nan, dv_init=nan)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    idx = got["idx"]
    for n in ("o", "dq", "dk", "dv"):
        assert np.all(np.isfinite(got[n])), n
    t64 = {n: t[n].double().numpy() for n in t}
    rows, keys = _window_samples(w, window, np.random.default_rng(3))
    _say("  sampled rows", len(rows), "keys", len(keys))
    ref = oracle_share(w, w.rank, t64, rows=rows, window=window)
    assert_close(got["o"][rows], ref["o"][rows], f"{name} {window} O[rows]")
    assert_lse(got["lse"][:, rows], ref["lse"][:, rows], f"{name} {window} LSE[rows]")
    assert_close(got["dq"][rows], ref["dq"][rows], f"{name} {window} dQ[rows]")
    if keys:
        assert_close(got["dk"][keys], ref["dk"][keys], f"{name} {window} dK[keys]")
        assert_close(got["dv"][keys], ref["dv"][keys], f"{name} {window} dV[keys]")
    else:
        assert window == (-1, -1)   # every key is attended by a whole document
    # invariants at any size: untouched rows 0; per document sum dV = sum dO
    # of the local real rows, sum dK ~ 0
    touched = O.touched_keys(cu, cup, w.T, idx, window=window)
    assert np.all(got["dk"][~touched] == 0) and np.all(got["dv"][~touched] == 0)
    doc, _, valid = O.token_table(cu, cup, w.T)
    dol = t64["do"][idx]
    vloc = valid[idx]
    sv, sdo, sk, nk = [], [], [], []
    for d in range(w.B):
        a, b = cup[d], cup[d + 1]
        rd = np.flatnonzero(vloc & (doc[idx] == d))
        if len(rd) == 0:
            continue
        sv.append(got["dv"][a:b].astype(np.float64).sum(axis=0))
        sdo.append(dol[rd].sum(axis=0))
        sk.append(got["dk"][a:b].astype(np.float64).sum(axis=0))
        nk.append(np.linalg.norm(got["dk"][a:b]))
    _, rel = err(np.array(sv), np.array(sdo))
    assert rel < 5e-3, f"sum dV vs sum dO rel={rel:.2e}"
    assert np.linalg.norm(np.array(sk)) < 0.05 * np.linalg.norm(np.array(nk))
