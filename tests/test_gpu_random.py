"""Seeded random layouts, every rank, element by element against the oracle.

The fixed cases elsewhere pin chosen edge cases. Here a seeded generator draws
the rest of the space the plan accepts:
- both strategies, cp_size 1-4, head dims 64 and 128, 1-3 heads;
- 1-5 documents of 0-419 real tokens, with or without padding (DUAL_CHUNK_SWAP
  rounds every padded length up to a multiple of 2*cp_size);
- for NO_LOAD_BALANCE, an unused tail after the last document;
- causal, whole-document and banded key windows.

Each layout runs every rank through the product path (partition index,
gather, plan, forward, composite backward) and is compared with the fp64
oracle at the usual bar. Padding rows must come out exactly 0.
"""
import sys

import numpy as np
import pytest

import workloads as W
from _parity import assert_close, assert_lse, f64, oracle_share, run_share

import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")

N_LAYOUTS = 12


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def random_layout(i):
    rng = np.random.default_rng(20261202 + i)
    strategy = ("dual_chunk_swap", "no_load_balance")[int(rng.integers(0, 2))]
    cp = int(rng.integers(1, 5))
    D = (64, 128)[int(rng.integers(0, 2))]
    H = int(rng.integers(1, 4))
    lengths, padded = [], []
    for _ in range(int(rng.integers(1, 6))):
        n = 0 if rng.random() < 0.1 else int(rng.integers(1, 420))
        p = n + (int(rng.integers(0, 12)) if rng.random() < 0.6 else 0)
        if strategy == "dual_chunk_swap":
            p = -(-p // (2 * cp)) * (2 * cp)
        lengths.append(n)
        padded.append(p)
    if sum(padded) == 0:
        lengths[-1] = 1
        padded[-1] = 2 * cp
    if strategy == "dual_chunk_swap":
        T = None
    else:
        extra = int(rng.integers(0, 3 * cp))
        T = -(-(sum(padded) + extra) // cp) * cp
    windows = [(-1, 0), (-1, 0), (-1, -1), (int(rng.integers(0, 300)), 0),
               (int(rng.integers(0, 200)), int(rng.integers(1, 80)))]
    window = windows[int(rng.integers(0, len(windows)))]
    w = W.custom(f"rand{i}", lengths, padded, T, H, D, cp, 0, strategy, number=500 + i)
    return w, window


@pytest.mark.parametrize("i", range(N_LAYOUTS), ids=lambda i: f"layout{i}")
def test_random_layout_all_ranks(i):
    w, window = random_layout(i)
    _say(f"layout {i}: {w.strategy} cp={w.cp_size} H={w.H} D={w.D} T={w.T} "
         f"lengths={list(w.lengths)} padded={list(w.padded)} window={window}")
    t = W.bf16_tensors(w)
    t64 = f64(t)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    _, _, valid = O.token_table(cu, cup, w.T)
    for r in range(w.cp_size):
        _say("  rank", r)
        got = run_share(w, r, t, window=window)
        ref = oracle_share(w, r, t64, window=window)
        assert np.array_equal(got["idx"], ref["idx"])
        tag = f"rand{i} r{r}"
        assert_close(got["o"], ref["o"], f"{tag} O")
        assert_lse(got["lse"], ref["lse"], f"{tag} LSE")
        for n in ("dq", "dk", "dv"):
            assert_close(got[n], ref[n], f"{tag} {n}")
        pad_local = ~valid[ref["idx"]]
        assert np.all(got["o"][pad_local] == 0) and np.all(got["dq"][pad_local] == 0)
        assert np.all(got["dk"][~valid] == 0) and np.all(got["dv"][~valid] == 0)
