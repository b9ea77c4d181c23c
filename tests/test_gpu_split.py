"""GPU parity of split key walks.

A rank's forward and dQ are one launch each over its query tiles ("[PyTorch]
Add no-load-balance THD all-gather CP", "Why"). When the share's documents
are short that grid barely fills the chip and the longest tiles' key walks
set the launch's duration, so the plan divides those walks into parts of
consecutive key tiles computed by separate workgroups; the last part to
finish merges them in key order (softmax states for O/LSE, sums for dQ).

Checked here against the fp64 oracle element by element, at forced part
counts from 1 (never split) to 8, on layouts whose walks span many key
tiles and end in a ragged diagonal: one long document, padded
DUAL_CHUNK_SWAP documents (rank-major K/V too), a window, head dim 64 and
128. Split and unsplit results agree to rounding, repeated launches give the
same bits (the part counters are left at zero), and the separate dQ entry
point matches the composite backward. Bar: max-abs 2e-2, relative-L2 5e-3.
"""
import sys

import numpy as np
import pytest

import workloads as W
from _parity import assert_close, assert_lse, err, f64, oracle_share, run_share

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    W.custom("split_doc_d128", [4000], [4096], None, 2, 128, 1, 0, "no_load_balance"),
    W.custom("split_dcs_pad_d64", [1900, 3, 2801, 640], [1904, 8, 2808, 640], None, 2, 64, 2, 0,
             "dual_chunk_swap"),
    W.custom("split_nlb_tail_d128", [2500, 77, 1300], [2500, 80, 1300], 3884, 2, 128, 2, 0,
             "no_load_balance"),
]


def _check(got, ref, tag):
    assert_close(got["o"], ref["o"], tag + " O")
    assert_lse(got["lse"], ref["lse"], tag + " LSE")
    for n in ("dq", "dk", "dv"):
        assert_close(got[n], ref[n], f"{tag} {n}")


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_split_parts_elementwise(w):
    t = W.bf16_tensors(w)
    t64 = f64(t)
    for r in range(w.cp_size):
        ref = oracle_share(w, r, t64)
        base = None
        for parts in (1, 2, 3, 8, 0):
            _say("split", w.name, "rank", r, "max_key_splits", parts)
            got = run_share(w, r, t, max_key_splits=parts)
            info = got["plan"].info
            if parts == 1:
                assert info.n_split_tiles == 0 and info.n_fwd_parts == info.n_fwd_tiles
                base = got
            else:
                assert info.n_split_tiles > 0 and info.n_fwd_parts > info.n_fwd_tiles
            _check(got, ref, f"{w.name} r{r} parts<={parts}")
            # split vs unsplit: the same sums in another order. The forward
            # differs by fp32 rounding (O by at most a bf16 step); the
            # backward also rounds dS to bf16 from the slightly different
            # LSE, so its gradients agree to a few bf16 steps in norm.
            d_o = np.abs(got["o"] - base["o"]).max()
            assert d_o <= 2 ** -6, d_o
            for n in ("dq", "dk", "dv"):
                _, rel = err(got[n], base[n])
                assert rel <= 1e-3, (n, rel)


def test_split_window_and_rank_major():
    w = CASES[1]
    t = W.bf16_tensors(w)
    t64 = f64(t)
    for window in ((700, 0), (300, 45)):
        ref = oracle_share(w, 1, t64, window=window)
        got = run_share(w, 1, t, window=window, max_key_splits=4)
        assert got["plan"].info.n_split_tiles > 0
        _check(got, ref, f"{w.name} {window} split")
    g = run_share(w, 0, t, max_key_splits=8)
    m = run_share(w, 0, t, max_key_splits=8, kv_layout="rank_major")
    perm = m["perm"]
    for n in ("o", "lse", "dq"):
        assert np.array_equal(m[n], g[n]), n
    for n in ("dk", "dv"):
        assert np.array_equal(m[n], g[n][perm]), n


def test_split_repeat_launches_bit_identical():
    # the counters that pick each group's last part are back at zero after
    # every launch: the same plan and workspace, launched again, give the
    # same bits
    w = CASES[0]
    t = W.bf16_tensors(w)
    dev = torch.device("cuda", 0)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    plan = thd.Plan(cu, cup, w.T, 1, 0, w.strategy, w.H, w.D, max_key_splits=8)
    assert plan.info.n_split_tiles > 0
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    outs = []
    for i in range(3):
        _say("repeat launch", i)
        o, lse = thd.attn_fwd(plan, q, k, v)
        dq, dk, dv = thd.attn_bwd(plan, q, k, v, o, lse, do)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (o, lse, dq, dk, dv)])
    for later in outs[1:]:
        for a, b in zip(outs[0], later):
            assert torch.equal(a, b)


def test_split_dq_entry_matches_composite():
    w = CASES[2]
    t = W.bf16_tensors(w)
    dev = torch.device("cuda", 0)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    cup_dev = torch.from_numpy(cup).to(dev)
    idx = thd.partition_index(cup, cup_dev, w.T, w.cp_size, 1, w.strategy)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    ql, dol = thd.gather(q, idx), thd.gather(do, idx)
    plan = thd.Plan(cu, cup, w.T, w.cp_size, 1, w.strategy, w.H, w.D, max_key_splits=4)
    assert plan.info.n_split_tiles > 0
    o, lse = thd.attn_fwd(plan, ql, k, v)
    dq, dk, dv = thd.attn_bwd(plan, ql, k, v, o, lse, dol)
    n = plan.n_local
    dq2 = torch.empty_like(dq)
    dk2 = torch.empty_like(dk)
    dv2 = torch.empty_like(dv)
    scratch = torch.empty(int(plan.info.bwd_scratch_bytes) // 4 + 64, dtype=torch.float32,
                          device=dev)
    thd.attn_bwd_parts(plan, ql, k, v, o, lse, dol, dq2, dk2, dv2, scratch)
    torch.cuda.synchronize()
    assert n > 0
    # delta is summed in another order by the separate preprocess launch
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.allclose(a, b, rtol=0, atol=1e-4 * max(float(a.abs().max()), 1.0))


def test_split_auto_long_document_full_size():
    # one 16384-token document over 4 heads: the plan splits its longer walks
    # on its own; sampled rows against the oracle, the whole output against
    # the unsplit plan, and the per-head invariants sum dV = sum dO, sum dK = 0
    w = W.custom("doc16k_h4", [16384], [16384], None, 4, 128, 1, 0, "no_load_balance")
    t = W.bf16_tensors(w)
    split = run_share(w, 0, t)
    whole = run_share(w, 0, t, max_key_splits=1)
    assert split["plan"].info.fwd_tile_rows == 256
    assert split["plan"].info.n_split_tiles == 32
    assert whole["plan"].info.n_split_tiles == 0
    rng = np.random.default_rng(11)
    rows = sorted(set(rng.choice(w.T, size=48, replace=False).tolist()) | {0, w.T - 1})
    t64 = {n: t[n].double().numpy() for n in t}
    ref = oracle_share(w, 0, t64, rows=rows)
    assert_close(split["o"][rows], ref["o"][rows], "doc16k O[rows]")
    assert_lse(split["lse"][:, rows], ref["lse"][:, rows], "doc16k LSE[rows]")
    assert_close(split["dq"][rows], ref["dq"][rows], "doc16k dQ[rows]")
    assert np.abs(split["o"] - whole["o"]).max() <= 2 ** -6
    for n in ("dq", "dk", "dv"):
        _, rel = err(split[n], whole[n])
        assert rel <= 1e-3, (n, rel)
    sv = split["dv"].astype(np.float64).sum(axis=0)
    _, rel = err(sv, t64["do"].sum(axis=0))
    assert rel < 5e-3, rel
    sk = split["dk"].astype(np.float64).sum(axis=0)
    assert np.linalg.norm(sk) < 0.05 * np.linalg.norm(split["dk"])
