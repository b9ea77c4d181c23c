"""GPU parity of dense bshd / sbhd batches through their THD views.

Flat a2a is tested over bshd, sbhd and THD ("[PyTorch] Extend no-load-balance
CP to the a2a comm type", PR body). The library takes a dense batch as a THD
view with no copy (sbhd: one document of S tokens with B*H heads; bshd: B
documents of S tokens); the oracle defines the dense rank share directly, per
batch element. Compared element by element (max-abs 2e-2, rel-L2 5e-3), every
rank, both strategies, including S divisible by cp_size but not 2*cp_size;
at full size an sbhd batch is bit-identical to its batch elements run one by
one as single-document THD shares.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W
from _parity import assert_close, assert_lse, device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_dense(layout, B, S, H, D, cp, rank, strategy, t, window=(-1, 0), max_key_splits=0):
    """Product path for one rank of a dense batch; outputs batch-major like
    the oracle's: O/dQ [B, n, H, D], LSE [B, H, n], dK/dV [B, S, H, D]."""
    dev = device()
    plan = thd.dense_plan(layout, B, S, H, D, cp, rank, strategy, window=window,
                          max_key_splits=max_key_splits)
    cu, heads = thd.dense_as_thd(layout, B, S, H)
    T = int(cu[-1])
    q, k, v, do = (thd.dense_view(t[n].to(dev), layout) for n in ("q", "k", "v", "do"))
    cu_dev = torch.from_numpy(cu).to(dev)
    idx = thd.partition_index(cu, cu_dev, T, cp, rank, strategy)
    ql, dol = thd.gather(q, idx), thd.gather(do, idx)
    o, lse = thd.attn_fwd(plan, ql, k, v)
    dq, dk, dv = thd.attn_bwd(plan, ql, k, v, o, lse, dol)
    torch.cuda.synchronize()
    n = plan.n_local
    o, dq, dk, dv = (x.float().cpu().numpy() for x in (o, dq, dk, dv))
    lse = lse.cpu().numpy()
    if layout == "sbhd":
        o = o.reshape(n, B, H, D).transpose(1, 0, 2, 3)
        dq = dq.reshape(n, B, H, D).transpose(1, 0, 2, 3)
        dk = dk.reshape(S, B, H, D).transpose(1, 0, 2, 3)
        dv = dv.reshape(S, B, H, D).transpose(1, 0, 2, 3)
        lse = lse.reshape(B, H, n)
    else:
        nb = n // B
        o, dq = o.reshape(B, nb, H, D), dq.reshape(B, nb, H, D)
        dk, dv = dk.reshape(B, S, H, D), dv.reshape(B, S, H, D)
        lse = lse.reshape(H, B, nb).transpose(1, 0, 2)
    return idx.cpu().numpy(), o, lse, dq, dk, dv


CASES = [
    ("sbhd", 3, 520, 2, 128, 2, "dual_chunk_swap", (-1, 0)),
    ("sbhd", 2, 390, 3, 64, 3, "no_load_balance", (-1, 0)),
    ("sbhd", 2, 202, 2, 128, 2, "no_load_balance", (-1, -1)),   # S % 2cp != 0
    ("sbhd", 4, 256, 1, 128, 1, "no_load_balance", (100, 0)),
    ("bshd", 3, 416, 2, 128, 2, "dual_chunk_swap", (-1, 0)),
    ("bshd", 2, 256, 2, 64, 4, "dual_chunk_swap", (50, 50)),
    ("bshd", 1, 333, 2, 128, 3, "no_load_balance", (-1, 0)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) for x in c[:7]) +
                         f"-w{c[7][0]}_{c[7][1]}")
def test_dense_layout_elementwise_all_ranks(case):
    layout, B, S, H, D, cp, strategy, window = case
    t = W.dense_bf16(layout, B, S, H, D, seed=7000)
    t64 = {n: x.double().numpy() for n, x in t.items()}
    for r in range(cp):
        _say("dense", layout, B, S, H, D, cp, strategy, window, "rank", r)
        pos, o, lse, dq, dk, dv = O.dense_rank_share(t64["q"], t64["k"], t64["v"], t64["do"],
                                                     layout, cp, r, strategy, window=window)
        idx, go, glse, gdq, gdk, gdv = run_dense(layout, B, S, H, D, cp, r, strategy, t, window)
        tag = f"{layout} r{r}"
        # the view's local rows are the sequence shard (sbhd), or the shard of
        # every batch element, batch-major (bshd)
        if layout == "sbhd":
            assert idx.tolist() == pos.tolist()
        else:
            assert idx.tolist() == [b * S + p for b in range(B) for p in pos.tolist()]
        assert_close(go, o, tag + " O")
        assert_lse(glse, lse, tag + " LSE")
        assert_close(gdq, dq, tag + " dQ")
        assert_close(gdk, dk, tag + " dK")
        assert_close(gdv, dv, tag + " dV")


def test_dense_bshd_nlb_batch_refused():
    with pytest.raises(ValueError):
        thd.dense_plan("bshd", 2, 64, 1, 64, 2, 0, "no_load_balance", upload=False)


@pytest.mark.parametrize("cp,strategy", [(1, "no_load_balance"), (2, "no_load_balance"),
                                         (2, "dual_chunk_swap")])
def test_sbhd_full_size_equals_per_batch_element(cp, strategy):
    """sbhd [8192, 4, 5, 128] (the flat post-a2a share of 40 heads over 8
    ranks, four sequences): bit-identical to each sequence run alone as a
    single-document THD share with 5 heads, given the same key walks (the
    automatic walk split depends on the launch's head count, so both sides
    take max_key_splits = 1)."""
    layout, B, S, H, D = "sbhd", 4, 8192, 5, 128
    _say("sbhd full size", cp, strategy)
    t = W.dense_bf16(layout, B, S, H, D, seed=7100)
    r = cp - 1
    _, o, lse, dq, dk, dv = run_dense(layout, B, S, H, D, cp, r, strategy, t, max_key_splits=1)
    for b in range(B):
        tb = {n: x[:, b].contiguous() for n, x in t.items()}
        _, o1, l1, dq1, dk1, dv1 = run_dense("bshd", 1, S, H, D, cp, r, strategy,
                                             {n: x[None] for n, x in tb.items()},
                                             max_key_splits=1)
        for a, c, n in ((o[b], o1[0], "O"), (lse[b], l1[0], "LSE"), (dq[b], dq1[0], "dQ"),
                        (dk[b], dk1[0], "dK"), (dv[b], dv1[0], "dV")):
            assert np.array_equal(a, c), (b, n)


@pytest.mark.parametrize("strategy", ["no_load_balance", "dual_chunk_swap"])
def test_sbhd_a2a_exchange_then_attention(strategy):
    """The a2a around an sbhd batch: heads split per batch element, so the
    exchange runs on the [S*B, H, D] row view (one document of S*B rows, whose
    dual chunks are whole S positions); attention then runs on the received
    head group's [S, B*H/cp, D] view. Rank r's received tensor must be the
    head slice r of every batch element, bit for bit, and its attention the
    oracle's per-batch-element attention of that slice."""
    from _parity import a2a_round_trip
    S, B, H, D, cp = 1024, 3, 8, 128, 4
    hl = H // cp
    t = W.dense_bf16("sbhd", B, S, H, D, seed=7200)
    x = t["q"].to(device())
    full = a2a_round_trip([0, S * B], S * B, cp, H, strategy, [x.view(S * B, H, D)])
    for r in range(cp):
        assert torch.equal(full[0][r].view(S, B, hl, D), x[:, :, r * hl:(r + 1) * hl])
    # attention of rank 1's head group on the exchanged q (k, v, do sliced the
    # same way), cp_size 1 math after the exchange
    r = 1
    sl = {n: y[:, :, r * hl:(r + 1) * hl].contiguous() for n, y in t.items()}
    sl["q"] = full[0][r].view(S, B, hl, D).cpu()
    t64 = {n: y.double().numpy() for n, y in sl.items()}
    pos, o, lse, dq, dk, dv = O.dense_rank_share(t64["q"], t64["k"], t64["v"], t64["do"],
                                                 "sbhd", 1, 0, "no_load_balance")
    _, go, glse, gdq, gdk, gdv = run_dense("sbhd", B, S, hl, D, 1, 0, "no_load_balance", sl)
    assert_close(go, o, "sbhd a2a O")
    assert_lse(glse, lse, "sbhd a2a LSE")
    assert_close(gdq, dq, "sbhd a2a dQ")
    assert_close(gdk, dk, "sbhd a2a dK")
    assert_close(gdv, dv, "sbhd a2a dV")
