"""Whole-tensor parity at full size: every element of O, LSE, dQ, dK and dV
of the HIP path against the fp64 oracle, in the launch configuration the
benchmark times (rank-major K/V as the all-gather delivers them, the restore
and unrestore fused into the kernels, gated tail zeroing, two-launch
backward).

"[PyTorch] Add no-load-balance THD all-gather CP" ("Validation") validates
full forward and backward passes of both strategies; here that is done per
rank share against the oracle:

- the named-rank shares of dcs_8k, nlb_32k and pad_131k, and rank 0 of the
  two DUAL_CHUNK_SWAP workloads (the rank that holds their padding rows);
- flat_75k (one 75600-token document, 5 heads): every row and key of head 0,
  so the dK/dV of keys whose query walks span the whole document (up to ~2,400
  blocks of 32 queries) are compared element by element;
- one 32768-token document with 2 heads (walks of ~1,000 query blocks);
- every rank of dcs_8k with its dK/dV partial added on the device
  (accumulate_dkv) into one buffer, against the oracle's cp_size = 1 run.

Bar: max-abs 2e-2 and relative-L2 5e-3 per tensor; LSE on real rows, -inf on
padding rows; padding rows and untouched keys exactly 0.
"""
import sys
import time

import numpy as np
import pytest

import oracle as O
import workloads as W
from _parity import (assert_close, assert_lse, device, f64, oracle_share,
                     oracle_share_chunked, run_share)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _progress(label, total_rows, every=40.0):
    """Prints a line at most every ``every`` seconds while the oracle runs."""
    state = {"t": time.time(), "done": 0}

    def tick(_r0):
        state["done"] += 1
        if time.time() - state["t"] > every:
            state["t"] = time.time()
            _say(f"  oracle {label}: {state['done']} chunks done of ~{total_rows // 512 + 1}")
    return tick


def _compare_share(tag, got, ref, cu, cup, T, idx, rank_major_perm=None, heads=slice(None)):
    """Every element of one rank share (global-order oracle dK/dV mapped to
    the layout the kernels wrote)."""
    o, lse, dq = got["o"][:, heads], got["lse"][heads], got["dq"][:, heads]
    dk, dv = got["dk"][:, heads], got["dv"][:, heads]
    rk, rv = ref["dk"], ref["dv"]
    if rank_major_perm is not None:
        rk, rv = rk[rank_major_perm], rv[rank_major_perm]
    for name, x in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert np.all(np.isfinite(x)), f"{tag} {name}: non-finite values"
    assert_close(o, ref["o"], f"{tag} O whole")
    assert_lse(lse, ref["lse"], f"{tag} LSE whole")
    assert_close(dq, ref["dq"], f"{tag} dQ whole")
    assert_close(dk, rk, f"{tag} dK whole")
    assert_close(dv, rv, f"{tag} dV whole")
    # padding rows and untouched keys: exactly 0
    doc, pos, valid = O.token_table(cu, cup, T)
    pad_rows = ~valid[idx]
    assert np.all(o[pad_rows] == 0) and np.all(dq[pad_rows] == 0), f"{tag} padding rows"
    touched = O.touched_keys(cu, cup, T, idx)
    if rank_major_perm is not None:
        touched = touched[rank_major_perm]
    assert np.all(dk[~touched] == 0) and np.all(dv[~touched] == 0), f"{tag} untouched keys"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,rank", [("dcs_8k", 1), ("dcs_8k", 0), ("nlb_32k", 2),
                                       ("pad_131k", 3), ("pad_131k", 0)])
def test_whole_share_bench_config(name, rank):
    w = W.WORKLOADS[name]
    _say("whole share", name, "rank", rank)
    t = W.bf16_tensors(w)
    got = run_share(w, rank, t, kv_layout="rank_major")
    got["plan"].close()
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    t0 = time.time()
    ref = oracle_share(w, rank, f64(t))
    _say(f"  oracle {time.time() - t0:.1f} s")
    assert np.array_equal(got["idx"], ref["idx"])
    _compare_share(f"{name} r{rank}", got, ref, cu, cup, w.T, ref["idx"],
                   rank_major_perm=got["perm"])


@pytest.mark.timeout(900)
def test_flat_75k_one_head_whole():
    w = W.WORKLOADS["flat_75k"]
    _say("whole head 0 of flat_75k (75600 tokens, 5 heads on the GPU)")
    t = W.bf16_tensors(w)
    got = run_share(w, 0, t, kv_layout="rank_major")
    got["plan"].close()
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    t0 = time.time()
    ref = oracle_share_chunked(w, 0, f64(t), heads=slice(0, 1),
                               progress=_progress("flat_75k head 0", w.T))
    _say(f"  oracle {time.time() - t0:.1f} s")
    _compare_share("flat_75k h0", got, ref, cu, cup, w.T, ref["idx"], heads=slice(0, 1))


@pytest.mark.timeout(900)
def test_one_32k_document_whole():
    w = W.custom("one_doc_32k", (32768,), (32768,), None, 2, 128, 1, 0, "no_load_balance",
                 number=6)
    _say("whole share of one 32768-token document, 2 heads")
    t = W.bf16_tensors(w)
    got = run_share(w, 0, t)
    got["plan"].close()
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    t0 = time.time()
    ref = oracle_share_chunked(w, 0, f64(t), progress=_progress("32k document", w.T))
    _say(f"  oracle {time.time() - t0:.1f} s")
    _compare_share("one_doc_32k", got, ref, cu, cup, w.T, ref["idx"])


@pytest.mark.timeout(900)
def test_all_ranks_accumulated_on_device_equal_cp1():
    """Every rank of dcs_8k in turn on one pair of dK/dV buffers: the first
    rank writes (and zeroes untouched rows), later ranks add their partial on
    the device (accumulate_dkv), which is the reduce of the reduce-scatter.
    The sum, and every rank's O / dQ placed at its global rows, must equal the
    oracle's cp_size = 1 share."""
    w = W.WORKLOADS["dcs_8k"]
    _say("all ranks of dcs_8k accumulated on the device vs cp_size 1")
    t = W.bf16_tensors(w)
    dev = device()
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    cup_dev = torch.from_numpy(cup).to(dev)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    perm = thd.partition_index(cup, cup_dev, w.T, w.cp_size, -1, w.strategy)
    k_rm, v_rm = thd.gather(k, perm), thd.gather(v, perm)
    dk = torch.full((w.T, w.H, w.D), float("nan"), dtype=torch.float32, device=dev)
    dv = torch.full_like(dk, float("nan"))
    o_g = np.zeros((w.T, w.H, w.D))
    dq_g = np.zeros((w.T, w.H, w.D))
    lse_g = np.full((w.H, w.T), -np.inf)
    for r in range(w.cp_size):
        idx = thd.partition_index(cup, cup_dev, w.T, w.cp_size, r, w.strategy)
        ql, dol = thd.gather(q, idx), thd.gather(do, idx)
        plan = thd.Plan(cu, cup, w.T, w.cp_size, r, w.strategy, w.H, w.D,
                        kv_layout="rank_major")
        o, lse = thd.attn_fwd(plan, ql, k_rm, v_rm)
        dq, _, _ = thd.attn_bwd(plan, ql, k_rm, v_rm, o, lse, dol, dk=dk, dv=dv,
                                zero_untouched=(r == 0), accumulate_dkv=(r > 0))
        torch.cuda.synchronize()
        ii = idx.cpu().numpy()
        o_g[ii] = o.float().cpu().numpy()
        dq_g[ii] = dq.cpu().numpy()
        lse_g[:, ii] = lse.cpu().numpy()
        plan.close()
    pm = perm.cpu().numpy()
    dk_g = np.empty((w.T, w.H, w.D))
    dv_g = np.empty((w.T, w.H, w.D))
    dk_g[pm] = dk.cpu().numpy()   # rank-major position p holds global row pm[p]
    dv_g[pm] = dv.cpu().numpy()
    w1 = W.custom("dcs_8k_cp1", w.lengths, w.padded, w.T, w.H, w.D, 1, 0, "no_load_balance",
                  number=w.number)
    t0 = time.time()
    ref = oracle_share(w1, 0, f64(t))
    _say(f"  oracle {time.time() - t0:.1f} s")
    assert_close(o_g, ref["o"], "dcs_8k union O")
    assert_lse(lse_g, ref["lse"], "dcs_8k union LSE")
    assert_close(dq_g, ref["dq"], "dcs_8k union dQ")
    assert_close(dk_g, ref["dk"], "dcs_8k union dK (on-device sum)")
    assert_close(dv_g, ref["dv"], "dcs_8k union dV (on-device sum)")
