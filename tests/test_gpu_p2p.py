"""GPU parity of the P2P (ring) steps against the fp64 oracle.

Under P2P context parallelism ("[PyTorch][Attention] THD P2P context-parallel
regression ...", "Describe the bug") a rank's attention runs as one step per
peer's K/V, merged through the log-sum-exp. Each step's forward (O_part,
LSE_part), the merge, each step's backward (dQ accumulated, dK/dV of the
source rank's rows) and the merged result are compared with the oracle's
step definitions, element by element on small layouts (every rank, every
step), and on sampled rows at full size plus against the all-gather path.
Bar: max-abs 2e-2 and relative-L2 5e-3 per tensor, as everywhere; rows with
no key in a step must be exactly O = 0, LSE = -inf; gradient rows no local
query reaches must be exactly 0 (or untouched when the gate is off).
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W
from _parity import (assert_close, assert_lse, device, f64, oracle_share, run_share,
                     sample_plan)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = [
    W.custom("p2p_dcs_pad_d128", [200, 1, 513, 77], [208, 8, 520, 80], None, 2, 128, 2, 0,
             "dual_chunk_swap"),
    W.custom("p2p_dcs_cp4_d64", [129, 3, 700, 64], [136, 8, 704, 64], None, 2, 64, 4, 0,
             "dual_chunk_swap"),
    W.custom("p2p_nlb_tail_d128", [250, 5, 900, 333], [256, 5, 900, 340], 1548, 2, 128, 3, 0,
             "no_load_balance"),
    W.custom("p2p_nlb_nopad_d64", [37, 91, 200, 2], [37, 91, 200, 2], None, 2, 64, 3, 0,
             "no_load_balance"),
]


def run_p2p(w, rank, tensors, fill=None, zero_untouched=True, keep_steps=True, merge="stepwise"):
    """The ring on one GPU for one rank: every peer's local K/V is gathered
    (what the ring delivers), then forward steps + merge (after every step
    into an fp32 accumulator, or merge="parts": all steps at once), delta of
    the merged output, backward steps. Returns numpy arrays (per-step ones in
    the source rank's local order) and the global-order sums of dK/dV."""
    dev = device()
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    cp = w.cp_size
    cup_dev = torch.from_numpy(cup).to(dev)
    q, k, v, do = (tensors[n].to(dev) for n in ("q", "k", "v", "do"))
    idxs = [thd.partition_index(cup, cup_dev, w.T, cp, s, w.strategy) for s in range(cp)]
    ql, dol = thd.gather(q, idxs[rank]), thd.gather(do, idxs[rank])
    kl = [thd.gather(k, i) for i in idxs]
    vl = [thd.gather(v, i) for i in idxs]
    plan = thd.Plan(cu, cup, w.T, cp, rank, w.strategy, w.H, w.D, p2p=True)
    n, H, D = plan.n_local, w.H, w.D
    o_acc = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    lse_acc = torch.empty((H, n), dtype=torch.float32, device=dev)
    o = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    o_parts = torch.empty((cp, n, H, D), dtype=torch.bfloat16, device=dev)
    lse_parts = torch.empty((cp, H, n), dtype=torch.float32, device=dev)
    fwd_steps = []
    for i in range(cp):
        src = O.p2p_source(rank, i, cp)
        op, lp = thd.attn_fwd_step(plan, src, ql, kl[src], vl[src], o_part=o_parts[i],
                                   lse_part=lse_parts[i])
        if keep_steps:
            fwd_steps.append((src, op.float().cpu().numpy(), lp.cpu().numpy()))
        if merge == "stepwise":
            thd.lse_merge(op, lp, o_acc, lse_acc, first=(i == 0),
                          o_out=o if i == cp - 1 else None)
    if merge == "parts":
        thd.lse_merge_parts(o_parts, lse_parts, o_out=o, lse_out=lse_acc)
        o_acc.copy_(o.float())
    scratch = torch.empty(max(int(plan.info.bwd_scratch_bytes), 256), dtype=torch.uint8,
                          device=dev)
    thd.bwd_preprocess(plan, o, lse_acc, dol, scratch)
    dq = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    bwd_steps = []
    dk = np.zeros((w.T, H, D), dtype=np.float64)
    dv = np.zeros((w.T, H, D), dtype=np.float64)
    for i in range(cp):
        src = O.p2p_source(rank, i, cp)
        dk_s = dv_s = None
        if fill is not None:
            dk_s = torch.full((n, H, D), fill, dtype=torch.float32, device=dev)
            dv_s = dk_s.clone()
        _, dk_s, dv_s = thd.attn_bwd_step(plan, src, ql, kl[src], vl[src], lse_acc, dol, scratch,
                                          dq, accumulate_dq=(i > 0), dk_src=dk_s, dv_src=dv_s,
                                          zero_untouched=zero_untouched)
        a, b = dk_s.cpu().numpy(), dv_s.cpu().numpy()
        if keep_steps:
            bwd_steps.append((src, dq.cpu().numpy(), a, b))
        gi = idxs[src].cpu().numpy()
        dk[gi] += a
        dv[gi] += b
    torch.cuda.synchronize()
    return dict(idx=idxs[rank].cpu().numpy(), idxs=[x.cpu().numpy() for x in idxs],
                o=o.float().cpu().numpy(), o_acc=o_acc.cpu().numpy(), lse=lse_acc.cpu().numpy(),
                dq=dq.cpu().numpy(), dk=dk, dv=dv, fwd_steps=fwd_steps, bwd_steps=bwd_steps,
                plan=plan)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_p2p_steps_elementwise_all_ranks(w):
    t = W.bf16_tensors(w)
    t64 = f64(t)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    _, _, valid = O.token_table(cu, cup, w.T)
    owner = O.owner_ranks(cup, w.T, w.cp_size, w.strategy)
    for r in range(w.cp_size):
        _say("p2p", w.name, "rank", r)
        got = run_p2p(w, r, t, fill=float("nan"))
        idx = got["idx"]
        ql, dol = t64["q"][idx], t64["do"][idx]
        o_ref, lse_ref = O.attention_fwd(ql, t64["k"], t64["v"], idx, cu, cup, w.T)
        delta = np.einsum("nhd,nhd->hn", o_ref, dol)
        touched = O.touched_keys(cu, cup, w.T, idx)
        dq_ref = np.zeros_like(ql)
        for (src, op, lp), (src_b, dq_got, dk_got, dv_got) in zip(got["fwd_steps"],
                                                                  got["bwd_steps"]):
            assert src == src_b
            tag = f"{w.name} r{r} src{src}"
            ok = owner == src
            op_ref, lp_ref = O.attention_fwd_keys(ql, t64["k"], t64["v"], idx, cu, cup, w.T, ok)
            empty = np.isneginf(lp_ref)
            assert np.all(np.isneginf(lp[empty])), tag + " LSE_part -inf rows"
            assert np.all(op.transpose(1, 0, 2)[empty] == 0), tag + " O_part empty rows"
            if (~empty).any():
                assert_close(op.transpose(1, 0, 2)[~empty], op_ref.transpose(1, 0, 2)[~empty],
                             tag + " O_part")
                assert_lse(lp, lp_ref, tag + " LSE_part")
            a, b, c = O.attention_bwd_keys(ql, t64["k"], t64["v"], dol, idx, cu, cup, w.T, ok,
                                           lse_ref, delta)
            dq_ref = dq_ref + a
            assert_close(dq_got, dq_ref, tag + " dQ (accumulated)")
            gi = got["idxs"][src]
            assert np.all(np.isfinite(dk_got)) and np.all(np.isfinite(dv_got)), tag
            assert_close(dk_got, b[gi], tag + " dK_src")
            assert_close(dv_got, c[gi], tag + " dV_src")
            # rows of rank src that no local query attends are exactly zero
            unt = ~touched[gi]
            assert np.all(dk_got[unt] == 0) and np.all(dv_got[unt] == 0), tag
        # merged result against the whole-key-set attention
        assert_close(got["o"], o_ref, f"{w.name} r{r} merged O")
        assert_close(got["o_acc"], o_ref, f"{w.name} r{r} merged O (fp32)")
        assert_lse(got["lse"], lse_ref, f"{w.name} r{r} merged LSE")
        pad_local = ~valid[idx]
        assert np.all(got["o"][pad_local] == 0) and np.all(got["dq"][pad_local] == 0)
        dq1, dk1, dv1 = O.attention_bwd(ql, t64["k"], t64["v"], dol, idx, cu, cup, w.T)
        assert_close(got["dq"], dq1, f"{w.name} r{r} dQ")
        assert_close(got["dk"], dk1, f"{w.name} r{r} dK (summed steps)")
        assert_close(got["dv"], dv1, f"{w.name} r{r} dV (summed steps)")
        # the same ring with all steps merged at once
        par = run_p2p(w, r, t, keep_steps=False, merge="parts")
        assert_close(par["o"], o_ref, f"{w.name} r{r} one-pass merged O")
        assert_lse(par["lse"], lse_ref, f"{w.name} r{r} one-pass merged LSE")
        assert np.all(par["o"][pad_local] == 0)
        for nm, ref_ in (("dq", dq1), ("dk", dk1), ("dv", dv1)):
            assert_close(par[nm], ref_, f"{w.name} r{r} one-pass {nm}")


def test_p2p_zero_gate_and_determinism():
    w = SMALL[0]
    t = W.bf16_tensors(w)
    r = 1
    a = run_p2p(w, r, t, fill=7.0, zero_untouched=False)
    b = run_p2p(w, r, t, fill=7.0, zero_untouched=True)
    c = run_p2p(w, r, t, fill=7.0, zero_untouched=True)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    touched = O.touched_keys(cu, cup, w.T, a["idx"])
    some_untouched = False
    for (src, _, ka, va), (_, _, kb, vb), (_, _, kc, vc) in zip(a["bwd_steps"], b["bwd_steps"],
                                                                c["bwd_steps"]):
        tch = touched[a["idxs"][src]]
        some_untouched |= bool((~tch).any())
        assert np.all(ka[~tch] == 7.0) and np.all(va[~tch] == 7.0)
        assert np.all(kb[~tch] == 0) and np.all(vb[~tch] == 0)
        assert np.array_equal(ka[tch], kb[tch]) and np.array_equal(va[tch], vb[tch])
        assert np.array_equal(kb, kc) and np.array_equal(vb, vc)  # no atomics: bit-identical
    assert some_untouched
    for n in ("o", "lse", "dq"):
        assert np.array_equal(b[n], c[n]), n


def _random_parts(rng, n, H, D, steps):
    """Step results with rows empty in some steps and in every step."""
    parts = []
    for s in range(steps):
        o = torch.from_numpy(rng.standard_normal((n, H, D))).to(torch.bfloat16)
        lse = rng.standard_normal((H, n)) * 4
        lse[rng.random((H, n)) < 0.3] = -np.inf   # rows with no key in this step
        lse[:, :7] = -np.inf                      # rows with no key in any step
        o_np = o.double().numpy()
        o_np[np.isneginf(lse).T] = 0.0
        o = torch.from_numpy(o_np).to(torch.bfloat16)
        parts.append((o, torch.from_numpy(lse).float()))
    return parts


@pytest.mark.parametrize("D,steps", [(128, 4), (64, 8), (128, 1)])
def test_lse_merge_parts_kernel_vs_oracle(D, steps):
    # all steps merged at once; the oracle's merge is the log-sum-exp over
    # parts written out (pinned on the CPU against pairwise and closed forms)
    dev = device()
    parts = _random_parts(np.random.default_rng(5 + steps), 263, 3, D, steps)
    o_parts = torch.stack([o for o, _ in parts]).to(dev)
    lse_parts = torch.stack([l for _, l in parts]).to(dev)
    o_out, lse_out = thd.lse_merge_parts(o_parts, lse_parts)
    o2, l2 = thd.lse_merge_parts(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert torch.equal(o_out, o2) and torch.equal(lse_out, l2)   # fixed summation order
    ref_o, ref_l = O.lse_merge([(o.double().numpy(), l.double().numpy()) for o, l in parts])
    got_l = lse_out.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(got_l[fin] - ref_l[fin]).max() < 1e-5
    got_o = o_out.float().cpu().numpy()
    assert np.all(got_o[:7] == 0)
    assert np.abs(got_o - ref_o).max() <= 2 ** -7 * np.abs(ref_o).max()
    if steps == 1:   # one part: weight 1, the part itself
        assert torch.equal(o_out.cpu(), parts[0][0])
        assert torch.equal(lse_out.cpu(), parts[0][1])


def test_lse_merge_kernel_vs_oracle():
    dev = device()
    rng = np.random.default_rng(3)
    n, H, D, steps = 301, 3, 128, 4
    parts = []
    for s in range(steps):
        o = torch.from_numpy(rng.standard_normal((n, H, D))).to(torch.bfloat16)
        lse = rng.standard_normal((H, n)) * 4
        lse[rng.random((H, n)) < 0.3] = -np.inf   # rows with no key in this step
        lse[:, :7] = -np.inf                      # rows with no key in any step
        o_np = o.double().numpy()
        o_np[np.isneginf(lse).T] = 0.0
        o = torch.from_numpy(o_np).to(torch.bfloat16)
        parts.append((o, torch.from_numpy(lse).float()))
    o_acc = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    lse_acc = torch.empty((H, n), dtype=torch.float32, device=dev)
    o_out = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    for s, (o, l) in enumerate(parts):
        thd.lse_merge(o.to(dev), l.to(dev), o_acc, lse_acc, first=(s == 0),
                      o_out=o_out if s == steps - 1 else None)
    torch.cuda.synchronize()
    ref_o, ref_l = O.lse_merge([(o.double().numpy(), l.double().numpy()) for o, l in parts])
    got_l = lse_acc.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(got_l[fin] - ref_l[fin]).max() < 1e-5
    assert np.abs(o_acc.cpu().numpy() - ref_o).max() < 1e-5
    assert np.all(o_acc.cpu().numpy()[:7] == 0)
    assert np.abs(o_out.float().cpu().numpy() - ref_o).max() <= 2 ** -7 * np.abs(ref_o).max()


@pytest.mark.parametrize("name", ["dcs_8k", "nlb_32k", "pad_131k"])
def test_p2p_full_size(name):
    """The ring at full size for the workload's rank: sampled rows against the
    oracle, and every element against the all-gather path of the same rank."""
    w = W.WORKLOADS[name]
    _say("p2p full-size", name)
    t = W.bf16_tensors(w)
    got = run_p2p(w, w.rank, t, fill=float("nan"), keep_steps=False, merge="parts")
    ag = run_share(w, w.rank, t)
    assert np.array_equal(got["idx"], ag["idx"])
    for n in ("o", "dq", "dk", "dv"):
        assert np.all(np.isfinite(got[n])), n
        assert_close(got[n], ag[n], f"{name} p2p vs all-gather {n}")
    assert_lse(got["lse"], ag["lse"], f"{name} p2p vs all-gather LSE")
    t64 = {n: t[n].double().numpy() for n in t}
    rows, keys = sample_plan(w, w.rank, np.random.default_rng(2))
    ref = oracle_share(w, w.rank, t64, rows=rows)
    assert_close(got["o"][rows], ref["o"][rows], f"{name} p2p O[rows]")
    assert_lse(got["lse"][:, rows], ref["lse"][:, rows], f"{name} p2p LSE[rows]")
    assert_close(got["dq"][rows], ref["dq"][rows], f"{name} p2p dQ[rows]")
    assert_close(got["dk"][keys], ref["dk"][keys], f"{name} p2p dK[keys]")
    assert_close(got["dv"][keys], ref["dv"][keys], f"{name} p2p dV[keys]")
