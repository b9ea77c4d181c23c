"""cp_attn_bwd_noalloc (scratch in the library's fixed device array) gives
exactly what cp_attn_bwd (scratch from the caller) gives, through the C ABI:
two calls in a row on one GPU, the second on a smaller input, so the second
reuses the array the first left behind."""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _pair(w, rank, kv_layout, accumulate):
    dev = torch.device("cuda", 0)
    t = W.bf16_tensors(w)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    cup_dev = torch.from_numpy(cup).to(dev)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    idx = thd.partition_index(cup, cup_dev, w.T, w.cp_size, rank, w.strategy)
    ql, dol = thd.gather(q, idx), thd.gather(do, idx)
    if kv_layout == "rank_major":
        perm = thd.partition_index(cup, cup_dev, w.T, w.cp_size, -1, w.strategy)
        k, v = thd.gather(k, perm), thd.gather(v, perm)
    plan = thd.Plan(cu, cup, w.T, w.cp_size, rank, w.strategy, w.H, w.D, kv_layout=kv_layout)
    o, lse = thd.attn_fwd(plan, ql, k, v)
    n, H, D, T = plan.n_local, w.H, w.D, w.T
    g = torch.Generator(device=dev).manual_seed(3)
    init = torch.randn((T, H, D), generator=g, device=dev)
    outs = []
    for which in ("caller scratch", "no alloc"):
        dq = torch.full((n, H, D), float("nan"), device=dev)
        dk = init.clone() if accumulate else torch.full((T, H, D), float("nan"), device=dev)
        dv = init.clone() if accumulate else torch.full((T, H, D), float("nan"), device=dev)
        if which == "caller scratch":
            thd.attn_bwd(plan, ql, k, v, o, lse, dol, dq=dq, dk=dk, dv=dv,
                         zero_untouched=not accumulate, accumulate_dkv=accumulate)
        else:
            thd.attn_bwd_noalloc(plan, ql, k, v, o, lse, dol, dq, dk, dv,
                                 zero_untouched=not accumulate, accumulate_dkv=accumulate)
        torch.cuda.synchronize()
        outs.append((dq, dk, dv))
    for name, a, b in zip(("dQ", "dK", "dV"), outs[0], outs[1]):
        assert torch.isfinite(b).all(), f"{w.name} {name}: rows left unwritten"
        assert torch.equal(a, b), f"{w.name} {name}: differs from cp_attn_bwd"
    plan.close()


def test_noalloc_equals_cp_attn_bwd_two_calls():
    # 1) the dcs_8k share in the benchmark's layout (n_local * H = 65,536)
    w1 = W.WORKLOADS["dcs_8k"]
    _say("no-alloc backward, call 1: dcs_8k rank 1, rank-major K/V")
    _pair(w1, 1, "rank_major", accumulate=False)
    # 2) a smaller share (n_local * H = 1,200) right after, adding into
    #    existing partials: the array keeps the first call's values, which
    #    the second must not read
    w2 = W.custom("noalloc_small", (250, 0, 180, 90), (256, 0, 184, 160), None, 3, 64, 2, 0,
                  "dual_chunk_swap", number=8)
    _say("no-alloc backward, call 2: a 600-token padded share, D = 64, accumulate")
    _pair(w2, 0, "global", accumulate=True)
