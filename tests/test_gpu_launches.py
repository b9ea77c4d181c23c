"""Launch counts of the hot path, recorded by the PyTorch profiler.

"[PyTorch][Attention] THD P2P context-parallel regression when padded
cu_seqlens are value-equal but not object-identical" ("Describe the bug",
"Expected behavior") traces the regression to launches: an identity test on
cu_seqlens_padded sent a value-equal copy down the padded path, which added
per-step sequence-length helper launches and tail-zeroing launches. Here the
padding decision is by value and every per-step table comes from the plan, so:

- a value-equal copy of cu_seqlens_padded, the same array, and an omitted
  cu_seqlens give the same kernel list, launch for launch;
- the all-gather forward + backward is exactly three attention launches
  (forward; dQ carrying delta and the gated zeroing; dK/dV);
- the separate zeroing call launches only when the plan has untouched rows;
- a P2P ring of cp steps is cp forward steps, one merge, one delta launch and
  per step at most one dQ and one dK/dV launch, the same for both arrays.
"""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")

OURS = ("attn_", "move_rows", "partition", "zero_rows", "copy16", "lse_merge", "bwd_prep")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _launches(fn):
    """Names of this library's kernels launched by fn(), in order."""
    from torch.autograd import DeviceType
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    ev = [e for e in prof.events() if e.device_type == DeviceType.CUDA]
    ev.sort(key=lambda e: e.time_range.start)
    return [e.name for e in ev if any(k in e.name for k in OURS)]


def _short(names):
    out = []
    for n in names:
        for k in ("attn_fwd_kernel", "attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel",
                  "lse_merge_parts_kernel", "lse_merge_kernel", "bwd_prep_kernel",
                  "zero_rows_kernel", "move_rows_kernel", "partition_kernel", "copy16_kernel"):
            if k in n:
                out.append(k)
                break
    return out


def _tensors(w, dev):
    t = W.bf16_tensors(w)
    return [t[n].to(dev) for n in ("q", "k", "v", "do")]


def _allgather_step(w, cu_arg, cup_arg, tensors):
    q, k, v, do = tensors
    dev = q.device
    cup = w.cu_seqlens_padded()
    cup_dev = torch.from_numpy(cup).to(dev)
    idx = thd.partition_index(cup, cup_dev, w.T, w.cp_size, w.rank, w.strategy)
    ql, dol = thd.gather(q, idx), thd.gather(do, idx)
    plan = thd.Plan(cu_arg, cup_arg, w.T, w.cp_size, w.rank, w.strategy, w.H, w.D)
    torch.cuda.synchronize()

    def run():
        o, lse = thd.attn_fwd(plan, ql, k, v)
        thd.attn_bwd(plan, ql, k, v, o, lse, dol)
    return plan, run


def test_value_equal_copy_same_launches_allgather():
    # nlb_32k's rank 2: cu_seqlens_padded holds the same values as cu_seqlens
    w = W.WORKLOADS["nlb_32k"]
    dev = torch.device("cuda", 0)
    tensors = _tensors(w, dev)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    runs = {}
    for tag, a, b in (("copy", cu, cup.copy()), ("same", cup, cup), ("omitted", None, cup)):
        if tag != "copy" and not np.array_equal(cu, cup):
            continue   # the same-array forms only describe layouts without padding
        plan, run = _allgather_step(w, a, b, tensors)
        run()   # first launches set per-device attributes; record a later one
        runs[tag] = _short(_launches(run))
        _say(tag, runs[tag])
    first = next(iter(runs.values()))
    assert first == ["attn_fwd_kernel", "attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel"]
    for v in runs.values():
        assert v == first


def test_value_equal_copy_same_launches_no_padding():
    # one layout without padding, where cu_seqlens and cu_seqlens_padded are
    # equal: a copy, the same array and an omitted cu_seqlens launch alike
    w = W.custom("launch_nopad", [37, 91, 200, 2], [37, 91, 200, 2], None, 2, 64, 2, 1,
                 "no_load_balance")
    dev = torch.device("cuda", 0)
    tensors = _tensors(w, dev)
    cup = w.cu_seqlens_padded()
    runs = []
    for a, b in ((cup.copy(), cup), (cup, cup), (None, cup)):
        plan, run = _allgather_step(w, a, b, tensors)
        assert plan.info.padding_present == 0
        run()
        runs.append(_short(_launches(run)))
    assert runs[0] == runs[1] == runs[2]
    assert runs[0] == ["attn_fwd_kernel", "attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel"]


def test_zeroing_launch_gated():
    dev = torch.device("cuda", 0)
    for name, expect in (("flat_75k", 0), ("dcs_8k", 1)):
        w = W.WORKLOADS[name]
        plan = thd.Plan(w.cu_seqlens(), w.cu_seqlens_padded(), w.T, w.cp_size, w.rank,
                        w.strategy, w.H, w.D)
        assert (plan.info.untouched_rows > 0) == (expect == 1)
        dk = torch.zeros((w.T, w.H, w.D), dtype=torch.float32, device=dev)
        dv = torch.zeros_like(dk)
        names = _short(_launches(
            lambda: thd.lib().thdcp_zero_untouched(plan.handle, thd._dev_ptr(dk, "dk"),
                                                   thd._dev_ptr(dv, "dv"), thd._stream())))
        assert names == ["zero_rows_kernel"] * expect, (name, names)


def test_p2p_ring_launches():
    w = W.custom("launch_p2p", [250, 5, 900, 333], [256, 8, 904, 336], None, 2, 64, 2, 1,
                 "dual_chunk_swap")
    dev = torch.device("cuda", 0)
    q, k, v, do = _tensors(w, dev)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    cp, r = w.cp_size, w.rank
    cup_dev = torch.from_numpy(cup).to(dev)
    idxs = [thd.partition_index(cup, cup_dev, w.T, cp, s, w.strategy) for s in range(cp)]
    ql, dol = thd.gather(q, idxs[r]), thd.gather(do, idxs[r])
    kl = [thd.gather(k, i) for i in idxs]
    vl = [thd.gather(v, i) for i in idxs]
    lists = []
    for cup_arg in (cup.copy(), cup):
        plan = thd.Plan(cu, cup_arg, w.T, cp, r, w.strategy, w.H, w.D, p2p=True)
        n, H, D = plan.n_local, w.H, w.D
        o_parts = torch.empty((cp, n, H, D), dtype=torch.bfloat16, device=dev)
        lse_parts = torch.empty((cp, H, n), dtype=torch.float32, device=dev)
        scratch = torch.empty(int(plan.info.bwd_scratch_bytes) + 256, dtype=torch.uint8,
                              device=dev)
        dq = torch.empty((n, H, D), dtype=torch.float32, device=dev)

        def ring():
            srcs = [(r - i) % cp for i in range(cp)]
            for i, s in enumerate(srcs):
                thd.attn_fwd_step(plan, s, ql, kl[s], vl[s], o_part=o_parts[i],
                                  lse_part=lse_parts[i])
            o, lse = thd.lse_merge_parts(o_parts, lse_parts)
            thd.bwd_preprocess(plan, o, lse, dol, scratch)
            for i, s in enumerate(srcs):
                thd.attn_bwd_step(plan, s, ql, kl[s], vl[s], lse, dol, scratch, dq, i > 0)
        ring()
        lists.append(_short(_launches(ring)))
        _say("p2p launches", lists[-1])
    assert lists[0] == lists[1]
    names = lists[0]
    assert names[:cp] == ["attn_fwd_kernel"] * cp
    assert names[cp:cp + 2] == ["lse_merge_parts_kernel", "bwd_prep_kernel"]
    rest = names[cp + 2:]
    assert set(rest) <= {"attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel"}
    assert 1 <= len(rest) <= 2 * cp
    assert "zero_rows_kernel" not in names and "partition_kernel" not in names
