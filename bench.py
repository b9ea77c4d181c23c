"""Benchmark: one CP rank's share of causal THD attention on one MI355X.

A step is one pass of the whole hot path for the measured rank over one batch:
  validate + build the rank plan (host) and upload it,
  partition index for every rank (the all-ranks permutation),
  gather the rank's local Q and dO,
  attention forward (O, LSE) on K and V as the all-gather delivers them
    (rank-major): the restore to global order is fused into the kernels'
    K/V loads through the plan's row map,
  attention backward in two launches: dQ (which also computes the
    preprocess term delta = rowsum(dO * O), and whose grid ends with the
    gated zeroing of untouched dK/dV rows), then dK/dV; the dK/dV stores go
    straight to rank-major order for the reduce-scatter (the unrestore fused
    the same way).
Inputs are synthetic and already resident in HBM when timing starts.

The headline workload (default flat_75k: the post-exchange share of one
75600-token sequence, 5 heads of 128, the largest of the five) gives
value = 14 * D * H * causal_pairs / step time (TFLOP/s; masked-in FLOPs only),
the steps timed with no events inside. A second pass puts an event pair around
each step (mean / median / p90). A third pass runs the same steps with the
backward as its separate launches (preprocess, dK/dV, dQ, gated zeroing) and
an event pair around each attention kernel: from those in-step durations the
"roofline" object names the step's longest kernel with its own algorithmic
work (forward 4, dK/dV 8, dQ 2 x D x H x pairs FLOPs; the dQ kernel's S and
dP recompute is reported beside it as executed work), and the other kernels'
figures sit beside it. The standalone K+V restore (warm and cold) and the plan
upload are timed apart. "configs" holds the same block for each of the other
four workloads, measured in the same run; "cpu_baseline" times the fp64
oracle on a bounded sample of the headline share on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload flat_75k] [--no-cpu-baseline]
    python bench.py --gather-only --workload dcs_8k --steps 40   # gather launches alone
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal THD attn fwd+bwd TFLOP/s per CP-rank share; % bf16 MFMA peak; gather GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="flat_75k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window", type=int, nargs=2, default=(-1, 0), metavar=("LEFT", "RIGHT"),
                    help="attention window of the timed step: real keys at document "
                         "positions [p-LEFT, p+RIGHT], -1 unbounded; (-1, 0) causal")
    ap.add_argument("--max-key-splits", type=int, default=0,
                    help="the plan's max_key_splits for the timed step: 0 automatic, "
                         "1 never split a forward / dQ key walk, n at most n parts")
    ap.add_argument("--no-masks", action="store_true",
                    help="skip the mask-variant measurement on the flat share")
    ap.add_argument("--no-p2p", action="store_true",
                    help="skip the P2P (ring) step measurement")
    ap.add_argument("--no-a2a", action="store_true",
                    help="skip the all-to-all layout measurement (flat vs dual-chunk)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload blocks of the other four workloads")
    ap.add_argument("--gather-only", action="store_true",
                    help="time only the workload's restore gather (--steps launches, cold); "
                         "for a rocprofv3 kernel trace of the gather alone")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 512 MiB device copy (a known-size reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library simulates every CP rank on a single "
              f"device and has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import context_causal_attention_thd_amd as thd
    import workloads as W

    thd.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.int16, device=dev)   # 512 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.gather_only:
        print(json.dumps(gather_only(W.WORKLOADS[args.workload], stream, args.steps)), flush=True)
        return

    w = W.WORKLOADS[args.workload]
    t = W.bf16_tensors(w)
    block = measure_workload(w, t, args, dev, stream, args.steps, args.warmup,
                             tuple(args.window), args.max_key_splits)
    head = block.pop("_head")
    result = {
        "metric": METRIC,
        "value": block["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": block["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
    }
    result.update(block)
    # Side measurements, each on a clean allocator cache: a block that frees
    # gigabytes of buffers (mask_variants) left the P2P ring's Python loop up
    # to 3x slower afterwards, with every kernel and phase of it unchanged.
    q, k, v, do, cup_dev = head["tensors"]
    ms_step, flops, reps = block["ms_per_step"], head["flops"], head["reps"]
    del head

    def fresh():
        import gc
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    window = tuple(args.window)
    if w.cp_size > 1 and not args.no_p2p and window == (-1, 0):
        fresh()
        result["p2p_ring"] = p2p_ring(w, q, k, v, do, cup_dev, stream, args.warmup, args.steps,
                                      reps, flops, ms_step)
    del q, k, v, do, cup_dev
    if not args.no_masks:
        fresh()
        result["mask_variants"] = mask_variants(stream, args.warmup)
    if not args.no_a2a:
        fresh()
        result["a2a_layout"] = a2a_layout(stream)
        if w.name == "flat_75k":
            # the gather this workload is quoted on: the dual-chunk reorder of
            # q, k and v that flat sharding removes (s = 75600, cp = 8)
            row = result["a2a_layout"]["s75600"]
            result["roofline_gather"] = {
                "bound": "hbm", "kernel": "move_rows_kernel (q, k, v dual-chunk reorder, one launch)",
                "achieved": row["reorder_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(row["reorder_gbs"] / PEAK_HBM_GBS, 4), "bytes": row["reorder_bytes"],
                "note": "cold: launches rotate over buffer sets the 256 MB cache cannot hold"}
    if not args.no_configs:
        # The other workloads, each a parity-tested configuration: the same
        # step, timed the same way, in one block per workload.
        others = {}
        for name in W.ORDER:
            if name == w.name:
                continue
            fresh()
            wo = W.WORKLOADS[name]
            b = measure_workload(wo, W.bf16_tensors(wo), args, dev, stream,
                                 max(10, args.steps // 2), max(3, args.warmup // 2), (-1, 0), 0)
            hb = b.pop("_head")
            b["config"] = hb["config"]
            del hb
            others[name] = b
        result["configs"] = others
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, t)
    print(json.dumps(result), flush=True)


def measure_workload(w, t, args, dev, stream, steps, warmup, window, splits):
    """One workload's step, timed bare, evented, and kernel by kernel, with its
    rooflines; the standalone restore gather timed warm and cold. Returns the
    block; "_head" holds what the caller needs besides the JSON fields."""
    import torch

    import context_causal_attention_thd_amd as thd

    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    cup_dev = torch.from_numpy(cup).to(dev)
    T, H, D, cp, r = w.T, w.H, w.D, w.cp_size, w.rank
    n_local = T // cp

    # The all-gathered K/V as the rank receives it: every rank's share, rank-major.
    perm0 = thd.partition_index(cup, cup_dev, T, cp, -1, w.strategy)
    k_rm = thd.gather(k, perm0)
    v_rm = thd.gather(v, perm0)
    torch.cuda.synchronize()

    # Persistent buffers (allocation is outside the step).
    perm = torch.empty(T, dtype=torch.int32, device=dev)
    q_local = torch.empty((n_local, H, D), dtype=torch.bfloat16, device=dev)
    do_local = torch.empty_like(q_local)
    o = torch.empty_like(q_local)
    lse = torch.empty((H, n_local), dtype=torch.float32, device=dev)
    dq = torch.empty((n_local, H, D), dtype=torch.float32, device=dev)
    dk_rm = torch.empty((T, H, D), dtype=torch.float32, device=dev)   # rank-major partials
    dv_rm = torch.empty_like(dk_rm)
    probe = thd.Plan(cu, cup, T, cp, r, w.strategy, H, D, upload=False, kv_layout="rank_major",
                     window=window, max_key_splits=splits)
    ws = torch.empty(int(probe.info.workspace_bytes) + 4096, dtype=torch.uint8, device=dev)
    scratch = torch.empty(int(probe.info.bwd_scratch_bytes) + 256, dtype=torch.uint8, device=dev)
    pairs = int(probe.info.causal_pairs)
    touched = int(probe.info.touched_rows)
    probe.close()

    def new_plan():
        return thd.Plan(cu, cup, T, cp, r, w.strategy, H, D, upload=False,
                        kv_layout="rank_major", window=window, max_key_splits=splits)

    def step():
        plan = new_plan()
        plan.upload_into(ws, stream)
        thd.partition_index(cup, cup_dev, T, cp, -1, w.strategy, out=perm)
        mine = perm[r * n_local:(r + 1) * n_local]
        thd.gather_many([q, do], mine, [q_local, do_local])
        thd.attn_fwd(plan, q_local, k_rm, v_rm, o=o, lse=lse)
        thd.attn_bwd(plan, q_local, k_rm, v_rm, o, lse, do_local, dq=dq, dk=dk_rm, dv=dv_rm,
                     zero_untouched=True, scratch=scratch, stream=stream)
        return plan  # keep alive until the stream is synchronized

    # Whole steps: no events inside the timed region.
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    plans = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    wall0 = time.perf_counter()
    for _ in range(steps):
        plans.append(step())
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    plans.clear()
    ms_step = t_start.elapsed_time(t_end) / steps

    # Spread of the step time: a second pass with an event pair around each
    # step (the events add a little queue time, so value stays the bare mean).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        plans.append(step())
        b.record(stream)
    torch.cuda.synchronize()
    plans.clear()
    per_step = sorted(a.elapsed_time(b) for a, b in evs)
    # Host cost of the plan (validate, tiles, queues) and its upload, apart.
    t0 = time.perf_counter()
    for _ in range(20):
        new_plan().close()
    plan_host_us = (time.perf_counter() - t0) / 20 * 1e6

    plan = new_plan()
    plan.upload_into(ws, stream)
    reps = max(5, min(50, int(20.0 / max(ms_step, 1e-3))))

    def timed(fn):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_upload = timed(lambda: plan.upload_into(ws, stream))
    restore = restore_gather(w, k_rm, v_rm, perm, stream, reps)

    # Per-kernel durations inside steps: the same steps with the backward as
    # its separate launches (preprocess, dK/dV, dQ, gated zeroing -- the same
    # dK/dV launch as the composite call, whose dQ launch carries the delta
    # and the zeroing workgroups) and an event pair around each attention
    # kernel. Each kernel runs on the cache state a step leaves,
    # not on that of its own previous launch.
    kev = {n: [] for n in ("fwd", "dkdv", "dq")}

    def step_evented():
        pl = new_plan()
        pl.upload_into(ws, stream)
        thd.partition_index(cup, cup_dev, T, cp, -1, w.strategy, out=perm)
        mine = perm[r * n_local:(r + 1) * n_local]
        thd.gather_many([q, do], mine, [q_local, do_local])
        ev = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for n in kev}
        ev["fwd"][0].record(stream)
        thd.attn_fwd(pl, q_local, k_rm, v_rm, o=o, lse=lse)
        ev["fwd"][1].record(stream)
        thd.attn_bwd_parts(pl, q_local, k_rm, v_rm, o, lse, do_local, dq, dk_rm, dv_rm, scratch,
                           zero_untouched=True, stream=stream, events=ev)
        for n in kev:
            kev[n].append(ev[n])
        return pl

    for _ in range(steps):
        plans.append(step_evented())
    torch.cuda.synchronize()
    plans.clear()
    kms = {n: sorted(a.elapsed_time(b) for a, b in kev[n]) for n in kev}
    t_k = {n: sum(kms[n]) / len(kms[n]) for n in kms}

    flop_fwd = 4.0 * D * H * pairs      # QK^T, PV
    flop_bwd = 10.0 * D * H * pairs     # S, dP, dV, dK, dQ
    # Each kernel's own algorithmic work (what an ideal fused backward computes
    # once): the forward 4 units; dK/dV's kernel S, dP, dV, dK (8); the dQ
    # kernel only dQ (2) -- it recomputes S and dP (4 more units it executes).
    own = {"fwd": flop_fwd, "dkdv": 8.0 * D * H * pairs, "dq": 2.0 * D * H * pairs}
    executed = {"fwd": flop_fwd, "dkdv": own["dkdv"], "dq": 6.0 * D * H * pairs}
    names = {"fwd": "attn_fwd_kernel", "dkdv": "attn_bwd_dkdv_kernel", "dq": "attn_bwd_dq_kernel"}
    tflops_step = (flop_fwd + flop_bwd) / (ms_step * 1e-3) / 1e12
    t_bwd = t_k["dkdv"] + t_k["dq"]

    def kroof(n):
        a = own[n] / (t_k[n] * 1e-3) / 1e12
        x = executed[n] / (t_k[n] * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": names[n], "achieved": round(a, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(a / PEAK_BF16_TFLOPS, 4),
                "ms": round(t_k[n], 4), "executed_achieved": round(x, 2),
                "executed_frac": round(x / PEAK_BF16_TFLOPS, 4)}

    # The roofline object names the kernel that takes longest in the step.
    dominant = max(t_k, key=lambda n: t_k[n])
    roof = kroof(dominant)
    roof["traffic"] = _traffic(w.name, names[dominant])
    roof["note"] = ("the step's longest kernel; achieved = its own algorithmic FLOPs "
                    "(fwd 4, dK/dV 8, dQ 2 x D x H x pairs) over its in-step duration; "
                    "executed_* count the dQ kernel's S and dP recompute too")
    row_bytes = H * D * 2
    # Algorithmic HBM bytes of the step (each tensor once): local Q, O, dO
    # (bf16) and dQ (fp32); K, V (bf16) and dK, dV (fp32) of the touched key
    # rows, plus zeros written to the untouched ones; LSE and delta (fp32);
    # the gather of local Q and dO (read + write).
    step_bytes = (3 * n_local * row_bytes + n_local * row_bytes * 2
                  + 2 * touched * row_bytes + 2 * touched * row_bytes * 2
                  + 2 * (T - touched) * row_bytes * 2 + 2 * 4 * H * n_local
                  + 2 * 2 * n_local * row_bytes)
    hbm = step_bytes / (ms_step * 1e-3) / 1e9
    block = {
        "ms_per_step": round(ms_step, 4),
        "tflops": round(tflops_step, 3),
        "mfma_frac": round(tflops_step / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "roofline_fwd": dict(kroof("fwd"), **(
            {"includes": "v_transpose_kernel (the plan's V^T pre-pass, inside the forward call)"}
            if int(plan.info.fwd_tile_rows) == 256 and D == 128 else {})),
        "roofline_bwd_dkdv": kroof("dkdv"),
        "roofline_bwd_dq": kroof("dq"),
        "bwd_algorithmic": {"achieved": round(flop_bwd / (t_bwd * 1e-3) / 1e12, 2),
                            "unit": "TFLOP/s",
                            "frac": round(flop_bwd / (t_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "attn_kernels": {"ms": round(t_k["fwd"] + t_bwd, 4),
                         "tflops": round((flop_fwd + flop_bwd)
                                         / ((t_k["fwd"] + t_bwd) * 1e-3) / 1e12, 2),
                         "frac": round((flop_fwd + flop_bwd) / ((t_k["fwd"] + t_bwd) * 1e-3)
                                       / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "roofline_gather": restore,
        "step_hbm": {"bytes": step_bytes, "achieved": round(hbm, 1), "unit": "GB/s",
                     "frac": round(hbm / PEAK_HBM_GBS, 4)},
        "times_ms": {"step": round(ms_step, 4),
                     "step_mean_evented": round(sum(per_step) / len(per_step), 4),
                     "step_median_evented": round(per_step[len(per_step) // 2], 4),
                     "step_p90_evented": round(per_step[int(0.9 * (len(per_step) - 1))], 4),
                     "plan_build_host_us": round(plan_host_us, 1),
                     "plan_upload": round(t_upload, 4),
                     "fwd": round(t_k["fwd"], 4),
                     "bwd_dkdv": round(t_k["dkdv"], 4), "bwd_dq": round(t_k["dq"], 4),
                     "host_wall_per_step": round(wall / steps * 1e3, 4),
                     "kernel_reps": reps},
        "_head": {"config": {"workload": w.name, "T": T, "heads": H, "head_dim": D,
                             "cp_size": cp, "window": list(window), "max_key_splits": splits,
                             "rank": r, "strategy": w.strategy, "docs": w.B,
                             "causal_pairs_per_head": pairs,
                             "parallelism": "one simulated CP rank on one GPU"},
                  "flops": flop_fwd + flop_bwd, "reps": reps,
                  "tensors": (q, k, v, do, cup_dev)},
    }
    plan.close()
    return block


def _prepared(kind, srcs, idx, outs, stream, cp_size=0):
    """One row-movement launch with its C arguments built once: the binding's
    call (with its shape checks) runs first, then the returned callable repeats
    exactly that launch through the exported entry point. Timing loops of
    launches that last ~20-30 us then measure the kernels rather than the
    binding's per-call argument marshalling, which takes about as long."""
    import numpy as np
    import torch

    import context_causal_attention_thd_amd as thd
    L = thd.lib()
    st = thd._stream(stream)
    src_p, out_p = thd._ptr_list(srcs, "src"), thd._ptr_list(outs, "out")
    if kind == "scatter":
        thd.scatter_many(srcs, idx, outs, stream=stream)
        args = (len(srcs), src_p, srcs[0].shape[0], thd._dev_ptr(idx, "idx", torch.int32),
                thd._row_bytes(srcs[0]), out_p, outs[0].shape[0], st)
        fn = L.thd_scatter_batched
    elif kind == "gather":
        thd.gather_many(srcs, idx, outs, stream=stream)
        args = (len(srcs), src_p, srcs[0].shape[0], thd._dev_ptr(idx, "idx", torch.int32),
                idx.shape[0], thd._row_bytes(srcs[0]), out_p, st)
        fn = L.thd_gather_batched
    elif kind == "pack":
        thd.a2a_pack(srcs, cp_size, outs=outs, stream=stream)
        n = srcs[0].shape[0]
        args = (len(srcs), src_p, n, cp_size, thd._row_bytes(srcs[0]) // cp_size, out_p, st)
        fn = L.thd_a2a_pack
    else:  # unpack
        thd.a2a_unpack(srcs, outs=outs, stream=stream)
        cp, n = srcs[0].shape[0], srcs[0].shape[1]
        gb = max(1, int(np.prod(srcs[0].shape[2:])) * srcs[0].element_size())
        args = (len(srcs), src_p, n, cp, gb, out_p, st)
        fn = L.thd_a2a_unpack
    keep = (srcs, idx, outs)

    def call():
        _ = keep
        thd._check(fn(*args))
    return call


def restore_gather(w, k_rm, v_rm, perm, stream, reps):
    """The K and V restore (rank-major to global order) as one standalone
    batched gather launch, warm (back-to-back on the same buffers) and cold
    (buffer sets rotated through more than twice the 256 MB last-level cache,
    so no launch finds its rows cached by the one before). Under
    NO_LOAD_BALANCE and cp_size 1 the restore is the identity; it is timed
    all the same, as the copy it would be."""
    import torch

    import context_causal_attention_thd_amd as thd
    T = w.T
    row_bytes = w.H * w.D * 2
    k_g = torch.empty_like(k_rm)
    v_g = torch.empty_like(v_rm)

    def timed(fn):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_warm = timed(_prepared("scatter", [k_rm, v_rm], perm, [k_g, v_g], stream))
    set_bytes = 4 * k_rm.numel() * k_rm.element_size()
    n_sets = max(3, -(-(600 << 20) // set_bytes))
    sets = [[torch.empty_like(k_rm) for _ in range(4)] for _ in range(n_sets - 1)]
    sets.insert(0, [k_rm, v_rm, k_g, v_g])
    for st_ in sets[1:]:
        st_[0].copy_(k_rm)
        st_[1].copy_(v_rm)
    # One untimed pass touches every destination once: the first write to a
    # freshly allocated buffer costs extra (measured 37 us against 24 us per
    # launch), which is allocation, not bandwidth.
    calls = [_prepared("scatter", [a_, b_], perm, [c_, d_], stream) for a_, b_, c_, d_ in sets]
    torch.cuda.synchronize()
    ec0 = torch.cuda.Event(enable_timing=True)
    ec1 = torch.cuda.Event(enable_timing=True)
    cold_reps = 3 * n_sets
    ec0.record(stream)
    for i in range(cold_reps):
        calls[i % n_sets]()
    ec1.record(stream)
    torch.cuda.synchronize()
    t_cold = ec0.elapsed_time(ec1) / cold_reps
    del sets
    nbytes = 2 * (2 * T * row_bytes + 4 * T)    # K and V: read + write rows, read idx
    cold = nbytes / (t_cold * 1e-3) / 1e9
    warm = nbytes / (t_warm * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": "move_rows_kernel (K and V restore, one launch)",
            "achieved": round(cold, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(cold / PEAK_HBM_GBS, 4), "bytes": nbytes, "ms": round(t_cold, 4),
            "warm_achieved": round(warm, 1), "warm_frac": round(warm / PEAK_HBM_GBS, 4),
            "warm_ms": round(t_warm, 4),
            "note": "achieved: buffer sets rotated through > 512 MB so every launch reads and "
                    "writes HBM (cold); warm: back-to-back on the same buffers, served largely "
                    "from the 256 MB cache"}


def gather_only(w, stream, launches):
    """Only the workload's gathers, for a kernel trace whose per-launch figures
    need no unpicking: the cold K and V restore of the all-gather (or, for the
    flat share, the dual-chunk reorder of q, k and v that flat sharding
    removes), repeated ``launches`` times over rotated buffer sets."""
    import numpy as np
    import torch

    import context_causal_attention_thd_amd as thd
    dev = torch.device("cuda", 0)
    if w.name == "flat_75k":
        cp, heads = 8, 40
        s, hl = w.T, heads // cp
        cup = np.array([0, s], dtype=np.int32)
        perm = thd.partition_index(cup, torch.from_numpy(cup).to(dev), s, cp, -1,
                                   "dual_chunk_swap")
        n_t, row_bytes, T = 3, hl * w.D * 2, s
        what = "q, k, v dual-chunk reorder (s = 75600, cp_size 8, 5 heads of 128 per rank)"
    else:
        cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
        perm = thd.partition_index(cup, torch.from_numpy(cup).to(dev), w.T, w.cp_size, -1,
                                   w.strategy)
        n_t, row_bytes, T = 2, w.H * w.D * 2, w.T
        what = "K and V restore from rank-major order"
    one = T * row_bytes // 2
    set_bytes = 2 * n_t * T * row_bytes
    n_sets = max(3, -(-(600 << 20) // set_bytes))
    sets = [([torch.randn(one, device=dev).to(torch.bfloat16).view(T, -1) for _ in range(n_t)],
             [torch.empty(T, row_bytes // 2, dtype=torch.bfloat16, device=dev)
              for _ in range(n_t)]) for _ in range(n_sets)]
    calls = [_prepared("scatter", a, perm, b, stream) for a, b in sets]
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(launches):
        calls[i % n_sets]()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    nbytes = n_t * (2 * T * row_bytes + 4 * T)
    return {"gather_only": w.name, "what": what, "launches": launches, "warmup_launches": n_sets,
            "buffer_sets": n_sets, "bytes_per_launch": nbytes, "ms_per_launch": round(ms, 4),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def _traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` from profiles/traffic.json, when they
    were measured on the kernel's current source (hash check); else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = {"attn_bwd_dkdv_kernel": "attn_bwd.hip", "attn_bwd_dq_kernel": "attn_bwd_dq.hip",
           "attn_fwd_kernel": "attn_fwd.hip"}.get(kernel)
    if not src or not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            entry = json.load(f).get(workload, {}).get(kernel)
        if entry and entry.get("source_hash") == _source_hash(src):
            return entry["bytes_per_launch"]
    except Exception:
        return None
    return None


def p2p_ring(w, q, k, v, do, cup_dev, stream, warmup, steps, reps, flops, ms_allgather):
    """The same rank's fwd+bwd as P2P (ring) steps on one GPU: every peer's
    local K/V is already resident (what the ring's sends deliver). A ring
    step = p2p plan + upload, partition index, gather of local Q and dO,
    cp forward steps (each step's result kept), one LSE merge of all of them,
    delta of the merged output, cp backward steps (dQ accumulated, the peer's
    dK/dV into its own buffer for the return trip). The transfers themselves
    are not here. The forward with a merge after every step into an fp32
    accumulator is timed beside it."""
    import torch
    import context_causal_attention_thd_amd as thd
    dev = q.device
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    T, H, D, cp, r = w.T, w.H, w.D, w.cp_size, w.rank
    n = T // cp
    idxs = [thd.partition_index(cup, cup_dev, T, cp, s, w.strategy) for s in range(cp)]
    kl = [thd.gather(k, i) for i in idxs]
    vl = [thd.gather(v, i) for i in idxs]
    probe = thd.Plan(cu, cup, T, cp, r, w.strategy, H, D, upload=False, p2p=True)
    ws = torch.empty(int(probe.info.workspace_bytes) + 4096, dtype=torch.uint8, device=dev)
    scratch = torch.empty(int(probe.info.bwd_scratch_bytes) + 256, dtype=torch.uint8,
                          device=dev)
    probe.close()
    idx = torch.empty(n, dtype=torch.int32, device=dev)
    ql = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    dol = torch.empty_like(ql)
    o_parts = torch.empty((cp, n, H, D), dtype=torch.bfloat16, device=dev)
    lse_parts = torch.empty((cp, H, n), dtype=torch.float32, device=dev)
    o_acc = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((H, n), dtype=torch.float32, device=dev)
    o = torch.empty_like(ql)
    dq = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    dkp = torch.empty((cp, n, H, D), dtype=torch.float32, device=dev)
    dvp = torch.empty_like(dkp)
    srcs = [(r - i) % cp for i in range(cp)]

    def fwd(plan):
        for i, s in enumerate(srcs):
            thd.attn_fwd_step(plan, s, ql, kl[s], vl[s], o_part=o_parts[i],
                              lse_part=lse_parts[i])
        thd.lse_merge_parts(o_parts, lse_parts, o_out=o, lse_out=lse)

    def fwd_stepwise(plan):
        for i, s in enumerate(srcs):
            thd.attn_fwd_step(plan, s, ql, kl[s], vl[s], o_part=o_parts[0],
                              lse_part=lse_parts[0])
            thd.lse_merge(o_parts[0], lse_parts[0], o_acc, lse, first=(i == 0),
                          o_out=o if i == cp - 1 else None)

    def bwd(plan):
        thd.bwd_preprocess(plan, o, lse, dol, scratch)
        for i, s in enumerate(srcs):
            thd.attn_bwd_step(plan, s, ql, kl[s], vl[s], lse, dol, scratch, dq, i > 0,
                              dk_src=dkp[s], dv_src=dvp[s])

    def step():
        plan = thd.Plan(cu, cup, T, cp, r, w.strategy, H, D, upload=False, p2p=True)
        plan.upload_into(ws, stream)
        thd.partition_index(cup, cup_dev, T, cp, r, w.strategy, out=idx)
        thd.gather_many([q, do], idx, [ql, dol])
        fwd(plan)
        bwd(plan)
        return plan

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    plans = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        plans.append(step())
    e1.record(stream)
    torch.cuda.synchronize()
    plans.clear()
    ms = e0.elapsed_time(e1) / steps

    plan = thd.Plan(cu, cup, T, cp, r, w.strategy, H, D, upload=False, p2p=True)
    plan.upload_into(ws, stream)

    def timed(fn):
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_fwd = timed(lambda: fwd(plan))
    t_merge = timed(lambda: thd.lse_merge_parts(o_parts, lse_parts, o_out=o, lse_out=lse))
    t_fwd_stepwise = timed(lambda: fwd_stepwise(plan))
    t_step_merge = timed(lambda: thd.lse_merge(o_parts[0], lse_parts[0], o_acc, lse,
                                               first=False))
    fwd(plan)  # leave the one-pass merge's O and LSE for the backward
    t_bwd = timed(lambda: bwd(plan))
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "vs_allgather_step": round(ms_allgather / ms, 4), "ring_steps": cp,
            "times_ms": {"fwd_steps_and_merge": round(t_fwd, 4),
                         "merge_all_steps": round(t_merge, 4),
                         "fwd_with_stepwise_merges": round(t_fwd_stepwise, 4),
                         "one_stepwise_merge": round(t_step_merge, 4),
                         "bwd_preprocess_and_steps": round(t_bwd, 4)},
            "note": "per-rank compute of the ring on one GPU; peer K/V resident, "
                    "transfers not included"}


def mask_variants(stream, warmup, windows=((-1, 0), (-1, -1), (4096, 0), (512, 512))):
    """The flat post-a2a share (one 75600-token sequence, 5 heads x 128: cp_size
    1 math) under masks other than causal. Per window: the pairs the mask
    allows, the forward and backward (dQ + dK/dV) times from back-to-back
    launches on the same inputs, and the algorithmic TFLOP/s (4 and 10 FLOP per
    pair and head dim)."""
    import torch
    import context_causal_attention_thd_amd as thd
    import workloads as W
    w = W.WORKLOADS["flat_75k"]
    dev = torch.device("cuda", 0)
    t = W.bf16_tensors(w)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    T, H, D = w.T, w.H, w.D
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    dq = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    out = {"workload": "flat_75k", "note": "forward / backward kernels of one share, "
           "back-to-back launches; backward = dQ (with delta) + dK/dV"}
    for win in windows:
        plan = thd.Plan(cu, cup, T, 1, 0, w.strategy, H, D, window=win)
        scratch = torch.empty(int(plan.info.bwd_scratch_bytes) + 256, dtype=torch.uint8,
                              device=dev)
        pairs = int(plan.info.causal_pairs)

        def fwd():
            thd.attn_fwd(plan, q, k, v, o=o, lse=lse)

        def bwd():
            thd.attn_bwd(plan, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, scratch=scratch)

        for _ in range(max(2, warmup // 10)):
            fwd()
            bwd()
        torch.cuda.synchronize()
        times = []
        for fn in (fwd, bwd):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            reps = 5
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / reps)
        tf = 4.0 * D * H * pairs / (times[0] * 1e-3) / 1e12
        tb = 10.0 * D * H * pairs / (times[1] * 1e-3) / 1e12
        out[f"w{win[0]}_{win[1]}"] = {
            "window": list(win), "pairs_per_head": pairs, "fwd_ms": round(times[0], 4),
            "bwd_ms": round(times[1], 4), "fwd_tflops": round(tf, 2), "bwd_tflops": round(tb, 2),
            "fwd_bwd_tflops": round(14.0 * D * H * pairs / ((times[0] + times[1]) * 1e-3) / 1e12,
                                    2)}
        plan.close()
    return out


def a2a_layout(stream, seqlens=(8192, 32768, 75600), cp=8, heads=40, head_dim=128):
    """Local layout work of one before-attention all-to-all of q, k and v and
    of the return exchange of O, for bshd with batch 1 (one document), cp=8,
    h=40, d=128: the head-group pack every rank does before sending, and the
    dual-chunk reorder of the received sequence that flat sharding removes.
    The exchange itself (RCCL over xGMI) is not part of a one-GPU run.

    Every launch is timed cold: launches rotate over enough independent
    buffer sets that the 256 MB last-level cache holds none of them."""
    import math

    import numpy as np
    import torch

    import context_causal_attention_thd_amd as thd
    dev = torch.device("cuda", 0)
    hl = heads // cp
    out = {"config": {"layout": "bshd, batch 1", "cp_size": cp, "heads": heads,
                      "head_dim": head_dim, "tensors_before_attn": "q, k, v",
                      "tensors_after_attn": "o", "timing": "cold, rotated buffer sets"}}
    for s in seqlens:
        s_local = s // cp
        per_tensor = s_local * heads * head_dim * 2          # == s * hl * head_dim * 2
        sets = max(1, math.ceil((1536 << 20) / (12 * per_tensor)))
        cup = np.array([0, s], dtype=np.int32)
        cup_dev = torch.from_numpy(cup).to(dev)
        perm = thd.partition_index(cup, cup_dev, s, cp, -1, "dual_chunk_swap")
        bufs = []
        for _ in range(sets):
            shard = [torch.randn((s_local, heads, head_dim), device=dev).to(torch.bfloat16)
                     for _ in range(3)]
            packed = [torch.empty((cp, s_local, hl, head_dim), dtype=torch.bfloat16, device=dev)
                      for _ in range(3)]
            recv = [torch.randn((s, hl, head_dim), device=dev).to(torch.bfloat16)
                    for _ in range(3)]
            glob = [torch.empty_like(x) for x in recv]
            bufs.append((shard, packed, recv, glob))
        torch.cuda.synchronize()
        reps = max(2 * sets, 20)

        def timed(make):
            calls = [make(b) for b in bufs]  # each runs its launch once, untimed
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                calls[i % sets]()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        t_pack = timed(lambda b: _prepared("pack", b[0], None, b[1], stream, cp_size=cp))
        t_reorder = timed(lambda b: _prepared("scatter", b[2], perm, b[3], stream))
        # return direction, O only: rank-major gather (dual-chunk only), unpack
        t_unorder = timed(lambda b: _prepared("gather", b[3][:1], perm, b[2][:1], stream))
        t_unpack = timed(lambda b: _prepared("unpack", [b[1][0]], None, [b[0][0]], stream))
        pack_bytes = 3 * 2 * per_tensor
        reorder_bytes = 3 * (2 * per_tensor + 4 * s)
        out[f"s{s}"] = {
            "pack_ms": round(t_pack, 4),
            "pack_gbs": round(pack_bytes / (t_pack * 1e-3) / 1e9, 1),
            "reorder_ms": round(t_reorder, 4),
            "reorder_gbs": round(reorder_bytes / (t_reorder * 1e-3) / 1e9, 1),
            "reorder_bytes": reorder_bytes,
            "before_attn_flat_ms": round(t_pack, 4),
            "before_attn_dual_chunk_ms": round(t_pack + t_reorder, 4),
            "before_attn_local_saving": round(t_reorder / (t_pack + t_reorder), 4),
            "after_attn_flat_ms": round(t_unpack, 4),
            "after_attn_dual_chunk_ms": round(t_unpack + t_unorder, 4),
            "buffer_sets": sets,
        }
        del bufs
        torch.cuda.empty_cache()
    return out


def _source_hash(name: str) -> str:
    import hashlib
    p = os.path.join(ROOT, "context_causal_attention_thd_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_baseline(w, t, min_seconds=10.0, max_run_seconds=20.0, nominal_tflops=0.07):
    """The fp64 oracle, as it stands, on the host cores: the same rank share's
    forward + backward, on a bounded sample. When one run of the whole share
    would take more than max_run_seconds at the nominal rate, the sample keeps
    every k-th local row and a prefix of the heads; the sample is then run
    until min_seconds have passed (at least once), and the rate is the
    sample's causal-masked FLOPs over the time."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    idx = O.partition_index(cup, w.T, w.cp_size, w.rank, w.strategy)
    pairs_all = O.causal_pairs(cu, cup, w.T, idx)
    est = 14.0 * w.D * w.H * pairs_all / (nominal_tflops * 1e12)
    heads, step = w.H, 1
    while est * (heads / w.H) / step > max_run_seconds and heads > 1:
        heads = max(1, heads // 2)
    while est * (heads / w.H) / step > max_run_seconds:
        step *= 2
    rows = np.arange(0, len(idx), step)
    t64 = {n: x[:, :heads].double().numpy() for n, x in t.items()}
    ql, dol = t64["q"][idx], t64["do"][idx]
    sel = None if step == 1 else rows
    pairs = pairs_all if step == 1 else O.causal_pairs(cu, cup, w.T, idx[rows])
    runs, dt = 0, 0.0
    while runs == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        O.attention_fwd(ql, t64["k"], t64["v"], idx, cu, cup, w.T, rows=sel)
        O.attention_bwd(ql, t64["k"], t64["v"], dol, idx, cu, cup, w.T, rows=sel)
        dt += time.perf_counter() - t0
        runs += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    what = (f"{w.name} rank-{w.rank} share, fwd+bwd, {len(rows)} of {len(idx)} local rows "
            f"({'all' if step == 1 else f'every {step}th'}), {heads} of {w.H} heads")
    return {"value": round(14.0 * w.D * heads * pairs * runs / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{what}; fp64 numpy, {runs} runs in {dt:.1f} s",
            "seconds": round(dt, 3), "cpu_model": cpu,
            "affinity_cores": len(os.sched_getaffinity(0))}

if __name__ == "__main__":
    main()
