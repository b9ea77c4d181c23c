"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Integer work (partition indices, gathers, scatters) must be bit-exact.
Attention outputs must be within max-abs 2e-2 and relative-L2 5e-3 of the
oracle, per tensor: element by element on layouts the oracle finishes in
seconds (several tiles and a ragged tail), and on sampled rows plus
size-independent invariants at the full sizes of the five workloads, in the
same launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W
from _parity import (a2a_round_trip, assert_close, assert_lse, err, f64, oracle_share,
                     run_share, sample_plan, device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
thd = pytest.importorskip("context_causal_attention_thd_amd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------- partition / rows

@pytest.mark.parametrize("name", W.ORDER)
def test_partition_bit_exact(name):
    w = W.WORKLOADS[name]
    _say("partition", name)
    cup = w.cu_seqlens_padded()
    cup_dev = torch.from_numpy(cup).to(device())
    allr = []
    for r in range(w.cp_size):
        got = thd.partition_index(cup, cup_dev, w.T, w.cp_size, r, w.strategy).cpu().numpy()
        exp = O.partition_index(cup, w.T, w.cp_size, r, w.strategy)
        assert np.array_equal(got, exp), f"rank {r}"
        allr.append(exp)
    perm = thd.partition_index(cup, cup_dev, w.T, w.cp_size, -1, w.strategy).cpu().numpy()
    assert np.array_equal(perm, np.concatenate(allr))


def _random_layout(rng, strategy, cp):
    mult = 2 * cp if strategy == "dual_chunk_swap" else 1
    n = int(rng.integers(1, 12))
    L = rng.integers(0, 300, size=n)
    P = ((L + mult - 1) // mult) * mult + rng.integers(0, 3, size=n) * mult
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cup = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
    T = int(cup[-1])
    if strategy == "no_load_balance":
        T = ((T + int(rng.integers(0, 40)) + cp - 1) // cp) * cp
    return cu, cup, T


@pytest.mark.parametrize("strategy", ["dual_chunk_swap", "no_load_balance"])
def test_partition_random_layouts(strategy):
    rng = np.random.default_rng(5)
    for trial in range(30):
        cp = int(rng.integers(1, 9))
        cu, cup, T = _random_layout(rng, strategy, cp)
        if T == 0:
            continue
        cup_dev = torch.from_numpy(cup).to(device())
        for r in range(cp):
            got = thd.partition_index(cup, cup_dev, T, cp, r, strategy).cpu().numpy()
            assert np.array_equal(got, O.partition_index(cup, T, cp, r, strategy)), (trial, r)


@pytest.mark.parametrize("row_shape,dtype", [((16, 128), torch.bfloat16), ((5, 128), torch.bfloat16),
                                             ((8, 128), torch.float32), ((1,), torch.int64),
                                             ((3,), torch.int16), ((3,), torch.uint8),
                                             ((40, 16), torch.bfloat16)])
def test_gather_scatter_byte_exact(row_shape, dtype):
    g = torch.Generator().manual_seed(1)
    n_src = 1037
    if dtype.is_floating_point:
        src = torch.randn((n_src,) + row_shape, generator=g).to(dtype)
    else:
        src = torch.randint(-100, 100, (n_src,) + row_shape, generator=g).to(dtype)
    idx = torch.randint(0, n_src, (777,), generator=g, dtype=torch.int32)
    idx[5] = -1          # out of range -> zero row
    idx[6] = n_src + 3   # out of range -> zero row
    sd = src.to(device())
    got = thd.gather(sd, idx.to(device())).cpu()
    exp = O.gather(src.view(torch.uint8).numpy() if dtype == torch.bfloat16 else src.numpy(),
                   np.clip(idx.numpy(), 0, n_src - 1))
    exp = np.array(exp, copy=True)
    exp[5] = 0
    exp[6] = 0
    gv = got.view(torch.uint8).numpy() if dtype == torch.bfloat16 else got.numpy()
    assert np.array_equal(gv, exp)
    # scatter with a permutation (no duplicates)
    perm = torch.randperm(n_src, generator=g).to(torch.int32)
    dst = torch.zeros_like(sd)
    thd.scatter(sd, perm.to(device()), dst)
    expd = O.scatter(src.view(torch.uint8).numpy() if dtype == torch.bfloat16 else src.numpy(),
                     perm.numpy(), n_src)
    dv = dst.cpu()
    dv = dv.view(torch.uint8).numpy() if dtype == torch.bfloat16 else dv.numpy()
    assert np.array_equal(dv, expd)


@pytest.mark.parametrize("n_tensors", [1, 2, 4])
def test_batched_gather_scatter_byte_exact(n_tensors):
    g = torch.Generator().manual_seed(7)
    n_src = 2053
    srcs = [torch.randn((n_src, 5, 128), generator=g).to(torch.bfloat16) for _ in range(n_tensors)]
    idx = torch.randint(0, n_src, (1500,), generator=g, dtype=torch.int32)
    idx[3] = -7
    dev_srcs = [x.to(device()) for x in srcs]
    outs = thd.gather_many(dev_srcs, idx.to(device()))
    for x, o in zip(srcs, outs):
        exp = np.array(O.gather(x.view(torch.int16).numpy(), np.clip(idx.numpy(), 0, n_src - 1)))
        exp[3] = 0
        assert np.array_equal(o.cpu().view(torch.int16).numpy(), exp)
    perm = torch.randperm(n_src, generator=g).to(torch.int32)
    dsts = [torch.zeros_like(x) for x in dev_srcs]
    thd.scatter_many(dev_srcs, perm.to(device()), dsts)
    for x, d in zip(srcs, dsts):
        exp = O.scatter(x.view(torch.int16).numpy(), perm.numpy(), n_src)
        assert np.array_equal(d.cpu().view(torch.int16).numpy(), exp)


@pytest.mark.parametrize("name", ["dcs_8k", "nlb_32k", "pad_131k"])
def test_kv_restore_round_trip(name):
    """Simulated all-gather: rank-major buffer of every rank's share, restored
    to global order with one scatter by the all-ranks permutation."""
    w = W.WORKLOADS[name]
    _say("restore", name)
    cup = w.cu_seqlens_padded()
    dev = device()
    cup_dev = torch.from_numpy(cup).to(dev)
    t = W.bf16_tensors(w, ("k", "v"))
    k, v = t["k"].to(dev), t["v"].to(dev)
    perm = thd.partition_index(cup, cup_dev, w.T, w.cp_size, -1, w.strategy)
    k_rm = thd.gather(k, perm)                  # all-gather output, rank-major
    k_glob = torch.empty_like(k)
    thd.scatter(k_rm, perm, k_glob)             # restore
    assert torch.equal(k_glob, k)
    # K and V together in one launch
    k_rm2, v_rm2 = thd.gather_many([k, v], perm)
    k_g2, v_g2 = torch.empty_like(k), torch.empty_like(v)
    thd.scatter_many([k_rm2, v_rm2], perm, [k_g2, v_g2])
    assert torch.equal(k_g2, k) and torch.equal(v_g2, v) and torch.equal(k_rm2, k_rm)
    exp = O.gather(k.view(torch.int16).cpu().numpy(),
                   O.partition_index(cup, w.T, w.cp_size, 0, w.strategy))
    assert np.array_equal(k_rm[: w.T // w.cp_size].view(torch.int16).cpu().numpy(), exp)


# ---------------------------------------------------------------- a2a layout kernels

@pytest.mark.parametrize("n,cp,hl,tail,dtype,n_tensors", [
    (1037, 8, 5, (128,), torch.bfloat16, 3),   # the bshd cp=8, h=40, d=128 shape
    (37, 3, 2, (7,), torch.bfloat16, 1),       # 28-byte groups: 4-byte vectors
    (50, 4, 1, (3,), torch.uint8, 2),          # 3-byte groups: byte path
    (129, 1, 4, (64,), torch.float32, 1),      # cp_size = 1: pack is a copy
    (0, 4, 2, (16,), torch.bfloat16, 1),       # no tokens
])
def test_a2a_pack_unpack_byte_exact(n, cp, hl, tail, dtype, n_tensors):
    _say("a2a pack/unpack", n, cp, hl, tail, dtype, n_tensors)
    g = torch.Generator().manual_seed(n + cp)
    shape = (n, cp * hl) + tail
    if dtype.is_floating_point:
        xs = [torch.randn(shape, generator=g).to(dtype) for _ in range(n_tensors)]
    else:
        xs = [torch.randint(0, 255, shape, generator=g).to(dtype) for _ in range(n_tensors)]
    bits = (lambda t: t.view(torch.int16).numpy()) if dtype == torch.bfloat16 else (
        lambda t: t.numpy())
    packed = thd.a2a_pack([x.to(device()) for x in xs], cp)
    for x, pk in zip(xs, packed):
        assert tuple(pk.shape) == (cp, n, hl) + tail
        assert np.array_equal(bits(pk.cpu()), O.a2a_pack(bits(x), cp))
    back = thd.a2a_unpack(packed)
    for x, b in zip(xs, back):
        assert np.array_equal(bits(b.cpu()), bits(x))


@pytest.mark.parametrize("strategy", ["dual_chunk_swap", "no_load_balance"])
def test_a2a_exchange_small_vs_oracle(strategy):
    cup, T, cp, H, D = [0, 48, 176, 192, 320], 320, 4, 8, 64
    _say("a2a exchange small", strategy)
    x = torch.randn((T, H, D), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    full = a2a_round_trip(cup, T, cp, H, strategy, [x.to(device())])
    shards = [x.view(torch.int16).numpy()[O.partition_index(cup, T, cp, r, strategy)]
              for r in range(cp)]
    exp = O.a2a_before_attn(shards, cup, T, cp, strategy)
    for r in range(cp):
        assert np.array_equal(full[0][r].cpu().view(torch.int16).numpy(), exp[r])


@pytest.mark.parametrize("s", [8192, 75600])
@pytest.mark.parametrize("strategy", ["dual_chunk_swap", "no_load_balance"])
def test_a2a_exchange_bshd_full_size(s, strategy):
    """bshd, cp=8, h=40, d=128 (batch 1 = one document) at the benchmarked
    sequence lengths: q, k and v through pack, exchange, (reorder), return."""
    _say("a2a exchange full", s, strategy)
    g = torch.Generator(device=device()).manual_seed(s)
    qkv = [torch.randn((s, 40, 128), generator=g, device=device()).to(torch.bfloat16)
           for _ in range(3)]
    a2a_round_trip([0, s], s, 8, 40, strategy, qkv)


# ---------------------------------------------------------------- attention, element by element

SMALL = [
    W.custom("dcs_pad_d128", [300, 517, 0, 1000, 77], [304, 520, 0, 1000, 80], None, 3, 128, 2, 0,
             "dual_chunk_swap"),
    W.custom("dcs_cp4_d64", [129, 3, 700, 64], [136, 8, 704, 64], None, 2, 64, 4, 0,
             "dual_chunk_swap"),
    W.custom("nlb_tail_d128", [250, 5, 900, 333], [256, 5, 900, 340], 1548, 2, 128, 3, 0,
             "no_load_balance"),
    W.custom("nlb_nopad_d64", [37, 91, 200, 2], [37, 91, 200, 2], None, 2, 64, 3, 0,
             "no_load_balance"),
]


def _cmp_all(got, ref, tag):
    res = {}
    res["o"] = assert_close(got["o"], ref["o"], f"{tag} O")
    res["lse"] = assert_lse(got["lse"], ref["lse"], f"{tag} LSE")
    for n in ("dq", "dk", "dv"):
        res[n] = assert_close(got[n], ref[n], f"{tag} {n}")
    return res


@pytest.mark.parametrize("w", SMALL + [W.WORKLOADS["tiny_nlb"]], ids=lambda w: w.name)
def test_attention_elementwise_all_ranks(w):
    t = W.bf16_tensors(w)
    t64 = f64(t)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    _, _, valid = O.token_table(cu, cup, w.T)
    o_u = np.zeros((w.T, w.H, w.D))
    dk_u = np.zeros((w.T, w.H, w.D))
    for r in range(w.cp_size):
        _say("attention", w.name, "rank", r)
        got = run_share(w, r, t)
        ref = oracle_share(w, r, t64)
        assert np.array_equal(got["idx"], ref["idx"])
        res = _cmp_all(got, ref, f"{w.name} r{r}")
        _say("  ", {k: (f"{a:.2e}", f"{b:.2e}") for k, (a, b) in res.items()})
        pad_local = ~valid[ref["idx"]]
        assert np.all(got["o"][pad_local] == 0) and np.all(got["dq"][pad_local] == 0)
        assert np.all(got["dk"][~valid] == 0) and np.all(got["dv"][~valid] == 0)
        o_u[got["idx"]] = got["o"]
        dk_u += got["dk"]
    # union of ranks against the oracle's cp_size=1 result
    ref1 = O.attention_fwd(t64["q"], t64["k"], t64["v"], np.arange(w.T), cu, cup, w.T)[0]
    assert_close(o_u, ref1, f"{w.name} union O")
    dk1 = O.attention_bwd(t64["q"], t64["k"], t64["v"], t64["do"], np.arange(w.T), cu, cup, w.T)[1]
    assert_close(dk_u, dk1, f"{w.name} union dK")


def test_padding_poison():
    w = SMALL[0]
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    _, _, valid = O.token_table(cu, cup, w.T)
    t = W.bf16_tensors(w)
    bad = {n: x.clone() for n, x in t.items()}
    for x in bad.values():
        x[torch.from_numpy(~valid)] = float("nan")
    for r in range(w.cp_size):
        _say("poison rank", r)
        clean = run_share(w, r, t)
        dirty = run_share(w, r, bad)
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert np.array_equal(clean[n], dirty[n]), n


def test_determinism_run_to_run():
    # Every output row has one writer (split key walks are merged in key
    # order), so every output is bit-identical across runs.
    w = SMALL[2]
    t = W.bf16_tensors(w)
    a = run_share(w, 1, t)
    b = run_share(w, 1, t)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


def test_zero_untouched_gate_and_accumulate():
    w = SMALL[0]
    t = W.bf16_tensors(w)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    r = 1
    idx = O.partition_index(cup, w.T, w.cp_size, r, w.strategy)
    touched = O.touched_keys(cu, cup, w.T, idx)
    fill = torch.full((w.T, w.H, w.D), 7.0)
    kept = run_share(w, r, t, zero_untouched=False, dk_init=fill, dv_init=fill)
    zeroed = run_share(w, r, t, zero_untouched=True, dk_init=fill, dv_init=fill)
    assert kept["plan"].info.n_zero_ranges > 0
    assert np.all(kept["dk"][~touched] == 7.0) and np.all(kept["dv"][~touched] == 7.0)
    assert np.all(zeroed["dk"][~touched] == 0) and np.all(zeroed["dv"][~touched] == 0)
    assert np.array_equal(kept["dk"][touched], zeroed["dk"][touched])
    acc = run_share(w, r, t, zero_untouched=False, dk_init=fill, dv_init=fill, accumulate=True)
    assert np.allclose(acc["dk"][touched], zeroed["dk"][touched] + 7.0, atol=1e-5)
    assert np.all(acc["dk"][~touched] == 7.0)
    # a layout with no untouched rows has no zeroing ranges at all
    f = W.WORKLOADS["flat_75k"]
    p = thd.Plan(f.cu_seqlens(), f.cu_seqlens_padded(), f.T, 1, 0, f.strategy, f.H, f.D,
                 upload=False)
    assert p.info.n_zero_ranges == 0 and p.info.untouched_rows == 0


@pytest.mark.parametrize("name", ["dcs_pad_d128", "dcs_cp4_d64", "nlb_tail_d128", "dcs_8k",
                                  "pad_131k"])
def test_rank_major_kv_fuses_restore(name):
    """K/V passed as the all-gather delivers them (rank-major) and dK/dV
    returned in that order: the restore and unrestore are fused into the
    kernels' loads and stores, so every output is bit-identical to the
    global-order call (dK/dV permuted), which the other tests check against
    the oracle; one small layout is also checked against the oracle directly."""
    small = {x.name: x for x in SMALL}
    w = small.get(name) or W.WORKLOADS[name]
    t = W.bf16_tensors(w)
    ranks = range(w.cp_size) if name in small else [w.rank]
    for r in ranks:
        _say("rank-major K/V", name, "rank", r)
        g = run_share(w, r, t)
        m = run_share(w, r, t, kv_layout="rank_major")
        perm = m["perm"]
        assert sorted(perm.tolist()) == list(range(w.T))
        for n in ("o", "lse", "dq"):
            assert np.array_equal(m[n], g[n]), n
        for n in ("dk", "dv"):
            assert np.array_equal(m[n], g[n][perm]), n
        if name == "dcs_pad_d128":
            ref = oracle_share(w, r, f64(t))
            ref["dk"], ref["dv"] = ref["dk"][perm], ref["dv"][perm]
            _cmp_all(m, ref, f"{name} r{r} rank-major")


@pytest.mark.parametrize("kv_layout", ["global", "rank_major"])
def test_bwd_parts_match_composite(kv_layout):
    """cp_attn_bwd (two launches: dQ computing delta, dK/dV with the zeroing
    workgroups) against its separate launches (preprocess, dK/dV, dQ, zeroing):
    the same gradients up to the summation order of delta."""
    w = SMALL[0]
    t = W.bf16_tensors(w)
    dev = device()
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    cup_dev = torch.from_numpy(cup).to(dev)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    if kv_layout == "rank_major":
        perm = thd.partition_index(cup, cup_dev, w.T, w.cp_size, -1, w.strategy)
        k, v = thd.gather(k, perm), thd.gather(v, perm)
    for r in range(w.cp_size):
        _say("bwd parts vs composite", kv_layout, "rank", r)
        idx = thd.partition_index(cup, cup_dev, w.T, w.cp_size, r, w.strategy)
        ql, dol = thd.gather(q, idx), thd.gather(do, idx)
        plan = thd.Plan(cu, cup, w.T, w.cp_size, r, w.strategy, w.H, w.D, kv_layout=kv_layout)
        o, lse = thd.attn_fwd(plan, ql, k, v)
        fill = torch.full((w.T, w.H, w.D), 3.0, device=dev)
        a = thd.attn_bwd(plan, ql, k, v, o, lse, dol, dk=fill.clone(), dv=fill.clone())
        scratch = torch.empty(int(plan.info.bwd_scratch_bytes), dtype=torch.uint8, device=dev)
        dq = torch.empty_like(a[0])
        b = thd.attn_bwd_parts(plan, ql, k, v, o, lse, dol, dq, fill.clone(), fill.clone(),
                               scratch)
        torch.cuda.synchronize()
        # rows that must be exactly zero: padding query rows of dQ; untouched
        # key rows of dK/dV (zeroed by the composite, by the zeroing launch in
        # the parts), in the layout of dk/dv
        _, _, valid = O.token_table(cu, cup, w.T)
        gidx = idx.cpu().numpy()
        untouched = ~O.touched_keys(cu, cup, w.T, gidx)
        if kv_layout == "rank_major":
            untouched = untouched[perm.cpu().numpy()]
        must_zero = {"dq": ~valid[gidx], "dk": untouched, "dv": untouched}
        for x, y, n in zip(a, b, ("dq", "dk", "dv")):
            x, y = x.cpu().numpy(), y.cpu().numpy()
            assert np.all(np.isfinite(x)), n
            assert np.all(x[must_zero[n]] == 0) and np.all(y[must_zero[n]] == 0), n
            assert np.abs(x - y).max() <= 1e-4 * max(1.0, np.abs(y).max()), n


# ---------------------------------------------------------------- full sizes

FULL = ["tiny_nlb", "dcs_8k", "nlb_32k", "flat_75k", "pad_131k"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    w = W.WORKLOADS[name]
    _say("full-size", name)
    t = W.bf16_tensors(w)
    got = run_share(w, w.rank, t)
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    idx = got["idx"]
    assert np.array_equal(idx, O.partition_index(cup, w.T, w.cp_size, w.rank, w.strategy))
    for n in ("o", "lse", "dq", "dk", "dv"):
        x = got[n]
        assert np.all(np.isfinite(x) | np.isneginf(x)), n
    t64 = {n: t[n].double().numpy() for n in t}
    rng = np.random.default_rng(1)
    rows, keys = sample_plan(w, w.rank, rng)
    _say("  sampled rows", len(rows), "keys", len(keys))
    ref = oracle_share(w, w.rank, t64, rows=rows)
    assert_close(got["o"][rows], ref["o"][rows], f"{name} O[rows]")
    assert_lse(got["lse"][:, rows], ref["lse"][:, rows], f"{name} LSE[rows]")
    assert_close(got["dq"][rows], ref["dq"][rows], f"{name} dQ[rows]")
    assert keys, "no sampled keys"
    assert_close(got["dk"][keys], ref["dk"][keys], f"{name} dK[keys]")
    assert_close(got["dv"][keys], ref["dv"][keys], f"{name} dV[keys]")
    # Size-independent invariants per document: sum_j dV_j = sum of the local
    # rows' dO; sum_j dK_j ~ 0; untouched rows are zero.
    doc, pos, valid = O.token_table(cu, cup, w.T)
    dol = t64["do"][idx]
    vloc = valid[idx]
    touched = O.touched_keys(cu, cup, w.T, idx)
    assert np.all(got["dk"][~touched] == 0) and np.all(got["dv"][~touched] == 0)
    sums_v, sums_do, sums_k, norms_k = [], [], [], []
    for d in range(w.B):
        a, b = cup[d], cup[d + 1]
        rowsd = np.nonzero(vloc & (doc[idx] == d))[0]
        if len(rowsd) == 0:
            continue
        sums_v.append(got["dv"][a:b].astype(np.float64).sum(axis=0))
        sums_do.append(dol[rowsd].sum(axis=0))
        sums_k.append(got["dk"][a:b].astype(np.float64).sum(axis=0))
        norms_k.append(np.linalg.norm(got["dk"][a:b]))
    a_, r_ = err(np.array(sums_v), np.array(sums_do))
    assert r_ < 5e-3, f"sum dV vs sum dO rel={r_:.2e}"
    assert np.linalg.norm(np.array(sums_k)) < 0.05 * np.linalg.norm(np.array(norms_k))


@pytest.mark.parametrize("name", ["dcs_8k", "pad_131k", "nlb_32k"])
def test_union_of_ranks_equals_cp1_full_size(name):
    """Every rank of the workload, simulated one after another on the GPU:
    scattered O and summed dK/dV partials equal a cp_size=1 run."""
    w = W.WORKLOADS[name]
    _say("union", name)
    t = W.bf16_tensors(w)
    dev = device()
    w1 = W.custom(name + "_cp1", w.lengths, w.padded, w.T, w.H, w.D, 1, 0, "no_load_balance",
                  number=w.number)
    ref = run_share(w1, 0, t)
    o_u = np.zeros_like(ref["o"])
    dk_u = np.zeros_like(ref["dk"])
    dv_u = np.zeros_like(ref["dv"])
    dq_u = np.zeros_like(ref["dq"])
    for r in range(w.cp_size):
        got = run_share(w, r, t)
        o_u[got["idx"]] = got["o"]
        dq_u[got["idx"]] = got["dq"]
        dk_u += got["dk"]
        dv_u += got["dv"]
    assert_close(o_u, ref["o"], "union O")
    assert_close(dq_u, ref["dq"], "union dQ")
    assert_close(dk_u, ref["dk"], "union dK")
    assert_close(dv_u, ref["dv"], "union dV")
