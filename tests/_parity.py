"""Shared helpers for the GPU parity tests: run one rank's share through the
HIP library (via the C ABI binding) and compare with the fp64 oracle."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle as O

# Bar for floating-point outputs (bf16 inputs, fp32 accumulation).
MAX_ABS = 2e-2
REL_L2 = 5e-3


def err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def _log(name, a, r, bar):
    """Append measured errors and the bars they were held to to
    $THDCP_PARITY_LOG (JSON lines) when set."""
    path = os.environ.get("THDCP_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"check": name, "max_abs": a, "rel_l2": r,
                                "bar": [bar[0], bar[1] if np.isfinite(bar[1]) else None]})
                    + "\n")


def assert_close(got, ref, name, max_abs=MAX_ABS, rel_l2=REL_L2):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    a, r = err(got, ref)
    _log(name, a, r, (max_abs, rel_l2))
    assert a <= max_abs and r <= rel_l2, f"{name}: max_abs={a:.3e} rel_l2={r:.3e}"
    return a, r


def assert_lse(got, ref, name="lse"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    pad = np.isneginf(ref)
    assert np.all(np.isneginf(got[pad])), f"{name}: padding rows must be -inf"
    return assert_close(got[~pad], ref[~pad], name)


def device():
    import torch
    return torch.device("cuda", 0)


def run_share(w, rank, tensors, zero_untouched=True, dk_init=None, dv_init=None,
              accumulate=False, kv_layout="global", window=(-1, 0), max_key_splits=0):
    """Product path on cuda:0 for one rank: partition index -> gather local Q
    and dO -> plan -> forward -> backward. Returns numpy arrays. With
    kv_layout="rank_major" K/V are passed in the all-gathered (rank-major)
    order and dK/dV come back in that order; "perm" is the all-ranks
    permutation (rank-major position p holds global row perm[p])."""
    import torch
    import context_causal_attention_thd_amd as thd
    dev = device()
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    cup_dev = torch.from_numpy(cup).to(dev)
    q, k, v, do = (tensors[n].to(dev) for n in ("q", "k", "v", "do"))
    idx = thd.partition_index(cup, cup_dev, w.T, w.cp_size, rank, w.strategy)
    q_local = thd.gather(q, idx)
    do_local = thd.gather(do, idx)
    perm = None
    if kv_layout == "rank_major":
        perm = thd.partition_index(cup, cup_dev, w.T, w.cp_size, -1, w.strategy)
        k, v = thd.gather(k, perm), thd.gather(v, perm)
    plan = thd.Plan(cu, cup, w.T, w.cp_size, rank, w.strategy, w.H, w.D, kv_layout=kv_layout,
                    window=window, max_key_splits=max_key_splits)
    o, lse = thd.attn_fwd(plan, q_local, k, v)
    dk = None if dk_init is None else dk_init.to(dev).clone()
    dv = None if dv_init is None else dv_init.to(dev).clone()
    dq, dk, dv = thd.attn_bwd(plan, q_local, k, v, o, lse, do_local, dk=dk, dv=dv,
                              zero_untouched=zero_untouched, accumulate_dkv=accumulate)
    torch.cuda.synchronize()
    out = dict(idx=idx.cpu().numpy(), o=o.float().cpu().numpy(), lse=lse.cpu().numpy(),
               dq=dq.cpu().numpy(), dk=dk.cpu().numpy(), dv=dv.cpu().numpy(), plan=plan,
               perm=None if perm is None else perm.cpu().numpy())
    return out


def f64(tensors):
    return {n: t.double().numpy() for n, t in tensors.items()}


def oracle_share(w, rank, t64, rows=None, window=(-1, 0)):
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    idx = O.partition_index(cup, w.T, w.cp_size, rank, w.strategy)
    ql = t64["q"][idx]
    dol = t64["do"][idx]
    o, lse = O.attention_fwd(ql, t64["k"], t64["v"], idx, cu, cup, w.T, rows=rows,
                             window=window)
    dq, dk, dv = O.attention_bwd(ql, t64["k"], t64["v"], dol, idx, cu, cup, w.T, rows=rows,
                                 window=window)
    return dict(idx=idx, o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def sample_plan(w, rank, rng, n_rows=96, max_attending=400):
    """Pick local query rows and key rows whose oracle values are cheap to get
    one by one at full size: keys attended by few local queries (near the last
    attended key of a document), and the local rows attending them."""
    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    idx = O.partition_index(cup, w.T, w.cp_size, rank, w.strategy)
    doc, pos, valid = O.token_table(cu, cup, w.T)
    gl = idx
    vl = valid[gl]
    rows = set(rng.choice(len(idx), size=min(n_rows, len(idx)), replace=False).tolist())
    rows |= {0, len(idx) - 1}
    keys = []
    docs = sorted(set(doc[gl[vl]].tolist()))
    for d in rng.permutation(docs)[:6]:
        local = np.nonzero(vl & (doc[gl] == d))[0]
        gmax = int(gl[local].max())
        a = cup[d]
        cand = [gmax, gmax - 1, gmax - 7, gmax - 33, gmax - 100, a]
        for j in cand:
            if j < a:
                continue
            attending = local[gl[local] >= j]
            if 0 < len(attending) <= max_attending:
                keys.append(j)
                rows |= set(attending.tolist())
    return sorted(rows), sorted(set(keys))


def exchange(send):
    """The all-to-all itself (communication, simulated with device copies):
    rank r receives block r of every rank's send buffer, rank-major."""
    import torch
    cp = len(send)
    return [torch.cat([send[c][r] for c in range(cp)], dim=0) for r in range(cp)]


def a2a_round_trip(cup, T, cp, H, strategy, tensors):
    """Forward exchange of every rank, checked against the global head
    slices, then the return exchange, checked against the local shards."""
    import torch
    import context_causal_attention_thd_amd as thd
    dev = device()
    cup_dev = torch.from_numpy(np.asarray(cup, dtype=np.int32)).to(dev)
    perm = thd.partition_index(np.asarray(cup, dtype=np.int32), cup_dev, T, cp, -1, strategy)
    s_local, hl = T // cp, H // cp
    shards = [thd.gather_many(tensors, perm[r * s_local:(r + 1) * s_local]) for r in range(cp)]
    send = [thd.a2a_pack(sh, cp) for sh in shards]           # per rank: list over tensors
    full = []
    for i in range(len(tensors)):
        recv = exchange([send[r][i] for r in range(cp)])     # [T, hl, D], rank-major
        if strategy == "dual_chunk_swap":
            glob = [torch.empty_like(x) for x in recv]
            for r in range(cp):
                thd.scatter(recv[r], perm, glob[r])
            recv = glob
        full.append(recv)
    for i, x in enumerate(tensors):
        for r in range(cp):
            assert torch.equal(full[i][r], x[:, r * hl:(r + 1) * hl]), (i, r)
    # return exchange of the (unchanged) full-sequence head slices
    for i, x in enumerate(tensors):
        outs = full[i]
        if strategy == "dual_chunk_swap":
            outs = [thd.gather(o, perm) for o in outs]        # global -> rank-major
        send_back = [[o[c * s_local:(c + 1) * s_local] for c in range(cp)] for o in outs]
        recv = [torch.stack([send_back[c][r] for c in range(cp)]) for r in range(cp)]
        for r in range(cp):
            (local,) = thd.a2a_unpack([recv[r]])
            assert torch.equal(local, shards[r][i]), (i, r)
    return full


def oracle_share_chunked(w, rank, t64, heads=None, chunk_rows=512, workers=None,
                         window=(-1, 0), idx=None, progress=None):
    """The oracle's whole rank share (O, LSE, dQ, dK, dV over every row and
    key), evaluated in chunks of local rows on a thread pool. Rows are
    independent in the forward and the backward's dK/dV is a sum over rows,
    so the chunks' results are assembled (O, LSE, dQ by row) and summed (dK,
    dV); the oracle's arithmetic is unchanged. ``heads`` (a slice) restricts
    the heads the oracle sees. Each chunk's key range ends at its last row,
    which keeps the work near the causal pair count on long documents.
    ``progress`` (callable) is told every chunk that finished."""
    import concurrent.futures
    import threading

    cu, cup = w.cu_seqlens(), w.cu_seqlens_padded()
    if idx is None:
        idx = O.partition_index(cup, w.T, w.cp_size, rank, w.strategy)
    idx = np.asarray(idx, dtype=np.int64)
    sl = slice(None) if heads is None else heads
    q, k, v, do = (np.ascontiguousarray(t64[x][:, sl]) for x in ("q", "k", "v", "do"))
    ql, dol = q[idx], do[idx]
    n, H, D = ql.shape
    cupl = np.asarray(cup, dtype=np.int64)
    nb = len(cupl) - 1
    # Keys a chunk can reach lie in the documents of its rows: from the first
    # one's start to the last one's end (rows of the buffer tail have none).
    doc_of = np.searchsorted(cupl, idx, side="right") - 1
    o = np.zeros((n, H, D))
    lse = np.full((H, n), -np.inf)
    dq = np.zeros((n, H, D))
    dk = np.zeros((w.T, H, D))
    dv = np.zeros((w.T, H, D))
    lock = threading.Lock()

    def one(r0):
        rows = list(range(r0, min(n, r0 + chunk_rows)))
        of, lf = O.attention_fwd(ql, k, v, idx, cu, cup, w.T, rows=rows, window=window)
        gq, gk, gv = O.attention_bwd(ql, k, v, dol, idx, cu, cup, w.T, rows=rows,
                                     window=window)
        docs = doc_of[rows]
        docs = docs[(docs >= 0) & (docs < nb)]
        k0 = int(cupl[docs.min()]) if len(docs) else 0
        k1 = int(cupl[docs.max() + 1]) if len(docs) else 0
        with lock:
            o[rows], lse[:, rows], dq[rows] = of[rows], lf[:, rows], gq[rows]
            dk[k0:k1] += gk[k0:k1]
            dv[k0:k1] += gv[k0:k1]
        if progress is not None:
            progress(r0)

    if workers is None:
        workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(0, n, chunk_rows)))
    return dict(idx=idx, o=o, lse=lse, dq=dq, dk=dk, dv=dv)
