"""Plain fp64 definitions of one CP rank's share of causal THD attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
library imports, links or runs this file.

Pages cited (by title and section):
  [AG]  "[PyTorch] Add no-load-balance THD all-gather CP"
  [A2A] "[PyTorch] Extend no-load-balance CP to the a2a comm type"
  [PAD] "[PyTorch][Attention] THD P2P context-parallel regression when padded
         cu_seqlens are value-equal but not object-identical"

Vocabulary follows the pages: ``cu_seqlens`` (cumulative actual lengths),
``cu_seqlens_padded`` (cumulative physical offsets into the THD buffer),
``cp_size``, ``rank``, ``s_local``, DUAL_CHUNK_SWAP and NO_LOAD_BALANCE.

Readings of points the pages leave open (each is listed in the design notes):
  * DUAL_CHUNK_SWAP gives rank r the chunks r and 2*cp_size-1-r of every
    document ([AG] "Why" says only "2 * cp_size chunks" and "two attention
    steps per rank"; the mirrored pair is the one that balances causal work,
    which is the point of the load-balanced default).
  * Local row order under DUAL_CHUNK_SWAP: document-major, chunk r before
    chunk 2*cp_size-1-r, ascending token order inside a chunk.
  * Padding of a document sits at its end: the first L_i rows of
    [cu_seqlens_padded[i], cu_seqlens_padded[i+1]) are valid.
  * Partitions cover the physical buffer, padding rows included ([AG]
    "What changed": "one contiguous physical-token chunk"; "Why": "the
    complete physical buffer").
  * NO_LOAD_BALANCE: s_local = T / cp_size; rows at or past
    cu_seqlens_padded[B] are a padding tail ([A2A] body: only the packed
    total must divide).
  * Causality is by position inside the document, diagonal included
    (window_size = (-1, 0), [AG] "Scope and constraints"), and the mask is
    identical to cp_size = 1 ([A2A] body).
  * Other masks ([A2A] body: after the a2a exchange every attn_mask_type and
    window_size stays valid): window = (left, right) lets a real query at
    position p attend the real tokens of its document at positions
    [p - left, p + right], -1 meaning no bound on that side. (-1, 0) is the
    causal mask (every causal variant, since queries and keys share one
    layout), (-1, -1) the padding-only mask (the whole document), (w, 0) a
    causal sliding window.
  * softmax scale 1/sqrt(D); LSE is the natural log; padding rows give
    O = 0 and LSE = -inf; gradients of padding rows and of keys that no
    local query attends are 0.

Every function below is pinned by tests in ``tests/test_oracle_*.py`` against
hand examples, closed forms, brute force, a library routine on special cases
and finite differences; none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

DUAL_CHUNK_SWAP = "dual_chunk_swap"
NO_LOAD_BALANCE = "no_load_balance"

# Row chunk size for the dense per-document score matrices (rows are
# independent, so chunking rows changes no arithmetic).
_MAX_SCORE_ELEMS = 1 << 24


# --------------------------------------------------------------------------
# Metadata
# --------------------------------------------------------------------------

def _as_list(a) -> list:
    return [int(x) for x in np.asarray(a).reshape(-1)]


def check_layout(cu_seqlens, cu_seqlens_padded, T: int, cp_size: int, rank: int,
                 strategy: str) -> None:
    """Raise ValueError when the THD metadata breaks a rule the pages state.

    [AG] "Why": DUAL_CHUNK_SWAP divides every sequence into 2*cp_size chunks,
    so every padded document length must divide by 2*cp_size; NO_LOAD_BALANCE
    only needs the packed total to divide by cp_size ([A2A] body).
    """
    cu = _as_list(cu_seqlens)
    cup = _as_list(cu_seqlens_padded)
    if len(cu) != len(cup) or len(cup) < 1:
        raise ValueError("cu_seqlens and cu_seqlens_padded must have the same length B+1")
    if cp_size < 1 or not (0 <= rank < cp_size):
        raise ValueError("rank must lie in [0, cp_size)")
    if cup[0] != 0 or cu[0] != 0:
        raise ValueError("cumulative arrays must start at 0")
    for i in range(len(cup) - 1):
        p = cup[i + 1] - cup[i]
        n = cu[i + 1] - cu[i]
        if p < 0 or n < 0:
            raise ValueError("cumulative arrays must be non-decreasing")
        if n > p:
            raise ValueError("a document's actual length exceeds its padded length")
        if strategy == DUAL_CHUNK_SWAP and p % (2 * cp_size) != 0:
            raise ValueError("DUAL_CHUNK_SWAP needs every padded length divisible by 2*cp_size")
    if cup[-1] > T:
        raise ValueError("cu_seqlens_padded[-1] exceeds T")
    if strategy == DUAL_CHUNK_SWAP and cup[-1] != T:
        raise ValueError("DUAL_CHUNK_SWAP needs T == cu_seqlens_padded[-1]")
    if T % cp_size != 0:
        raise ValueError("T must divide by cp_size")
    if strategy not in (DUAL_CHUNK_SWAP, NO_LOAD_BALANCE):
        raise ValueError("unknown strategy")


def padding_present(cu_seqlens, cu_seqlens_padded, T: int) -> bool:
    """Inter-sequence padding decided by value, never by object identity.

    [PAD] "Expected behavior": equal values must mean "no padding" even when
    the two arrays are separate objects.
    """
    cu = _as_list(cu_seqlens)
    cup = _as_list(cu_seqlens_padded)
    for i in range(len(cup) - 1):
        if (cu[i + 1] - cu[i]) != (cup[i + 1] - cup[i]):
            return True
    return T > cup[-1]


def token_table(cu_seqlens, cu_seqlens_padded, T: int):
    """Per physical row t: document index (-1 in the tail), position inside
    the document, and whether the row is a real (non-padding) token."""
    cu = _as_list(cu_seqlens)
    cup = _as_list(cu_seqlens_padded)
    doc = np.full(T, -1, dtype=np.int64)
    pos = np.zeros(T, dtype=np.int64)
    valid = np.zeros(T, dtype=bool)
    for i in range(len(cup) - 1):
        start, end = cup[i], cup[i + 1]
        length = cu[i + 1] - cu[i]
        doc[start:end] = i
        pos[start:end] = np.arange(end - start)
        valid[start:end] = pos[start:end] < length
    return doc, pos, valid


def partition_index(cu_seqlens_padded, T: int, cp_size: int, rank: int,
                    strategy: str) -> np.ndarray:
    """Global physical row of each local row of ``rank`` (int64 [T/cp_size]).

    NO_LOAD_BALANCE ([AG] "What changed"; [A2A] body): rank r owns the
    contiguous range [r*s_local, (r+1)*s_local) with s_local = T/cp_size.

    DUAL_CHUNK_SWAP ([AG] "Why"): every padded document is cut into
    2*cp_size equal chunks; rank r takes chunk r and chunk 2*cp_size-1-r.
    A layout that breaks the strategy's divisibility rules raises ValueError.
    """
    cup = _as_list(cu_seqlens_padded)
    check_layout(cup, cup, T, cp_size, rank, strategy)
    if strategy == NO_LOAD_BALANCE:
        s_local = T // cp_size
        return np.arange(rank * s_local, (rank + 1) * s_local, dtype=np.int64)
    rows = []
    for i in range(len(cup) - 1):
        chunk = (cup[i + 1] - cup[i]) // (2 * cp_size)
        for c in (rank, 2 * cp_size - 1 - rank):
            first = cup[i] + c * chunk
            rows.extend(range(first, first + chunk))
    return np.asarray(rows, dtype=np.int64)


def local_valid_lengths(cu_seqlens, cu_seqlens_padded, T: int, cp_size: int, rank: int,
                        strategy: str) -> np.ndarray:
    """Number of real tokens of each document held by ``rank`` (int64 [B]).

    The per-rank valid length the P2P path asks for ([PAD] "Describe the
    bug", get_cu_seqlens_on_cp_rank), counted from the token table.
    """
    doc, _, valid = token_table(cu_seqlens, cu_seqlens_padded, T)
    idx = partition_index(cu_seqlens_padded, T, cp_size, rank, strategy)
    B = len(_as_list(cu_seqlens_padded)) - 1
    out = np.zeros(B, dtype=np.int64)
    for g in idx:
        if valid[g]:
            out[doc[g]] += 1
    return out


CAUSAL = (-1, 0)


def key_bounds(g, a: int, e: int, window=CAUSAL):
    """First and last key (global rows, inclusive) that real query row(s) g of
    a document with real tokens [a, e) attend: the positions within
    [g - left, g + right] of that range, -1 meaning unbounded."""
    left, right = int(window[0]), int(window[1])
    g = np.asarray(g, dtype=np.int64)
    lo = np.full_like(g, a) if left < 0 else np.maximum(a, g - left)
    hi = np.full_like(g, e - 1) if right < 0 else np.minimum(e - 1, g + right)
    return lo, hi


def _doc_real_end(cu_seqlens, cu_seqlens_padded, d: int) -> int:
    cu, cup = _as_list(cu_seqlens), _as_list(cu_seqlens_padded)
    return cup[d] + (cu[d + 1] - cu[d])


def causal_pairs(cu_seqlens, cu_seqlens_padded, T: int, idx, window=CAUSAL) -> int:
    """Number of (query, key) pairs the mask allows, summed over local rows
    (per head): under the causal mask query g attends keys j of its own
    document with j <= g; in general the keys of ``key_bounds``."""
    doc, pos, valid = token_table(cu_seqlens, cu_seqlens_padded, T)
    cup = _as_list(cu_seqlens_padded)
    total = 0
    for g in _as_list(idx):
        if valid[g]:
            d = int(doc[g])
            lo, hi = key_bounds(g, cup[d], _doc_real_end(cu_seqlens, cu_seqlens_padded, d),
                                window)
            total += int(hi) - int(lo) + 1
    return total


def touched_keys(cu_seqlens, cu_seqlens_padded, T: int, idx, window=CAUSAL) -> np.ndarray:
    """bool [T]: key rows attended by at least one local query."""
    doc, pos, valid = token_table(cu_seqlens, cu_seqlens_padded, T)
    cup = _as_list(cu_seqlens_padded)
    out = np.zeros(T, dtype=bool)
    for g in _as_list(idx):
        if valid[g]:
            d = int(doc[g])
            lo, hi = key_bounds(g, cup[d], _doc_real_end(cu_seqlens, cu_seqlens_padded, d),
                                window)
            out[int(lo):int(hi) + 1] = True
    return out


# --------------------------------------------------------------------------
# Row movement
# --------------------------------------------------------------------------

def gather(src: np.ndarray, idx) -> np.ndarray:
    """dst[m] = src[idx[m]] (the rank slicing of [AG] "How to use" and the
    K/V restore of its sequence diagram)."""
    return np.asarray(src)[np.asarray(idx, dtype=np.int64)]


def scatter(src: np.ndarray, idx, n_dst: int, fill=0) -> np.ndarray:
    """dst[idx[m]] = src[m]; rows not named keep ``fill``."""
    src = np.asarray(src)
    dst = np.full((n_dst,) + src.shape[1:], fill, dtype=src.dtype)
    dst[np.asarray(idx, dtype=np.int64)] = src
    return dst


def a2a_pack(x: np.ndarray, cp_size: int) -> np.ndarray:
    """Split every token's heads into cp_size equal groups and make group c one
    contiguous block: [n, H, ...] -> [cp_size, n, H / cp_size, ...]. Block c
    is what this rank sends to rank c in the all-to-all before attention
    ([A2A] body: after the exchange each rank holds only its own head slice)."""
    x = np.asarray(x)
    n, H = x.shape[0], x.shape[1]
    if H % cp_size != 0:
        raise ValueError("heads not divisible by cp_size")
    hl = H // cp_size
    out = np.empty((cp_size, n, hl) + x.shape[2:], dtype=x.dtype)
    for c in range(cp_size):
        for m in range(n):
            out[c, m] = x[m, c * hl:(c + 1) * hl]
    return out


def a2a_unpack(y: np.ndarray) -> np.ndarray:
    """Inverse of a2a_pack: block c of [cp, n, Hl, ...] becomes heads
    c*Hl .. c*Hl+Hl-1 of every token of [n, cp*Hl, ...] (the last step of
    the [A2A] diagram: local token shard, full heads)."""
    y = np.asarray(y)
    cp, n, hl = y.shape[0], y.shape[1], y.shape[2]
    out = np.empty((n, cp * hl) + y.shape[3:], dtype=y.dtype)
    for c in range(cp):
        for m in range(n):
            out[m, c * hl:(c + 1) * hl] = y[c, m]
    return out


def _all_ranks_index(cu_seqlens_padded, T: int, cp_size: int, strategy: str) -> np.ndarray:
    return np.concatenate([partition_index(cu_seqlens_padded, T, cp_size, r, strategy)
                           for r in range(cp_size)]).astype(np.int64)


def a2a_before_attn(local_shards, cu_seqlens_padded, T: int, cp_size: int,
                    strategy: str = DUAL_CHUNK_SWAP):
    """The forward exchange of [A2A], simulated for all ranks at once.

    local_shards[r] is rank r's [T/cp, H, ...] token shard (its partition, all
    heads). Each rank packs, the all-to-all hands block c of rank r to rank c
    (placed at position r of rank c's receive buffer), and the receive buffer
    is read as one sequence in rank-major order. Under NO_LOAD_BALANCE that is
    already global order; under DUAL_CHUNK_SWAP the rank-major rows are put
    back into global order (the reorder that flat sharding removes, [A2A]
    body). Returns, per rank, the full sequence [T, H/cp, ...] of its head
    group."""
    send = [a2a_pack(x, cp_size) for x in local_shards]
    out = []
    for r in range(cp_size):
        rank_major = np.concatenate([send[c][r] for c in range(cp_size)], axis=0)
        if strategy == NO_LOAD_BALANCE:
            out.append(rank_major)
        else:
            perm = _all_ranks_index(cu_seqlens_padded, T, cp_size, strategy)
            out.append(scatter(rank_major, perm, T))
    return out


def a2a_after_attn(full_outputs, cu_seqlens_padded, T: int, cp_size: int,
                   strategy: str = DUAL_CHUNK_SWAP):
    """The return exchange of [A2A] (diagram: split the sequence by CP rank,
    exchange, local token shard with full heads), simulated for all ranks.
    full_outputs[r] is rank r's [T, H/cp, ...] result for head group r in
    global order; returns every rank's [T/cp, H, ...] shard."""
    s_local = T // cp_size
    send = []
    for r in range(cp_size):
        x = np.asarray(full_outputs[r])
        if strategy != NO_LOAD_BALANCE:
            x = gather(x, _all_ranks_index(cu_seqlens_padded, T, cp_size, strategy))
        send.append([x[c * s_local:(c + 1) * s_local] for c in range(cp_size)])
    return [a2a_unpack(np.stack([send[c][r] for c in range(cp_size)])) for r in range(cp_size)]


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _groups(idx, cu_seqlens, cu_seqlens_padded, T: int, rows: Optional[Sequence[int]]):
    """Valid local rows grouped by document: (doc start, local rows, globals,
    end of the document's real tokens)."""
    doc, _, valid = token_table(cu_seqlens, cu_seqlens_padded, T)
    cup = _as_list(cu_seqlens_padded)
    idx = np.asarray(idx, dtype=np.int64)
    sel = np.arange(len(idx)) if rows is None else np.asarray(sorted(set(_as_list(rows))),
                                                               dtype=np.int64)
    by_doc = {}
    for m in sel:
        g = int(idx[m])
        if valid[g]:
            by_doc.setdefault(int(doc[g]), []).append(int(m))
    out = []
    for d in sorted(by_doc):
        ms = np.asarray(by_doc[d], dtype=np.int64)
        out.append((cup[d], ms, idx[ms], _doc_real_end(cu_seqlens, cu_seqlens_padded, d)))
    return out


def _scores(q_rows, k_keys, lo_rows, hi_rows, key0: int, scale: float):
    """scale * q k^T over keys key0.. with keys outside a row's [lo, hi] set
    to -inf (under the causal mask: the keys j > g of the future)."""
    s = (q_rows @ k_keys.T) * scale
    keys = key0 + np.arange(k_keys.shape[0])
    s[(keys[None, :] > hi_rows[:, None]) | (keys[None, :] < lo_rows[:, None])] = -np.inf
    return s


def _chunks(n_rows: int, n_keys: int):
    step = max(1, _MAX_SCORE_ELEMS // max(1, n_keys))
    for r0 in range(0, n_rows, step):
        yield r0, min(n_rows, r0 + step)


def attention_fwd(q_local, k, v, idx, cu_seqlens, cu_seqlens_padded, T: int,
                  scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
                  window=CAUSAL):
    """O [n, H, D] and LSE [H, n] of local queries against the full K/V.

    A local row m with global row g = idx[m] that is a real token attends the
    keys j of its own document with j <= g (all real, since padding sits at
    the end of a document): s_j = scale * <Q_m, K_j>, LSE = log sum_j exp s_j,
    O_m = sum_j exp(s_j - LSE) V_j. Padding rows: O = 0, LSE = -inf.
    ``rows`` restricts the computation to those local rows (others stay 0/-inf).
    ``window`` (see ``key_bounds``) replaces j <= g by the window's keys.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, H, D = q_local.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((n, H, v.shape[2]), dtype=np.float64)
    lse = np.full((H, n), -np.inf, dtype=np.float64)
    for a, ms, gs, e_doc in _groups(idx, cu_seqlens, cu_seqlens_padded, T, rows):
        lo, hi = key_bounds(gs, a, e_doc, window)
        k0, kend = int(lo.min()), int(hi.max()) + 1
        for h in range(H):
            kk = k[k0:kend, h]
            vv = v[k0:kend, h]
            for r0, r1 in _chunks(len(ms), kend - k0):
                s = _scores(q_local[ms[r0:r1], h], kk, lo[r0:r1], hi[r0:r1], k0, scale)
                mx = s.max(axis=1)
                e = np.exp(s - mx[:, None])
                tot = e.sum(axis=1)
                lse[h, ms[r0:r1]] = mx + np.log(tot)
                out[ms[r0:r1], h] = (e / tot[:, None]) @ vv
    return out, lse


def attention_bwd(q_local, k, v, do_local, idx, cu_seqlens, cu_seqlens_padded, T: int,
                  scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
                  window=CAUSAL):
    """Gradients of sum(dO * O) for ``attention_fwd``: dQ [n,H,D] (local rows)
    and this rank's partial dK, dV [T,H,D] in global order.

    With P the softmax rows and dP_j = <dO_m, V_j>, the softmax Jacobian gives
    dS_j = P_j (dP_j - sum_i P_i dP_i); then dQ_m = scale sum_j dS_j K_j,
    dK_j += scale dS_j Q_m, dV_j += P_j dO_m. These partials are what the
    rank hands to the reduce-scatter ([AG] sequence diagram: dK/dV are
    unrestored for reduce-scatter). Rows that are padding or that no local
    query attends stay 0. ``rows`` restricts the query rows that contribute;
    ``window`` is the mask of ``attention_fwd``.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do_local = np.asarray(do_local, dtype=np.float64)
    n, H, D = q_local.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = np.zeros((n, H, D), dtype=np.float64)
    dk = np.zeros((T, H, D), dtype=np.float64)
    dv = np.zeros((T, H, D), dtype=np.float64)
    for a, ms, gs, e_doc in _groups(idx, cu_seqlens, cu_seqlens_padded, T, rows):
        lo, hi = key_bounds(gs, a, e_doc, window)
        k0, kend = int(lo.min()), int(hi.max()) + 1
        for h in range(H):
            kk = k[k0:kend, h]
            vv = v[k0:kend, h]
            for r0, r1 in _chunks(len(ms), kend - k0):
                m_sel = ms[r0:r1]
                qq = q_local[m_sel, h]
                dd = do_local[m_sel, h]
                s = _scores(qq, kk, lo[r0:r1], hi[r0:r1], k0, scale)
                mx = s.max(axis=1)
                e = np.exp(s - mx[:, None])
                p = e / e.sum(axis=1)[:, None]
                dp = dd @ vv.T
                ds = p * (dp - (p * dp).sum(axis=1)[:, None])
                dq[m_sel, h] = scale * (ds @ kk)
                dk[k0:kend, h] += scale * (ds.T @ qq)
                dv[k0:kend, h] += p.T @ dd
    return dq, dk, dv


# --------------------------------------------------------------------------
# P2P (ring) context parallelism
# --------------------------------------------------------------------------
# [PAD] "Describe the bug": under P2P context parallelism a rank's attention
# runs in steps, each against the K/V one peer holds, with per-step sequence
# metadata (get_cu_seqlens_on_cp_rank) and gradient tails to clear. The pages
# do not spell out the ring, so the plainest reading is taken: at step i rank
# r works on the keys held by rank (r - i) mod cp_size; the step results are
# merged through their log-sum-exp; the backward of a step uses the softmax of
# the whole key set (its LSE and delta = rowsum(dO * O) of the merged output).

def owner_ranks(cu_seqlens_padded, T: int, cp_size: int, strategy: str) -> np.ndarray:
    """owner[g] = the rank whose local share holds global row g."""
    owner = np.full(T, -1, dtype=np.int64)
    for r in range(cp_size):
        owner[partition_index(cu_seqlens_padded, T, cp_size, r, strategy)] = r
    return owner


def p2p_source(rank: int, step: int, cp_size: int) -> int:
    """Rank whose K/V rank ``rank`` attends at ring step ``step``."""
    return (rank - step) % cp_size


def attention_fwd_keys(q_local, k, v, idx, cu_seqlens, cu_seqlens_padded, T: int, key_ok,
                       scale: Optional[float] = None):
    """``attention_fwd`` restricted to the keys j with key_ok[j] (one P2P step:
    the keys one rank holds). A row with no allowed key gets O = 0, LSE = -inf."""
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    key_ok = np.asarray(key_ok, dtype=bool)
    n, H, D = q_local.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((n, H, v.shape[2]), dtype=np.float64)
    lse = np.full((H, n), -np.inf, dtype=np.float64)
    for a, ms, gs, _ in _groups(idx, cu_seqlens, cu_seqlens_padded, T, None):
        kend = int(gs.max()) + 1
        drop = ~key_ok[a:kend]
        for h in range(H):
            kk = k[a:kend, h]
            vv = v[a:kend, h]
            for r0, r1 in _chunks(len(ms), kend - a):
                s = _scores(q_local[ms[r0:r1], h], kk, np.full(r1 - r0, a), gs[r0:r1], a,
                            scale)
                s[:, drop] = -np.inf
                mx = s.max(axis=1)
                some = np.isfinite(mx)
                e = np.zeros_like(s)
                e[some] = np.exp(s[some] - mx[some, None])
                tot = e.sum(axis=1)
                rows = ms[r0:r1]
                lse[h, rows[some]] = mx[some] + np.log(tot[some])
                out[rows[some], h] = (e[some] / tot[some, None]) @ vv
    return out, lse


def lse_merge(parts):
    """Merge (O_i, LSE_i) of attention over disjoint key sets into the result
    over their union: LSE = log sum_i exp LSE_i, O = sum_i exp(LSE_i - LSE) O_i.
    O has shape [n, H, D] and LSE [H, n]; a part with LSE = -inf adds nothing."""
    lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])
    mx = lses.max(axis=0)
    some = np.isfinite(mx)
    safe = np.where(some, mx, 0.0)
    w = np.exp(lses - safe[None])  # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    lse = np.where(some, safe + np.log(np.where(some, tot, 1.0)), -np.inf)
    o = np.zeros_like(np.asarray(parts[0][0], dtype=np.float64))
    for (oi, li), wi in zip(parts, w):
        coef = np.where(some, wi / np.where(some, tot, 1.0), 0.0)  # [H, n]
        o += np.asarray(oi, dtype=np.float64) * coef.T[:, :, None]
    return o, lse


def attention_bwd_keys(q_local, k, v, do_local, idx, cu_seqlens, cu_seqlens_padded, T: int,
                       key_ok, lse, delta, scale: Optional[float] = None):
    """One P2P step of the backward: the part of ``attention_bwd`` that flows
    through the keys j with key_ok[j]. The probabilities are those of the whole
    key set, P_j = exp(s_j - LSE) with the merged LSE [H, n], and
    dS_j = P_j (dP_j - delta) with delta [H, n] = rowsum(dO * O) of the merged
    output; then dQ_m = scale sum_j dS_j K_j over the step's keys, and dK_j,
    dV_j for those keys (0 elsewhere)."""
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do_local = np.asarray(do_local, dtype=np.float64)
    key_ok = np.asarray(key_ok, dtype=bool)
    lse = np.asarray(lse, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    n, H, D = q_local.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = np.zeros((n, H, D), dtype=np.float64)
    dk = np.zeros((T, H, D), dtype=np.float64)
    dv = np.zeros((T, H, D), dtype=np.float64)
    for a, ms, gs, _ in _groups(idx, cu_seqlens, cu_seqlens_padded, T, None):
        kend = int(gs.max()) + 1
        drop = ~key_ok[a:kend]
        for h in range(H):
            kk = k[a:kend, h]
            vv = v[a:kend, h]
            for r0, r1 in _chunks(len(ms), kend - a):
                m_sel = ms[r0:r1]
                qq = q_local[m_sel, h]
                dd = do_local[m_sel, h]
                s = _scores(qq, kk, np.full(r1 - r0, a), gs[r0:r1], a, scale)
                p = np.exp(s - lse[h, m_sel][:, None])
                p[:, drop] = 0.0
                dp = dd @ vv.T
                ds = p * (dp - delta[h, m_sel][:, None])
                dq[m_sel, h] = scale * (ds @ kk)
                dk[a:kend, h] += scale * (ds.T @ qq)
                dv[a:kend, h] += p.T @ dd
    return dq, dk, dv


def sequence_shard(S: int, cp_size: int, rank: int, strategy: str) -> np.ndarray:
    """Positions of one sequence of S tokens that ``rank`` holds: chunks r and
    2*cp_size-1-r of 2*cp_size under DUAL_CHUNK_SWAP ([AG] "Why"), the range
    [r*S/cp_size, (r+1)*S/cp_size) under NO_LOAD_BALANCE ([A2A] body)."""
    if strategy == DUAL_CHUNK_SWAP:
        if S % (2 * cp_size):
            raise ValueError("DUAL_CHUNK_SWAP needs S divisible by 2*cp_size")
        c = S // (2 * cp_size)
        return np.concatenate([np.arange(rank * c, (rank + 1) * c),
                               np.arange((2 * cp_size - 1 - rank) * c,
                                         (2 * cp_size - rank) * c)]).astype(np.int64)
    if S % cp_size:
        raise ValueError("NO_LOAD_BALANCE needs S divisible by cp_size")
    s = S // cp_size
    return np.arange(rank * s, (rank + 1) * s, dtype=np.int64)


def dense_rank_share(q, k, v, do, layout: str, cp_size: int, rank: int, strategy: str,
                     window=CAUSAL, scale: Optional[float] = None):
    """One rank's share of attention over a dense batch, bshd [B, S, H, D] or
    sbhd [S, B, H, D] ([A2A] body: flat a2a is tested over bshd, sbhd and
    THD). Every batch element is its own sequence of S tokens, sharded along S
    by ``sequence_shard`` and attended with ``window`` as one document.
    Returns (pos, O [B, n, H, D], LSE [B, H, n], dQ [B, n, H, D],
    dK [B, S, H, D], dV [B, S, H, D]) with pos the rank's positions (n of
    them), batch-major whatever the input layout."""
    def bsd(x):
        x = np.asarray(x, dtype=np.float64)
        return x if layout == "bshd" else x.transpose(1, 0, 2, 3)
    if layout not in ("bshd", "sbhd"):
        raise ValueError(layout)
    q, k, v, do = bsd(q), bsd(k), bsd(v), bsd(do)
    B, S = q.shape[:2]
    pos = sequence_shard(S, cp_size, rank, strategy)
    cu = [0, S]
    outs = [], [], [], [], []
    for b in range(B):
        o, lse = attention_fwd(q[b][pos], k[b], v[b], pos, cu, cu, S, scale, window=window)
        dq, dk, dv = attention_bwd(q[b][pos], k[b], v[b], do[b][pos], pos, cu, cu, S, scale,
                                   window=window)
        for lst, x in zip(outs, (o, lse, dq, dk, dv)):
            lst.append(x)
    return (pos,) + tuple(np.stack(x) for x in outs)


def rank_share(q, k, v, do, cu_seqlens, cu_seqlens_padded, T: int, cp_size: int,
               rank: int, strategy: str, scale: Optional[float] = None, window=CAUSAL):
    """Everything one rank computes, from global-order inputs: idx, O, LSE,
    dQ (local rows) and the dK/dV partials (global rows)."""
    idx = partition_index(cu_seqlens_padded, T, cp_size, rank, strategy)
    q_local = gather(q, idx)
    do_local = gather(do, idx)
    o, lse = attention_fwd(q_local, k, v, idx, cu_seqlens, cu_seqlens_padded, T, scale,
                           window=window)
    dq, dk, dv = attention_bwd(q_local, k, v, do_local, idx, cu_seqlens, cu_seqlens_padded,
                               T, scale, window=window)
    return idx, o, lse, dq, dk, dv
