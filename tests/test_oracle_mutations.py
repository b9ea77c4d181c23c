"""Planted mistakes in a copy of the oracle each fail at least one pin.

The oracle is pinned to things other than itself (hand-worked fixtures, a
library routine on special cases, brute force, closed forms, invariants).
This file checks that those pins have teeth: it loads the oracle's source,
plants one plausible mistake (a strict mask, a wrong chunk pairing, a dropped
Jacobian term, a dropped scale, a wrong operand, an off-by-one validity, a
halved LSE, a disabled tail detection, ...), runs the pins against the
mutated copy, and requires at least one of them to fail. The unmutated copy
must pass every pin. All of it runs on the CPU; the oracle on disk is never
changed.
"""
import json
import math
import os
import types
import warnings

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "thd.py")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(source: str, name: str) -> types.ModuleType:
    mod = types.ModuleType(name)
    exec(compile(source, f"<{name}>", "exec"), mod.__dict__)
    return mod


# ------------------------------------------------------------------ pins
# Each takes the oracle module under test and raises AssertionError when the
# module disagrees with what the pages or the mathematics fix.

def pin_partition_golden(M):
    with open(os.path.join(GOLDEN, "partition_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = M.partition_index(c["cu_seqlens_padded"], c["T"], c["cp_size"], c["rank"],
                                c["strategy"]).tolist()
        exp = c["expected"]
        if isinstance(exp, str):
            _, a, b = exp.split(":")
            exp = list(range(int(a), int(b)))
        assert got == exp, c["name"]


def pin_metadata_golden(M):
    with open(os.path.join(GOLDEN, "metadata_examples.json")) as f:
        ex = json.load(f)
    for c in ex["padding"]:
        assert M.padding_present(c["cu_seqlens"], c["cu_seqlens_padded"], c["T"]) == c["padding"]
    for c in ex["pairs"]:
        idx = M.partition_index(c["cu_seqlens_padded"], c["T"], c["cp_size"], c["rank"],
                                c["strategy"])
        assert M.causal_pairs(c["cu_seqlens"], c["cu_seqlens_padded"], c["T"], idx) == c["pairs"]


def pin_dcs_balance(M):
    # the mirrored pairing gives every rank the same causal work (no padding)
    cup = [0, 64, 192]
    pairs = [M.causal_pairs(cup, cup, 192, M.partition_index(cup, 192, 4, r, "dual_chunk_swap"))
             for r in range(4)]
    assert len(set(pairs)) == 1, pairs


def _sdpa_doc(q, k, v, mask):
    """torch float64 SDPA of one document and head-batch ([H, n, D]) with a
    boolean mask (True = attend)."""
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)


def pin_sdpa_fwd_bwd(M):
    # cp_size 1, documents without padding: per document and head, torch's
    # float64 SDPA with a causal (or band) mask and its autograd.
    cu = [0, 13, 40, 41, 70]
    T, H, D = 70, 2, 8
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((T, H, D)) for _ in range(4))
    idx = M.partition_index(cu, T, 1, 0, "no_load_balance")
    for window in ((-1, 0), (5, 2)):
        o, lse = M.attention_fwd(q[idx], k, v, idx, cu, cu, T, window=window)
        dq, dk, dv = M.attention_bwd(q[idx], k, v, do[idx], idx, cu, cu, T, window=window)
        for i in range(len(cu) - 1):
            a, b = cu[i], cu[i + 1]
            n = b - a
            pos = np.arange(n)
            allow = pos[None, :] <= pos[:, None] + window[1]
            if window[0] >= 0:
                allow &= pos[None, :] >= pos[:, None] - window[0]
            mask = torch.from_numpy(allow)
            tq, tk, tv = (torch.from_numpy(x[a:b]).permute(1, 0, 2).contiguous()
                          .requires_grad_(True) for x in (q, k, v))
            ot = _sdpa_doc(tq, tk, tv, mask)
            ot.backward(torch.from_numpy(do[a:b]).permute(1, 0, 2).contiguous())
            np.testing.assert_allclose(o[a:b], ot.detach().permute(1, 0, 2).numpy(),
                                       rtol=1e-9, atol=1e-11)
            np.testing.assert_allclose(dq[a:b], tq.grad.permute(1, 0, 2).numpy(),
                                       rtol=1e-8, atol=1e-10)
            np.testing.assert_allclose(dk[a:b], tk.grad.permute(1, 0, 2).numpy(),
                                       rtol=1e-8, atol=1e-10)
            np.testing.assert_allclose(dv[a:b], tv.grad.permute(1, 0, 2).numpy(),
                                       rtol=1e-8, atol=1e-10)
            # LSE from the scores written out
            s = np.einsum("hnd,hmd->hnm", q[a:b].transpose(1, 0, 2),
                          k[a:b].transpose(1, 0, 2)) / math.sqrt(D)
            s = np.where(allow[None], s, -np.inf)
            ref = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
            np.testing.assert_allclose(lse[:, a:b], ref, rtol=1e-12, atol=1e-12)


def pin_lse_closed_form(M):
    # K = 0: every allowed score is 0, so LSE = log(number of allowed keys)
    cu, cup, T = [0, 5, 13], [0, 7, 15], 18
    rng = np.random.default_rng(3)
    q, v = rng.standard_normal((T, 1, 4)), rng.standard_normal((T, 1, 4))
    k = np.zeros((T, 1, 4))
    idx = M.partition_index(cup, T, 3, 1, "no_load_balance")
    _, lse = M.attention_fwd(q[idx], k, v, idx, cu, cup, T)
    doc, pos, valid = M.token_table(cu, cup, T)
    for m, g in enumerate(idx):
        if g < 13 and (g < 5 or 7 <= g < 15) and pos[g] < (cu[doc[g] + 1] - cu[doc[g]]):
            assert abs(lse[0, m] - math.log(pos[g] + 1)) < 1e-12
        else:
            assert lse[0, m] == -np.inf


def pin_padding_poison(M):
    # Poison in padding rows (actual length < padded length, and a tail)
    # leaves every real output unchanged; padding outputs are exactly 0.
    cu, cup, T = [0, 5, 5, 16], [0, 8, 8, 24], 24
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((T, 2, 4)) for _ in range(4))
    pad = np.array([i for i in range(T) if not (i < 5 or 8 <= i < 19)])
    qp, kp, vp, dop = (x.copy() for x in (q, k, v, do))
    for x in (qp, kp, vp, dop):
        x[pad] = 1e4
    for r in range(2):
        idx = M.partition_index(cup, T, 2, r, "dual_chunk_swap")
        clean = M.attention_fwd(q[idx], k, v, idx, cu, cup, T)[0], \
            M.attention_bwd(q[idx], k, v, do[idx], idx, cu, cup, T)
        dirty = M.attention_fwd(qp[idx], kp, vp, idx, cu, cup, T)[0], \
            M.attention_bwd(qp[idx], kp, vp, dop[idx], idx, cu, cup, T)
        np.testing.assert_array_equal(clean[0], dirty[0])
        for a, b in zip(clean[1], dirty[1]):
            np.testing.assert_array_equal(a, b)
        padl = np.isin(idx, pad)
        assert np.all(clean[0][padl] == 0)
        assert np.all(clean[1][1][pad] == 0) and np.all(clean[1][2][pad] == 0)


def pin_union_cp1(M):
    # all ranks of a padded layout together equal the cp_size 1 run
    cu, cup, T = [0, 5, 5, 16], [0, 8, 8, 24], 24
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.standard_normal((T, 2, 4)) for _ in range(4))
    i1 = M.partition_index(cup, T, 1, 0, "no_load_balance")
    o1, _ = M.attention_fwd(q[i1], k, v, i1, cu, cup, T)
    _, dk1, dv1 = M.attention_bwd(q[i1], k, v, do[i1], i1, cu, cup, T)
    o_u, dk_u, dv_u = np.zeros_like(o1), np.zeros_like(dk1), np.zeros_like(dv1)
    for r in range(2):
        idx = M.partition_index(cup, T, 2, r, "dual_chunk_swap")
        o_u[idx] = M.attention_fwd(q[idx], k, v, idx, cu, cup, T)[0]
        _, a, b = M.attention_bwd(q[idx], k, v, do[idx], idx, cu, cup, T)
        dk_u += a
        dv_u += b
    np.testing.assert_allclose(o_u, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk_u, dk1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv_u, dv1, rtol=1e-12, atol=1e-12)


PINS = [pin_partition_golden, pin_metadata_golden, pin_dcs_balance, pin_sdpa_fwd_bwd,
        pin_lse_closed_form, pin_padding_poison, pin_union_cp1]

# (name, text in oracle/thd.py, planted replacement)
MUTATIONS = [
    ("strict causal mask (diagonal dropped)",
     "np.minimum(e - 1, g + right)", "np.minimum(e - 1, g + right - 1)"),
    ("window left bound off by one",
     "np.maximum(a, g - left)", "np.maximum(a, g - left + 1)"),
    ("chunk pairing r, cp + r",
     "for c in (rank, 2 * cp_size - 1 - rank):", "for c in (rank, cp_size + rank):"),
    ("chunk order swapped",
     "for c in (rank, 2 * cp_size - 1 - rank):", "for c in (2 * cp_size - 1 - rank, rank):"),
    ("NO_LOAD_BALANCE range shifted",
     "np.arange(rank * s_local, (rank + 1) * s_local, dtype=np.int64)",
     "np.arange(rank * s_local + 1, (rank + 1) * s_local + 1, dtype=np.int64) % T"),
    ("softmax Jacobian term dropped",
     "ds = p * (dp - (p * dp).sum(axis=1)[:, None])", "ds = p * dp"),
    ("score scale dropped", "s = (q_rows @ k_keys.T) * scale", "s = (q_rows @ k_keys.T)"),
    ("dQ scale dropped", "dq[m_sel, h] = scale * (ds @ kk)", "dq[m_sel, h] = ds @ kk"),
    ("dV from Q instead of dO", "dv[k0:kend, h] += p.T @ dd", "dv[k0:kend, h] += p.T @ qq"),
    ("dK from dO instead of Q", "dk[k0:kend, h] += scale * (ds.T @ qq)",
     "dk[k0:kend, h] += scale * (ds.T @ dd)"),
    ("validity off by one", "valid[start:end] = pos[start:end] < length",
     "valid[start:end] = pos[start:end] <= length"),
    ("halved LSE", "lse[h, ms[r0:r1]] = mx + np.log(tot)",
     "lse[h, ms[r0:r1]] = 0.5 * (mx + np.log(tot))"),
    ("tail detection disabled", "return T > cup[-1]", "return False"),
]


def _failing_pins(M):
    failed = []
    for pin in PINS:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore", RuntimeWarning)  # a mutant may make NaNs
                pin(M)
        except (AssertionError, ValueError, IndexError) as e:
            failed.append((pin.__name__, type(e).__name__))
    return failed


def test_unmutated_copy_passes_every_pin():
    M = _load(open(SRC).read(), "oracle_copy")
    assert _failing_pins(M) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, old, new):
    src = open(SRC).read()
    # the first occurrence is the all-gather path's (the P2P step functions
    # that follow repeat some lines)
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    M = _load(src.replace(old, new, 1), "oracle_mutant")
    failed = _failing_pins(M)
    assert failed, f"no pin caught the planted mistake: {name}"
