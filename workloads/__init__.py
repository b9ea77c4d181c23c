"""Seeded synthetic THD workloads: document layouts and bf16 input tensors.

This module only *builds inputs*. It holds none of the method's arithmetic
(no partitioning, masking or attention); both the fp64 oracle and the HIP
path receive the arrays it returns.

Five workloads are defined (sizes and distributions follow the five
configurations the benchmark is quoted on):

  tiny_nlb   2 packed docs [37, 91] (128 tokens, no inter-sequence padding),
             H=2, D=64, cp_size=2 NO_LOAD_BALANCE, both ranks.
  dcs_8k     8 docs, lengths uniform in [256, 2048], each padded to a multiple
             of 2*cp_size=4, 8192 padded tokens, H=16, D=128, cp_size=2
             DUAL_CHUNK_SWAP, rank 1.
  nlb_32k    32768 tokens, doc lengths lognormal(mu=7, sigma=1) clipped to
             [64, 16384], no per-doc padding, H=32, D=128, cp_size=4
             NO_LOAD_BALANCE, rank 2. cu_seqlens_padded is a value-equal copy
             of cu_seqlens (the case from the THD P2P regression page).
  flat_75k   one 75600-token sequence (bshd with batch 1 == THD with one doc),
             H=5 (40 heads / cp_size 8 after the a2a exchange), D=128, the
             post-exchange share, i.e. cp_size=1 math.
  pad_131k   64 docs, lengths uniform in [128, 4096], each padded to a multiple
             of 2*cp_size=16 (padding gaps in cu_seqlens_padded), ~131k tokens,
             H=8, D=128, cp_size=8 DUAL_CHUNK_SWAP, rank 3.

Tensors: Q, K, V, dO are drawn i.i.d. N(0, 1) in float32 with
numpy.random.default_rng(1000 * config_number + tensor_id) and rounded to
bfloat16 (round-to-nearest-even). They are laid out [T, H, D] in global token
order; a rank's local Q / dO are gathers of these.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

STRATEGY_DCS = "dual_chunk_swap"
STRATEGY_NLB = "no_load_balance"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    number: int               # 1..5, used in the tensor seeds
    lengths: tuple            # actual (unpadded) document lengths
    padded: tuple             # physical (padded) document lengths
    T: int                    # physical THD buffer length
    H: int
    D: int
    cp_size: int
    rank: int                 # the rank whose share is measured
    strategy: str
    value_equal_clone: bool   # cu_seqlens_padded is a separate, value-equal array

    @property
    def B(self) -> int:
        return len(self.lengths)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    def cu_seqlens_padded(self) -> np.ndarray:
        # Always a freshly allocated array, even when equal in value.
        return np.concatenate([[0], np.cumsum(self.padded)]).astype(np.int32)


def _round_up(x: np.ndarray, m: int) -> np.ndarray:
    return ((x + m - 1) // m) * m


def _lengths_dcs_8k(seed: int = 0):
    rng = np.random.default_rng(seed)
    while True:
        L = rng.integers(256, 2049, size=7)
        P = _round_up(L, 4)
        last_p = 8192 - int(P.sum())
        if 256 <= last_p <= 2048:
            last_l = max(256, last_p - int(rng.integers(0, 4)))
            break
    return [int(x) for x in L] + [last_l], [int(x) for x in P] + [last_p]


def _lengths_nlb_32k(seed: int = 0, total: int = 32768):
    rng = np.random.default_rng(seed)
    out: List[int] = []
    remaining = total
    while remaining > 0:
        n = int(np.clip(np.rint(rng.lognormal(7.0, 1.0)), 64, 16384))
        n = min(n, remaining)
        out.append(n)
        remaining -= n
    return out, list(out)


def _lengths_pad_131k(seed: int = 1):
    rng = np.random.default_rng(seed)
    L = rng.integers(128, 4097, size=64)
    P = _round_up(L, 16)
    return [int(x) for x in L], [int(x) for x in P]


def _build() -> Dict[str, Workload]:
    w: Dict[str, Workload] = {}
    w["tiny_nlb"] = Workload("tiny_nlb", 1, (37, 91), (37, 91), 128, 2, 64, 2, 0,
                             STRATEGY_NLB, True)
    L, P = _lengths_dcs_8k()
    w["dcs_8k"] = Workload("dcs_8k", 2, tuple(L), tuple(P), int(sum(P)), 16, 128, 2, 1,
                           STRATEGY_DCS, False)
    L, P = _lengths_nlb_32k()
    w["nlb_32k"] = Workload("nlb_32k", 3, tuple(L), tuple(P), int(sum(P)), 32, 128, 4, 2,
                            STRATEGY_NLB, True)
    w["flat_75k"] = Workload("flat_75k", 4, (75600,), (75600,), 75600, 5, 128, 1, 0,
                             STRATEGY_NLB, True)
    L, P = _lengths_pad_131k()
    w["pad_131k"] = Workload("pad_131k", 5, tuple(L), tuple(P), int(sum(P)), 8, 128, 8, 3,
                             STRATEGY_DCS, False)
    return w


WORKLOADS: Dict[str, Workload] = _build()
ORDER = ["tiny_nlb", "dcs_8k", "nlb_32k", "flat_75k", "pad_131k"]


def custom(name: str, lengths, padded, T: Optional[int], H: int, D: int, cp_size: int,
           rank: int, strategy: str, number: int = 9) -> Workload:
    """A small ad-hoc layout (used by tests); T defaults to sum(padded)."""
    lengths = tuple(int(x) for x in lengths)
    padded = tuple(int(x) for x in padded)
    T = int(sum(padded)) if T is None else int(T)
    return Workload(name, number, lengths, padded, T, H, D, cp_size, rank, strategy,
                    lengths == padded)


TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4}


def normal_f32(w: Workload, tensor: str, seed_offset: int = 0) -> np.ndarray:
    """N(0,1) float32 array [T, H, D] for tensor 'q', 'k', 'v' or 'do'."""
    seed = 1000 * w.number + TENSOR_IDS[tensor] + seed_offset
    rng = np.random.default_rng(seed)
    return rng.standard_normal((w.T, w.H, w.D), dtype=np.float32)


def bf16_tensors(w: Workload, names=("q", "k", "v", "do"), seed_offset: int = 0):
    """Dict of torch.bfloat16 CPU tensors [T, H, D] (round-to-nearest-even)."""
    import torch
    return {n: torch.from_numpy(normal_f32(w, n, seed_offset)).to(torch.bfloat16)
            for n in names}


def dense_bf16(layout: str, B: int, S: int, H: int, D: int, seed: int,
               names=("q", "k", "v", "do")):
    """Dict of torch.bfloat16 CPU tensors of a dense batch, bshd [B, S, H, D]
    or sbhd [S, B, H, D]: i.i.d. N(0,1) float32 from numpy's default_rng(seed
    + tensor id), rounded to bf16."""
    import torch
    shape = (B, S, H, D) if layout == "bshd" else (S, B, H, D)
    out = {}
    for n in names:
        rng = np.random.default_rng(seed + TENSOR_IDS[n])
        out[n] = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(
            torch.bfloat16)
    return out


def stair_bf16(w: Workload, step_keys: int = 256, jump_log2: float = 10.0, q_mag: float = 2.0,
               noise: float = 0.05):
    """Dict of torch.bfloat16 CPU tensors [T, H, D] whose attention scores
    climb in steps along each document: every ``step_keys`` keys the score of
    a key rises by about ``jump_log2`` in log2 units at the usual 1/sqrt(D)
    scale. Q = q_mag (1 + noise n), K = c(pos) (1 + noise n) with
    c(pos) = step * (pos // step_keys), pos the key's offset in its padded
    document and step = jump_log2 / (q_mag sqrt(D) log2(e)); V ~ N(0, 1),
    dO ~ N(0, 1) / 4 (n: i.i.d. N(0, 1) float32 from default_rng(1000 *
    number + tensor id + 50), all rounded to bf16). It only builds inputs;
    the scores are named to say what the layout is for."""
    import torch
    cup = w.cu_seqlens_padded()
    pos = np.zeros(w.T, dtype=np.int64)
    for d in range(len(cup) - 1):
        pos[cup[d]:cup[d + 1]] = np.arange(cup[d + 1] - cup[d])
    step = jump_log2 / (q_mag * np.sqrt(w.D) * np.log2(np.e))
    c = (step * (pos // step_keys)).astype(np.float32)[:, None, None]
    n = {x: normal_f32(w, x, seed_offset=50) for x in ("q", "k", "v", "do")}
    arrs = {
        "q": q_mag * (1.0 + noise * n["q"]),
        "k": c * (1.0 + noise * n["k"]),
        "v": n["v"],
        "do": 0.25 * n["do"],
    }
    return {x: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16) for x, a in arrs.items()}
