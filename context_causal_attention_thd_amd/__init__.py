"""Python binding of libthdcp (one CP rank's share of causal THD attention on
MI355X / gfx950).

Argument marshalling only: every step runs in the HIP library through its C
ABI (include/thdcp.h). PyTorch supplies device memory and the current HIP
stream. There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libthdcp.so")

DUAL_CHUNK_SWAP = 0
NO_LOAD_BALANCE = 1
_STRATEGY_NAMES = {"dual_chunk_swap": DUAL_CHUNK_SWAP, "no_load_balance": NO_LOAD_BALANCE,
                   DUAL_CHUNK_SWAP: DUAL_CHUNK_SWAP, NO_LOAD_BALANCE: NO_LOAD_BALANCE}

EXPORTED_SYMBOLS = (
    "thdcp_last_error", "thdcp_version", "thdcp_validate", "thd_partition_index", "thd_gather",
    "thd_scatter", "thd_gather_batched", "thd_scatter_batched", "thd_a2a_pack",
    "thd_a2a_unpack", "thdcp_plan_create", "thdcp_plan_get_info", "thdcp_plan_local_seqlens",
    "thdcp_plan_upload", "thdcp_plan_destroy", "cp_attn_fwd", "cp_attn_bwd",
    "cp_attn_bwd_preprocess", "cp_attn_bwd_dkdv", "cp_attn_bwd_dq", "thdcp_zero_untouched",
    "cp_attn_fwd_step", "thdcp_lse_merge", "thdcp_lse_merge_parts", "cp_attn_bwd_step",
    "cp_attn_bwd_noalloc",
)


class ThdcpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libthdcp status {status}: {msg}")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_padded_host", ctypes.POINTER(ctypes.c_int32)),
        ("B", ctypes.c_int32),
        ("T", ctypes.c_int64),
        ("cp_size", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("strategy", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("pad_between_seqs", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("p2p", ctypes.c_int32),
        ("max_key_splits", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("n_local", ctypes.c_int64),
        ("causal_pairs", ctypes.c_int64),
        ("touched_rows", ctypes.c_int64),
        ("untouched_rows", ctypes.c_int64),
        ("padding_present", ctypes.c_int32),
        ("n_fwd_tiles", ctypes.c_int32),
        ("n_bwd_tiles", ctypes.c_int32),
        ("n_zero_ranges", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("bwd_scratch_bytes", ctypes.c_size_t),
        ("n_split_tiles", ctypes.c_int32),
        ("n_fwd_parts", ctypes.c_int32),
        ("fwd_tile_rows", ctypes.c_int32),
        ("bwd_tile_keys", ctypes.c_int32),
    ]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libthdcp.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libthdcp is not built ({LIB_PATH} missing); run "
                          "`python -m context_causal_attention_thd_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    L.thdcp_last_error.restype = ctypes.c_char_p
    L.thdcp_last_error.argtypes = []
    L.thdcp_version.restype = i32
    L.thdcp_validate.restype = i32
    L.thdcp_validate.argtypes = [pi32, pi32, i32, i64, i32, i32, i32, i32, i32, i32, pi32]
    L.thd_partition_index.restype = i32
    L.thd_partition_index.argtypes = [pi32, vp, i32, i64, i32, i32, i32, vp, vp]
    L.thd_gather.restype = i32
    L.thd_gather.argtypes = [vp, i64, vp, i64, i64, vp, vp]
    L.thd_scatter.restype = i32
    L.thd_scatter.argtypes = [vp, i64, vp, i64, vp, i64, vp]
    pvp = ctypes.POINTER(vp)
    L.thd_gather_batched.restype = i32
    L.thd_gather_batched.argtypes = [i32, pvp, i64, vp, i64, i64, pvp, vp]
    L.thd_scatter_batched.restype = i32
    L.thd_scatter_batched.argtypes = [i32, pvp, i64, vp, i64, pvp, i64, vp]
    for name in ("thd_a2a_pack", "thd_a2a_unpack"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = [i32, pvp, i64, i32, i64, pvp, vp]
    L.thdcp_plan_create.restype = i32
    L.thdcp_plan_create.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(vp)]
    L.thdcp_plan_get_info.restype = i32
    L.thdcp_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.thdcp_plan_local_seqlens.restype = i32
    L.thdcp_plan_local_seqlens.argtypes = [vp, pi32]
    L.thdcp_plan_upload.restype = i32
    L.thdcp_plan_upload.argtypes = [vp, vp, sz, vp]
    L.thdcp_plan_destroy.restype = None
    L.thdcp_plan_destroy.argtypes = [vp]
    L.cp_attn_fwd.restype = i32
    L.cp_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.cp_attn_bwd.restype = i32
    L.cp_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp]
    L.cp_attn_bwd_noalloc.restype = i32
    L.cp_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp]
    L.cp_attn_bwd_preprocess.restype = i32
    L.cp_attn_bwd_preprocess.argtypes = [vp, vp, vp, vp, vp, sz, vp]
    L.cp_attn_bwd_dkdv.restype = i32
    L.cp_attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.cp_attn_bwd_dq.restype = i32
    L.cp_attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.thdcp_zero_untouched.restype = i32
    L.thdcp_zero_untouched.argtypes = [vp, vp, vp, vp]
    L.cp_attn_fwd_step.restype = i32
    L.cp_attn_fwd_step.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
    L.thdcp_lse_merge.restype = i32
    L.thdcp_lse_merge.argtypes = [i64, i32, i32, vp, vp, vp, vp, i32, vp, vp]
    L.thdcp_lse_merge_parts.restype = i32
    L.thdcp_lse_merge_parts.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp]
    L.cp_attn_bwd_step.restype = i32
    L.cp_attn_bwd_step.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, sz, vp, i32, vp, vp, i32,
                                   vp]
    _lib_handle = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise ThdcpError(status, lib().thdcp_last_error().decode(errors="replace"))


def _i32_host(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i32_ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _strategy(s) -> int:
    try:
        return _STRATEGY_NAMES[s]
    except KeyError:
        raise ValueError(f"unknown strategy {s!r}") from None


# Row order of K/V in and dK/dV out of the attention calls (thdcp_kv_layout_t).
KV_LAYOUTS = {"global": 0, "rank_major": 1}


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name: str, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# Metadata
# ---------------------------------------------------------------------------

def validate(cu_seqlens, cu_seqlens_padded, T: int, cp_size: int, rank: int, strategy,
             window=(-1, 0), pad_between_seqs: int = -1) -> bool:
    """Check the THD layout rules; returns whether padding is present (by value)."""
    cup = _i32_host(cu_seqlens_padded)
    cu = None if cu_seqlens is None else _i32_host(cu_seqlens)
    out = ctypes.c_int32(0)
    _check(lib().thdcp_validate(_i32_ptr(cu), _i32_ptr(cup), len(cup) - 1, int(T), int(cp_size),
                                int(rank), _strategy(strategy), int(window[0]), int(window[1]),
                                int(pad_between_seqs), ctypes.byref(out)))
    return bool(out.value)


def partition_index(cu_seqlens_padded_host, cu_seqlens_padded_dev, T: int, cp_size: int,
                    rank: int, strategy, out=None, stream=None, validate_host: bool = True):
    """int32 device tensor [T/cp_size] (rank >= 0) or [T] (rank == -1, rank-major)."""
    import torch
    cup = _i32_host(cu_seqlens_padded_host)
    n = int(T) if rank < 0 else int(T) // int(cp_size)
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=cu_seqlens_padded_dev.device)
    _check(lib().thd_partition_index(_i32_ptr(cup) if validate_host else None,
                                     _dev_ptr(cu_seqlens_padded_dev, "cu_seqlens_padded_dev",
                                              torch.int32),
                                     len(cup) - 1, int(T), int(cp_size), int(rank),
                                     _strategy(strategy),
                                     _dev_ptr(out, "out", torch.int32), _stream(stream)))
    return out


def _row_bytes(t) -> int:
    return t[0].numel() * t.element_size() if t.shape[0] > 0 else (
        int(np.prod(t.shape[1:])) * t.element_size())


def gather(src, idx, out=None, stream=None):
    """out[m] = src[idx[m]] over the leading dimension (any dtype)."""
    import torch
    if out is None:
        out = torch.empty((idx.shape[0],) + tuple(src.shape[1:]), dtype=src.dtype,
                          device=src.device)
    rb = _row_bytes(src)
    if _row_bytes(out) != rb:
        raise ValueError("src and out rows differ in size")
    _idx_rows(idx, out.shape[0], "out")
    _check(lib().thd_gather(_dev_ptr(src, "src"), src.shape[0], _dev_ptr(idx, "idx", torch.int32),
                            idx.shape[0], rb, _dev_ptr(out, "out"), _stream(stream)))
    return out


def scatter(src, idx, out, stream=None):
    """out[idx[m]] = src[m] over the leading dimension (any dtype)."""
    import torch
    rb = _row_bytes(src)
    if _row_bytes(out) != rb:
        raise ValueError("src and out rows differ in size")
    _idx_rows(idx, src.shape[0], "src")
    _check(lib().thd_scatter(_dev_ptr(src, "src"), src.shape[0],
                             _dev_ptr(idx, "idx", torch.int32), rb, _dev_ptr(out, "out"),
                             out.shape[0], _stream(stream)))
    return out


def _idx_rows(idx, rows: int, name: str):
    """The index is 1-D with one entry per row of ``name`` (the gather's
    output or the scatter's input): the kernel walks idx.shape[0] rows of it."""
    if idx.dim() != 1:
        raise ValueError(f"idx must be 1-D, got shape {tuple(idx.shape)}")
    if idx.shape[0] != rows:
        raise ValueError(f"idx has {idx.shape[0]} entries but {name} has {rows} rows")


def _ptr_list(ts, name):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _dev_ptr(t, f"{name}[{i}]").value
    return arr


def gather_many(srcs, idx, outs=None, stream=None):
    """outs[i][m] = srcs[i][idx[m]] for 1..4 same-shaped tensors, one launch."""
    import torch
    if outs is None:
        outs = [torch.empty((idx.shape[0],) + tuple(s.shape[1:]), dtype=s.dtype,
                            device=s.device) for s in srcs]
    rb = _row_bytes(srcs[0])
    if any(_row_bytes(x) != rb for x in list(srcs) + list(outs)):
        raise ValueError("all rows must have the same size")
    if any(x.shape[0] != srcs[0].shape[0] for x in srcs):
        raise ValueError("all sources must have the same number of rows")
    for i, x in enumerate(outs):
        _idx_rows(idx, x.shape[0], f"outs[{i}]")
    _check(lib().thd_gather_batched(len(srcs), _ptr_list(srcs, "src"), srcs[0].shape[0],
                                    _dev_ptr(idx, "idx", torch.int32), idx.shape[0], rb,
                                    _ptr_list(outs, "out"), _stream(stream)))
    return outs


def scatter_many(srcs, idx, outs, stream=None):
    """outs[i][idx[m]] = srcs[i][m] for 1..4 same-shaped tensors, one launch."""
    import torch
    rb = _row_bytes(srcs[0])
    if any(_row_bytes(x) != rb for x in list(srcs) + list(outs)):
        raise ValueError("all rows must have the same size")
    if any(x.shape[0] != outs[0].shape[0] for x in outs):
        raise ValueError("all destinations must have the same number of rows")
    for i, x in enumerate(srcs):
        _idx_rows(idx, x.shape[0], f"srcs[{i}]")
    _check(lib().thd_scatter_batched(len(srcs), _ptr_list(srcs, "src"), srcs[0].shape[0],
                                     _dev_ptr(idx, "idx", torch.int32), rb,
                                     _ptr_list(outs, "out"), outs[0].shape[0], _stream(stream)))
    return outs


def a2a_pack(srcs, cp_size: int, outs=None, stream=None):
    """Head-group pack before the all-to-all: each src [n, H, ...] becomes
    [cp_size, n, H // cp_size, ...] with block c = head group c of every token
    (the send buffer for rank c). 1..4 same-shaped tensors, one launch."""
    import torch
    n, H = srcs[0].shape[0], srcs[0].shape[1]
    if H % cp_size != 0:
        raise ValueError(f"heads ({H}) not divisible by cp_size ({cp_size})")
    shape = (cp_size, n, H // cp_size) + tuple(srcs[0].shape[2:])
    if any(tuple(x.shape) != tuple(srcs[0].shape) or x.dtype != srcs[0].dtype for x in srcs):
        raise ValueError("all sources must have the same shape and dtype")
    if outs is None:
        outs = [torch.empty(shape, dtype=x.dtype, device=x.device) for x in srcs]
    if any(tuple(o.shape) != shape or o.dtype != srcs[0].dtype for o in outs):
        raise ValueError(f"outputs must be {shape}")
    gb = (_row_bytes(srcs[0]) // cp_size) if n > 0 else 1
    _check(lib().thd_a2a_pack(len(srcs), _ptr_list(srcs, "src"), n, cp_size, gb,
                              _ptr_list(outs, "out"), _stream(stream)))
    return outs


def a2a_unpack(srcs, outs=None, stream=None):
    """Inverse of a2a_pack: each src [cp, n, Hl, ...] (block c = head group c
    received from rank c) becomes [n, cp * Hl, ...]."""
    import torch
    cp, n, Hl = srcs[0].shape[0], srcs[0].shape[1], srcs[0].shape[2]
    shape = (n, cp * Hl) + tuple(srcs[0].shape[3:])
    if any(tuple(x.shape) != tuple(srcs[0].shape) or x.dtype != srcs[0].dtype for x in srcs):
        raise ValueError("all sources must have the same shape and dtype")
    if outs is None:
        outs = [torch.empty(shape, dtype=x.dtype, device=x.device) for x in srcs]
    if any(tuple(o.shape) != shape or o.dtype != srcs[0].dtype for o in outs):
        raise ValueError(f"outputs must be {shape}")
    gb = int(np.prod(srcs[0].shape[2:])) * srcs[0].element_size()
    _check(lib().thd_a2a_unpack(len(srcs), _ptr_list(srcs, "src"), n, cp, max(gb, 1),
                                _ptr_list(outs, "out"), _stream(stream)))
    return outs


# ---------------------------------------------------------------------------
# Plan + attention
# ---------------------------------------------------------------------------

class Plan:
    """Host plan + its device workspace (a torch uint8 tensor)."""

    def __init__(self, cu_seqlens, cu_seqlens_padded, T: int, cp_size: int, rank: int, strategy,
                 H: int, D: int, softmax_scale: float = 0.0, window=(-1, 0),
                 pad_between_seqs: int = -1, device=None, stream=None, upload: bool = True,
                 kv_layout: str = "global", p2p: bool = False, max_key_splits: int = 0):
        self._cup = _i32_host(cu_seqlens_padded)
        self._cu = None if cu_seqlens is None else _i32_host(cu_seqlens)
        d = _Desc()
        d.cu_seqlens_host = _i32_ptr(self._cu)
        d.cu_seqlens_padded_host = _i32_ptr(self._cup)
        d.B = len(self._cup) - 1
        d.T = int(T)
        d.cp_size = int(cp_size)
        d.rank = int(rank)
        d.strategy = _strategy(strategy)
        d.H = int(H)
        d.D = int(D)
        d.softmax_scale = float(softmax_scale)
        d.window_left, d.window_right = int(window[0]), int(window[1])
        d.pad_between_seqs = int(pad_between_seqs)
        if kv_layout not in KV_LAYOUTS:
            raise ValueError(f"unknown kv_layout {kv_layout!r} (one of {sorted(KV_LAYOUTS)})")
        d.kv_layout = KV_LAYOUTS[kv_layout]
        self.kv_layout = kv_layout
        d.p2p = int(bool(p2p))
        self.p2p = bool(p2p)
        d.max_key_splits = int(max_key_splits)
        self._handle = ctypes.c_void_p()
        _check(lib().thdcp_plan_create(ctypes.byref(d), ctypes.byref(self._handle)))
        self.T, self.H, self.D, self.cp_size, self.rank = int(T), int(H), int(D), cp_size, rank
        self.info = PlanInfo()
        _check(lib().thdcp_plan_get_info(self._handle, ctypes.byref(self.info)))
        self.n_local = int(self.info.n_local)
        self.workspace = None
        if upload:
            self.upload(device=device, stream=stream)

    def upload(self, device=None, stream=None):
        import torch
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        nbytes = int(self.info.workspace_bytes)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        base = self.workspace.data_ptr()
        aligned = (base + 255) & ~255
        _check(lib().thdcp_plan_upload(self._handle, ctypes.c_void_p(aligned), nbytes,
                                       _stream(stream)))
        return self

    def upload_into(self, workspace, stream=None):
        """Upload into a caller-owned uint8 device tensor (no allocation)."""
        import torch
        nbytes = int(self.info.workspace_bytes)
        base = _dev_ptr(workspace, "workspace", torch.uint8).value
        aligned = (base + 255) & ~255
        if aligned + nbytes > base + workspace.numel():
            raise ValueError("workspace too small")
        self.workspace = workspace
        _check(lib().thdcp_plan_upload(self._handle, ctypes.c_void_p(aligned), nbytes,
                                       _stream(stream)))
        return self

    def local_seqlens(self) -> np.ndarray:
        out = np.zeros(len(self._cup) - 1, dtype=np.int32)
        _check(lib().thdcp_plan_local_seqlens(self._handle, _i32_ptr(out)))
        return out

    def close(self):
        if self._handle is not None and self._handle.value:
            lib().thdcp_plan_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._handle


def attn_fwd(plan: Plan, q_local, k, v, o=None, lse=None, stream=None):
    """O bf16 [n_local,H,D] and LSE fp32 [H,n_local]."""
    import torch
    n, H, D, T = plan.n_local, plan.H, plan.D, plan.T
    if o is None:
        o = torch.empty((n, H, D), dtype=torch.bfloat16, device=q_local.device)
    if lse is None:
        lse = torch.empty((H, n), dtype=torch.float32, device=q_local.device)
    bf, f32 = torch.bfloat16, torch.float32
    ptrs = _args((q_local, (n, H, D), bf, "q_local"), (k, (T, H, D), bf, "k"),
                 (v, (T, H, D), bf, "v"), (o, (n, H, D), bf, "o"), (lse, (H, n), f32, "lse"))
    _check(lib().cp_attn_fwd(plan.handle, *ptrs, _stream(stream)))
    return o, lse


def attn_bwd(plan: Plan, q_local, k, v, o, lse, d_o, dq=None, dk=None, dv=None,
             zero_untouched: bool = True, accumulate_dkv: bool = False, scratch=None,
             stream=None):
    """dQ fp32 [n_local,H,D]; dK, dV fp32 [T,H,D] (this rank's partials)."""
    import torch
    n, H, D, T = plan.n_local, plan.H, plan.D, plan.T
    dev = q_local.device
    if dq is None:
        dq = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    if dk is None:
        dk = (torch.empty if zero_untouched else torch.zeros)((T, H, D), dtype=torch.float32,
                                                              device=dev)
    if dv is None:
        dv = (torch.empty if zero_untouched else torch.zeros)((T, H, D), dtype=torch.float32,
                                                              device=dev)
    need = int(plan.info.bwd_scratch_bytes)
    if scratch is None:
        scratch = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    q_p, k_p, v_p, lse_p, do_p, o_p, dq_p, dk_p, dv_p = _bwd_ptrs(
        plan, q_local, k, v, lse, d_o, o, dq, dk, dv)
    _check(lib().cp_attn_bwd(plan.handle, q_p, k_p, v_p, o_p, lse_p, do_p, dq_p, dk_p, dv_p,
                             int(bool(zero_untouched)), int(bool(accumulate_dkv)),
                             _dev_ptr(scratch, "scratch"),
                             scratch.numel() * scratch.element_size(), _stream(stream)))
    return dq, dk, dv


def attn_bwd_noalloc(plan: Plan, q_local, k, v, o, lse, d_o, dq, dk, dv,
                     zero_untouched: bool = True, accumulate_dkv: bool = False, stream=None):
    """cp_attn_bwd_noalloc: attn_bwd with its scratch in the library's fixed
    device array (no scratch argument, nothing allocated). dq, dk and dv are
    the caller's preallocated outputs."""
    q_p, k_p, v_p, lse_p, do_p, o_p, dq_p, dk_p, dv_p = _bwd_ptrs(
        plan, q_local, k, v, lse, d_o, o, dq, dk, dv)
    _check(lib().cp_attn_bwd_noalloc(plan.handle, q_p, k_p, v_p, o_p, lse_p, do_p, dq_p, dk_p,
                                     dv_p, int(bool(zero_untouched)), int(bool(accumulate_dkv)),
                                     _stream(stream)))
    return dq, dk, dv


def _bwd_ptrs(plan: Plan, q_local, k, v, lse, d_o, o, dq, dk, dv):
    """Checked pointers of a backward call's tensors, in this order."""
    import torch
    n, H, D, T = plan.n_local, plan.H, plan.D, plan.T
    bf, f32 = torch.bfloat16, torch.float32
    return _args((q_local, (n, H, D), bf, "q_local"), (k, (T, H, D), bf, "k"),
                 (v, (T, H, D), bf, "v"), (lse, (H, n), f32, "lse"),
                 (d_o, (n, H, D), bf, "d_o"), (o, (n, H, D), bf, "o"),
                 (dq, (n, H, D), f32, "dq"), (dk, (T, H, D), f32, "dk"),
                 (dv, (T, H, D), f32, "dv"))


def attn_bwd_parts(plan: Plan, q_local, k, v, o, lse, d_o, dq, dk, dv, scratch,
                   zero_untouched: bool = True, accumulate_dkv: bool = False, stream=None,
                   events=None):
    """cp_attn_bwd as its separate launches. ``events`` (optional dict of
    torch.cuda.Event pairs, keys "dkdv" and "dq") are recorded around those
    two kernels."""
    import torch
    L = lib()
    ptrs = _bwd_ptrs(plan, q_local, k, v, lse, d_o, o, dq, dk, dv)
    args, (o_p, dq_p, dk_p, dv_p) = ptrs[:5], ptrs[5:]
    st = _stream(stream)
    nbytes = scratch.numel() * scratch.element_size()
    sp = _dev_ptr(scratch, "scratch")
    _check(L.cp_attn_bwd_preprocess(plan.handle, o_p, args[3], args[4], sp, nbytes, st))
    ev = events or {}
    if "dkdv" in ev:
        ev["dkdv"][0].record()
    _check(L.cp_attn_bwd_dkdv(plan.handle, *args, dk_p, dv_p, int(bool(accumulate_dkv)), sp,
                              nbytes, st))
    if "dkdv" in ev:
        ev["dkdv"][1].record()
    if "dq" in ev:
        ev["dq"][0].record()
    _check(L.cp_attn_bwd_dq(plan.handle, *args, dq_p, sp, nbytes, st))
    if "dq" in ev:
        ev["dq"][1].record()
    if zero_untouched:
        _check(L.thdcp_zero_untouched(plan.handle, dk_p, dv_p, st))
    return dq, dk, dv


def bwd_preprocess(plan: Plan, o, lse, d_o, scratch, stream=None):
    """delta = rowsum(O * dO) into ``scratch`` (cp_attn_bwd_preprocess)."""
    import torch
    n, H, D = plan.n_local, plan.H, plan.D
    _check(lib().cp_attn_bwd_preprocess(plan.handle,
                                        *_args((o, (n, H, D), torch.bfloat16, "o"),
                                               (lse, (H, n), torch.float32, "lse"),
                                               (d_o, (n, H, D), torch.bfloat16, "d_o")),
                                        _dev_ptr(scratch, "scratch"),
                                        scratch.numel() * scratch.element_size(),
                                        _stream(stream)))
    return scratch


# ---------------------------------------------------------------------------
# Dense layouts as THD views (no copies)
# ---------------------------------------------------------------------------
# Attention is independent per (batch element, head), so a dense tensor is a
# THD buffer under a reshape: bshd [B, S, H, D] is B documents of S tokens
# with H heads; sbhd [S, B, H, D] is one document of S tokens with B*H heads
# (the row of position s holds every batch element's heads). CP shards the
# sequence dimension of every batch element: for sbhd under either strategy,
# and for bshd under DUAL_CHUNK_SWAP, that is the THD partition of the view.
# bshd with B > 1 under NO_LOAD_BALANCE is not (the THD partition would cut
# the packed B*S rows instead of each sequence) and is refused.

def dense_as_thd(layout: str, B: int, S: int, H: int):
    """(cu_seqlens int32 [docs+1], heads) of the THD view of a dense layout."""
    if layout == "bshd":
        return np.arange(0, (B + 1) * S, S, dtype=np.int32)[:B + 1], int(H)
    if layout == "sbhd":
        return np.array([0, S], dtype=np.int32), int(B) * int(H)
    raise ValueError(f"unknown dense layout {layout!r} (bshd or sbhd)")


def dense_view(x, layout: str):
    """[rows, heads, D] view of a contiguous bshd or sbhd tensor."""
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError("expected a contiguous 4-D tensor")
    a, b, h, d = x.shape
    if layout == "bshd":
        return x.view(a * b, h, d)
    if layout == "sbhd":
        return x.view(a, b * h, d)
    raise ValueError(f"unknown dense layout {layout!r} (bshd or sbhd)")


def dense_plan(layout: str, B: int, S: int, H: int, D: int, cp_size: int, rank: int, strategy,
               **kw) -> "Plan":
    """Plan for one rank of a dense bshd/sbhd batch (its THD view)."""
    cu, heads = dense_as_thd(layout, B, S, H)
    if layout == "bshd" and B > 1 and _strategy(strategy) == 1:
        raise ValueError("bshd with batch > 1 under NO_LOAD_BALANCE shards each sequence, "
                         "which its THD view does not: pass the batch as sbhd")
    T = int(cu[-1])
    return Plan(cu, cu, T, cp_size, rank, strategy, heads, D, **kw)


# ---------------------------------------------------------------------------
# P2P (ring) steps: the plan must be made with p2p=True
# ---------------------------------------------------------------------------

def attn_fwd_step(plan: Plan, src_rank: int, q_local, k_src, v_src, o_part=None, lse_part=None,
                  stream=None):
    """One ring step: local queries against rank src_rank's local K/V
    ([n_local,H,D] each, in that rank's local order). Returns (o_part bf16
    [n_local,H,D], lse_part fp32 [H,n_local]); rows with no key in the step
    get O = 0, LSE = -inf."""
    import torch
    n, H, D = plan.n_local, plan.H, plan.D
    _shape(q_local, (n, H, D), "q_local")
    _shape(k_src, (n, H, D), "k_src")
    _shape(v_src, (n, H, D), "v_src")
    dev = q_local.device
    if o_part is None:
        o_part = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    if lse_part is None:
        lse_part = torch.empty((H, n), dtype=torch.float32, device=dev)
    _shape(o_part, (n, H, D), "o_part")
    _shape(lse_part, (H, n), "lse_part")
    _check(lib().cp_attn_fwd_step(plan.handle, int(src_rank),
                                  _dev_ptr(q_local, "q_local", torch.bfloat16),
                                  _dev_ptr(k_src, "k_src", torch.bfloat16),
                                  _dev_ptr(v_src, "v_src", torch.bfloat16),
                                  _dev_ptr(o_part, "o_part", torch.bfloat16),
                                  _dev_ptr(lse_part, "lse_part", torch.float32),
                                  _stream(stream)))
    return o_part, lse_part


def lse_merge(o_part, lse_part, o_acc, lse_acc, first: bool, o_out=None, stream=None):
    """Fold one step's (o_part, lse_part) into (o_acc fp32, lse_acc fp32);
    o_out (bf16, optional) receives the merged output."""
    import torch
    n, H, D = o_part.shape
    _shape(lse_part, (H, n), "lse_part")
    _shape(o_acc, (n, H, D), "o_acc")
    _shape(lse_acc, (H, n), "lse_acc")
    if o_out is not None:
        _shape(o_out, (n, H, D), "o_out")
    _check(lib().thdcp_lse_merge(int(n), int(H), int(D),
                                 _dev_ptr(o_part, "o_part", torch.bfloat16),
                                 _dev_ptr(lse_part, "lse_part", torch.float32),
                                 _dev_ptr(o_acc, "o_acc", torch.float32),
                                 _dev_ptr(lse_acc, "lse_acc", torch.float32), int(bool(first)),
                                 None if o_out is None else _dev_ptr(o_out, "o_out",
                                                                     torch.bfloat16),
                                 _stream(stream)))
    return o_acc, lse_acc


def lse_merge_parts(o_parts, lse_parts, o_out=None, lse_out=None, stream=None):
    """Merge all step results at once: o_parts bf16 [parts, n, H, D], lse_parts
    fp32 [parts, H, n] -> (o_out bf16 [n, H, D], lse_out fp32 [H, n])."""
    import torch
    parts, n, H, D = o_parts.shape
    _shape(lse_parts, (parts, H, n), "lse_parts")
    if o_out is None:
        o_out = torch.empty((n, H, D), dtype=torch.bfloat16, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty((H, n), dtype=torch.float32, device=o_parts.device)
    _shape(o_out, (n, H, D), "o_out")
    _shape(lse_out, (H, n), "lse_out")
    _check(lib().thdcp_lse_merge_parts(int(n), int(H), int(D), int(parts),
                                       _dev_ptr(o_parts, "o_parts", torch.bfloat16),
                                       _dev_ptr(lse_parts, "lse_parts", torch.float32),
                                       _dev_ptr(o_out, "o_out", torch.bfloat16),
                                       _dev_ptr(lse_out, "lse_out", torch.float32),
                                       _stream(stream)))
    return o_out, lse_out


def attn_bwd_step(plan: Plan, src_rank: int, q_local, k_src, v_src, lse, d_o, scratch, dq,
                  accumulate_dq: bool, dk_src=None, dv_src=None, zero_untouched: bool = True,
                  stream=None):
    """Backward of one ring step with the merged LSE; ``scratch`` holds delta
    of the merged output (bwd_preprocess). dq fp32 [n_local,H,D] is written or
    added to; returns (dq, dk_src, dv_src), the last two fp32 [n_local,H,D] in
    rank src_rank's local order."""
    import torch
    n, H, D = plan.n_local, plan.H, plan.D
    _shape(q_local, (n, H, D), "q_local")
    _shape(k_src, (n, H, D), "k_src")
    _shape(v_src, (n, H, D), "v_src")
    _shape(lse, (H, n), "lse")
    _shape(d_o, (n, H, D), "d_o")
    _shape(dq, (n, H, D), "dq")
    dev = q_local.device
    mk = torch.empty if zero_untouched else torch.zeros
    if dk_src is None:
        dk_src = mk((n, H, D), dtype=torch.float32, device=dev)
    if dv_src is None:
        dv_src = mk((n, H, D), dtype=torch.float32, device=dev)
    _shape(dk_src, (n, H, D), "dk_src")
    _shape(dv_src, (n, H, D), "dv_src")
    _check(lib().cp_attn_bwd_step(plan.handle, int(src_rank),
                                  _dev_ptr(q_local, "q_local", torch.bfloat16),
                                  _dev_ptr(k_src, "k_src", torch.bfloat16),
                                  _dev_ptr(v_src, "v_src", torch.bfloat16),
                                  _dev_ptr(lse, "lse", torch.float32),
                                  _dev_ptr(d_o, "d_o", torch.bfloat16),
                                  _dev_ptr(scratch, "scratch"),
                                  scratch.numel() * scratch.element_size(),
                                  _dev_ptr(dq, "dq", torch.float32), int(bool(accumulate_dq)),
                                  _dev_ptr(dk_src, "dk_src", torch.float32),
                                  _dev_ptr(dv_src, "dv_src", torch.float32),
                                  int(bool(zero_untouched)), _stream(stream)))
    return dq, dk_src, dv_src


def _shape(t, shape: Sequence[int], name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _args(*specs):
    """Device pointers of tensor arguments given as (tensor, shape, dtype,
    name): every shape is checked first (ValueError), then dtype, device and
    contiguity (TypeError / ValueError). The C ABI takes raw pointers with no
    sizes, so an undersized buffer must be refused here, before a kernel
    writes past its end."""
    for t, shape, _, name in specs:
        _shape(t, shape, name)
    return tuple(_dev_ptr(t, name, dtype) for t, _, dtype, name in specs)
