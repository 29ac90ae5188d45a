"""Python binding of libdlrm_mi355x.so, the MI355X (gfx950) DLRMv1 forward hot path.

Thin ctypes marshalling over the C ABI declared in ``include/dlrm_mi355x.h``:
every step of the computation runs in the library's HIP kernels.  PyTorch is
used only to hold device memory and to name the current HIP stream.  The
binding never falls back to another implementation: if the library is missing
or a call fails, it raises.

Functions take CUDA (HIP) torch tensors:

* ``embbag_sum(tables, indices, offsets)`` -> (B, T, D)
* ``interact_lower_tri(x, emb, concat_dense=True)`` -> (B, D + P) or (B, P)
* ``linear_bias_act(x, W, bias, act)`` -> (M, N)
* ``Model(...)`` holding DLRMv1 parameters, with ``forward(dense, indices, offsets)``
* ``check_indices(...)``, ``pair_index_map(F)``, ``workspace_bytes``
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libdlrm_mi355x.so")

DLRM_OK, DLRM_E_NULL, DLRM_E_SHAPE, DLRM_E_WORKSPACE, DLRM_E_UNSUPPORTED, DLRM_E_HIP, DLRM_E_INDEX = range(7)
ACT_NONE, ACT_RELU, ACT_SIGMOID = 0, 1, 2
MAX_TABLES = 64
ABI_VERSION = 3

_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


class DlrmError(RuntimeError):
    def __init__(self, code: int, what: str, msg: str):
        super().__init__(f"{what}: {msg}")
        self.code = code


class _BagOptions(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("include_last_offset", ctypes.c_int32), ("index_bytes", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("padding_idx", _i64p), ("per_sample_weights", ctypes.POINTER(_vp))]


BAG_MODES = {"sum": 0, "mean": 1, "max": 2}


class _Model(ctypes.Structure):
    _fields_ = [
        ("n_bot", ctypes.c_int32), ("ln_bot", _i64p),
        ("n_top", ctypes.c_int32), ("ln_top", _i64p),
        ("num_tables", ctypes.c_int32), ("emb_dim", ctypes.c_int32),
        ("rows", _i64p),
        ("emb_w", ctypes.POINTER(_vp)),
        ("bot_w", ctypes.POINTER(_vp)), ("bot_b", ctypes.POINTER(_vp)),
        ("top_w", ctypes.POINTER(_vp)), ("top_b", ctypes.POINTER(_vp)),
        ("packed_w", _vp),
        ("emb_stacked", _vp), ("emb_row_base", _i64p),
    ]


_LIB = None


def library_path() -> str:
    return LIBRARY


def load(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load the HIP library (building it with hipcc only if it does not exist)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIBRARY):
        if not build_if_missing:
            raise ImportError(f"{LIBRARY} is not built")
        from . import _build
        _build.build_library()
    L = ctypes.CDLL(LIBRARY)
    L.dlrm_status_string.argtypes = [ctypes.c_int]
    L.dlrm_status_string.restype = ctypes.c_char_p
    L.dlrm_abi_version.argtypes = []
    L.dlrm_abi_version.restype = ctypes.c_int32
    L.dlrm_embbag_sum.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_vp), _i64p,
                                  ctypes.POINTER(_vp), _i64p, ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp]
    L.dlrm_embbag_sum_stacked.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _vp, _i64p, _i64p,
                                          ctypes.POINTER(_vp), _i64p, ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp]
    L.dlrm_embbag.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_vp), _i64p,
                              ctypes.POINTER(_vp), _i64p, ctypes.POINTER(_vp), ctypes.POINTER(_BagOptions), _vp, _vp]
    L.dlrm_interact_lower_tri.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64,
                                          _vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp]
    L.dlrm_embbag_interact.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_vp), _i64p,
                                       ctypes.POINTER(_vp), _i64p, ctypes.POINTER(_vp), ctypes.c_int32, _vp,
                                       ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int32, _vp]
    L.dlrm_linear_bias_act.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp, ctypes.c_int64, _vp,
                                       _vp, ctypes.c_int32, _vp, ctypes.c_int64, _vp]
    L.dlrm_forward_workspace_bytes.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64]
    L.dlrm_forward_workspace_bytes.restype = ctypes.c_size_t
    L.dlrm_forward.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64, _vp, ctypes.POINTER(_vp), _i64p,
                               ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp, ctypes.c_size_t, _vp]
    L.dlrm_forward_layered.argtypes = L.dlrm_forward.argtypes
    L.dlrm_forward_noalloc.argtypes = L.dlrm_forward_fused.argtypes = [
        ctypes.POINTER(_Model), ctypes.c_int64, _vp, ctypes.POINTER(_vp), _i64p, ctypes.POINTER(_vp), ctypes.c_int32,
        _vp, _vp]
    L.dlrm_forward_noalloc_max_bytes.argtypes = []
    L.dlrm_forward_noalloc_max_bytes.restype = ctypes.c_size_t
    L.dlrm_forward_path.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64]
    L.dlrm_forward_path.restype = ctypes.c_int32
    L.dlrm_pack_weights_bytes.argtypes = [ctypes.POINTER(_Model)]
    L.dlrm_pack_weights_bytes.restype = ctypes.c_size_t
    L.dlrm_pack_weights.argtypes = [ctypes.POINTER(_Model), _vp, ctypes.c_size_t, _vp]
    L.dlrm_forward_fused.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64, _vp, ctypes.POINTER(_vp), _i64p,
                                     ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp]
    L.dlrm_embbag_check_indices.argtypes = [ctypes.c_int32, ctypes.c_int64, _i64p, ctypes.POINTER(_vp), _i64p,
                                            ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp]
    L.dlrm_probe_sink_floats.argtypes = []
    L.dlrm_probe_sink_floats.restype = ctypes.c_int64
    L.dlrm_probe_read_stream.argtypes = [_vp, ctypes.c_int64, _vp, _vp]
    L.dlrm_probe_gather_rows.argtypes = [_vp, ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_int64, _vp, _vp]
    L.dlrm_probe_l2_stream.argtypes = [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp]
    L.dlrm_pair_index_map.argtypes = [ctypes.c_int32, _vp, _vp, _vp]
    for f in ("dlrm_embbag_sum", "dlrm_embbag_sum_stacked", "dlrm_embbag", "dlrm_interact_lower_tri",
              "dlrm_embbag_interact", "dlrm_linear_bias_act", "dlrm_forward", "dlrm_forward_layered",
              "dlrm_forward_fused", "dlrm_forward_noalloc", "dlrm_pack_weights", "dlrm_embbag_check_indices",
              "dlrm_pair_index_map",
              "dlrm_probe_read_stream", "dlrm_probe_gather_rows", "dlrm_probe_l2_stream"):
        getattr(L, f).restype = ctypes.c_int
    if L.dlrm_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIBRARY}: ABI version {L.dlrm_abi_version()} != {ABI_VERSION}")
    _LIB = L
    return L


def _check(rc: int, what: str):
    if rc != DLRM_OK:
        msg = load().dlrm_status_string(rc).decode()
        raise DlrmError(rc, what, msg)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _cuda(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    return t


def _index_bytes(indices: Sequence[torch.Tensor], offsets: Sequence[torch.Tensor]) -> int:
    """Check that every index and offset tensor is a contiguous CUDA int32 or
    int64 tensor of one common dtype; return its width in bytes."""
    itype = indices[0].dtype if len(indices) else torch.int64
    if itype not in (torch.int32, torch.int64):
        raise TypeError("indices must be int32 or int64")
    for i, (ix, of) in enumerate(zip(indices, offsets)):
        _dev(ix, itype, f"indices[{i}]")
        _dev(of, itype, f"offsets[{i}]")
    return 4 if itype == torch.int32 else 8


def _ptrs(ts: Sequence[torch.Tensor]):
    return (_vp * max(len(ts), 1))(*[t.data_ptr() for t in ts])


def _i64s(vs: Sequence[int]):
    return (ctypes.c_int64 * max(len(vs), 1))(*[int(v) for v in vs])


# --- the four hot-path calls -----------------------------------------------------


def embbag_sum(tables: List[torch.Tensor], indices: List[torch.Tensor], offsets: List[torch.Tensor],
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sum-pooled bags of every table in one launch -> (B, T, D) fp32.
    Indices and offsets are all int64 or all int32."""
    L = load()
    T = len(tables)
    if not (T == len(indices) == len(offsets)) or T == 0:
        raise ValueError("tables, indices and offsets must have the same non-zero length")
    for i, t in enumerate(tables):
        _dev(t, torch.float32, f"tables[{i}]")
        if t.dim() != 2:
            raise ValueError(f"tables[{i}] must be 2-D")
    ib = _index_bytes(indices, offsets)
    D = tables[0].shape[1]
    B = offsets[0].shape[0]
    if out is None:
        out = torch.empty((B, T, D), device=tables[0].device, dtype=torch.float32)
    _dev(out, torch.float32, "out")
    if tuple(out.shape) != (B, T, D) or any(t.shape[1] != D for t in tables) or any(o.shape[0] != B for o in offsets):
        raise ValueError("shape mismatch")
    rc = L.dlrm_embbag_sum(T, B, D, _ptrs(tables), _i64s([t.shape[0] for t in tables]), _ptrs(indices),
                           _i64s([i.numel() for i in indices]), _ptrs(offsets), ib, out.data_ptr(),
                           _stream(out.device))
    _check(rc, "dlrm_embbag_sum")
    return out


def embbag_sum_stacked(stacked: torch.Tensor, rows: Sequence[int], indices: List[torch.Tensor],
                       offsets: List[torch.Tensor], row_base: Optional[Sequence[int]] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dlrm_embbag_sum over tables stacked in one (sum of rows, D) tensor:
    table t is rows [row_base[t], row_base[t] + rows[t]) (row_base defaults to
    the running sum of rows).  Indices are relative to their own table."""
    L = load()
    T = len(rows)
    if not (T == len(indices) == len(offsets)) or T == 0:
        raise ValueError("rows, indices and offsets must have the same non-zero length")
    _dev(stacked, torch.float32, "stacked")
    if stacked.dim() != 2:
        raise ValueError("stacked must be 2-D")
    if row_base is None:
        row_base = [sum(rows[:t]) for t in range(T)]
    if any(int(b) < 0 or int(b) + int(r) > stacked.shape[0] for b, r in zip(row_base, rows)):
        raise ValueError("a table's rows run past the stacked tensor")
    ib = _index_bytes(indices, offsets)
    D = stacked.shape[1]
    B = offsets[0].shape[0]
    if out is None:
        out = torch.empty((B, T, D), device=stacked.device, dtype=torch.float32)
    _dev(out, torch.float32, "out")
    if tuple(out.shape) != (B, T, D) or any(o.shape[0] != B for o in offsets):
        raise ValueError("shape mismatch")
    rc = L.dlrm_embbag_sum_stacked(T, B, D, stacked.data_ptr(), _i64s(row_base), _i64s(rows), _ptrs(indices),
                                   _i64s([i.numel() for i in indices]), _ptrs(offsets), ib, out.data_ptr(),
                                   _stream(out.device))
    _check(rc, "dlrm_embbag_sum_stacked")
    return out


def embbag(tables: List[torch.Tensor], indices: List[torch.Tensor], offsets: List[torch.Tensor],
           mode: str = "sum", include_last_offset: bool = False, padding_idx=None,
           per_sample_weights: Optional[List[torch.Tensor]] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """General bags of every table in one launch -> (B, T, D) fp32.

    mode 'sum' | 'mean' | 'max'; per_sample_weights (sum only) one fp32 tensor
    per table; include_last_offset: offsets hold B + 1 entries; padding_idx an
    int or one int / None per table.  Indices and offsets are all int64 or all
    int32."""
    L = load()
    T = len(tables)
    if not (T == len(indices) == len(offsets)) or T == 0:
        raise ValueError("tables, indices and offsets must have the same non-zero length")
    itype = indices[0].dtype
    if itype not in (torch.int32, torch.int64):
        raise TypeError("indices must be int32 or int64")
    for i, t in enumerate(tables):
        _dev(t, torch.float32, f"tables[{i}]")
        _dev(indices[i], itype, f"indices[{i}]")
        _dev(offsets[i], itype, f"offsets[{i}]")
    D = tables[0].shape[1]
    B = offsets[0].shape[0] - (1 if include_last_offset else 0)
    if out is None:
        out = torch.empty((B, T, D), device=tables[0].device, dtype=torch.float32)
    _dev(out, torch.float32, "out")
    if tuple(out.shape) != (B, T, D) or any(t.shape[1] != D for t in tables):
        raise ValueError("shape mismatch")
    opts = _BagOptions(BAG_MODES[mode], int(bool(include_last_offset)), 4 if itype == torch.int32 else 8, 0)
    keep = []
    if padding_idx is not None:
        pads = padding_idx if isinstance(padding_idx, (list, tuple)) else [padding_idx] * T
        arr = _i64s([-1 if p is None else int(p) for p in pads])
        keep.append(arr)
        opts.padding_idx = ctypes.cast(arr, _i64p)
    if per_sample_weights is not None:
        for i, w in enumerate(per_sample_weights):
            _dev(w, torch.float32, f"per_sample_weights[{i}]")
        arr = _ptrs(per_sample_weights)
        keep.append(arr)
        opts.per_sample_weights = ctypes.cast(arr, ctypes.POINTER(_vp))
    rc = L.dlrm_embbag(T, B, D, _ptrs(tables), _i64s([t.shape[0] for t in tables]), _ptrs(indices),
                       _i64s([i.numel() for i in indices]), _ptrs(offsets), ctypes.byref(opts), out.data_ptr(),
                       _stream(out.device))
    _check(rc, "dlrm_embbag")
    return out


def n_pairs(n_feat: int) -> int:
    return n_feat * (n_feat - 1) // 2


def interact_lower_tri(x: torch.Tensor, emb: torch.Tensor, concat_dense: bool = True,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Strict-lower-triangle dots over [x, emb[:, 0], ...] -> [x | Z] (or Z)."""
    L = load()
    if x.dim() != 2 or emb.dim() != 3:
        raise ValueError("x must be (B, >=D) and emb (B, T, D)")
    B, T, D = emb.shape
    if x.device.type != "cuda" or x.dtype != torch.float32 or x.stride(1) != 1 or x.shape[0] != B or x.shape[1] < D:
        raise ValueError("x must be a (B, >=D) fp32 CUDA tensor with unit column stride")
    _dev(emb, torch.float32, "emb")
    P = n_pairs(T + 1)
    width = D + P if concat_dense else P
    if out is None:
        out = torch.empty((B, width), device=emb.device, dtype=torch.float32)
    _cuda(out, "out")
    if out.dtype != torch.float32 or out.stride(1) != 1 or out.shape[0] != B or out.shape[1] < width:
        raise ValueError("out must be (B, >= width) fp32 with unit column stride")
    rc = L.dlrm_interact_lower_tri(B, T, D, x.data_ptr(), x.stride(0), emb.data_ptr(), out.data_ptr(),
                                   out.stride(0), int(bool(concat_dense)), _stream(emb.device))
    _check(rc, "dlrm_interact_lower_tri")
    return out


def embbag_interact(tables: List[torch.Tensor], indices: List[torch.Tensor], offsets: List[torch.Tensor],
                    x: torch.Tensor, concat_dense: bool = True, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Bags gathered and dotted in one launch -> [x | Z] (or Z); E is never materialised."""
    L = load()
    T = len(tables)
    if not (T == len(indices) == len(offsets)) or T == 0:
        raise ValueError("tables, indices and offsets must have the same non-zero length")
    for i, t in enumerate(tables):
        _dev(t, torch.float32, f"tables[{i}]")
        if t.dim() != 2:
            raise ValueError(f"tables[{i}] must be 2-D")
    ib = _index_bytes(indices, offsets)
    D = tables[0].shape[1]
    B = offsets[0].shape[0]
    if any(t.shape[1] != D for t in tables) or any(o.shape[0] != B for o in offsets):
        raise ValueError("shape mismatch")
    _cuda(x, "x")
    if x.dim() != 2 or x.dtype != torch.float32 or x.stride(1) != 1 or x.shape[0] != B or x.shape[1] < D:
        raise ValueError("x must be a (B, >=D) fp32 CUDA tensor with unit column stride")
    P = n_pairs(T + 1)
    width = D + P if concat_dense else P
    if out is None:
        out = torch.empty((B, width), device=x.device, dtype=torch.float32)
    _cuda(out, "out")
    if out.dtype != torch.float32 or out.stride(1) != 1 or out.shape[0] != B or out.shape[1] < width:
        raise ValueError("out must be (B, >= width) fp32 with unit column stride")
    rc = L.dlrm_embbag_interact(T, B, D, _ptrs(tables), _i64s([t.shape[0] for t in tables]), _ptrs(indices),
                                _i64s([i.numel() for i in indices]), _ptrs(offsets), ib, x.data_ptr(), x.stride(0),
                                out.data_ptr(), out.stride(0), int(bool(concat_dense)), _stream(x.device))
    _check(rc, "dlrm_embbag_interact")
    return out


def linear_bias_act(x: torch.Tensor, W: torch.Tensor, bias: Optional[torch.Tensor], act: int,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """act(x W^T + bias) with W (N, K) -> (M, N) fp32."""
    L = load()
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype != torch.float32 or x.device.type != "cuda":
        raise ValueError("x must be a 2-D fp32 CUDA tensor with unit column stride")
    _dev(W, torch.float32, "W")
    M, K = x.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be (N, K)")
    if bias is not None:
        _dev(bias, torch.float32, "bias")
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((M, N), device=x.device, dtype=torch.float32)
    _cuda(out, "out")
    if out.dtype != torch.float32 or out.stride(1) != 1 or tuple(out.shape[:1]) != (M,) or out.shape[1] < N:
        raise ValueError("out must be (M, >= N) fp32 with unit column stride")
    rc = L.dlrm_linear_bias_act(M, N, K, x.data_ptr(), x.stride(0), W.data_ptr(),
                                bias.data_ptr() if bias is not None else None, int(act), out.data_ptr(),
                                out.stride(0), _stream(x.device))
    _check(rc, "dlrm_linear_bias_act")
    return out


FORWARD_PATHS = {"auto": "dlrm_forward", "fused": "dlrm_forward_fused", "layered": "dlrm_forward_layered",
                 "noalloc": "dlrm_forward_noalloc"}


class Model:
    """DLRMv1 parameters resident on one GPU, with the fused ``forward``.

    ``tables`` T x (V_t, D); ``bot_w[l]`` (out, in) and ``bot_b[l]``; same for
    the top MLP, whose last layer has one output.  Alternatively ``stacked``
    (sum of V_t, D) with ``rows`` [V_0, ...]: every table in one allocation,
    table t starting at row V_0 + ... + V_{t-1} (``tables`` is then None).
    The descriptor passed to the library is built once; tensors are kept
    alive by this object.
    """

    def __init__(self, tables, bot_w, bot_b, top_w, top_b, n_dense: Optional[int] = None, pack: bool = True,
                 stacked: Optional[torch.Tensor] = None, rows: Optional[Sequence[int]] = None):
        L = load()
        if stacked is not None:
            if tables is not None or rows is None:
                raise ValueError("give either tables, or stacked with rows")
            _dev(stacked, torch.float32, "stacked")
            if stacked.dim() != 2 or sum(int(r) for r in rows) > stacked.shape[0] or any(int(r) < 1 for r in rows):
                raise ValueError("stacked must be 2-D with at least sum(rows) rows")
            self.stacked = stacked
            self.tables = [stacked[sum(rows[:t]):sum(rows[:t + 1])] for t in range(len(rows))]
        else:
            self.stacked = None
            self.tables = [_dev(t, torch.float32, "table") for t in tables]
        if not self.tables:
            raise ValueError("at least one table")
        self.dim = int(self.tables[0].shape[1])
        if any(t.dim() != 2 or t.shape[1] != self.dim for t in self.tables):
            raise ValueError("every table must be 2-D with the same row width")
        self.bot_w = [_dev(w, torch.float32, "bot_w") for w in bot_w]
        self.bot_b = [_dev(b, torch.float32, "bot_b") for b in bot_b]
        self.top_w = [_dev(w, torch.float32, "top_w") for w in top_w]
        self.top_b = [_dev(b, torch.float32, "top_b") for b in top_b]
        self.device = self.tables[0].device
        n0 = n_dense if n_dense is not None else self.bot_w[0].shape[1]
        self.ln_bot = [int(n0)] + [int(w.shape[0]) for w in self.bot_w]
        self.ln_top = [int(self.top_w[0].shape[1])] + [int(w.shape[0]) for w in self.top_w]
        self.num_tables = len(self.tables)
        nrows = [int(t.shape[0]) for t in self.tables]
        self._keep = (_i64s(self.ln_bot), _i64s(self.ln_top), _i64s(nrows),
                      _ptrs(self.tables), _ptrs(self.bot_w), _ptrs(self.bot_b), _ptrs(self.top_w), _ptrs(self.top_b),
                      _i64s([sum(nrows[:t]) for t in range(len(nrows))]))
        lb, lt, rws, emb, bw, bb, tw, tb, base = self._keep
        self._desc = _Model(len(self.ln_bot), ctypes.cast(lb, _i64p), len(self.ln_top), ctypes.cast(lt, _i64p),
                            self.num_tables, self.dim, ctypes.cast(rws, _i64p), emb, bw, bb, tw, tb, None)
        if self.stacked is not None:
            # the library addresses the tables through one base pointer and row bases
            self._desc.emb_w = None
            self._desc.emb_stacked = self.stacked.data_ptr()
            self._desc.emb_row_base = ctypes.cast(base, _i64p)
        self._ws: Optional[torch.Tensor] = None
        # weights packed once for the single-launch forward (when the model fits it)
        self.packed: Optional[torch.Tensor] = None
        if pack:
            self.repack()

    def repack(self) -> bool:
        """(Re)write the packed weights of the single-launch forward from the
        current Linear weights; False when the model is outside that path."""
        L = load()
        self._desc.packed_w = None
        n = int(L.dlrm_pack_weights_bytes(ctypes.byref(self._desc)))
        if n == 0:
            self.packed = None
            return False
        if self.packed is None or self.packed.numel() * 4 < n:
            self.packed = torch.empty((n + 3) // 4, dtype=torch.float32, device=self.device)
        _check(L.dlrm_pack_weights(ctypes.byref(self._desc), self.packed.data_ptr(), n, _stream(self.device)),
               "dlrm_pack_weights")
        self._desc.packed_w = self.packed.data_ptr()
        return True

    @classmethod
    def from_inputs(cls, inp, pack: bool = True) -> "Model":
        return cls(inp.tables, inp.bot_w, inp.bot_b, inp.top_w, inp.top_b, n_dense=inp.workload.n_dense, pack=pack)

    def path(self, batch: int) -> str:
        """The path dlrm_forward takes for `batch` samples: "fused" or "layered"."""
        p = load().dlrm_forward_path(ctypes.byref(self._desc), int(batch))
        if p == 0:
            raise DlrmError(DLRM_E_SHAPE, "dlrm_forward_path", "invalid model or batch")
        return "fused" if p == 2 else "layered"

    def workspace_bytes(self, batch: int) -> int:
        n = load().dlrm_forward_workspace_bytes(ctypes.byref(self._desc), int(batch))
        if n == 0:
            raise DlrmError(DLRM_E_SHAPE, "dlrm_forward_workspace_bytes", "invalid model or batch")
        return int(n)

    def workspace(self, batch: int) -> torch.Tensor:
        need = self.workspace_bytes(batch)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def forward_args(self, dense, indices, offsets):
        """Marshal the per-call pointer arrays once (reusable across calls on the same tensors)."""
        B = dense.shape[0]
        return (B, dense.data_ptr(), _ptrs(indices), _i64s([i.numel() for i in indices]), _ptrs(offsets),
                _index_bytes(indices, offsets))

    def forward(self, dense: torch.Tensor, indices: List[torch.Tensor], offsets: List[torch.Tensor],
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                args=None, path: str = "auto") -> torch.Tensor:
        """The whole forward.  ``path``: "auto" (dlrm_forward: the library picks),
        "fused" (dlrm_forward_fused, one launch), "layered" (dlrm_forward_layered)
        or "noalloc" (dlrm_forward_noalloc: dlrm_forward with the library's
        static workspace instead of one passed in)."""
        if path not in FORWARD_PATHS:
            raise ValueError(f"path must be one of {sorted(FORWARD_PATHS)}")
        L = load()
        _dev(dense, torch.float32, "dense")
        if len(indices) != self.num_tables or len(offsets) != self.num_tables:
            raise ValueError("one index and one offset tensor per table")
        _index_bytes(indices, offsets)
        B = dense.shape[0]
        if dense.shape[1] != self.ln_bot[0] or any(o.shape[0] != B for o in offsets):
            raise ValueError("shape mismatch")
        if out is None:
            out = torch.empty((B,), device=self.device, dtype=torch.float32)
        _dev(out, torch.float32, "out")
        if out.numel() != B:
            raise ValueError("out must hold B values")
        if args is None:
            args = self.forward_args(dense, indices, offsets)
        b, dp, ip, nn_, op, ib = args
        if path in ("fused", "noalloc"):
            fn = FORWARD_PATHS[path]
            rc = getattr(L, fn)(ctypes.byref(self._desc), b, dp, ip, nn_, op, ib, out.data_ptr(),
                                _stream(self.device))
            _check(rc, fn)
            return out
        ws = workspace if workspace is not None else self.workspace(B)
        fn = FORWARD_PATHS[path]
        rc = getattr(L, fn)(ctypes.byref(self._desc), b, dp, ip, nn_, op, ib, out.data_ptr(), ws.data_ptr(),
                            ws.numel() * ws.element_size(), _stream(self.device))
        _check(rc, fn)
        return out


def check_indices(tables_rows: Sequence[int], indices: List[torch.Tensor], offsets: List[torch.Tensor]) -> int:
    """Count malformed indices / offsets on the device (synchronises to read the count)."""
    L = load()
    T = len(indices)
    dev = indices[0].device
    bad = torch.empty(1, dtype=torch.int32, device=dev)
    B = offsets[0].shape[0]
    ib = _index_bytes(indices, offsets)
    rc = L.dlrm_embbag_check_indices(T, B, _i64s(tables_rows), _ptrs(indices), _i64s([i.numel() for i in indices]),
                                     _ptrs(offsets), ib, bad.data_ptr(), _stream(dev))
    _check(rc, "dlrm_embbag_check_indices")
    return int(bad.item())


def pair_index_map(n_feat: int, device="cuda"):
    """The interaction kernels' own decoding p -> (i, j), as two int32 tensors."""
    L = load()
    P = n_pairs(n_feat)
    i = torch.empty(max(P, 1), dtype=torch.int32, device=device)
    j = torch.empty(max(P, 1), dtype=torch.int32, device=device)
    rc = L.dlrm_pair_index_map(int(n_feat), i.data_ptr(), j.data_ptr(), _stream(i.device))
    _check(rc, "dlrm_pair_index_map")
    return i[:P], j[:P]


def probe_read_stream(src: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Enqueue one sequential read of the fp32 CUDA tensor `src` (numel a multiple
    of 4): the library's own HBM read ceiling kernel.  Returns the sink."""
    L = load()
    _dev(src, torch.float32, "src")
    if sink is None:
        sink = torch.zeros(int(L.dlrm_probe_sink_floats()), dtype=torch.float32, device=src.device)
    _check(L.dlrm_probe_read_stream(src.data_ptr(), src.numel(), sink.data_ptr(), _stream(src.device)),
           "dlrm_probe_read_stream")
    return sink


def probe_gather_rows(table: torch.Tensor, idx: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Enqueue a read of the rows idx (int64) of the (rows, dim) fp32 table: the
    random-row gather ceiling of one-index bags.  Returns the sink."""
    L = load()
    _dev(table, torch.float32, "table")
    _dev(idx, torch.int64, "idx")
    if sink is None:
        sink = torch.zeros(int(L.dlrm_probe_sink_floats()), dtype=torch.float32, device=table.device)
    _check(L.dlrm_probe_gather_rows(table.data_ptr(), table.shape[0], table.shape[1], idx.data_ptr(), idx.numel(),
                                    sink.data_ptr(), _stream(table.device)), "dlrm_probe_gather_rows")
    return sink


def probe_l2_stream(src: torch.Tensor, blocks: int = 256, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Enqueue `blocks` blocks that each read all of the fp32 CUDA tensor `src`
    (numel a multiple of 4): one block per CU measures the L2 -> CU rate."""
    L = load()
    _dev(src, torch.float32, "src")
    if sink is None:
        sink = torch.zeros(int(L.dlrm_probe_sink_floats()), dtype=torch.float32, device=src.device)
    _check(L.dlrm_probe_l2_stream(src.data_ptr(), src.numel(), int(blocks), sink.data_ptr(), _stream(src.device)),
           "dlrm_probe_l2_stream")
    return sink
