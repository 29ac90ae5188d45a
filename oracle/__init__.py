"""fp64 CPU oracle of the DLRMv1 forward hot path (ctypes wrapper over dlrm_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check of the entry
module and the CPU-baseline leg of the benchmark, never by the product path.
It shares no code with the HIP library; the only thing both sides use is the
seeded input generator module.

All functions take numpy arrays (or torch CPU tensors, converted with
``numpy()``) and return float64 numpy arrays.  Shapes:
  tables    T x (V, D) float32
  indices   T x (N_t,) int64
  offsets   T x (B,)   int64 (last bag ends at N_t)
  dense     (B, n0)    float32
  weights   (out, in)  float32, biases (out,) float32
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "dlrm_oracle.c")
LIBRARY = os.path.join(HERE, "libdlrm_oracle.so")

E_NULL, E_SHAPE, E_INDEX, E_NOMEM = -1, -2, -3, -4
ACT_NONE, ACT_RELU, ACT_SIGMOID = 0, 1, 2

_i64p = ctypes.POINTER(ctypes.c_int64)
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle error {code}")
        self.code = code


class _Model(ctypes.Structure):
    _fields_ = [
        ("n_bot", ctypes.c_int32), ("ln_bot", _i64p),
        ("n_top", ctypes.c_int32), ("ln_top", _i64p),
        ("T", ctypes.c_int32), ("D", ctypes.c_int32),
        ("rows", _i64p),
        ("emb", ctypes.POINTER(_fp)),
        ("bot_w", ctypes.POINTER(_fp)), ("bot_b", ctypes.POINTER(_fp)),
        ("top_w", ctypes.POINTER(_fp)), ("top_b", ctypes.POINTER(_fp)),
    ]


def compile_library(source: str = SOURCE, out: str = LIBRARY, extra_flags: Sequence[str] = ()) -> str:
    """Build the oracle with gcc (-O2, no fast-math, OpenMP over samples)."""
    import subprocess
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           *extra_flags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _np(a, dtype) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, lib_path: str = LIBRARY):
        if not os.path.exists(lib_path):
            compile_library(out=lib_path)
        self.path = lib_path
        L = ctypes.CDLL(lib_path)
        self._L = L
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_n_pairs.argtypes = [ctypes.c_int64]
        L.oracle_n_pairs.restype = ctypes.c_int64
        L.oracle_pair_closed_form.argtypes = [ctypes.c_int64, _i64p, _i64p]
        L.oracle_linear.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dp, ctypes.c_int64,
                                    _fp, _fp, ctypes.c_int, _dp, ctypes.c_int64]
        L.oracle_embbag_sum.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.POINTER(_fp), _i64p, ctypes.POINTER(_i64p), _i64p,
                                        ctypes.POINTER(_i64p), _dp]
        L.oracle_embbag_ex.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_fp), _i64p,
                                       ctypes.POINTER(_i64p), _i64p, ctypes.POINTER(_i64p), ctypes.c_int32,
                                       ctypes.c_int32, _i64p, ctypes.POINTER(_fp), _dp]
        L.oracle_interact.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _dp, ctypes.c_int64,
                                      _dp, _dp, ctypes.c_int64]
        L.oracle_gram.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _dp, ctypes.c_int64,
                                  _dp, _dp]
        L.oracle_validate.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64]
        L.oracle_forward.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64, _fp, ctypes.POINTER(_i64p),
                                     _i64p, ctypes.POINTER(_i64p), _dp, _dp, _dp, _dp]
        for f in ("oracle_pair_closed_form", "oracle_linear", "oracle_embbag_sum", "oracle_embbag_ex", "oracle_interact",
                  "oracle_gram", "oracle_validate", "oracle_forward"):
            getattr(L, f).restype = ctypes.c_int

    # -- helpers -----------------------------------------------------------------
    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise OracleError(rc, what)

    def set_threads(self, n: int) -> int:
        return self._L.oracle_set_threads(int(n))

    def n_pairs(self, n_feat: int) -> int:
        return int(self._L.oracle_n_pairs(int(n_feat)))

    def pair_closed_form(self, p: int):
        i, j = ctypes.c_int64(), ctypes.c_int64()
        self._check(self._L.oracle_pair_closed_form(int(p), ctypes.byref(i), ctypes.byref(j)), "pair")
        return int(i.value), int(j.value)

    # -- stages --------------------------------------------------------------------
    def linear(self, x, W, b, act: int) -> np.ndarray:
        x = _np(x, np.float64)
        W = _np(W, np.float32)
        M, K = x.shape
        N = W.shape[0]
        assert W.shape[1] == K
        bp = None
        if b is not None:
            b = _np(b, np.float32)
            bp = b.ctypes.data_as(_fp)
        y = np.empty((M, N), np.float64)
        rc = self._L.oracle_linear(M, N, K, x.ctypes.data_as(_dp), K, W.ctypes.data_as(_fp), bp, int(act),
                                   y.ctypes.data_as(_dp), N)
        self._check(rc, "linear")
        return y

    def _tables(self, tables, indices, offsets):
        T = len(tables)
        tabs = [_np(t, np.float32) for t in tables]
        idxs = [_np(i, np.int64) for i in indices]
        offs = [_np(o, np.int64) for o in offsets]
        keep = (tabs, idxs, offs)
        W = (_fp * T)(*[t.ctypes.data_as(_fp) for t in tabs])
        rows = (ctypes.c_int64 * T)(*[t.shape[0] for t in tabs])
        I = (_i64p * T)(*[i.ctypes.data_as(_i64p) for i in idxs])
        N = (ctypes.c_int64 * T)(*[i.shape[0] for i in idxs])
        O = (_i64p * T)(*[o.ctypes.data_as(_i64p) for o in offs])
        return keep, W, rows, I, N, O

    def embbag_sum(self, tables, indices, offsets) -> np.ndarray:
        T = len(tables)
        keep, W, rows, I, N, O = self._tables(tables, indices, offsets)
        D = keep[0][0].shape[1]
        B = keep[2][0].shape[0]
        out = np.empty((B, T, D), np.float64)
        rc = self._L.oracle_embbag_sum(T, B, D, W, rows, I, N, O, out.ctypes.data_as(_dp))
        self._check(rc, "embbag_sum")
        return out

    MODES = {"sum": 0, "mean": 1, "max": 2}

    def embbag_ex(self, tables, indices, offsets, mode="sum", include_last_offset=False, padding_idx=None,
                  per_sample_weights=None) -> np.ndarray:
        """General bags: mode sum / mean / max, optional per-sample weights (sum only),
        include_last_offset, per-table padding index (None or -1: none).  Indices and
        offsets may be int32 or int64; they are widened to int64 exactly."""
        T = len(tables)
        widen = lambda a: np.ascontiguousarray(a.detach().cpu().numpy() if hasattr(a, "detach") else a).astype(np.int64)
        keep, W, rows, I, N, O = self._tables(tables, [widen(i) for i in indices], [widen(o) for o in offsets])
        D = keep[0][0].shape[1]
        B = keep[2][0].shape[0] - (1 if include_last_offset else 0)
        out = np.empty((max(B, 0), T, D), np.float64)
        pad = None
        if padding_idx is not None:
            pads = padding_idx if isinstance(padding_idx, (list, tuple)) else [padding_idx] * T
            pad = (ctypes.c_int64 * T)(*[(-1 if p is None else int(p)) for p in pads])
        psw = None
        keep_w = None
        if per_sample_weights is not None:
            keep_w = [_np(w, np.float32) for w in per_sample_weights]
            psw = (_fp * T)(*[w.ctypes.data_as(_fp) for w in keep_w])
        rc = self._L.oracle_embbag_ex(T, B, D, W, rows, I, N, O, self.MODES[mode], int(bool(include_last_offset)),
                                      ctypes.cast(pad, _i64p) if pad is not None else None, psw,
                                      out.ctypes.data_as(_dp))
        self._check(rc, "embbag_ex")
        return out

    def interact(self, x, E) -> np.ndarray:
        x = _np(x, np.float64)
        E = _np(E, np.float64)
        B, T, D = E.shape
        assert x.shape == (B, D)
        P = self.n_pairs(T + 1)
        Z = np.empty((B, P), np.float64)
        rc = self._L.oracle_interact(B, T, D, x.ctypes.data_as(_dp), D, E.ctypes.data_as(_dp),
                                     Z.ctypes.data_as(_dp), P)
        self._check(rc, "interact")
        return Z

    def gram(self, x, E) -> np.ndarray:
        x = _np(x, np.float64)
        E = _np(E, np.float64)
        B, T, D = E.shape
        G = np.empty((B, T + 1, T + 1), np.float64)
        rc = self._L.oracle_gram(B, T, D, x.ctypes.data_as(_dp), D, E.ctypes.data_as(_dp),
                                 G.ctypes.data_as(_dp))
        self._check(rc, "gram")
        return G

    def _model(self, ln_bot, ln_top, tables, bot_w, bot_b, top_w, top_b):
        bw = [_np(w, np.float32) for w in bot_w]
        bb = [_np(b, np.float32) for b in bot_b]
        tw = [_np(w, np.float32) for w in top_w]
        tb = [_np(b, np.float32) for b in top_b]
        tabs = [_np(t, np.float32) for t in tables]
        lb = (ctypes.c_int64 * len(ln_bot))(*ln_bot)
        lt = (ctypes.c_int64 * len(ln_top))(*ln_top)
        arr = lambda xs: (_fp * max(len(xs), 1))(*[x.ctypes.data_as(_fp) for x in xs])
        rows = (ctypes.c_int64 * len(tabs))(*[t.shape[0] for t in tabs])
        D = tabs[0].shape[1] if tabs else 0
        m = _Model(len(ln_bot), ctypes.cast(lb, _i64p), len(ln_top), ctypes.cast(lt, _i64p), len(tabs), D,
                   ctypes.cast(rows, _i64p), arr(tabs), arr(bw), arr(bb), arr(tw), arr(tb))
        keep = (bw, bb, tw, tb, tabs, lb, lt, rows)
        return m, keep

    def validate(self, ln_bot, ln_top, num_tables: int, dim: int, batch: int) -> int:
        lb = (ctypes.c_int64 * len(ln_bot))(*ln_bot)
        lt = (ctypes.c_int64 * len(ln_top))(*ln_top)
        m = _Model(len(ln_bot), ctypes.cast(lb, _i64p), len(ln_top), ctypes.cast(lt, _i64p), num_tables, dim)
        return int(self._L.oracle_validate(ctypes.byref(m), batch))

    def forward(self, dense, tables, indices, offsets, bot_w, bot_b, top_w, top_b,
                ln_bot=None, ln_top=None, intermediates: bool = False):
        dense = _np(dense, np.float32)
        B = dense.shape[0]
        if ln_bot is None:
            ln_bot = [dense.shape[1]] + [int(w.shape[0]) for w in bot_w]
        if ln_top is None:
            ln_top = [int(top_w[0].shape[1])] + [int(w.shape[0]) for w in top_w]
        m, keep_m = self._model(ln_bot, ln_top, tables, bot_w, bot_b, top_w, top_b)
        keep_t, W, rows, I, N, O = self._tables(tables, indices, offsets)
        T = len(tables)
        D = int(ln_bot[-1])
        P = self.n_pairs(T + 1)
        out = np.empty((B,), np.float64)
        x = e = r = None
        xp = ep = rp = None
        if intermediates:
            x = np.empty((B, D), np.float64)
            e = np.empty((B, T, D), np.float64)
            r = np.empty((B, D + P), np.float64)
            xp, ep, rp = x.ctypes.data_as(_dp), e.ctypes.data_as(_dp), r.ctypes.data_as(_dp)
        rc = self._L.oracle_forward(ctypes.byref(m), B, dense.ctypes.data_as(_fp), I, N, O,
                                    out.ctypes.data_as(_dp), xp, ep, rp)
        self._check(rc, "forward")
        if intermediates:
            return out, {"x": x, "E": e, "R": r}
        return out


_DEFAULT: Optional[Oracle] = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def forward_inputs(inp, intermediates: bool = False, oracle: Optional[Oracle] = None):
    """Run the oracle forward on a ``dlrm_inputs.Inputs`` (tensors moved to the CPU)."""
    o = oracle or default()
    cpu = lambda xs: [x.detach().cpu() for x in xs]
    return o.forward(inp.dense.cpu(), cpu(inp.tables), cpu(inp.indices), cpu(inp.offsets),
                     cpu(inp.bot_w), cpu(inp.bot_b), cpu(inp.top_w), cpu(inp.top_b),
                     ln_bot=list(inp.workload.ln_bot), ln_top=list(inp.workload.ln_top),
                     intermediates=intermediates)
