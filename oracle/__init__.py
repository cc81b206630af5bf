"""ctypes binding of the CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package.
Inputs are numpy arrays (bf16 and fp16 as uint16 bit patterns); every call
raises ``OracleError`` on a nonzero status.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_lib_path = None

SCORE = {"sigmoid": 0, "sqrt_softplus": 1}
DTYPE = {"f32": 0, "bf16": 1, "q8b32": 2}


class OracleError(RuntimeError):
    pass


class RefConfig(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_expert", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("score", ctypes.c_int32),
                ("route_scale", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32)]


class RefMat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class RefWeights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("gate", RefMat), ("up", RefMat), ("down", RefMat),
                ("s_gate", RefMat), ("s_up", RefMat), ("s_down", RefMat)]


class RefDebug(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p),
                ("topk_w", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("perm_rows", ctypes.c_void_p), ("inv_perm", ctypes.c_void_p)]


def load(path: str | None = None):
    """Load the oracle library (building it if absent); ``path`` selects a mutant build."""
    global _lib, _lib_path
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(_build.LIB):
            _build.build(force=False)
        path = _build.LIB
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int32
    C = ctypes.POINTER(RefConfig)
    W = ctypes.POINTER(RefWeights)
    lib.moe_ref_route.argtypes = [C, P, P, P, P, P, P]
    lib.moe_ref_select.argtypes = [C, P, P, P, P]
    lib.moe_ref_permute.argtypes = [C, P, P, P, P]
    lib.moe_ref_expert_ffn.argtypes = [C, P, W, P, P, P, P, P]
    lib.moe_ref_combine.argtypes = [C, P, P, P]
    lib.moe_ref_layer_forward.argtypes = [C, P, W, P, ctypes.POINTER(RefDebug)]
    lib.moe_ref_topk_rows.argtypes = [I, I, I, P, P, P]
    lib.moe_ref_dense_swiglu.argtypes = [I, I, I, I, I, P, RefMat, RefMat, RefMat, I, P]
    lib.moe_ref_bf16_from_f64.argtypes = [ctypes.c_double]
    lib.moe_ref_bf16_from_f64.restype = ctypes.c_uint16
    lib.moe_ref_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.moe_ref_f16_to_f32.restype = ctypes.c_float
    lib.moe_ref_score.argtypes = [I, ctypes.c_float]
    lib.moe_ref_score.restype = ctypes.c_float
    lib.moe_ref_status_str.argtypes = [ctypes.c_int]
    lib.moe_ref_status_str.restype = ctypes.c_char_p
    lib.moe_ref_mutant.restype = ctypes.c_int
    lib.moe_ref_threads.restype = ctypes.c_int
    lib.moe_ref_set_threads.argtypes = [ctypes.c_int]
    lib.moe_ref_set_threads.restype = ctypes.c_int
    if path == _build.LIB:
        _lib, _lib_path = lib, path
    return lib


class Oracle:
    """Numpy-level wrapper around one oracle build (the real one by default)."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # ---- marshalling -------------------------------------------------
    @staticmethod
    def config(cfg: dict, T: int | None = None) -> RefConfig:
        return RefConfig(n_tokens=cfg["T"] if T is None else T, d_model=cfg["d"],
                         n_expert=cfg["E"], top_k=cfg["k"], d_ff=cfg["F"],
                         n_shared=cfg["n_shared"], d_ff_shared=cfg["Fs"],
                         score=SCORE[cfg["score"]], route_scale=cfg["scale"],
                         act_dtype=DTYPE[cfg["act"]], w_dtype=DTYPE[cfg["w"]])

    @staticmethod
    def _p(a):
        if a is None:
            return None
        assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], type(a)
        return a.ctypes.data

    def _mat(self, m):
        if m is None:
            return RefMat(None, None)
        if isinstance(m, tuple):
            return RefMat(self._p(m[0]), self._p(m[1]))
        return RefMat(self._p(m), None)

    def weights(self, L) -> RefWeights:
        return RefWeights(self._p(L["w_router"]), self._p(L.get("bias")),
                          self._mat(L["gate"]), self._mat(L["up"]), self._mat(L["down"]),
                          self._mat(L.get("s_gate")), self._mat(L.get("s_up")),
                          self._mat(L.get("s_down")))

    def _check(self, st):
        if st != 0:
            raise OracleError("oracle status %d (%s)" % (st, self.lib.moe_ref_status_str(st).decode()))

    # ---- calls -------------------------------------------------------
    def route(self, cfg, x, w_router, bias=None):
        T = x.shape[0]
        c = self.config(cfg, T)
        logits = np.empty((T, cfg["E"]), np.float32)
        idx = np.empty((T, cfg["k"]), np.int32)
        w = np.empty((T, cfg["k"]), np.float32)
        self._check(self.lib.moe_ref_route(ctypes.byref(c), self._p(x), self._p(w_router),
                                           self._p(bias), self._p(logits), self._p(idx), self._p(w)))
        return logits, idx, w

    def select(self, cfg, logits, bias=None):
        T = logits.shape[0]
        c = self.config(cfg, T)
        idx = np.empty((T, cfg["k"]), np.int32)
        w = np.empty((T, cfg["k"]), np.float32)
        self._check(self.lib.moe_ref_select(ctypes.byref(c), self._p(logits), self._p(bias),
                                            self._p(idx), self._p(w)))
        return idx, w

    def topk_rows(self, scores, k):
        """Per row of ``scores`` [rows, n] f32: the k chosen candidate indices in
        ascending order [rows, k] i32, and their scores [rows, k] f32."""
        rows, n = scores.shape
        idx = np.empty((rows, k), np.int32)
        vals = np.empty((rows, k), np.float32)
        self._check(self.lib.moe_ref_topk_rows(rows, n, k, self._p(scores), self._p(idx),
                                               self._p(vals)))
        return idx, vals

    def permute(self, cfg, topk_idx):
        T = topk_idx.shape[0]
        c = self.config(cfg, T)
        n = T * cfg["k"]
        off = np.empty(cfg["E"] + 1, np.int32)
        perm = np.empty(n, np.int32)
        inv = np.empty(n, np.int32)
        self._check(self.lib.moe_ref_permute(ctypes.byref(c), self._p(np.ascontiguousarray(topk_idx)),
                                             self._p(off), self._p(perm), self._p(inv)))
        return off, perm, inv

    def expert_ffn(self, cfg, L, offsets, perm_rows, topk_w):
        x = L["x"]
        T = x.shape[0]
        c = self.config(cfg, T)
        W = self.weights(L)
        slot = np.empty((T * cfg["k"], cfg["d"]), np.float32)
        shared = np.empty((T, cfg["d"]), np.float32) if cfg["n_shared"] else None
        self._check(self.lib.moe_ref_expert_ffn(ctypes.byref(c), self._p(x), ctypes.byref(W),
                                                self._p(offsets), self._p(perm_rows),
                                                self._p(np.ascontiguousarray(topk_w)),
                                                self._p(slot), self._p(shared)))
        return slot, shared

    def combine(self, cfg, slot, shared, T=None):
        T = slot.shape[0] // cfg["k"] if T is None else T
        c = self.config(cfg, T)
        y = np.empty((T, cfg["d"]), np.float32)
        self._check(self.lib.moe_ref_combine(ctypes.byref(c), self._p(slot), self._p(shared), self._p(y)))
        return y

    def layer_forward(self, cfg, L, debug=True):
        x = L["x"]
        T = x.shape[0]
        c = self.config(cfg, T)
        W = self.weights(L)
        y = np.empty((T, cfg["d"]), np.float32)
        out = dict(y=y)
        dbg = None
        if debug:
            n = T * cfg["k"]
            out.update(logits=np.empty((T, cfg["E"]), np.float32),
                       topk_idx=np.empty((T, cfg["k"]), np.int32),
                       topk_w=np.empty((T, cfg["k"]), np.float32),
                       offsets=np.empty(cfg["E"] + 1, np.int32),
                       perm_rows=np.empty(n, np.int32), inv_perm=np.empty(n, np.int32))
            dbg = RefDebug(*(self._p(out[k]) for k in
                             ("logits", "topk_idx", "topk_w", "offsets", "perm_rows", "inv_perm")))
        self._check(self.lib.moe_ref_layer_forward(ctypes.byref(c), self._p(x), ctypes.byref(W),
                                                   self._p(y), ctypes.byref(dbg) if dbg else None))
        return out

    def dense_swiglu(self, cfg, x, gate, up, down, expert=0, F=None):
        T = x.shape[0]
        y = np.empty((T, cfg["d"]), np.float64)
        self._check(self.lib.moe_ref_dense_swiglu(T, cfg["d"], cfg["F"] if F is None else F,
                                                  DTYPE[cfg["act"]], DTYPE[cfg["w"]], self._p(x),
                                                  self._mat(gate), self._mat(up), self._mat(down),
                                                  expert, self._p(y)))
        return y

    def score(self, kind, logit):
        return self.lib.moe_ref_score(SCORE[kind], float(logit))

    def bf16_from_f64(self, v):
        return self.lib.moe_ref_bf16_from_f64(float(v))

    def f16_to_f32(self, h):
        return self.lib.moe_ref_f16_to_f32(int(h))

    def mutant(self):
        return self.lib.moe_ref_mutant()

    def threads(self):
        return self.lib.moe_ref_threads()

    def set_threads(self, n):
        """Threads of the token loops from now on; returns the previous count."""
        return self.lib.moe_ref_set_threads(int(n))
