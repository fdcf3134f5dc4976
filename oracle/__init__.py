"""Oracle for the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Plain, slow CPU reference written in C (``oracle.c``), loaded with ctypes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the library path never does.
Floating point is double except the router logits, which are fp32 by
definition (``oracle.c`` states every reading taken and the page each
function follows).

``Oracle(so_path)`` binds one compiled copy; the module-level functions use
the default build (``liboracle.so`` beside this file). The tests also bind
deliberately broken copies to show that the pins catch planted mistakes.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

_P = np.ctypeslib.ndpointer
_I32 = ctypes.c_int32


def compile_oracle(src, so_path):
    """gcc, OpenMP, no floating-point contraction, no fast-math."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", src, "-o", so_path + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(so_path + ".tmp", so_path)


def build():
    compile_oracle(SOURCE, _SO)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


class Oracle:
    def __init__(self, so_path):
        L = ctypes.CDLL(so_path)
        f32, f64, i32, u16 = (_P(np.float32, flags="C"), _P(np.float64, flags="C"),
                              _P(np.int32, flags="C"), _P(np.uint16, flags="C"))
        vp = ctypes.c_void_p
        L.oracle_partition.argtypes = [_I32, _I32, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]
        L.oracle_partition.restype = ctypes.c_int
        L.oracle_owner.argtypes = [_I32, _I32, _I32]
        L.oracle_owner.restype = _I32
        L.oracle_router_logits.argtypes = [u16, f32, vp, _I32, _I32, _I32, f32]
        L.oracle_router_logits.restype = None
        L.oracle_route.argtypes = [f32, _I32, _I32, _I32, i32, f64]
        L.oracle_route.restype = ctypes.c_int
        L.oracle_permute.argtypes = [i32, _I32, _I32, _I32, _I32, _I32, i32, i32, i32, i32]
        L.oracle_permute.restype = ctypes.c_int
        L.oracle_expert_row.argtypes = [u16, u16, u16, _I32, _I32, f64]
        L.oracle_expert_row.restype = None
        L.oracle_grouped_ffn.argtypes = [u16, i32, i32, _I32, _I32, _I32, _I32, _I32, u16, u16,
                                         f64]
        L.oracle_grouped_ffn.restype = ctypes.c_int
        u8 = _P(np.uint8, flags="C")
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_expert_row_fp8.argtypes = [u16, u8, f32, u8, f32, _I32, _I32, f64]
        L.oracle_expert_row_fp8.restype = None
        L.oracle_grouped_ffn_fp8.argtypes = [u16, i32, i32, _I32, _I32, _I32, _I32, _I32, u8, f32,
                                             u8, f32, f64]
        L.oracle_grouped_ffn_fp8.restype = ctypes.c_int
        L.oracle_combine.argtypes = [f64, i32, f64, _I32, _I32, _I32, f64]
        L.oracle_combine.restype = None
        L.oracle_forward.argtypes = [u16, f32, vp, u16, u16, _I32, _I32, _I32, _I32, _I32, _I32,
                                     _I32, i32, _I32, f32, i32, f64, f64]
        L.oracle_forward.restype = ctypes.c_int
        self.lib = L

    def partition(self, E, S, s):
        """(first_expert, count) of share s when E experts are split over S shares."""
        f, c = _I32(), _I32()
        if self.lib.oracle_partition(E, S, s, ctypes.byref(f), ctypes.byref(c)) != 0:
            raise ValueError("invalid partition arguments")
        return f.value, c.value

    def owner(self, E, S, e):
        return self.lib.oracle_owner(E, S, e)

    def router_logits(self, x, wg, bias=None):
        x = _c(x, np.uint16)
        wg = _c(wg, np.float32)
        T, H = x.shape
        E = wg.shape[0]
        out = np.empty((T, E), np.float32)
        b = _c(bias, np.float32) if bias is not None else None
        self.lib.oracle_router_logits(x, wg, b.ctypes.data if b is not None else None, T, H, E,
                                      out)
        return out

    def route(self, logits, k):
        logits = _c(logits, np.float32)
        T, E = logits.shape
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        if self.lib.oracle_route(logits, T, E, k, ids, w) != 0:
            raise ValueError("invalid routing arguments")
        return ids, w

    def permute(self, ids, E, first=0, L=None):
        """(counts [E], offsets [L+1], permuted_rows [N_L], expanded_to_permuted [T*k])."""
        ids = _c(ids, np.int32)
        T, k = ids.shape
        L = E - first if L is None else L
        counts = np.empty(E, np.int32)
        offsets = np.empty(L + 1, np.int32)
        perm = np.full(max(T * k, 1), -7, np.int32)
        e2p = np.empty(max(T * k, 1), np.int32)
        if self.lib.oracle_permute(ids if ids.size else np.zeros((1, 1), np.int32), T, k, E, first,
                                   L, counts, offsets, perm, e2p) != 0:
            raise ValueError("invalid permutation arguments")
        return counts, offsets, perm[: offsets[L]].copy(), e2p[: T * k].copy()

    def expert_row(self, xrow, w1e, w2e):
        xrow = _c(xrow, np.uint16)
        H = xrow.shape[0]
        I = w2e.shape[1]
        out = np.empty(H, np.float64)
        self.lib.oracle_expert_row(xrow, _c(w1e, np.uint16), _c(w2e, np.uint16), H, I, out)
        return out

    def grouped_ffn(self, x, permuted_rows, offsets, k, w1, w2):
        x = _c(x, np.uint16)
        T, H = x.shape
        L = len(offsets) - 1
        I = w2.shape[2]
        n = int(offsets[L]) if L > 0 else 0
        out = np.empty((max(n, 1), H), np.float64)
        pr = _c(permuted_rows, np.int32)
        if pr.size == 0:
            pr = np.zeros(1, np.int32)
        if self.lib.oracle_grouped_ffn(x, pr, _c(offsets, np.int32), L, T, k, H, I,
                                       _c(w1, np.uint16), _c(w2, np.uint16), out) != 0:
            raise ValueError("invalid grouped FFN arguments")
        return out[:n]

    def e4m3_value(self, code):
        """Value of one FP8 E4M3 code (uint8)."""
        return self.lib.oracle_e4m3_value(int(code))

    def expert_row_fp8(self, xrow, w1q, w1s, w2q, w2s):
        xrow = _c(xrow, np.uint16)
        H = xrow.shape[0]
        I = w2q.shape[1]
        out = np.empty(H, np.float64)
        self.lib.oracle_expert_row_fp8(xrow, _c(w1q, np.uint8), _c(w1s, np.float32),
                                       _c(w2q, np.uint8), _c(w2s, np.float32), H, I, out)
        return out

    def grouped_ffn_fp8(self, x, permuted_rows, offsets, k, w1q, w1s, w2q, w2s):
        """grouped_ffn with FP8 E4M3 weight codes and per-row fp32 scales:
        w1q [L, 2I, H], w1s [L, 2I], w2q [L, H, I], w2s [L, H]."""
        x = _c(x, np.uint16)
        T, H = x.shape
        L = len(offsets) - 1
        I = w2q.shape[2]
        n = int(offsets[L]) if L > 0 else 0
        out = np.empty((max(n, 1), H), np.float64)
        pr = _c(permuted_rows, np.int32)
        if pr.size == 0:
            pr = np.zeros(1, np.int32)
        if self.lib.oracle_grouped_ffn_fp8(x, pr, _c(offsets, np.int32), L, T, k, H, I,
                                           _c(w1q, np.uint8), _c(w1s, np.float32),
                                           _c(w2q, np.uint8), _c(w2s, np.float32), out) != 0:
            raise ValueError("invalid grouped FFN arguments")
        return out[:n]

    def combine(self, expert_out, e2p, weights, T, k, H):
        eo = _c(expert_out, np.float64).reshape(-1, H)
        y = np.empty((T, H), np.float64)
        if eo.size == 0:
            eo = np.zeros((1, H), np.float64)
        self.lib.oracle_combine(eo, _c(e2p, np.int32), _c(weights, np.float64), T, k, H, y)
        return y

    def forward(self, x, wg, w1, w2, k, first=0, L=None, bias=None, sample=None):
        """Router logits, routing, and the layer output for the sampled tokens.

        w1/w2 hold the L local experts only. Returns (logits [T,E] fp32,
        ids [T,k], weights [T,k] fp64, y [n_sample,H] fp64).
        """
        x = _c(x, np.uint16)
        wg = _c(wg, np.float32)
        T, H = x.shape
        E = wg.shape[0]
        L = E - first if L is None else L
        I = w2.shape[2]
        sample = np.arange(T, dtype=np.int32) if sample is None else _c(sample, np.int32)
        logits = np.empty((T, E), np.float32)
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        y = np.empty((max(len(sample), 1), H), np.float64)
        b = _c(bias, np.float32) if bias is not None else None
        rc = self.lib.oracle_forward(x, wg, b.ctypes.data if b is not None else None,
                                     _c(w1, np.uint16), _c(w2, np.uint16), T, H, I, E, k, first, L,
                                     sample if len(sample) else np.zeros(1, np.int32), len(sample),
                                     logits, ids, w, y)
        if rc != 0:
            raise ValueError("invalid forward arguments")
        return logits, ids, w, y[: len(sample)]


_default = None


def default():
    global _default
    if _default is None:
        if not os.path.exists(_SO):
            build()
        _default = Oracle(_SO)
    return _default


def partition(*a, **kw):
    return default().partition(*a, **kw)


def owner(*a, **kw):
    return default().owner(*a, **kw)


def router_logits(*a, **kw):
    return default().router_logits(*a, **kw)


def route(*a, **kw):
    return default().route(*a, **kw)


def permute(*a, **kw):
    return default().permute(*a, **kw)


def expert_row(*a, **kw):
    return default().expert_row(*a, **kw)


def grouped_ffn(*a, **kw):
    return default().grouped_ffn(*a, **kw)


def e4m3_value(*a, **kw):
    return default().e4m3_value(*a, **kw)


def expert_row_fp8(*a, **kw):
    return default().expert_row_fp8(*a, **kw)


def grouped_ffn_fp8(*a, **kw):
    return default().grouped_ffn_fp8(*a, **kw)


def combine(*a, **kw):
    return default().combine(*a, **kw)


def forward(*a, **kw):
    return default().forward(*a, **kw)
