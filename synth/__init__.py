"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Holds none of the layer's arithmetic: it only draws numbers (``synth.c``).
Tensor ids keep the streams of different tensors apart.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

X, WG, W1, W2, BIAS, LOGITS, IDS, EXPERT_OUT, WEIGHTS = 1, 2, 3, 4, 5, 6, 7, 8, 9

_P = np.ctypeslib.ndpointer


def build():
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", os.path.join(_HERE, "synth.c"), "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, u32, i64, i32, d = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                 ctypes.c_int32, ctypes.c_double)
        vp = ctypes.c_void_p
        L.synth_normal_f32.argtypes = [u64, u32, u32, i64, d, vp]
        L.synth_normal_bf16.argtypes = [u64, u32, u32, u32, i64, d, vp]
        L.synth_tie_levels_f32.argtypes = [u64, u32, u32, i64, vp]
        L.synth_topk_ids.argtypes = [u64, u32, i32, i32, i32, vp]
        L.synth_uniform_int.argtypes = [u64, u32, i64, i64, vp]
        L.synth_fp8_rows.argtypes = [u64, u32, u32, u32, i64, i64, d, vp, vp]
        for f in (L.synth_normal_f32, L.synth_normal_bf16, L.synth_tie_levels_f32,
                  L.synth_topk_ids, L.synth_uniform_int, L.synth_fp8_rows):
            f.restype = None
        _lib = L
    return _lib


def normal_f32(seed, tensor, shape, sigma, expert=0):
    out = np.empty(shape, np.float32)
    lib().synth_normal_f32(seed, tensor, expert, out.size, float(sigma), out.ctypes.data)
    return out


def normal_bf16(seed, tensor, shape, sigma, first_expert=0):
    """bf16 bit patterns (uint16). For an expert-stacked tensor the leading
    dimension is the expert: expert e's block is drawn from its own stream
    (first_expert + local index), so a share's experts equal the same experts
    of the full tensor."""
    out = np.empty(shape, np.uint16)
    if len(shape) >= 3:
        ne, per = shape[0], int(np.prod(shape[1:]))
    else:
        ne, per = 1, out.size
    lib().synth_normal_bf16(seed, tensor, first_expert, ne, per, float(sigma), out.ctypes.data)
    return out


def fp8_rows(seed, tensor, shape, sigma, first_expert=0):
    """Per-row quantised FP8 E4M3 weights for an expert-stacked [L, R, C]
    tensor: (codes uint8 [L, R, C], scales float32 [L, R]); the weight is
    scale * value(code). Drawn from the same normals as normal_bf16."""
    ne, rows, cols = shape
    q = np.empty(shape, np.uint8)
    s = np.empty((ne, rows), np.float32)
    lib().synth_fp8_rows(seed, tensor, first_expert, ne, rows, cols, float(sigma), q.ctypes.data,
                         s.ctypes.data)
    return q, s


def tie_levels_f32(seed, tensor, shape):
    out = np.empty(shape, np.float32)
    lib().synth_tie_levels_f32(seed, tensor, 0, out.size, out.ctypes.data)
    return out


def topk_ids(seed, tensor, T, E, k):
    out = np.empty((T, k), np.int32)
    lib().synth_topk_ids(seed, tensor, T, E, k, out.ctypes.data)
    return out


def uniform_int(seed, tensor, n, m):
    out = np.empty(n, np.int64)
    lib().synth_uniform_int(seed, tensor, n, m, out.ctypes.data)
    return out


def bf16_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f):
    """Round float32 to bf16 (nearest even) -- input preparation only."""
    u = np.ascontiguousarray(f, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(f, np.float32))
    if nan.any():
        r[nan] = 0x7FC0
    return r
