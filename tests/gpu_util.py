"""Helpers for the GPU parity tests: device copies of numpy inputs, read-back,
and the tolerance checks, all in one place."""
import sys

import numpy as np

import routing_grouped_expert_amd as moe


def torch():
    import torch as t
    return t


def dev(a):
    """numpy -> torch tensor on cuda:0 holding the same bytes (bf16 bit
    patterns travel as int16)."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).to("cuda:0")


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty(shape, dtype):
    t = torch()
    return t.empty(shape, dtype=dtype, device="cuda:0")


def sync():
    torch().cuda.synchronize()


def note(msg):
    """Name the case on stdout before a GPU step (flushed)."""
    sys.stdout.write(f"[case] {msg}\n")
    sys.stdout.flush()


def bf16_to_f64(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def layer_tolerance(y_bf16, ref):
    """The layer-output bar: max|err| <= 2e-2 max|ref| and
    mean|err| <= 2e-3 mean|ref| (bf16 output against the fp64 oracle)."""
    y = bf16_to_f64(y_bf16)
    err = np.abs(y - ref)
    mx, mean = err.max() / np.abs(ref).max(), err.mean() / np.abs(ref).mean()
    return mx, mean


def assert_layer_ok(y_bf16, ref, what=""):
    mx, mean = layer_tolerance(y_bf16, ref)
    assert mx <= 2e-2 and mean <= 2e-3, f"{what}: max ratio {mx:.3e}, mean ratio {mean:.3e}"
    return mx, mean


def workspace(T, H, I, E, k, L):
    return moe.alloc_workspace(T, H, I, E, k, L)
