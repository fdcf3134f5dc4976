"""Python binding of libmoe.so: the MI355X MoE layer forward (C ABI in include/moe.h).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors on the GPU (PyTorch supplies device memory and the
stream); bf16 tensors may be torch.bfloat16 or 16-bit integer views of the
bit patterns. Every call checks the returned status and raises MoeError.
There is no fallback: without the compiled library every call fails.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

STATUS = {0: "MOE_SUCCESS", 1: "MOE_ERROR_INVALID_VALUE", 2: "MOE_ERROR_UNSUPPORTED",
          3: "MOE_ERROR_WORKSPACE", 4: "MOE_ERROR_LAUNCH"}


class MoeError(RuntimeError):
    def __init__(self, fn, status, detail=""):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}{detail}")
        self.status = status


_lib = None
_I32 = ctypes.c_int32
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_last_launch_error": ([], ctypes.c_char_p),
    "moe_partition": ([_I32, _I32, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)], ctypes.c_int),
    "moe_workspace_size": ([_I32] * 6 + [ctypes.POINTER(_SZ)], ctypes.c_int),
    "moe_router_logits": ([_VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "moe_route": ([_VP, _I32, _I32, _I32, _VP, _VP, _VP], ctypes.c_int),
    "moe_permute": ([_VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
                    ctypes.c_int),
    "moe_route_permute": ([_VP, _I32, _I32, _I32, _I32, _I32] + [_VP] * 7 + [_SZ, _VP],
                          ctypes.c_int),
    "moe_route_permute_variant": ([_VP, _I32, _I32, _I32, _I32, _I32] + [_VP] * 7 +
                                  [_SZ, _I32, _VP], ctypes.c_int),
    "moe_routing_plan": ([_I32, _I32, _I32, _I32, ctypes.POINTER(_I32)], ctypes.c_int),
    "moe_grouped_ffn": ([_VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _SZ,
                         _VP], ctypes.c_int),
    "moe_grouped_ffn_fp8": ([_VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                             _VP, _SZ, _VP], ctypes.c_int),
    "moe_combine": ([_VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP], ctypes.c_int),
    "moe_forward": ([_VP, _VP, _VP, _VP, _VP] + [_I32] * 7 + [_VP, _VP, _VP, _VP, _VP, _SZ, _VP],
                    ctypes.c_int),
    "moe_forward_fp8": ([_VP] * 7 + [_I32] * 7 + [_VP, _VP, _VP, _VP, _VP, _SZ, _VP],
                        ctypes.c_int),
    "moe_forward_no_alloc": ([_VP, _VP, _VP, _VP, _VP] + [_I32] * 7 + [_VP, _VP, _VP, _VP, _VP],
                             ctypes.c_int),
}

NO_ALLOC_SCRATCH_BYTES = 128 << 20


def lib():
    """Load libmoe.so (built in place by routing_grouped_expert_amd.build).

    torch is imported first: it carries its own HIP runtime under the same
    soname as the system one that libmoe.so names, and whichever is loaded
    first serves the whole process. Loading the library first would hand
    torch a runtime it was not built against (it then finds no GPU)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (see above)
        if not os.path.exists(LIB_PATH):
            from . import build
            build.build()
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn, st):
    if st != 0:
        detail = ""
        if st == 4:
            detail = f" ({lib().moe_last_launch_error().decode()})"
        raise MoeError(fn, st, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, esize, optional=False):
    """Raise ValueError unless t is a contiguous GPU tensor of `shape` whose
    elements are `esize` bytes (None allowed when optional). Checked before
    every call, so a host tensor, a strided view or a wrong shape never
    reaches a kernel."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() != esize:
        raise ValueError(f"{name} must have {esize}-byte elements, not {t.element_size()}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_ws(ws):
    if ws is None:
        return 0
    if not getattr(ws, "is_cuda", False) or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous GPU tensor")
    return ws.numel() * ws.element_size()


def _dims(t, name, nd):
    if t is None or t.dim() != nd:
        raise ValueError(f"{name} must be a {nd}-d tensor")
    return tuple(t.shape)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def partition(num_experts, num_shares, share):
    """(first_expert, num_local) of a contiguous ceil/floor expert share."""
    f, c = _I32(), _I32()
    _check("moe_partition", lib().moe_partition(num_experts, num_shares, share, ctypes.byref(f),
                                                ctypes.byref(c)))
    return f.value, c.value


def workspace_size(T, H, I, E, k, num_local):
    n = _SZ()
    _check("moe_workspace_size", lib().moe_workspace_size(T, H, I, E, k, num_local,
                                                          ctypes.byref(n)))
    return n.value


def router_logits(x, w_gate, bias, logits, ws, stream=None):
    T, H = _dims(x, "x", 2)
    E = _dims(w_gate, "w_gate", 2)[0]
    _need(x, "x", (T, H), 2)
    _need(w_gate, "w_gate", (E, H), 4)
    _need(bias, "bias", (E,), 4, optional=True)
    _need(logits, "logits", (T, E), 4)
    nws = _need_ws(ws)
    _check("moe_router_logits", lib().moe_router_logits(
        _ptr(x), _ptr(w_gate), _ptr(bias), T, H, E, _ptr(logits), _ptr(ws), nws,
        _stream(stream)))


def route(logits, k, topk_ids, topk_weights, stream=None):
    T, E = _dims(logits, "logits", 2)
    _need(logits, "logits", (T, E), 4)
    _need(topk_ids, "topk_ids", (T, k), 4)
    _need(topk_weights, "topk_weights", (T, k), 4)
    _check("moe_route", lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_ids),
                                        _ptr(topk_weights), _stream(stream)))


def permute(topk_ids, num_experts, first_expert, num_local, expert_counts, expert_offsets,
            permuted_rows, expanded_to_permuted, ws, stream=None):
    T, k = _dims(topk_ids, "topk_ids", 2)
    _need(topk_ids, "topk_ids", (T, k), 4)
    _need(expert_counts, "expert_counts", (num_experts,), 4)
    _need(expert_offsets, "expert_offsets", (num_local + 1,), 4)
    _need(permuted_rows, "permuted_rows", (T * k,), 4)
    _need(expanded_to_permuted, "expanded_to_permuted", (T * k,), 4)
    nws = _need_ws(ws)
    _check("moe_permute", lib().moe_permute(
        _ptr(topk_ids), T, k, num_experts, first_expert, num_local, _ptr(expert_counts),
        _ptr(expert_offsets), _ptr(permuted_rows), _ptr(expanded_to_permuted), _ptr(ws), nws,
        _stream(stream)))


ROUTING_VARIANTS = {"auto": 0, "one_block": 1, "two_kernels": 2, "tiled": 3}


def routing_plan(T, E, k, num_local):
    """Name of the routing variant moe_route_permute runs for these sizes."""
    v = _I32()
    _check("moe_routing_plan", lib().moe_routing_plan(T, E, k, num_local, ctypes.byref(v)))
    return {c: n for n, c in ROUTING_VARIANTS.items()}[v.value]


def route_permute(logits, k, first_expert, num_local, topk_ids, topk_weights, expert_counts,
                  expert_offsets, permuted_rows, expanded_to_permuted, ws, stream=None,
                  variant="auto"):
    """moe_route_permute: routing then the permutation, in one call (variant:
    a key of ROUTING_VARIANTS; "auto" is the plan)."""
    T, E = _dims(logits, "logits", 2)
    _need(logits, "logits", (T, E), 4)
    _need(topk_ids, "topk_ids", (T, k), 4)
    _need(topk_weights, "topk_weights", (T, k), 4)
    _need(expert_counts, "expert_counts", (E,), 4)
    _need(expert_offsets, "expert_offsets", (num_local + 1,), 4)
    _need(permuted_rows, "permuted_rows", (T * k,), 4)
    _need(expanded_to_permuted, "expanded_to_permuted", (T * k,), 4)
    nws = _need_ws(ws)
    if variant == "auto":
        _check("moe_route_permute", lib().moe_route_permute(
            _ptr(logits), T, E, k, first_expert, num_local, _ptr(topk_ids), _ptr(topk_weights),
            _ptr(expert_counts), _ptr(expert_offsets), _ptr(permuted_rows),
            _ptr(expanded_to_permuted), _ptr(ws), nws, _stream(stream)))
        return
    _check("moe_route_permute_variant", lib().moe_route_permute_variant(
        _ptr(logits), T, E, k, first_expert, num_local, _ptr(topk_ids), _ptr(topk_weights),
        _ptr(expert_counts), _ptr(expert_offsets), _ptr(permuted_rows),
        _ptr(expanded_to_permuted), _ptr(ws), nws, ROUTING_VARIANTS[variant], _stream(stream)))


def _ffn_common(x, permuted_rows, expert_offsets, k, w2, expert_out):
    T, H = _dims(x, "x", 2)
    L = _dims(expert_offsets, "expert_offsets", 1)[0] - 1
    I = _dims(w2, "w2", 3)[2]
    _need(x, "x", (T, H), 2)
    _need(permuted_rows, "permuted_rows", (T * k,), 4)
    _need(expert_offsets, "expert_offsets", (L + 1,), 4)
    _need(expert_out, "expert_out", (T * k, H), 4)
    return T, H, L, I


def grouped_ffn(x, permuted_rows, expert_offsets, k, w1, w2, expert_out, ws, stream=None):
    T, H, L, I = _ffn_common(x, permuted_rows, expert_offsets, k, w2, expert_out)
    _need(w1, "w1", (L, 2 * I, H), 2)
    _need(w2, "w2", (L, H, I), 2)
    nws = _need_ws(ws)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _ptr(x), _ptr(permuted_rows), _ptr(expert_offsets), L, T, k, H, I, _ptr(w1), _ptr(w2),
        _ptr(expert_out), _ptr(ws), nws, _stream(stream)))


def grouped_ffn_fp8(x, permuted_rows, expert_offsets, k, w1q, w1s, w2q, w2s, expert_out, ws,
                    stream=None):
    """moe_grouped_ffn_fp8: w1q [L, 2I, H] and w2q [L, H, I] uint8 E4M3 codes,
    w1s [L, 2I] and w2s [L, H] fp32 row scales."""
    T, H, L, I = _ffn_common(x, permuted_rows, expert_offsets, k, w2q, expert_out)
    _need(w1q, "w1q", (L, 2 * I, H), 1)
    _need(w1s, "w1s", (L, 2 * I), 4)
    _need(w2q, "w2q", (L, H, I), 1)
    _need(w2s, "w2s", (L, H), 4)
    nws = _need_ws(ws)
    _check("moe_grouped_ffn_fp8", lib().moe_grouped_ffn_fp8(
        _ptr(x), _ptr(permuted_rows), _ptr(expert_offsets), L, T, k, H, I, _ptr(w1q), _ptr(w1s),
        _ptr(w2q), _ptr(w2s), _ptr(expert_out), _ptr(ws), nws, _stream(stream)))


def combine(expert_out, expanded_to_permuted, topk_weights, y, stream=None):
    T, k = _dims(topk_weights, "topk_weights", 2)
    H = _dims(y, "y", 2)[1]
    _need(topk_weights, "topk_weights", (T, k), 4)
    _need(y, "y", (T, H), 2)
    _need(expert_out, "expert_out", (T * k, H), 4)
    _need(expanded_to_permuted, "expanded_to_permuted", (T * k,), 4)
    _check("moe_combine", lib().moe_combine(_ptr(expert_out), _ptr(expanded_to_permuted),
                                            _ptr(topk_weights), T, k, H, _ptr(y),
                                            _stream(stream)))


def _forward_common(x, w_gate, router_bias, k, y, logits_out, topk_ids_out, topk_weights_out):
    T, H = _dims(x, "x", 2)
    E = _dims(w_gate, "w_gate", 2)[0]
    _need(x, "x", (T, H), 2)
    _need(w_gate, "w_gate", (E, H), 4)
    _need(router_bias, "router_bias", (E,), 4, optional=True)
    _need(y, "y", (T, H), 2)
    _need(logits_out, "logits_out", (T, E), 4, optional=True)
    _need(topk_ids_out, "topk_ids_out", (T, k), 4, optional=True)
    _need(topk_weights_out, "topk_weights_out", (T, k), 4, optional=True)
    return T, H, E


def forward(x, w_gate, router_bias, w1, w2, k, first_expert, num_local, y, ws, logits_out=None,
            topk_ids_out=None, topk_weights_out=None, stream=None):
    T, H, E = _forward_common(x, w_gate, router_bias, k, y, logits_out, topk_ids_out,
                              topk_weights_out)
    I = _dims(w2, "w2", 3)[2]
    _need(w1, "w1", (num_local, 2 * I, H), 2)
    _need(w2, "w2", (num_local, H, I), 2)
    nws = _need_ws(ws)
    _check("moe_forward", lib().moe_forward(
        _ptr(x), _ptr(w_gate), _ptr(router_bias), _ptr(w1), _ptr(w2), T, H, I, E, k,
        first_expert, num_local, _ptr(y), _ptr(logits_out), _ptr(topk_ids_out),
        _ptr(topk_weights_out), _ptr(ws), nws, _stream(stream)))


def forward_fp8(x, w_gate, router_bias, w1q, w1s, w2q, w2s, k, first_expert, num_local, y, ws,
                logits_out=None, topk_ids_out=None, topk_weights_out=None, stream=None):
    """moe_forward_fp8: the layer with FP8 expert weights (codes and row scales
    as for grouped_ffn_fp8)."""
    T, H, E = _forward_common(x, w_gate, router_bias, k, y, logits_out, topk_ids_out,
                              topk_weights_out)
    I = _dims(w2q, "w2q", 3)[2]
    _need(w1q, "w1q", (num_local, 2 * I, H), 1)
    _need(w1s, "w1s", (num_local, 2 * I), 4)
    _need(w2q, "w2q", (num_local, H, I), 1)
    _need(w2s, "w2s", (num_local, H), 4)
    nws = _need_ws(ws)
    _check("moe_forward_fp8", lib().moe_forward_fp8(
        _ptr(x), _ptr(w_gate), _ptr(router_bias), _ptr(w1q), _ptr(w1s), _ptr(w2q), _ptr(w2s), T,
        H, I, E, k, first_expert, num_local, _ptr(y), _ptr(logits_out), _ptr(topk_ids_out),
        _ptr(topk_weights_out), _ptr(ws), nws, _stream(stream)))


def forward_no_alloc(x, w_gate, router_bias, w1, w2, k, first_expert, num_local, y,
                     logits_out=None, topk_ids_out=None, topk_weights_out=None, stream=None):
    """moe_forward_no_alloc: the layer on the library's own device scratch
    (no workspace argument; sizes whose workspace exceeds
    NO_ALLOC_SCRATCH_BYTES are rejected)."""
    T, H, E = _forward_common(x, w_gate, router_bias, k, y, logits_out, topk_ids_out,
                              topk_weights_out)
    I = _dims(w2, "w2", 3)[2]
    _need(w1, "w1", (num_local, 2 * I, H), 2)
    _need(w2, "w2", (num_local, H, I), 2)
    _check("moe_forward_no_alloc", lib().moe_forward_no_alloc(
        _ptr(x), _ptr(w_gate), _ptr(router_bias), _ptr(w1), _ptr(w2), T, H, I, E, k,
        first_expert, num_local, _ptr(y), _ptr(logits_out), _ptr(topk_ids_out),
        _ptr(topk_weights_out), _stream(stream)))


def alloc_workspace(T, H, I, E, k, num_local, device="cuda"):
    """A uint8 torch tensor of moe_workspace_size bytes (torch allocations are
    256-byte aligned)."""
    import torch
    n = workspace_size(T, H, I, E, k, num_local)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
