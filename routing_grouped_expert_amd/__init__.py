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
    "moe_grouped_ffn": ([_VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _SZ,
                         _VP], ctypes.c_int),
    "moe_grouped_ffn_fp8": ([_VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                             _VP, _SZ, _VP], ctypes.c_int),
    "moe_combine": ([_VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP], ctypes.c_int),
    "moe_forward": ([_VP, _VP, _VP, _VP, _VP] + [_I32] * 7 + [_VP, _VP, _VP, _VP, _VP, _SZ, _VP],
                    ctypes.c_int),
    "moe_forward_fp8": ([_VP] * 7 + [_I32] * 7 + [_VP, _VP, _VP, _VP, _VP, _SZ, _VP],
                        ctypes.c_int),
}


def lib():
    """Load libmoe.so (built in place by routing_grouped_expert_amd.build)."""
    global _lib
    if _lib is None:
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
    T, H = x.shape
    E = w_gate.shape[0]
    _check("moe_router_logits", lib().moe_router_logits(
        _ptr(x), _ptr(w_gate), _ptr(bias), T, H, E, _ptr(logits), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def route(logits, k, topk_ids, topk_weights, stream=None):
    T, E = logits.shape
    _check("moe_route", lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_ids),
                                        _ptr(topk_weights), _stream(stream)))


def permute(topk_ids, num_experts, first_expert, num_local, expert_counts, expert_offsets,
            permuted_rows, expanded_to_permuted, ws, stream=None):
    T, k = topk_ids.shape
    _check("moe_permute", lib().moe_permute(
        _ptr(topk_ids), T, k, num_experts, first_expert, num_local, _ptr(expert_counts),
        _ptr(expert_offsets), _ptr(permuted_rows), _ptr(expanded_to_permuted), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def grouped_ffn(x, permuted_rows, expert_offsets, k, w1, w2, expert_out, ws, stream=None):
    T, H = x.shape
    L = expert_offsets.shape[0] - 1
    I = w2.shape[-1]
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _ptr(x), _ptr(permuted_rows), _ptr(expert_offsets), L, T, k, H, I, _ptr(w1), _ptr(w2),
        _ptr(expert_out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def grouped_ffn_fp8(x, permuted_rows, expert_offsets, k, w1q, w1s, w2q, w2s, expert_out, ws,
                    stream=None):
    """moe_grouped_ffn_fp8: w1q [L, 2I, H] and w2q [L, H, I] uint8 E4M3 codes,
    w1s [L, 2I] and w2s [L, H] fp32 row scales."""
    T, H = x.shape
    L = expert_offsets.shape[0] - 1
    I = w2q.shape[-1]
    _check("moe_grouped_ffn_fp8", lib().moe_grouped_ffn_fp8(
        _ptr(x), _ptr(permuted_rows), _ptr(expert_offsets), L, T, k, H, I, _ptr(w1q), _ptr(w1s),
        _ptr(w2q), _ptr(w2s), _ptr(expert_out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def combine(expert_out, expanded_to_permuted, topk_weights, y, stream=None):
    T, k = topk_weights.shape
    H = y.shape[1]
    _check("moe_combine", lib().moe_combine(_ptr(expert_out), _ptr(expanded_to_permuted),
                                            _ptr(topk_weights), T, k, H, _ptr(y),
                                            _stream(stream)))


def forward(x, w_gate, router_bias, w1, w2, k, first_expert, num_local, y, ws, logits_out=None,
            topk_ids_out=None, topk_weights_out=None, stream=None):
    T, H = x.shape
    E = w_gate.shape[0]
    I = w2.shape[-1]
    _check("moe_forward", lib().moe_forward(
        _ptr(x), _ptr(w_gate), _ptr(router_bias), _ptr(w1), _ptr(w2), T, H, I, E, k,
        first_expert, num_local, _ptr(y), _ptr(logits_out), _ptr(topk_ids_out),
        _ptr(topk_weights_out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def forward_fp8(x, w_gate, router_bias, w1q, w1s, w2q, w2s, k, first_expert, num_local, y, ws,
                logits_out=None, topk_ids_out=None, topk_weights_out=None, stream=None):
    """moe_forward_fp8: the layer with FP8 expert weights (codes and row scales
    as for grouped_ffn_fp8)."""
    T, H = x.shape
    E = w_gate.shape[0]
    I = w2q.shape[-1]
    _check("moe_forward_fp8", lib().moe_forward_fp8(
        _ptr(x), _ptr(w_gate), _ptr(router_bias), _ptr(w1q), _ptr(w1s), _ptr(w2q), _ptr(w2s), T,
        H, I, E, k, first_expert, num_local, _ptr(y), _ptr(logits_out), _ptr(topk_ids_out),
        _ptr(topk_weights_out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def alloc_workspace(T, H, I, E, k, num_local, device="cuda"):
    """A uint8 torch tensor of moe_workspace_size bytes (torch allocations are
    256-byte aligned)."""
    import torch
    n = workspace_size(T, H, I, E, k, num_local)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
