"""The C-ABI library on the host: it loads, exports every symbol include/moe.h
declares, and rejects bad arguments before anything is launched (no GPU)."""
import ctypes
import os
import re

import pytest

import routing_grouped_expert_amd as moe
from conftest import golden


def _declared():
    src = open(moe.HEADER).read()
    return set(re.findall(r"^(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", src, re.M))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"moe_partition", "moe_workspace_size", "moe_router_logits", "moe_route",
            "moe_permute", "moe_grouped_ffn", "moe_grouped_ffn_fp8", "moe_combine", "moe_forward",
            "moe_forward_fp8", "moe_status_string", "moe_last_launch_error"} <= names
    L = ctypes.CDLL(moe.LIB_PATH)
    for n in sorted(names):
        assert hasattr(L, n), n
    # and the library's own names match the header's (nothing undeclared)
    out = os.popen(f"nm -D --defined-only {moe.LIB_PATH}").read()
    exported = set(re.findall(r" T (moe_\w+)$", out, re.M))
    assert exported == names


def test_probe_library_exports_its_one_symbol():
    """The measurement-only read probe is a library of its own (not part of
    moe.h): it exports hbm_read_probe and nothing named moe_*."""
    path = os.path.join(os.path.dirname(moe.LIB_PATH), "libhbmprobe.so")
    L = ctypes.CDLL(path)
    assert hasattr(L, "hbm_read_probe")
    out = os.popen(f"nm -D --defined-only {path}").read()
    assert not re.findall(r" T (moe_\w+)$", out, re.M)


def test_status_strings():
    L = moe.lib()
    for code, name in moe.STATUS.items():
        assert L.moe_status_string(code).decode() == name
    assert L.moe_last_launch_error().decode() == "hipSuccess"


def test_partition_matches_worked_examples():
    rows = [l.split() for l in open(golden("partition_examples.txt"))
            if l.strip() and not l.startswith("#")]
    for E, S, s, f, c in (map(int, r) for r in rows):
        assert moe.partition(E, S, s) == (f, c)


def test_partition_agrees_with_oracle():
    import oracle
    for E in range(1, 70):
        for S in range(1, 12):
            for s in range(S):
                assert moe.partition(E, S, s) == oracle.partition(E, S, s)


def test_partition_rejects():
    for args in [(0, 4, 0), (8, 0, 0), (8, 4, 4), (8, 4, -1)]:
        with pytest.raises(moe.MoeError) as ei:
            moe.partition(*args)
        assert ei.value.status == 1
    L = moe.lib()
    assert L.moe_partition(8, 2, 0, None, None) == 1


def test_workspace_size():
    a = moe.workspace_size(32, 4096, 14336, 8, 2, 8)
    b = moe.workspace_size(64, 4096, 14336, 8, 2, 8)
    assert 0 < a < b and a % 256 == 0
    with pytest.raises(moe.MoeError):
        moe.workspace_size(4, 64, 64, 8, 9, 8)      # k > E
    with pytest.raises(moe.MoeError) as ei:
        moe.workspace_size(4, 64, 64, 8000, 2, 8)   # E beyond the limit
    assert ei.value.status == 2


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first


def test_calls_reject_bad_arguments_without_launching():
    L = moe.lib()
    # route: k > E, k > 32, E = 0, null pointers
    assert L.moe_route(FAKE, 4, 8, 9, FAKE, FAKE, None) == 1
    assert L.moe_route(FAKE, 4, 64, 33, FAKE, FAKE, None) == 2
    assert L.moe_route(FAKE, 4, 0, 1, FAKE, FAKE, None) == 1
    assert L.moe_route(None, 4, 8, 2, FAKE, FAKE, None) == 1
    assert L.moe_route(None, 0, 8, 2, None, None, None) == 0  # T = 0: nothing to do
    # permute: share out of range, missing workspace for T > 64
    assert L.moe_permute(FAKE, 4, 2, 8, 6, 3, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert L.moe_permute(FAKE, 100, 2, 8, 0, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 3
    assert L.moe_permute(FAKE, 100, 2, 8, 0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    misaligned = ctypes.c_void_p(0x1010)
    assert L.moe_permute(FAKE, 100, 2, 8, 0, 8, FAKE, FAKE, FAKE, FAKE, misaligned, 1 << 20,
                         None) == 3
    # grouped ffn: bad dims, workspace too small
    assert L.moe_grouped_ffn(FAKE, FAKE, FAKE, 2, 4, 2, 0, 64, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                             None) == 1
    assert L.moe_grouped_ffn(FAKE, FAKE, FAKE, 2, 4, 2, 64, 64, FAKE, FAKE, FAKE, FAKE, 8,
                             None) == 3
    # grouped ffn with FP8 weights: bad dims, missing scales, workspace too small
    assert L.moe_grouped_ffn_fp8(FAKE, FAKE, FAKE, 2, 4, 2, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, 1 << 20, None) == 1
    assert L.moe_grouped_ffn_fp8(FAKE, FAKE, FAKE, 2, 4, 2, 64, 64, FAKE, None, FAKE, FAKE, FAKE,
                                 FAKE, 1 << 20, None) == 1
    assert L.moe_grouped_ffn_fp8(FAKE, FAKE, FAKE, 2, 4, 2, 64, 64, FAKE, FAKE, FAKE, None, FAKE,
                                 FAKE, 1 << 20, None) == 1
    assert L.moe_grouped_ffn_fp8(FAKE, FAKE, FAKE, 2, 4, 2, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, 8, None) == 3
    # combine: H = 0, k = 0
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 2, 0, FAKE, None) == 1
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 0, 8, FAKE, None) == 1
    # forward: share past E, workspace too small, null y
    assert L.moe_forward(FAKE, FAKE, None, FAKE, FAKE, 4, 64, 64, 8, 2, 4, 5, FAKE, None, None,
                         None, FAKE, 1 << 30, None) == 1
    assert L.moe_forward(FAKE, FAKE, None, FAKE, FAKE, 4, 64, 64, 8, 2, 0, 8, FAKE, None, None,
                         None, FAKE, 256, None) == 3
    assert L.moe_forward(FAKE, FAKE, None, FAKE, FAKE, 4, 64, 64, 8, 2, 0, 8, None, None, None,
                         None, FAKE, 1 << 30, None) == 1
    # forward with FP8 weights: share past E, a missing scale, workspace too small
    assert L.moe_forward_fp8(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 8, 2, 4, 5,
                             FAKE, None, None, None, FAKE, 1 << 30, None) == 1
    assert L.moe_forward_fp8(FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 4, 64, 64, 8, 2, 0, 8,
                             FAKE, None, None, None, FAKE, 1 << 30, None) == 1
    assert L.moe_forward_fp8(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 8, 2, 0, 8,
                             FAKE, None, None, None, FAKE, 256, None) == 3
    assert L.moe_router_logits(FAKE, FAKE, None, 4, 0, 8, FAKE, None, 0, None) == 1
    assert L.moe_router_logits(FAKE, FAKE, None, 100, 64, 8, FAKE, None, 0, None) == 3
