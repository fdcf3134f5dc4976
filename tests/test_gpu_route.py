"""moe_route and moe_permute against the oracle, bit-exact for ids, counts,
offsets and the permutation; weights within the fp32 bound below.

Weight tolerance (derived): the GPU forms exp(l_j - l_0) in fp32 (the
difference rounds with |l_j - l_0| <= ~12, an absolute error <= 1e-6, and
expf adds ~1 ulp), sums at most 32 terms and divides; the relative error of
w_j is below 3e-6, and w_j <= 1, so |w_gpu - w_oracle| <= 4e-6.
"""
import numpy as np
import pytest

import oracle
import routing_grouped_expert_amd as moe
import synth
from gpu_util import dev, empty, host, note, sync, torch
from synth import configs

pytestmark = pytest.mark.gpu
W_TOL = 4e-6


def gpu_route(logits, k):
    t = torch()
    T, E = logits.shape
    ids = empty((T, k), t.int32)
    w = empty((T, k), t.float32)
    moe.route(dev(logits), k, ids, w)
    sync()
    return host(ids), host(w)


def check_route(logits, k, what):
    note(f"route {what} T={logits.shape[0]} E={logits.shape[1]} k={k}")
    ids, w = gpu_route(logits, k)
    rid, rw = oracle.route(logits, k)
    assert np.array_equal(ids, rid), f"{what}: ids differ at {np.argwhere(ids != rid)[:5]}"
    assert np.abs(w - rw).max() <= W_TOL, f"{what}: weights off by {np.abs(w - rw).max():.2e}"
    assert np.abs(w.astype(np.float64).sum(1) - 1.0).max() <= W_TOL


@pytest.mark.parametrize("T", configs.ROUTING["T"])
def test_routing_workload(T):
    check_route(configs.routing_logits(T), configs.ROUTING["k"], "normal logits")


@pytest.mark.parametrize("T", configs.ROUTING["T"])
def test_routing_workload_ties(T):
    lg = configs.routing_logits(T, ties=True)
    check_route(lg, configs.ROUTING["k"], "eight-level logits")


@pytest.mark.parametrize("E,k", [(1, 1), (5, 5), (8, 2), (63, 7), (64, 8), (65, 8), (300, 32),
                                 (1024, 1), (2049, 8), (4096, 32)])
def test_routing_edges(E, k):
    lg = synth.normal_f32(77, 200 + E, (37, E), 1.0)
    check_route(lg, k, "edge")


def test_routing_special_values():
    lg = np.full((3, 100), 0.5, np.float32)
    ids, w = gpu_route(lg, 8)
    assert (ids == np.arange(8)).all() and np.abs(w - 0.125).max() == 0
    lg = np.array([[0.0, -0.0, -1.0, -0.0], [-0.0, 0.0, 0.0, -3.0]], np.float32)
    check_route(lg, 3, "signed zeros")


def gpu_permute(ids, E, first, L):
    t = torch()
    T, k = ids.shape
    counts = empty((E,), t.int32)
    offsets = empty((L + 1,), t.int32)
    perm = t.full((T * k,), -5, dtype=t.int32, device="cuda:0")
    e2p = empty((T * k,), t.int32)
    ws = moe.alloc_workspace(T, 128, 128, E, k, L)
    moe.permute(dev(ids), E, first, L, counts, offsets, perm, e2p, ws)
    sync()
    return host(counts), host(offsets), host(perm), host(e2p)


CASES = [(1, 8, 2, 0, 8), (32, 8, 2, 0, 8), (16, 8, 2, 2, 3), (64, 1024, 8, 0, 1024),
         (65, 8, 2, 0, 8), (200, 40, 4, 13, 9), (512, 256, 8, 0, 256), (4096, 1024, 8, 0, 1024),
         (4096, 384, 8, 0, 77), (4096, 384, 8, 308, 76), (100, 4096, 32, 1000, 2000),
         (129, 16, 4, 5, 0), (3000, 1, 1, 0, 1)]


@pytest.mark.parametrize("T,E,k,first,L", CASES)
def test_permute(T, E, k, first, L):
    note(f"permute T={T} E={E} k={k} share=({first},{L})")
    ids = synth.topk_ids(31, 300 + T, T, E, k)
    c, o, p, e = gpu_permute(ids, E, first, L)
    rc, ro, rp, re = oracle.permute(ids, E, first, L)
    assert np.array_equal(c, rc)
    assert np.array_equal(o, ro)
    n = ro[-1]
    assert np.array_equal(p[:n], rp)
    assert (p[n:] == -5).all()  # positions past N_L are not written
    assert np.array_equal(e, re)


def test_permute_structured():
    T, E, k = 300, 16, 4
    shared = np.tile(np.array([3, 9, 0, 5], np.int32), (T, 1))
    disjoint = ((np.arange(T)[:, None] * k + np.arange(k)[None, :]) % E).astype(np.int32)
    for ids in (shared, disjoint):
        for first, L in [(0, 16), (4, 6)]:
            got = gpu_permute(ids, E, first, L)
            want = oracle.permute(ids, E, first, L)
            for g, w_ in zip(got, want):
                assert np.array_equal(g[: len(w_)], w_)


def test_route_then_permute_repeatable():
    lg = configs.routing_logits(4096)
    a = gpu_route(lg, 8)
    for _ in range(3):
        b = gpu_route(lg, 8)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    p1 = gpu_permute(a[0], 1024, 0, 1024)
    p2 = gpu_permute(a[0], 1024, 0, 1024)
    for x, y in zip(p1, p2):
        assert np.array_equal(x, y)


def gpu_route_permute(logits, k, first, L, variant="auto"):
    t = torch()
    T, E = logits.shape
    ids = empty((T, k), t.int32)
    w = empty((T, k), t.float32)
    counts = empty((E,), t.int32)
    offsets = empty((L + 1,), t.int32)
    perm = t.full((T * k,), -5, dtype=t.int32, device="cuda:0")
    e2p = empty((T * k,), t.int32)
    ws = moe.alloc_workspace(T, 128, 128, E, k, L)
    moe.route_permute(dev(logits), k, first, L, ids, w, counts, offsets, perm, e2p, ws,
                      variant=variant)
    sync()
    return host(ids), host(w), host(counts), host(offsets), host(perm), host(e2p)


def check_route_permute(logits, k, first, L, what, variant="auto"):
    T, E = logits.shape
    note(f"route_permute {what} T={T} E={E} k={k} share=({first},{L}) variant={variant}")
    ids, w, c, o, p, e = gpu_route_permute(logits, k, first, L, variant)
    rid, rw = oracle.route(logits, k)
    assert np.array_equal(ids, rid), f"{what}: ids differ at {np.argwhere(ids != rid)[:5]}"
    assert np.abs(w - rw).max() <= W_TOL
    rc, ro, rp, re = oracle.permute(rid, E, first, L)
    assert np.array_equal(c, rc)
    assert np.array_equal(o, ro)
    n = ro[-1]
    assert np.array_equal(p[:n], rp)
    assert (p[n:] == -5).all()
    assert np.array_equal(e, re)


# Every values-per-lane tier (E up to 64, 128, 256, 512, 1024, 2048, 4096),
# with E a multiple of 4 (16-byte loads) or not, on both sides of the
# single-block form (T <= 64: selection and permutation in one kernel; T > 64:
# selection kernel writing the tile masks, then scan and scatter), tiles and
# token slices cut by T, and shares starting inside the expert range.
RP_CASES = [(1, 8, 2, 0, 8), (1, 1024, 8, 0, 1024), (5, 33, 3, 4, 20), (16, 100, 8, 0, 100),
            (64, 1024, 8, 0, 1024), (64, 4096, 32, 100, 3000), (37, 2048, 8, 0, 2048),
            (65, 1024, 8, 0, 1024), (100, 256, 8, 0, 77), (130, 130, 4, 10, 50),
            (512, 256, 8, 0, 256), (4096, 1024, 8, 0, 1024), (4096, 384, 8, 0, 77),
            (4100, 512, 8, 200, 312), (1000, 4096, 8, 0, 4096), (777, 2049, 16, 5, 2000),
            (300, 64, 8, 0, 64), (96, 1, 1, 0, 1)]


@pytest.mark.parametrize("T,E,k,first,L", RP_CASES)
def test_route_permute(T, E, k, first, L):
    lg = synth.normal_f32(53, 600 + T + E, (T, E), 1.0)
    check_route_permute(lg, k, first, L, "normal")


# Ties at or above the threshold: eight levels (the top level holds more than
# 64 of 1024 logits, so the candidate selection gives way to the k rounds),
# all-equal rows (every lane's maximum ties), and two levels.
@pytest.mark.parametrize("T", [1, 64, 200, 4096])
def test_route_permute_ties(T):
    check_route_permute(configs.routing_logits(T, ties=True), 8, 0, 1024, "eight levels")
    eq = np.full((T, 512), 0.25, np.float32)
    check_route_permute(eq, 8, 0, 512, "all equal")
    two = np.where(synth.normal_f32(5, 900 + T, (T, 300), 1.0) > 1.5, 1.0, -1.0).astype(np.float32)
    check_route_permute(two, 16, 0, 300, "two levels")


def test_route_permute_matches_separate_calls():
    """The fused call and moe_route + moe_permute give identical outputs."""
    for T in (3, 64, 4096):
        lg = configs.routing_logits(T)
        ids, w, c, o, p, e = gpu_route_permute(lg, 8, 0, 1024)
        ids2, w2 = gpu_route(lg, 8)
        assert np.array_equal(ids, ids2) and np.array_equal(w.view(np.uint32), w2.view(np.uint32))
        c2, o2, p2, e2 = gpu_permute(ids2, 1024, 0, 1024)
        n = o2[-1]
        assert np.array_equal(c, c2) and np.array_equal(o, o2) and np.array_equal(e, e2)
        assert np.array_equal(p[:n], p2[:n])


def variants_for(T, E, L):
    """The routing variants that apply to these sizes (the library's rule)."""
    out = ["tiled"]
    if T <= 64:
        out.append("one_block")
    nb = (T + 63) // 64
    if nb * E * 12 + 2 * (L + 17) * 4 <= 65536:
        out.append("two_kernels")
    return out


# Every variant on every values-per-lane tier it serves, both sides of its
# limits, shares, and the tie-heavy logits.
@pytest.mark.parametrize("T,E,k,first,L", [(1, 8, 2, 0, 8), (1, 4096, 32, 0, 4096),
                                            (7, 100, 5, 3, 90), (64, 1024, 8, 0, 1024),
                                            (64, 2048, 8, 7, 1000), (65, 256, 8, 0, 256),
                                            (256, 1024, 8, 0, 1024), (300, 40, 8, 0, 40),
                                            (1300, 256, 8, 0, 77), (2000, 16, 4, 2, 10)])
def test_route_permute_variants(T, E, k, first, L):
    lg = synth.normal_f32(59, 700 + T + E, (T, E), 1.0)
    for v in variants_for(T, E, L):
        check_route_permute(lg, k, first, L, "normal", variant=v)
    lt = configs.routing_logits(T, E=E, ties=True)
    for v in variants_for(T, E, L):
        check_route_permute(lt, min(k, E), first, L, "eight levels", variant=v)


def test_route_permute_variant_limits():
    """A variant outside its limits is refused before anything runs."""
    t = torch()
    lg = dev(configs.routing_logits(65, E=64))
    bufs = [empty((65, 8), t.int32), empty((65, 8), t.float32), empty((64,), t.int32),
            empty((65,), t.int32), empty((65 * 8,), t.int32), empty((65 * 8,), t.int32)]
    ws = moe.alloc_workspace(65, 128, 128, 64, 8, 64)
    with pytest.raises(moe.MoeError) as ei:
        moe.route_permute(lg, 8, 0, 64, *bufs, ws, variant="one_block")
    assert ei.value.status == 2
    assert moe.routing_plan(65, 64, 8, 64) in ("two_kernels", "tiled")
