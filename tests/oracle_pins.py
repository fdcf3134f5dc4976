"""Pins that tie the oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix: the pages'
worked partition examples, brute-force enumeration on tiny inputs, closed
forms, exact results on inputs whose sums are exact, library routines
(numpy, a stable sort) on special cases, and invariants. The same pins run
against copies of the oracle with planted mistakes (test_oracle_mutants.py),
which shows that each plausible slip is caught by at least one of them.

Pages: [P-A2A] "FlashInfer MoE all-to-all optimisation: TRT-LLM's one-sided
A2A" (flashinfer PR #3697). [P-ACT] "FlashInfer MoE optimisation: overlapping
grouped activation staging on Ampere and Hopper" (flashinfer PR #7368).
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16(a):
    return synth.f32_to_bf16(np.asarray(a, np.float32))


def _silu(g):
    return g / (1.0 + math.exp(-g))


# ---------------------------------------------------------------- partition
def pin_partition_golden(orc):
    """[P-A2A] section 1, examples A (32 over 4) and B (384 over 5)."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "partition_examples.txt"))
            if l.strip() and not l.startswith("#")]
    assert rows
    for E, S, s, f, c in (map(int, r) for r in rows):
        assert orc.partition(E, S, s) == (f, c), (E, S, s)


def pin_partition_bruteforce(orc):
    """Shares tile [0, E) in order, sizes differ by at most one with the larger
    ones first, and the owner of e is the share whose range holds it; the owner
    also matches the arithmetic form base/remainder form of [P-A2A] section 1."""
    for E in range(1, 97):
        for S in range(1, 14):
            nxt = 0
            sizes = []
            for s in range(S):
                f, c = orc.partition(E, S, s)
                assert f == nxt, (E, S, s)
                nxt += c
                sizes.append(c)
            assert nxt == E
            assert max(sizes) - min(sizes) <= 1
            assert sizes == sorted(sizes, reverse=True)
            base, rem = divmod(E, S)
            for e in range(E):
                o = orc.owner(E, S, e)
                f, c = orc.partition(E, S, o)
                assert f <= e < f + c
                if e < rem * (base + 1):
                    assert o == e // (base + 1)
                else:
                    assert o == rem + (e - rem * (base + 1)) // base


# ------------------------------------------------------------------ routing
def _brute_topk(vals, k):
    """Among all k-subsets whose smallest value is >= every value left out,
    the one whose sorted id tuple is lexicographically smallest (= lower ids
    win ties); slots ordered by value descending, id ascending."""
    E = len(vals)
    best = None
    for sub in itertools.combinations(range(E), k):
        rest = [vals[e] for e in range(E) if e not in sub]
        if rest and min(vals[e] for e in sub) < max(rest):
            continue
        if best is None or sub < best:
            best = sub
    return sorted(best, key=lambda e: (-vals[e], e))


def pin_route_bruteforce(orc):
    rng = np.random.default_rng(7)
    levels = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.5], np.float32)
    for E in range(1, 8):
        for k in range(1, E + 1):
            lg = levels[rng.integers(0, len(levels), size=(40, E))].astype(np.float32)
            ids, _ = orc.route(lg, k)
            for t in range(lg.shape[0]):
                assert list(ids[t]) == _brute_topk([float(v) for v in lg[t]], k), (E, k, lg[t])


def pin_route_exhaustive_ties(orc):
    """Every logit pattern over three levels for E = 6, every k."""
    E = 6
    pats = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=E)), np.float32)
    for k in range(1, E + 1):
        ids, w = orc.route(pats, k)
        for t in range(pats.shape[0]):
            assert list(ids[t]) == _brute_topk([float(v) for v in pats[t]], k)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)


def pin_route_weights_closed_form(orc):
    """w_j = exp(l_j - l_max) / sum over the chosen of exp(l_i - l_max): the
    full-softmax normaliser cancels in the renormalisation."""
    lg = synth.normal_f32(5, 50, (200, 64), 2.0)
    ids, w = orc.route(lg, 8)
    for t in range(lg.shape[0]):
        sel = [float(lg[t, e]) for e in ids[t]]
        m = max(sel)
        ex = [math.exp(v - m) for v in sel]
        z = sum(ex)
        for j in range(8):
            assert abs(w[t, j] - ex[j] / z) <= 1e-13, (t, j)
        assert abs(sum(w[t]) - 1.0) <= 1e-13


def pin_route_special(orc):
    # all logits equal: ids 0..k-1, weights exactly 1/k
    ids, w = orc.route(np.full((3, 16), 0.75, np.float32), 8)
    assert (ids == np.arange(8)).all() and (w == 0.125).all()
    # k = 1 always weight 1
    lg = synth.normal_f32(3, 51, (50, 33), 1.0)
    ids, w = orc.route(lg, 1)
    assert (w == 1.0).all() and (ids[:, 0] == lg.argmax(1)).all()
    # k = E: the weights are the full softmax over all experts (numpy, fp64)
    lg = synth.normal_f32(3, 52, (20, 12), 1.5)
    ids, w = orc.route(lg, 12)
    l64 = lg.astype(np.float64)
    sm = np.exp(l64 - l64.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    assert np.allclose(np.take_along_axis(sm, ids, 1), w, rtol=0, atol=1e-14)
    # -0 ties +0: the lower id goes first
    ids, _ = orc.route(np.array([[0.0, -0.0, -1.0], [-0.0, 0.0, -1.0]], np.float32), 1)
    assert ids[0, 0] == 0 and ids[1, 0] == 0


# -------------------------------------------------------------- permutation
def _check_permute(orc, ids, E, first, L):
    T, k = ids.shape
    counts, offsets, perm, e2p = orc.permute(ids, E, first, L)
    flat = ids.reshape(-1)
    assert (counts == np.bincount(flat, minlength=E)).all()
    assert counts.sum() == T * k
    assert offsets[0] == 0 and (np.diff(offsets) == counts[first:first + L]).all()
    local = [r for r in range(T * k) if first <= flat[r] < first + L]
    want = sorted(local, key=lambda r: (flat[r], r))  # stable sort by expert
    assert list(perm) == want
    for p, r in enumerate(perm):
        assert e2p[r] == p
    for r in range(T * k):
        if not first <= flat[r] < first + L:
            assert e2p[r] == -1


def pin_permute_vs_stable_sort(orc):
    for (T, E, k, seed) in [(1, 8, 2, 1), (37, 8, 2, 2), (64, 64, 8, 3), (129, 1024, 8, 4),
                            (300, 5, 5, 5), (50, 300, 32, 6)]:
        ids = synth.topk_ids(seed, 60, T, E, k)
        for first, L in [(0, E), (0, E // 2), (E // 3, E - E // 3), (E - 1, 1), (E // 2, 0)]:
            _check_permute(orc, ids, E, first, L)


def pin_permute_structured(orc):
    T, E, k = 40, 16, 4
    shared = np.tile(np.array([3, 9, 0, 5], np.int32), (T, 1))
    disjoint = ((np.arange(T)[:, None] * k + np.arange(k)[None, :]) % E).astype(np.int32)
    for ids in (shared, disjoint):
        for first, L in [(0, E), (4, 6), (10, 0)]:
            _check_permute(orc, ids, E, first, L)
    counts, offsets, perm, e2p = orc.permute(shared, E, 0, E)
    assert list(perm[:T]) == [t * k + 2 for t in range(T)]  # expert 0 = slot 2 of each token


# ---------------------------------------------------------------------- FFN
def pin_expert_row_hand(orc):
    """H = 3, I = 2, chosen so that a swapped gate/up, a wrong silu or a
    transposed operand each change the answer."""
    x = _bf16([1.0, 2.0, -1.0])
    w1 = _bf16([[1, 0, 0],        # gate 0 -> g0 = 1
                [0, 1, 1],        # gate 1 -> g1 = 1
                [1, 1, 0],        # up 0   -> u0 = 3
                [0, 0.5, 0.5]])   # up 1   -> u1 = 0.5
    w2 = _bf16([[1, 0.5], [0, -1], [2, 0]])  # [H, I]
    out = orc.expert_row(x, w1, w2)
    a0, a1 = _silu(1.0) * 3.0, _silu(1.0) * 0.5
    want = [a0 + 0.5 * a1, -a1, 2 * a0]
    assert np.allclose(out, want, rtol=1e-15, atol=0), (out, want)
    x = _bf16([0.5, -2.0, 1.0])
    w1 = _bf16([[2, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 1]])
    out = orc.expert_row(x, w1, w2)
    a0, a1 = _silu(1.0) * 1.0, _silu(-2.0) * -0.5
    want = [a0 + 0.5 * a1, -a1, 2 * a0]
    assert np.allclose(out, want, rtol=1e-15, atol=1e-300), (out, want)


def pin_expert_row_vs_numpy(orc):
    H, I = 48, 80
    x = synth.normal_bf16(9, 61, (H,), 1.0)
    w1 = synth.normal_bf16(9, 62, (2 * I, H), 0.2)
    w2 = synth.normal_bf16(9, 63, (H, I), 0.2)
    xf, w1f, w2f = (synth.bf16_to_f32(a).astype(np.float64) for a in (x, w1, w2))
    g = w1f[:I] @ xf
    u = w1f[I:] @ xf
    want = w2f @ (g / (1.0 + np.exp(-g)) * u)
    out = orc.expert_row(x, w1, w2)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_expert_row_special(orc):
    H, I = 16, 8
    w1 = synth.normal_bf16(9, 64, (2 * I, H), 0.5)
    w2 = synth.normal_bf16(9, 65, (H, I), 0.5)
    assert (orc.expert_row(np.zeros(H, np.uint16), w1, w2) == 0).all()
    # gate rows = 8 * e_0, x = 5 e_0 -> g = 40, silu(g) = g up to e^-40
    x = _bf16([5.0] + [0.0] * (H - 1))
    w1s = synth.bf16_to_f32(w1).copy()
    w1s[:I] = 0.0
    w1s[:I, 0] = 8.0
    w1s = _bf16(w1s)
    u = synth.bf16_to_f32(w1s[I:]).astype(np.float64) @ synth.bf16_to_f32(x).astype(np.float64)
    want = synth.bf16_to_f32(w2).astype(np.float64) @ (40.0 * u)
    out = orc.expert_row(x, w1s, w2)
    assert np.allclose(out, want, rtol=1e-14, atol=1e-14 * np.abs(want).max())


def pin_grouped_ffn_structure(orc):
    """Entry p of local expert i uses token permuted_rows[p] // k ([P-ACT]
    section 1: route index divided by the route divisor) and expert i's weights."""
    T, H, I, E, k = 9, 16, 24, 5, 2
    x = synth.normal_bf16(4, 66, (T, H), 1.0)
    w1 = synth.normal_bf16(4, 67, (E, 2 * I, H), 0.3)
    w2 = synth.normal_bf16(4, 68, (E, H, I), 0.3)
    ids = synth.topk_ids(4, 69, T, E, k)
    first, L = 1, 3
    counts, offsets, perm, e2p = orc.permute(ids, E, first, L)
    out = orc.grouped_ffn(x, perm, offsets, k, w1[first:first + L], w2[first:first + L])
    assert out.shape == (offsets[-1], H)
    for p, r in enumerate(perm):
        t, e = r // k, ids.reshape(-1)[r]
        want = orc.expert_row(x[t], w1[e], w2[e])
        assert np.array_equal(out[p], want), p


# ------------------------------------------------------------- FP8 weights
def _e4m3_ref(codes):
    """Values of FP8 E4M3 codes by torch's float8_e4m3fn (a library decoder)."""
    import torch
    c = np.ascontiguousarray(codes, np.uint8)
    return torch.from_numpy(c.reshape(-1)).view(torch.float8_e4m3fn).double().numpy().reshape(c.shape)


def pin_e4m3_values(orc):
    """All 256 codes against torch's float8_e4m3fn, and the OCP FP8
    specification's landmarks: 448 (0x7E), the smallest normal 2^-6 (0x08),
    the smallest subnormal 2^-9 (0x01), 1 (0x38), -2 (0xC0), -0 (0x80), NaN
    (0x7F, 0xFF)."""
    ref = _e4m3_ref(np.arange(256))
    got = np.array([orc.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert (got[0x7E], got[0x08], got[0x01], got[0x38], got[0xC0]) == (448.0, 2.0**-6, 2.0**-9, 1.0, -2.0)
    assert got[0x80] == 0.0 and math.copysign(1.0, got[0x80]) < 0


def _fp8_layer(seed, T, H, I, E, k):
    """Random codes (no NaN) and per-row power-of-two scales, plus the same
    weights as bf16 bits: scale * value is exact in bf16 for these scales."""
    def codes(tensor, shape):
        c = synth.uniform_int(seed, tensor, int(np.prod(shape)), 254).astype(np.uint8)
        c[c >= 0x7F] += 1  # skip the NaN code 0x7F (0xFF is out of range)
        return c.reshape(shape)

    def scales(rows, e0):
        r = np.arange(rows)
        return np.stack([2.0 ** -(5 + (7 * r + 3 * e + e0) % 5) for e in range(E)]).astype(np.float32)

    x = synth.normal_bf16(seed, 70, (T, H), 1.0)
    q1, q2 = codes(71, (E, 2 * I, H)), codes(72, (E, H, I))
    s1, s2 = scales(2 * I, 0), scales(H, 1)
    w1 = _bf16(_e4m3_ref(q1) * s1[:, :, None])
    w2 = _bf16(_e4m3_ref(q2) * s2[:, :, None])
    assert np.array_equal(synth.bf16_to_f32(w1), (_e4m3_ref(q1) * s1[:, :, None]).astype(np.float32))
    return x, q1, s1, q2, s2, w1, w2


def pin_fp8_ffn_vs_bf16(orc):
    """With per-row power-of-two scales every dequantised weight scale *
    value is a bf16 number, so the FP8 grouped FFN equals the bf16 one on
    those bf16 weights exactly (same terms, same order); scales differ by row
    and by expert, so a scale taken from the wrong row or expert shows."""
    T, H, I, E, k = 7, 16, 24, 3, 2
    x, q1, s1, q2, s2, w1, w2 = _fp8_layer(11, T, H, I, E, k)
    ids = synth.topk_ids(11, 73, T, E, k)
    _, offsets, perm, _ = orc.permute(ids, E, 0, E)
    got = orc.grouped_ffn_fp8(x, perm, offsets, k, q1, s1, q2, s2)
    want = orc.grouped_ffn(x, perm, offsets, k, w1, w2)
    assert np.array_equal(got, want)
    # one expert row directly, and a share (experts 1..2)
    assert np.array_equal(orc.expert_row_fp8(x[0], q1[1], s1[1], q2[1], s2[1]),
                          orc.expert_row(x[0], w1[1], w2[1]))
    _, offsets, perm, _ = orc.permute(ids, E, 1, 2)
    got = orc.grouped_ffn_fp8(x, perm, offsets, k, q1[1:], s1[1:], q2[1:], s2[1:])
    want = orc.grouped_ffn(x, perm, offsets, k, w1[1:], w2[1:])
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ combine
def pin_combine(orc):
    T, k, H = 4, 2, 3
    eo = np.arange(1, 6 * H + 1, dtype=np.float64).reshape(6, H)
    e2p = np.array([0, -1, 2, 3, -1, -1, 5, 1], np.int32)
    w = np.array([0.25, 0.75, 0.5, 0.5, 0.1, 0.9, 1.0, 2.0])
    y = orc.combine(eo, e2p, w, T, k, H)
    want = np.stack([0.25 * eo[0], 0.5 * eo[2] + 0.5 * eo[3], np.zeros(H), eo[5] + 2.0 * eo[1]])
    assert np.array_equal(y, want)


# ------------------------------------------------------------------- router
def pin_router_exact(orc):
    """Inputs whose products and sums are exact in double: x in small
    integers/halves (bf16), W_g = m / 2^20 with |m| < 2^22 (fp32), bias = n / 2^20.
    The exact sum is an integer over 2^20, so the fp32 logit must equal one
    rounding of it (numpy float64 -> float32 of an exactly held double)."""
    rng = np.random.default_rng(11)
    T, H, E = 6, 64, 10
    xv = rng.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0, 3.0], size=(T, H))
    m = rng.integers(-(1 << 22) + 1, 1 << 22, size=(E, H))
    n = rng.integers(-(1 << 24), 1 << 24, size=E)
    wg = (m / float(1 << 20)).astype(np.float32)
    bias = (n / float(1 << 20)).astype(np.float32)
    assert np.array_equal(wg.astype(np.float64) * (1 << 20), m)
    x = _bf16(xv)
    assert np.array_equal(synth.bf16_to_f32(x), xv)
    lg = orc.router_logits(x, wg, bias)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(xv[t, h]) * Fraction(int(m[e, h]), 1 << 20) for h in range(H))
            exact += Fraction(int(n[e]), 1 << 20)
            assert float(exact) == exact  # held exactly in double
            assert lg[t, e] == np.float32(float(exact)), (t, e)
    # one-hot x picks a column of W_g; x = 0 gives the bias
    x1 = np.zeros((H, H), np.uint16)
    x1[np.arange(H), np.arange(H)] = _bf16([1.0])[0]
    lg = orc.router_logits(x1, wg)
    assert np.array_equal(lg, wg.T)
    lg = orc.router_logits(np.zeros((2, H), np.uint16), wg, bias)
    assert np.array_equal(lg, np.tile(bias, (2, 1)))


def pin_router_vs_numpy(orc):
    T, H, E = 12, 512, 24
    x = synth.normal_bf16(2, 70, (T, H), 1.0)
    wg = synth.normal_f32(2, 71, (E, H), 0.1)
    b = synth.normal_f32(2, 72, (E,), 1.0)
    ref = (synth.bf16_to_f32(x).astype(np.float64) @ wg.astype(np.float64).T
           + b.astype(np.float64))
    lg = orc.router_logits(x, wg, b)
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert (np.abs(lg - ref) <= ulp).all()
    assert (lg == ref.astype(np.float32)).mean() > 0.99


# ------------------------------------------------------------------ forward
def _small_layer(seed, T=24, H=32, I=40, E=10, k=3, bias=True):
    x = synth.normal_bf16(seed, 80, (T, H), 1.0)
    wg = synth.normal_f32(seed, 81, (E, H), 0.3)
    b = synth.normal_f32(seed, 82, (E,), 1.0) if bias else None
    w1 = synth.normal_bf16(seed, 83, (E, 2 * I, H), 0.2)
    w2 = synth.normal_bf16(seed, 84, (E, H, I), 0.2)
    return x, wg, b, w1, w2


def pin_forward_composition(orc):
    """The per-token forward equals route -> permute -> grouped FFN -> combine."""
    x, wg, b, w1, w2 = _small_layer(1)
    k, E = 3, wg.shape[0]
    lg, ids, w, y = orc.forward(x, wg, w1, w2, k, bias=b)
    assert np.array_equal(lg, orc.router_logits(x, wg, b))
    ids2, w2_ = orc.route(lg, k)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2_)
    counts, offsets, perm, e2p = orc.permute(ids, E)
    eo = orc.grouped_ffn(x, perm, offsets, k, w1, w2)
    y2 = orc.combine(eo, e2p, w, x.shape[0], k, x.shape[1])
    assert np.allclose(y, y2, rtol=1e-14, atol=1e-14 * np.abs(y).max())
    # a sample returns the same rows
    smp = np.array([5, 0, 23], np.int32)
    _, _, _, ys = orc.forward(x, wg, w1, w2, k, bias=b, sample=smp)
    assert np.array_equal(ys, y[smp])


def pin_forward_shares_sum(orc):
    """Weights are renormalised over all k before the share mask, so the
    outputs of all shares add up to the whole layer."""
    x, wg, b, w1, w2 = _small_layer(2, E=11, k=4)
    E, k, S = 11, 4, 3
    _, _, _, y_full = orc.forward(x, wg, w1, w2, k, bias=b)
    acc = np.zeros_like(y_full)
    for s in range(S):
        f, c = orc.partition(E, S, s)
        _, _, _, ys = orc.forward(x, wg, w1[f:f + c], w2[f:f + c], k, first=f, L=c, bias=b)
        acc += ys
    assert np.allclose(acc, y_full, rtol=1e-13, atol=1e-13 * np.abs(y_full).max())


def pin_forward_dense(orc):
    """E = k = 1: one expert with weight 1 is a dense SwiGLU FFN (numpy)."""
    x, wg, b, w1, w2 = _small_layer(3, E=1, k=1, T=7)
    _, ids, w, y = orc.forward(x, wg, w1, w2, 1, bias=b)
    assert (ids == 0).all() and (w == 1.0).all()
    I = w2.shape[2]
    xf = synth.bf16_to_f32(x).astype(np.float64)
    w1f = synth.bf16_to_f32(w1[0]).astype(np.float64)
    w2f = synth.bf16_to_f32(w2[0]).astype(np.float64)
    g, u = xf @ w1f[:I].T, xf @ w1f[I:].T
    want = (g / (1 + np.exp(-g)) * u) @ w2f.T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
