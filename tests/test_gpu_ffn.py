"""moe_grouped_ffn and moe_combine against the oracle.

Grouped FFN tolerance (derived): inputs are exact bf16, products exact in
the MFMA, fp32 accumulation over K <= 16384 terms (relative error ~1e-6 of
the term scale), silu in fp32, and the intermediate carried as hi + lo bf16
(2^-17 relative). The output error stays below 1e-4 of max|ref| and the mean
below 2e-5 of mean|ref|.

Combine: one fp32 sum of at most k products, then one round to bf16: the
result is within half a bf16 ulp of the exact value, plus fp32 slack.
"""
import numpy as np
import pytest

import oracle
import routing_grouped_expert_amd as moe
import synth
from gpu_util import bf16_to_f64, dev, empty, host, note, sync, torch

pytestmark = pytest.mark.gpu


def pad_rows(perm, n):
    """permuted_rows as the library takes it: [T * k], the local entries
    first (positions past them are never read)."""
    out = np.full(n, -1, np.int32)
    out[:len(perm)] = perm
    return out


def layer(seed, T, H, I, E, k, first, L):
    x = synth.normal_bf16(seed, synth.X, (T, H), 1.0)
    w1 = synth.normal_bf16(seed, synth.W1, (L, 2 * I, H), 0.02, first_expert=first)
    w2 = synth.normal_bf16(seed, synth.W2, (L, H, I), 0.02, first_expert=first)
    ids = synth.topk_ids(seed, synth.IDS, T, E, k)
    return x, w1, w2, ids


def run_ffn(x, perm, offsets, k, w1, w2, x_offset=0, out_offset=0):
    """x_offset > 0 places x at an element offset inside a larger buffer (not
    16-byte aligned), which takes the checked element-wise path; out_offset
    does the same for expert_out."""
    t = torch()
    T, H = x.shape
    L = len(offsets) - 1
    I = w2.shape[2]
    xb = dev(np.concatenate([np.zeros(x_offset, np.uint16), x.reshape(-1)]))
    xd = xb[x_offset:].view(T, H)
    ob = t.full((T * k * H + out_offset,), float("nan"), dtype=t.float32, device="cuda:0")
    out = ob[out_offset:].view(T * k, H)
    ws = moe.alloc_workspace(T, H, I, 1 + L, k, L)
    pd = dev(pad_rows(perm, T * k))
    moe.grouped_ffn(xd, pd, dev(offsets), k, dev(w1), dev(w2), out, ws)
    sync()
    return host(out)


def check_ffn(T, H, I, E, k, first, L, seed=1, x_offset=0, ids=None):
    note(f"ffn T={T} H={H} I={I} E={E} k={k} share=({first},{L}) x_offset={x_offset}")
    x, w1, w2, rnd = layer(seed, T, H, I, E, k, first, L)
    ids = rnd if ids is None else ids
    _, offsets, perm, _ = oracle.permute(ids, E, first, L)
    got = run_ffn(x, perm, offsets, k, w1, w2, x_offset)
    n = offsets[-1]
    ref = oracle.grouped_ffn(x, perm, offsets, k, w1, w2)
    g = got[:n].astype(np.float64)
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    assert err.max() <= 1e-4 * np.abs(ref).max(), err.max() / np.abs(ref).max()
    assert err.mean() <= 2e-5 * np.abs(ref).mean(), err.mean() / np.abs(ref).mean()
    assert np.isnan(got[n:]).all()  # rows past N_L untouched


# one 16-token tile, two, four, eight (+ a second pass when an expert has > 128 rows)
@pytest.mark.parametrize("T,E,k", [(12, 4, 2), (30, 8, 2), (60, 6, 2), (300, 2, 1)])
def test_ffn_fast_path_tiles(T, E, k):
    check_ffn(T, 256, 384, E, k, 0, E)


# K-split path (H a multiple of 512, I of 1024; at most 16 mean-doubled
# entries per expert, one 16-token tile per pass). On a 256-CU part (256
# blocks): whole tiles only when the rounds come out nearly even (24, 32, 200);
# stream-K over all tiles, every tile cut, for the up kernel (16, 4096, 1024)
# and the down kernel (16, 512, 4096); one whole round and then stream-K with
# cut tiles for the up kernel (40, 1024, 1024) and the down kernel
# (40, 4096, 2048); (60, 512, 768) doubles to 30 and takes the staged path.
@pytest.mark.parametrize("T,H,I,E,k", [(24, 512, 1024, 8, 2), (60, 512, 768, 8, 2),
                                       (32, 4096, 1024, 8, 2), (16, 512, 4096, 4, 1),
                                       (200, 1024, 1024, 64, 2), (16, 4096, 1024, 4, 1),
                                       (40, 1024, 1024, 20, 2), (40, 4096, 2048, 20, 2)])
def test_ffn_stream_k(T, H, I, E, k):
    check_ffn(T, H, I, E, k, 0, E)


def test_ffn_stream_k_skewed_passes():
    """One expert takes every token (three 16-token passes), others few."""
    T, E, k = 40, 16, 2
    ids = np.stack([np.zeros(T, np.int32), 1 + np.arange(T, dtype=np.int32) % 15], 1)
    check_ffn(T, 512, 1024, E, k, 0, E, ids=ids)


def test_ffn_stream_k_share():
    check_ffn(48, 512, 1024, 12, 2, 4, 5)


# Prefill path (many entries per expert: 4 or 8 token tiles per pass, the
# token rows staged in LDS per block; H a multiple of 512, I of 256): one
# pass, several passes, a skewed expert, a share.
@pytest.mark.parametrize("T,H,I,E,k", [(96, 512, 256, 8, 2), (256, 512, 512, 8, 2),
                                       (512, 512, 256, 4, 2), (200, 1024, 512, 16, 8)])
def test_ffn_prefill(T, H, I, E, k):
    check_ffn(T, H, I, E, k, 0, E)


def test_ffn_prefill_whole_rounds():
    """512 experts of ~64 entries: 1024 up tiles and 1024 down tiles, four
    even rounds of a 256-CU part, so every tile is dealt whole."""
    check_ffn(4096, 512, 256, 512, 8, 0, 512)


def test_ffn_prefill_rounds_then_cuts():
    """300 experts of ~85 entries: 600 up and 600 down tiles, 2.3 rounds of a
    256-CU part: one whole round, then the remaining tiles cut into equal unit
    ranges, most of them finished through the cross-block fixup."""
    check_ffn(3200, 512, 256, 300, 8, 0, 300)


def test_ffn_prefill_skewed():
    T, E, k = 300, 6, 2
    ids = np.stack([np.full(T, 2, np.int32), (3 + np.arange(T, dtype=np.int32) % 3)], 1)
    check_ffn(T, 512, 256, E, k, 0, E, ids=ids)


def partial_pass_ids(counts, seed=3):
    """Top-1 selections with the given entries per expert, tokens shuffled:
    passes that fill every number of 16-token tiles."""
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    return np.random.default_rng(seed).permutation(ids).reshape(-1, 1)


# Passes of the staged kernels multiply only their token tiles that hold
# entries: 8-tile passes holding 1 to 8 tiles (an expert of 169 entries takes
# a full pass and a 3-tile one), and 4-tile passes holding 1 to 4.
@pytest.mark.parametrize("counts", [[1, 17, 33, 49, 65, 81, 97, 169],
                                    [1, 16, 17, 32, 33, 48, 49, 64, 63, 50, 31, 18, 15, 2, 40,
                                     33]])
def test_ffn_prefill_partial_passes(counts):
    ids = partial_pass_ids(counts)
    check_ffn(len(ids), 512, 256, len(counts), 1, 0, len(counts), ids=ids)


def test_ffn_prefill_share():
    check_ffn(384, 512, 256, 20, 4, 5, 6)


# Dense path (at least 112 local entries per local expert on average, H a
# multiple of 256, I of 128): passes of 256 tokens, 256 x 256 tiles of weight rows and
# tokens with both operands staged in LDS. Two passes per expert, a share,
# passes filling every number of 16-token groups of the four token quarters,
# one expert taking every token (four passes), an empty expert.
@pytest.mark.parametrize("T,H,I,E,k,first,L", [(1024, 256, 256, 4, 2, 0, 4),
                                               (2048, 512, 384, 8, 2, 2, 3),
                                               (600, 768, 256, 2, 1, 0, 2)])
def test_ffn_dense(T, H, I, E, k, first, L):
    check_ffn(T, H, I, E, k, first, L)


@pytest.mark.parametrize("counts", [[1, 17, 65, 129, 200, 255, 256, 257, 300, 511, 513, 600, 700],
                                    [600, 0, 400]])
def test_ffn_dense_partial_passes(counts):
    ids = partial_pass_ids(counts)
    check_ffn(len(ids), 256, 256, len(counts), 1, 0, len(counts), ids=ids)


def test_ffn_dense_skewed():
    T, E, k = 1024, 4, 2
    ids = np.stack([np.zeros(T, np.int32), 1 + np.arange(T, dtype=np.int32) % 3], 1)
    check_ffn(T, 256, 256, E, k, 0, E, ids=ids)


def test_ffn_share_and_empty_experts():
    check_ffn(40, 128, 256, 16, 2, 3, 9)   # several local experts get no rows


@pytest.mark.parametrize("H,I", [(200, 72), (130, 260), (8, 24)])
def test_ffn_checked_path_ragged(H, I):
    check_ffn(37, H, I, 5, 2, 0, 5)


def test_ffn_checked_path_misaligned():
    check_ffn(20, 256, 256, 4, 2, 0, 4, x_offset=3)


def test_ffn_no_rows():
    x, w1, w2, ids = layer(3, 8, 128, 128, 8, 1, 0, 2)
    offsets = np.zeros(3, np.int32)
    got = run_ffn(x, np.zeros(0, np.int32), offsets, 1, w1, w2)
    assert np.isnan(got).all()


def run_combine(eo, e2p, w, H):
    t = torch()
    T, k = w.shape
    y = empty((T, H), t.int16)
    moe.combine(dev(eo), dev(e2p), dev(w), y)
    sync()
    return host(y, np.uint16)


@pytest.mark.parametrize("T,E,k,H,first,L", [(16, 8, 2, 128, 0, 8), (64, 40, 8, 300, 5, 20),
                                             (33, 12, 3, 7, 0, 0)])
def test_combine(T, E, k, H, first, L):
    note(f"combine T={T} k={k} H={H} share=({first},{L})")
    ids = synth.topk_ids(9, 400, T, E, k)
    _, offsets, perm, e2p = oracle.permute(ids, E, first, L)
    n = max(int(offsets[-1]), 1)
    eo = synth.normal_f32(9, synth.EXPERT_OUT, (T * k, H), 1.0)
    w = np.abs(synth.normal_f32(9, synth.WEIGHTS, (T, k), 0.4))
    y = run_combine(eo, e2p, w, H)
    ref = oracle.combine(eo[:n].astype(np.float64), e2p, w.astype(np.float64), T, k, H)
    got = bf16_to_f64(y)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 65536.0  # bf16 ulp
    slack = 1e-6 * (np.abs(w).sum(1, keepdims=True) * np.abs(eo).max())
    assert (np.abs(got - ref) <= 0.5 * ulp + slack).all()
    if L == 0:
        assert (got == 0).all()


def test_ffn_checked_path_misaligned_out():
    """expert_out 4 bytes past a 16-byte boundary: the element-wise path."""
    note("ffn misaligned expert_out")
    x, w1, w2, ids = layer(4, 24, 256, 256, 4, 2, 0, 4)
    _, offsets, perm, _ = oracle.permute(ids, 4, 0, 4)
    got = run_ffn(x, perm, offsets, 2, w1, w2, out_offset=1)
    n = offsets[-1]
    ref = oracle.grouped_ffn(x, perm, offsets, 2, w1, w2)
    err = np.abs(got[:n].astype(np.float64) - ref)
    assert err.max() <= 1e-4 * np.abs(ref).max()
    assert np.isnan(got[n:]).all()


# An entry whose expanded index lies outside [0, T k) gathers a zero row on
# every path: the element-wise kernels (ragged H), the K-split kernels (one
# 16-token tile per pass), the staged kernels (token rows in LDS) and the
# dense kernels.
@pytest.mark.parametrize("T,H,I,E,k", [(37, 200, 72, 5, 2), (32, 4096, 1024, 8, 2),
                                       (256, 512, 512, 8, 2), (1024, 256, 256, 4, 2)])
def test_ffn_out_of_range_rows_are_zero(T, H, I, E, k):
    note(f"ffn out-of-range rows T={T} H={H} I={I} E={E} k={k}")
    x, w1, w2, ids = layer(5, T, H, I, E, k, 0, E)
    _, offsets, perm, _ = oracle.permute(ids, E, 0, E)
    n = int(offsets[-1])
    ref = oracle.grouped_ffn(x, perm, offsets, k, w1, w2)
    bad = [0, n // 2, n - 1]  # first entry of expert 0, a middle one, the last one
    perm2 = perm.copy()
    perm2[bad[0]], perm2[bad[1]], perm2[bad[2]] = T * k, -1, T * k + 77
    got = run_ffn(x, perm2, offsets, k, w1, w2)
    assert (got[bad] == 0).all()
    keep = np.setdiff1d(np.arange(n), bad)
    err = np.abs(got[keep].astype(np.float64) - ref[keep])
    assert err.max() <= 1e-4 * np.abs(ref).max()
    assert np.isnan(got[n:]).all()


# The fixed order of every sum (in-block wave order, cross-block fixup in
# block order) makes the output bitwise repeatable, with tiles cut between
# blocks: the K-split up kernel cut by stream-K, and the staged kernels with a
# whole round followed by cut tiles; and on the dense kernels.
@pytest.mark.parametrize("T,H,I,E,k", [(32, 4096, 1024, 8, 2), (40, 4096, 2048, 20, 2),
                                       (3200, 512, 256, 300, 8), (1024, 256, 256, 4, 2)])
def test_ffn_bitwise_repeatable(T, H, I, E, k):
    note(f"ffn repeatability T={T} H={H} I={I} E={E} k={k}")
    x, w1, w2, ids = layer(6, T, H, I, E, k, 0, E)
    _, offsets, perm, _ = oracle.permute(ids, E, 0, E)
    n = int(offsets[-1])
    runs = [run_ffn(x, perm, offsets, k, w1, w2)[:n] for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(r.view(np.uint32), runs[0].view(np.uint32))


def sampled_entries(offsets, n_tiles):
    """Entries at the edges of passes and 16-token tiles: for the first,
    middle and last experts with entries, positions 0, 15, 16, 31, 32, the
    last entry of each pass of NT tiles and the expert's last entry."""
    L = len(offsets) - 1
    cnt = np.diff(offsets)
    with_rows = np.flatnonzero(cnt)
    picks = set()
    for e in {with_rows[0], with_rows[len(with_rows) // 2], with_rows[-1],
              int(np.argmax(cnt))}:
        b, c = int(offsets[e]), int(cnt[e])
        for q in (0, 15, 16, 31, 32, 16 * n_tiles - 1, 16 * n_tiles, c - 1):
            if q < c:
                picks.add(b + q)
    return sorted(picks)


@pytest.mark.parametrize("name,skew", [("fine", False), ("share0", True)])
def test_ffn_full_size_sampled(name, skew):
    """The grouped FFN alone at the fine-grained and share-0 sizes (staged
    kernels with 4 and 8 token tiles per pass), bench.py's launch
    configuration: every output row of entries at pass and tile edges against
    the oracle's single-entry FFN. share0 adds an expert chosen by 300 tokens
    (three passes)."""
    from synth import configs
    d = configs.layer_inputs(configs.WORKLOADS[name])
    T, H, I, E, k, first, L = (d[n] for n in ("T", "H", "I", "E", "k", "first", "L"))
    note(f"ffn full size {name} T={T} H={H} I={I} E={E} k={k} share=({first},{L})")
    ids = synth.topk_ids(d["seed"], synth.IDS, T, E, k)
    if skew:
        for t in range(300):
            if first not in ids[t]:
                ids[t, k - 1] = first
    _, offsets, perm, _ = oracle.permute(ids, E, first, L)
    got = run_ffn(d["x"], perm, offsets, k, d["w1"], d["w2"])
    n = int(offsets[-1])
    assert np.isnan(got[n:]).all()
    nt = 4 if name == "fine" else 8
    for p in sampled_entries(offsets, nt):
        e = int(np.searchsorted(offsets, p, side="right") - 1)
        ref = oracle.expert_row(d["x"][perm[p] // k], d["w1"][e], d["w2"][e])
        err = np.abs(got[p].astype(np.float64) - ref)
        assert err.max() <= 1e-4 * np.abs(ref).max(), (p, err.max() / np.abs(ref).max())
