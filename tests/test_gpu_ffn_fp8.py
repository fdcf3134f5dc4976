"""moe_grouped_ffn_fp8 against the oracle (FP8 E4M3 weights, per-row scales).

Tolerance (derived as for the bf16 FFN): every E4M3 code is a bf16 number,
so the widened weights are exact, the MFMA products are exact and the sums
are fp32 over K <= 16384 terms; each row sum is multiplied by its fp32 scale
once (2^-24 relative), silu in fp32, the intermediate carried as hi + lo
bf16. The output error stays below 1e-4 of max|ref| and the mean below 2e-5
of mean|ref|.
"""
import numpy as np
import pytest

import oracle
import routing_grouped_expert_amd as moe
import synth
from gpu_util import dev, host, note, sync, torch

pytestmark = pytest.mark.gpu


def pad_rows(perm, n):
    """permuted_rows as the library takes it: [T * k], the local entries
    first (positions past them are never read)."""
    out = np.full(n, -1, np.int32)
    out[:len(perm)] = perm
    return out


def layer_fp8(seed, T, H, I, E, k, first, L):
    x = synth.normal_bf16(seed, synth.X, (T, H), 1.0)
    w1q, w1s = synth.fp8_rows(seed, synth.W1, (L, 2 * I, H), 0.02, first_expert=first)
    w2q, w2s = synth.fp8_rows(seed, synth.W2, (L, H, I), 0.02, first_expert=first)
    ids = synth.topk_ids(seed, synth.IDS, T, E, k)
    return x, w1q, w1s, w2q, w2s, ids


def run_ffn_fp8(x, perm, offsets, k, w1q, w1s, w2q, w2s):
    t = torch()
    T, H = x.shape
    L = len(offsets) - 1
    out = t.full((T * k, H), float("nan"), dtype=t.float32, device="cuda:0")
    ws = moe.alloc_workspace(T, H, w2q.shape[2], 1 + L, k, L)
    pd = dev(pad_rows(perm, T * k))
    moe.grouped_ffn_fp8(dev(x), pd, dev(offsets), k, dev(w1q), dev(w1s), dev(w2q), dev(w2s), out,
                        ws)
    sync()
    return host(out)


def check_ffn_fp8(T, H, I, E, k, first, L, seed=1, ids=None):
    note(f"ffn fp8 T={T} H={H} I={I} E={E} k={k} share=({first},{L})")
    x, w1q, w1s, w2q, w2s, rnd = layer_fp8(seed, T, H, I, E, k, first, L)
    ids = rnd if ids is None else ids
    _, offsets, perm, _ = oracle.permute(ids, E, first, L)
    got = run_ffn_fp8(x, perm, offsets, k, w1q, w1s, w2q, w2s)
    n = offsets[-1]
    ref = oracle.grouped_ffn_fp8(x, perm, offsets, k, w1q, w1s, w2q, w2s)
    g = got[:n].astype(np.float64)
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    assert err.max() <= 1e-4 * np.abs(ref).max(), err.max() / np.abs(ref).max()
    assert err.mean() <= 2e-5 * np.abs(ref).mean(), err.mean() / np.abs(ref).mean()
    assert np.isnan(got[n:]).all()


# one to eight 16-token tiles, a second pass: the generic kernels for the
# first two (H below the K-split unit), the staged kernels for the others
@pytest.mark.parametrize("T,E,k", [(12, 4, 2), (30, 8, 2), (60, 6, 2), (300, 2, 1)])
def test_ffn_fp8_tiles(T, E, k):
    check_ffn_fp8(T, 256, 384, E, k, 0, E)


@pytest.mark.parametrize("H,I", [(200, 72), (130, 260)])
def test_ffn_fp8_checked_path_ragged(H, I):
    check_ffn_fp8(37, H, I, 5, 2, 0, 5)


@pytest.mark.parametrize("counts", [[1, 17, 33, 49, 65, 81, 97, 169],
                                    [1, 16, 17, 32, 33, 48, 49, 64, 63, 50, 31, 18, 15, 2, 40,
                                     33]])
def test_ffn_fp8_prefill_partial_passes(counts):
    """Staged passes holding every number of their 8 (or 4) token tiles."""
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    ids = np.random.default_rng(3).permutation(ids).reshape(-1, 1)
    check_ffn_fp8(len(ids), 512, 256, len(counts), 1, 0, len(counts), ids=ids)


def test_ffn_fp8_share_and_empty_experts():
    check_ffn_fp8(40, 128, 256, 16, 2, 3, 9)


# K-split kernels (H and I multiples of 1024, at most 16 mean-doubled entries
# per expert). On a 256-CU part (FP8 up kernel 512 blocks, down kernel 256):
# tiles dealt whole (24, 1024, 1024), stream-K with cut tiles for the up
# kernel (32, 4096, 1024), (16, 4096, 1024), (40, 2048, 1024) and the down
# kernel (16, 1024, 4096), one whole round then cut tiles in both (40, 4096,
# 2048).
@pytest.mark.parametrize("T,H,I,E,k", [(24, 1024, 1024, 8, 2), (32, 4096, 1024, 8, 2),
                                       (16, 4096, 1024, 4, 1), (16, 1024, 4096, 4, 1),
                                       (40, 2048, 1024, 20, 2), (40, 4096, 2048, 20, 2)])
def test_ffn_fp8_stream_k(T, H, I, E, k):
    check_ffn_fp8(T, H, I, E, k, 0, E)


def test_ffn_fp8_stream_k_share():
    check_ffn_fp8(12, 1024, 1024, 12, 2, 4, 5)


def test_ffn_fp8_decode_full_size_sampled():
    """The decode-shaped layer at full size (T32 H4096 I14336 E8 top-2) on
    FP8 weights, in the launch configuration bench.py times: every output row
    of four sampled entries against the oracle's single-entry FFN."""
    from synth import configs
    d = configs.layer_inputs(configs.WORKLOADS["decode"])
    T, H, I, E, k = d["T"], d["H"], d["I"], d["E"], d["k"]
    note(f"ffn fp8 decode full size T={T} H={H} I={I} E={E} k={k}")
    w1q, w1s, w2q, w2s = configs.fp8_weights(d)
    ids = synth.topk_ids(d["seed"], synth.IDS, T, E, k)
    _, offsets, perm, _ = oracle.permute(ids, E, 0, E)
    got = run_ffn_fp8(d["x"], perm, offsets, k, w1q, w1s, w2q, w2s)
    n = int(offsets[-1])
    assert np.isnan(got[n:]).all()
    for p in (0, n // 3, (2 * n) // 3, n - 1):
        e = int(np.searchsorted(offsets, p, side="right") - 1)
        ref = oracle.expert_row_fp8(d["x"][perm[p] // k], w1q[e], w1s[e], w2q[e], w2s[e])
        err = np.abs(got[p].astype(np.float64) - ref)
        assert err.max() <= 1e-4 * np.abs(ref).max(), (p, err.max() / np.abs(ref).max())


# Staged (prefill) kernels on FP8 codes: 4 token tiles per pass (128, 512,
# 512, 16, 4), 8 tiles dealt in whole rounds (4096 tokens, 512 experts), a
# whole round then cut tiles (3200 tokens, 300 experts), skewed experts with
# several passes, a share with empty experts.
def test_ffn_fp8_prefill_four_tiles():
    check_ffn_fp8(128, 512, 512, 16, 4, 0, 16)


def test_ffn_fp8_prefill_whole_rounds():
    check_ffn_fp8(4096, 512, 256, 512, 8, 0, 512)


def test_ffn_fp8_prefill_rounds_then_cuts():
    check_ffn_fp8(3200, 512, 256, 300, 8, 0, 300)


def test_ffn_fp8_prefill_skewed():
    T, E, k = 300, 6, 2
    ids = np.stack([np.full(T, 2, np.int32), (3 + np.arange(T, dtype=np.int32) % 3)], 1)
    check_ffn_fp8(T, 512, 256, E, k, 0, E, ids=ids)


def test_ffn_fp8_prefill_share():
    check_ffn_fp8(384, 512, 256, 20, 4, 5, 6)


def test_ffn_fp8_share0_full_size_sampled():
    """The share-0 prefill shape at full size (T4096 H7168 I2048, experts 0..76
    of 384, top-8) on FP8 codes, in the staged kernels bench.py times: every
    output row of five sampled entries against the oracle's single-entry FFN."""
    T, H, I, E, k, first, L = 4096, 7168, 2048, 384, 8, 0, 77
    note(f"ffn fp8 share-0 full size T={T} H={H} I={I} E={E} k={k} share=({first},{L})")
    x, w1q, w1s, w2q, w2s, ids = layer_fp8(7, T, H, I, E, k, first, L)
    _, offsets, perm, _ = oracle.permute(ids, E, first, L)
    got = run_ffn_fp8(x, perm, offsets, k, w1q, w1s, w2q, w2s)
    n = int(offsets[-1])
    assert np.isnan(got[n:]).all()
    for p in (0, n // 4, n // 2, (3 * n) // 4, n - 1):
        e = int(np.searchsorted(offsets, p, side="right") - 1)
        ref = oracle.expert_row_fp8(x[perm[p] // k], w1q[e], w1s[e], w2q[e], w2s[e])
        err = np.abs(got[p].astype(np.float64) - ref)
        assert err.max() <= 1e-4 * np.abs(ref).max(), (p, err.max() / np.abs(ref).max())
