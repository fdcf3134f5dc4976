"""moe_forward_fp8 against the oracle: the layer with FP8 E4M3 expert weights
(one fp32 scale per row). Routing is bit-exact, as for moe_forward; the bf16
output is held to the layer bound (max|err| <= 2e-2 max|ref|, mean|err| <=
2e-3 mean|ref|) against the oracle's FP8 FFN and combine in fp64. Reduced
sizes compare every output. The full decode size compares all routing and a
sample of tokens, each recomputed row by row."""
import numpy as np
import pytest

import oracle
import routing_grouped_expert_amd as moe
from gpu_util import assert_layer_ok, dev, empty, host, note, sync, torch
from synth import configs

pytestmark = pytest.mark.gpu
W_TOL = 4e-6


def gpu_forward_fp8(d, q):
    t = torch()
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    y = empty((T, H), t.int16)
    logits = empty((T, E), t.float32)
    ids = empty((T, k), t.int32)
    w = empty((T, k), t.float32)
    ws = moe.alloc_workspace(T, H, I, E, k, d["L"])
    w1q, w1s, w2q, w2s = (dev(a) for a in q)
    moe.forward_fp8(dev(d["x"]), dev(d["wg"]), None if d["bias"] is None else dev(d["bias"]),
                    w1q, w1s, w2q, w2s, k, d["first"], d["L"], y, ws, logits, ids, w)
    sync()
    return host(y, np.uint16), host(logits), host(ids), host(w)


def oracle_forward_fp8(d, q, sample=None):
    """Router, routing and permutation of the oracle, then its FP8 expert FFN
    and combine: every token when sample is None, else the sampled tokens,
    each selection's expert row recomputed on its own."""
    w1q, w1s, w2q, w2s = q
    x, k, first, L = d["x"], d["k"], d["first"], d["L"]
    lg = oracle.router_logits(x, d["wg"], d["bias"])
    ids, w = oracle.route(lg, k)
    T, H = x.shape
    if sample is None:
        _, offsets, perm, e2p = oracle.permute(ids, d["E"], first, L)
        eo = oracle.grouped_ffn_fp8(x, perm, offsets, k, w1q, w1s, w2q, w2s)
        full = np.zeros((max(T * k, 1), H), np.float64)
        full[: len(eo)] = eo
        return lg, ids, w, oracle.combine(full, e2p, w, T, k, H)
    y = np.zeros((len(sample), H), np.float64)
    for i, tok in enumerate(sample):
        for j in range(k):
            e = ids[tok, j] - first
            if 0 <= e < L:
                y[i] += w[tok, j] * oracle.expert_row_fp8(x[tok], w1q[e], w1s[e], w2q[e], w2s[e])
    return lg, ids, w, y


def check_forward_fp8(d, sample=None, what=""):
    note(f"forward fp8 {what} T={d['T']} H={d['H']} I={d['I']} E={d['E']} k={d['k']} "
         f"share=({d['first']},{d['L']})")
    q = configs.fp8_weights(d)
    y, lg, ids, w = gpu_forward_fp8(d, q)
    rlg, rids, rw, ry = oracle_forward_fp8(d, q, sample)
    assert (np.abs(lg.astype(np.float64) - rlg) <= np.spacing(np.abs(rlg))).all()
    assert np.array_equal(ids, rids), what
    assert np.abs(w - rw).max() <= W_TOL
    return assert_layer_ok(y if sample is None else y[sample], ry, what)


def test_forward_fp8_tiny():
    check_forward_fp8(configs.layer_inputs(configs.WORKLOADS["tiny"]), what="tiny")


# decode-shaped (K-split kernels), fine-grained and share-0 shaped (staged
# kernels at 4 and 8 token tiles), ragged shapes (the generic kernels)
@pytest.mark.parametrize("name,T,H,I", [("decode", 32, 1024, 2048), ("fine", 128, 512, 256),
                                        ("share0", 256, 512, 256), ("share0", 512, 512, 512)])
def test_forward_fp8_reduced(name, T, H, I):
    check_forward_fp8(configs.layer_inputs(configs.WORKLOADS[name], T=T, H=H, I=I), what=name)


def test_forward_fp8_odd_shapes():
    cfg = dict(configs.WORKLOADS["fine"], E=13, k=3, first=2, L=7)
    check_forward_fp8(configs.layer_inputs(cfg, T=45, H=200, I=72), what="odd shapes")


def test_forward_fp8_empty_share():
    """A share that no token selects: routing as the oracle's, output zero."""
    cfg = dict(configs.WORKLOADS["fine"], E=64, k=1, first=60, L=4)
    d = configs.layer_inputs(cfg, T=3, H=256, I=128)
    q = configs.fp8_weights(d)
    y, _, ids, _ = gpu_forward_fp8(d, q)
    rids, _ = oracle.route(oracle.router_logits(d["x"], d["wg"], d["bias"]), 1)
    assert np.array_equal(ids, rids) and (rids < 60).all()
    assert (y == 0).all()


def test_forward_fp8_decode_full_size_sampled():
    cfg = configs.WORKLOADS["decode"]
    d = configs.layer_inputs(cfg)
    T = d["T"]
    sample = np.unique(np.array([0, 1, T // 3, T // 2, T - 2, T - 1], np.int32))
    check_forward_fp8(d, sample=sample, what="decode full size")
