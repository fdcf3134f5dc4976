"""moe_forward against the oracle: routing bit-exact, the bf16 output within
max|err| <= 2e-2 max|ref| and mean|err| <= 2e-3 mean|ref| of the fp64 oracle
on the same bf16 inputs. Reduced sizes compare every output; the full
workload sizes compare all routing and a sample of token outputs, in the
launch configuration the benchmark times."""
import numpy as np
import pytest

import oracle
import routing_grouped_expert_amd as moe
from gpu_util import assert_layer_ok, bf16_to_f64, dev, empty, host, note, sync, torch
from synth import configs

pytestmark = pytest.mark.gpu
W_TOL = 4e-6


def gpu_forward(d):
    t = torch()
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    first, L = d["first"], d["L"]
    y = empty((T, H), t.int16)
    logits = empty((T, E), t.float32)
    ids = empty((T, k), t.int32)
    w = empty((T, k), t.float32)
    ws = moe.alloc_workspace(T, H, I, E, k, L)
    moe.forward(dev(d["x"]), dev(d["wg"]), None if d["bias"] is None else dev(d["bias"]),
                dev(d["w1"]), dev(d["w2"]), k, first, L, y, ws, logits, ids, w)
    sync()
    return host(y, np.uint16), host(logits), host(ids), host(w)


def check_forward(d, sample=None, what=""):
    note(f"forward {what} T={d['T']} H={d['H']} I={d['I']} E={d['E']} k={d['k']} "
         f"share=({d['first']},{d['L']})")
    y, lg, ids, w = gpu_forward(d)
    rlg, rids, rw, ry = oracle.forward(d["x"], d["wg"], d["w1"], d["w2"], d["k"], d["first"],
                                       d["L"], d["bias"], sample)
    ulp = np.spacing(np.abs(rlg))
    assert (np.abs(lg.astype(np.float64) - rlg) <= ulp).all()
    assert np.array_equal(ids, rids), f"{what}: routing differs for tokens {np.unique(np.argwhere(ids != rids)[:, 0])[:8]}"
    assert np.abs(w - rw).max() <= W_TOL
    ys = y if sample is None else y[sample]
    return assert_layer_ok(ys, ry, what)


def test_forward_tiny():
    check_forward(configs.layer_inputs(configs.WORKLOADS["tiny"]), what="tiny")


@pytest.mark.parametrize("name,T,H,I", [("decode", 32, 512, 1024), ("fine", 128, 512, 256),
                                        ("share0", 256, 512, 256)])
def test_forward_reduced(name, T, H, I):
    check_forward(configs.layer_inputs(configs.WORKLOADS[name], T=T, H=H, I=I), what=name)


# The dense grouped-FFN kernels through the whole layer, every output
# compared: the decode shape with 2048 tokens (512 entries per expert: two
# passes of 256 each), and share 0 of the share-0 workload with 8192 tokens
# (~170 local entries per local expert, chosen on the device from the counts).
@pytest.mark.parametrize("name,T,H,I", [("decode", 2048, 512, 256), ("share0", 8192, 256, 128)])
def test_forward_dense_complete(name, T, H, I):
    check_forward(configs.layer_inputs(configs.WORKLOADS[name], T=T, H=H, I=I), what=f"{name} dense")


def test_forward_odd_shapes():
    cfg = dict(configs.WORKLOADS["fine"], E=13, k=3, first=2, L=7)
    check_forward(configs.layer_inputs(cfg, T=45, H=200, I=72), what="odd shapes")


@pytest.mark.parametrize("T,E,k,first,L", [(1, 8, 2, 0, 8), (33, 64, 1, 5, 50),
                                            (17, 100, 4, 30, 20), (64, 200, 8, 0, 16),
                                            (40, 384, 8, 300, 12), (64, 1000, 8, 990, 10)])
def test_forward_small_batches(T, E, k, first, L):
    """Up to 64 tokens with H, I multiples of the persistent FFN kernels'
    tiles: every values-per-lane routing tier, K-split and token-staged FFN
    passes, shares that start inside the expert range."""
    cfg = dict(configs.WORKLOADS["fine"], E=E, k=k, first=first, L=L)
    check_forward(configs.layer_inputs(cfg, T=T, H=512, I=1024), what="small batch")


def test_forward_shares_sum_to_whole_layer():
    """Weights are renormalised before the share mask, so the shares' outputs
    add up to the whole layer (up to one bf16 rounding per share)."""
    cfg = dict(configs.WORKLOADS["share0"], E=20, S=5)
    full = configs.layer_inputs(cfg, T=64, H=256, I=128, first=0, L=20)
    y_full = bf16_to_f64(gpu_forward(full)[0])
    acc = np.zeros_like(y_full)
    for s in range(5):
        f, c = moe.partition(20, 5, s)
        d = configs.layer_inputs(cfg, T=64, H=256, I=128, first=f, L=c)
        acc += bf16_to_f64(gpu_forward(d)[0])
    err = np.abs(acc - y_full)
    assert err.max() <= 6 * 2 ** -8 * np.abs(y_full).max()
    assert err.mean() <= 2e-3 * np.abs(y_full).mean() * 3


@pytest.mark.parametrize("name,n_sample", [("decode", 32), ("fine", 128), ("share0", 256)])
def test_forward_full_size_sampled(name, n_sample):
    """The full workload in the launch configuration bench.py times: every
    token's routing, and the outputs of n_sample tokens spread over the batch
    (every token at decode size)."""
    cfg = configs.WORKLOADS[name]
    assert moe.partition(cfg["E"], cfg["S"], cfg["s"]) == (cfg["first"], cfg["L"])
    d = configs.layer_inputs(cfg)
    T = d["T"]
    sample = np.unique(np.concatenate([np.linspace(0, T - 1, n_sample).astype(np.int32),
                                       np.array([1, T - 2], np.int32)]))
    check_forward(d, sample=sample, what=name + " full size")


def test_forward_mfma_probe_sampled():
    """The MFMA-bound probe bench.py times: the share-0 expert weights with
    T = 32768 tokens (~683 entries per local expert). The GPU runs the whole
    batch; a token's logits, routing and output depend on that token alone, so
    256 sampled tokens are checked against the oracle run on those tokens."""
    cfg = configs.WORKLOADS["share0"]
    T = 32768
    d = configs.layer_inputs(cfg, T=T)
    note(f"forward mfma probe T={T} H={d['H']} I={d['I']} E={d['E']} k={d['k']} "
         f"share=({d['first']},{d['L']})")
    y, lg, ids, w = gpu_forward(d)
    sample = np.linspace(0, T - 1, 256).astype(np.int32)
    rlg, rids, rw, ry = oracle.forward(d["x"][sample], d["wg"], d["w1"], d["w2"], d["k"],
                                       d["first"], d["L"], d["bias"])
    assert (np.abs(lg[sample].astype(np.float64) - rlg) <= np.spacing(np.abs(rlg))).all()
    assert np.array_equal(ids[sample], rids)
    assert np.abs(w[sample] - rw).max() <= W_TOL
    assert_layer_ok(y[sample], ry, "mfma probe")


def structured_inputs(kind, T=256, H=512, I=256, E=16, k=4, seed=41):
    """Inputs whose routing is fixed by construction. shared: every token
    picks experts 0..k-1 (a router bias of 10 - e on them over tiny logits);
    disjoint: token t picks experts (t k + j) mod E, by a one-hot column per
    token in the last T columns of x and W_g rows that read it."""
    import synth
    cfg = dict(configs.WORKLOADS["share0"], E=E, k=k, first=0, L=E, S=1, s=0, bias=False)
    d = configs.layer_inputs(cfg, T=T, H=H, I=I, seed=seed)
    if kind == "shared":
        d["wg"] = (d["wg"] * 1e-3).astype(np.float32)
        b = np.zeros(E, np.float32)
        b[:k] = 10.0 - np.arange(k, dtype=np.float32)
        d["bias"] = b
    else:
        assert H > T
        x = d["x"].copy()
        x[:, H - T:] = 0
        x[np.arange(T), H - T + np.arange(T)] = synth.f32_to_bf16(np.array([8.0], np.float32))[0]
        wg = np.zeros((E, H), np.float32)
        for t in range(T):
            for j in range(k):
                wg[(t * k + j) % E, H - T + t] = 1.0 - 0.125 * j  # slot order j
        d["x"], d["wg"] = x, wg
    return d


@pytest.mark.parametrize("kind", ["shared", "disjoint"])
def test_forward_structured_routing(kind):
    """The two routing regimes the pages measure: all tokens on the same
    experts (4 experts of 256 entries: two staged passes each), and tokens
    spread evenly over all experts."""
    d = structured_inputs(kind)
    T, k, E = d["T"], d["k"], d["E"]
    want = (np.tile(np.arange(k), (T, 1)) if kind == "shared"
            else (np.arange(T)[:, None] * k + np.arange(k)[None, :]) % E)
    check_forward(d, what=kind + " routing")
    _, _, gids, _ = gpu_forward(d)
    assert np.array_equal(gids, want.astype(np.int32))
