"""moe_router_logits against the oracle.

Both sides sum the exact bf16 x fp32 products in fp64 and round once to fp32,
so they agree unless the exact value lies within ~1e-14 relative of an fp32
rounding midpoint: every logit is within one fp32 ulp and (all but a
vanishing fraction) bit-identical. On inputs whose sums are exact in fp64 the
results are identical.
"""
import numpy as np
import pytest

import oracle
import routing_grouped_expert_amd as moe
import synth
from gpu_util import dev, empty, host, note, sync, torch
from synth import configs

pytestmark = pytest.mark.gpu


def gpu_logits(x, wg, bias):
    t = torch()
    T, H = x.shape
    E = wg.shape[0]
    lg = empty((T, E), t.float32)
    ws = moe.alloc_workspace(T, H, 128, E, 1, 1)
    moe.router_logits(dev(x), dev(wg), None if bias is None else dev(bias), lg, ws)
    sync()
    return host(lg)


def check(x, wg, bias, what):
    note(f"router {what} T={x.shape[0]} H={x.shape[1]} E={wg.shape[0]}")
    got = gpu_logits(x, wg, bias)
    ref = oracle.router_logits(x, wg, bias)
    ulp = np.spacing(np.abs(ref))
    assert (np.abs(got.astype(np.float64) - ref) <= ulp).all(), what
    assert (got != ref).mean() <= 1e-5, f"{what}: {(got != ref).sum()} logits differ"


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("fine", 64),
                                    ("share0", 96)])
def test_router_workloads(name, T):
    cfg = configs.WORKLOADS[name]
    d = configs.layer_inputs(cfg, T=T, I=128, first=0, L=1)
    check(d["x"], d["wg"], d["bias"], name)


def test_router_ragged():
    x = synth.normal_bf16(5, 90, (67, 131), 1.0)
    wg = synth.normal_f32(5, 91, (65, 131), 0.1)
    b = synth.normal_f32(5, 92, (65,), 1.0)
    check(x, wg, b, "ragged")


def test_router_exact_sums():
    rng = np.random.default_rng(3)
    T, H, E = 70, 200, 66
    xv = rng.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 3.0], size=(T, H))
    m = rng.integers(-(1 << 22) + 1, 1 << 22, size=(E, H))
    wg = (m / float(1 << 20)).astype(np.float32)
    x = synth.f32_to_bf16(xv.astype(np.float32))
    assert np.array_equal(gpu_logits(x, wg, None), oracle.router_logits(x, wg, None))


@pytest.mark.parametrize("T,H,E", [(5, 130, 13), (40, 256, 21), (64, 7168, 384), (1, 4, 1)])
def test_router_few_tokens(T, H, E):
    """The few-token kernel (T <= 64): vector and element-wise loads, E not a
    multiple of its 8-expert groups."""
    x = synth.normal_bf16(6, 93, (T, H), 1.0)
    wg = synth.normal_f32(6, 94, (E, H), 0.1)
    b = synth.normal_f32(6, 95, (E,), 1.0)
    check(x, wg, b, "few tokens")
    check(x, wg, None, "few tokens, no bias")


@pytest.mark.parametrize("T,H,E", [(300, 1024, 100), (65, 7168, 256), (129, 200, 64)])
def test_router_many_tokens(T, H, E):
    """The fp64 MFMA kernel (T > 64): split K slices, partial tiles in T and E."""
    x = synth.normal_bf16(8, 96, (T, H), 1.0)
    wg = synth.normal_f32(8, 97, (E, H), 0.1)
    b = synth.normal_f32(8, 98, (E,), 1.0)
    check(x, wg, b, "many tokens")
