"""moe_forward_no_alloc (the layer on the library's own device scratch)
against moe_forward with a caller workspace: the same kernels on the same
inputs, so every output is bit-identical. Two calls in a row, the second with
fewer tokens, so the second call runs on scratch left by the first."""
import numpy as np
import pytest

import routing_grouped_expert_amd as moe
from gpu_util import dev, empty, host, note, sync, torch
from synth import configs

pytestmark = pytest.mark.gpu


def run(d, no_alloc):
    t = torch()
    T, H, I, E, k, first, L = (d[n] for n in ("T", "H", "I", "E", "k", "first", "L"))
    y = empty((T, H), t.int16)
    lg = empty((T, E), t.float32)
    ids = empty((T, k), t.int32)
    w = empty((T, k), t.float32)
    args = (dev(d["x"]), dev(d["wg"]), None if d["bias"] is None else dev(d["bias"]),
            dev(d["w1"]), dev(d["w2"]), k, first, L, y)
    if no_alloc:
        moe.forward_no_alloc(*args, lg, ids, w)
    else:
        moe.forward(*args, moe.alloc_workspace(T, H, I, E, k, L), lg, ids, w)
    sync()
    return [host(a) for a in (y, lg, ids, w)]


# FFN paths: K-split (decode, fine), element-wise (share0, I not a multiple
# of the K-split unit).
@pytest.mark.parametrize("name,T1,T2,H,I", [("decode", 32, 7, 1024, 2048),
                                             ("fine", 96, 33, 512, 1024),
                                             ("share0", 64, 16, 512, 256)])
def test_no_alloc_matches_forward_twice(name, T1, T2, H, I):
    for T in (T1, T2):
        d = configs.layer_inputs(configs.WORKLOADS[name], T=T, H=H, I=I, seed=77 + T)
        note(f"forward_no_alloc {name} T={T} H={H} I={I}")
        assert moe.workspace_size(T, H, I, d["E"], d["k"], d["L"]) <= moe.NO_ALLOC_SCRATCH_BYTES
        a = run(d, True)
        b = run(d, False)
        for u, v in zip(a, b):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_no_alloc_full_decode_layer():
    """The decode-shaped layer at full size (T32 H4096 I14336 E8 top-2) fits
    the scratch and matches moe_forward bit for bit."""
    d = configs.layer_inputs(configs.WORKLOADS["decode"])
    note("forward_no_alloc decode full size")
    a = run(d, True)
    b = run(d, False)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_no_alloc_rejects_sizes_beyond_scratch():
    """A prefill-sized layer needs more workspace than the scratch holds: the
    call fails with MOE_ERROR_WORKSPACE before launching anything."""
    t = torch()
    T, H, I, E, k = 512, 7168, 2048, 256, 8
    assert moe.workspace_size(T, H, I, E, k, E) > moe.NO_ALLOC_SCRATCH_BYTES
    x = empty((T, H), t.int16)
    wg = empty((E, H), t.float32)
    w1 = empty((1, 2 * I, H), t.int16)
    w2 = empty((1, H, I), t.int16)
    y = t.full((T, H), 7, dtype=t.int16, device="cuda:0")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_no_alloc(x, wg, None, w1, w2, k, 0, 1, y)
    assert ei.value.status == 3
    sync()
    assert (y == 7).all()
