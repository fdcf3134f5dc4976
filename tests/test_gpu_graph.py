"""The layer captured in a HIP graph (torch.cuda.graph over the library's
calls on the capture stream) and replayed: every replay must give outputs
bit-identical to the eager call. Between replays the program runs eager work
of its own (it refills the outputs and the workspace with garbage, since the
workspace needs no initialisation) and synchronises, so a replay cannot lean
on state a previous one left. The library records no memset nodes: every
counter it clears is cleared by one of its kernels."""
import numpy as np
import pytest

import routing_grouped_expert_amd as moe
from gpu_util import dev, empty, host, note, sync, torch
from synth import configs

pytestmark = pytest.mark.gpu
REPLAYS = 3


def outputs(d):
    t = torch()
    T, H, E, k = d["T"], d["H"], d["E"], d["k"]
    return [empty((T, H), t.int16), empty((T, E), t.float32), empty((T, k), t.int32),
            empty((T, k), t.float32)]


def check_replays(call, outs, ws, what):
    """Eager call, then a captured one replayed REPLAYS times; the outputs of
    every replay against the eager outputs, byte for byte."""
    t = torch()
    note(f"graph {what}: eager call")
    call()
    sync()
    ref = [host(o).copy() for o in outs]
    note(f"graph {what}: capture")
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        call()
    sync()
    for rep in range(REPLAYS):
        for o in outs:
            o.view(t.uint8).fill_(0xA5 + rep)
        if ws is not None:
            ws.fill_(0x5A + rep)
        sync()
        note(f"graph {what}: replay {rep}")
        g.replay()
        sync()
        for name, o, r in zip(("y", "logits", "ids", "weights"), outs, ref):
            got = host(o)
            assert np.array_equal(got.view(np.uint8), r.view(np.uint8)), \
                f"{what}: replay {rep}: {name} differs from the eager call"
    del g


# FFN paths: K-split (decode), token-staged with 4 and 8 tiles (fine,
# share 0), the dense kernels chosen on the device (decode with 2048 tokens).
@pytest.mark.parametrize("name,T,H,I", [("decode", 32, 1024, 2048), ("fine", 512, 512, 256),
                                        ("share0", 1024, 512, 256), ("decode", 2048, 512, 256)])
def test_forward_graph_replays(name, T, H, I):
    d = configs.layer_inputs(configs.WORKLOADS[name], T=T, H=H, I=I)
    outs = outputs(d)
    ws = moe.alloc_workspace(T, H, I, d["E"], d["k"], d["L"])
    x, wg, w1, w2 = dev(d["x"]), dev(d["wg"]), dev(d["w1"]), dev(d["w2"])
    bias = None if d["bias"] is None else dev(d["bias"])

    def call():
        moe.forward(x, wg, bias, w1, w2, d["k"], d["first"], d["L"], outs[0], ws, *outs[1:])

    check_replays(call, outs, ws, f"forward {name} T={T} H={H} I={I}")


@pytest.mark.parametrize("name,T,H,I", [("decode", 32, 1024, 2048), ("fine", 512, 512, 256)])
def test_forward_fp8_graph_replays(name, T, H, I):
    d = configs.layer_inputs(configs.WORKLOADS[name], T=T, H=H, I=I)
    q = [dev(a) for a in configs.fp8_weights(d)]
    outs = outputs(d)
    ws = moe.alloc_workspace(T, H, I, d["E"], d["k"], d["L"])
    x, wg = dev(d["x"]), dev(d["wg"])
    bias = None if d["bias"] is None else dev(d["bias"])

    def call():
        moe.forward_fp8(x, wg, bias, *q, d["k"], d["first"], d["L"], outs[0], ws, *outs[1:])

    check_replays(call, outs, ws, f"forward_fp8 {name} T={T} H={H} I={I}")


def test_forward_no_alloc_graph_replays():
    """The allocation-free entry point under capture (its scratch is the
    library's own device array; the graph holds its address)."""
    d = configs.layer_inputs(configs.WORKLOADS["decode"], T=32, H=1024, I=2048)
    assert moe.workspace_size(32, 1024, 2048, d["E"], d["k"], d["L"]) <= moe.NO_ALLOC_SCRATCH_BYTES
    outs = outputs(d)
    x, wg, w1, w2 = dev(d["x"]), dev(d["wg"]), dev(d["w1"]), dev(d["w2"])

    def call():
        moe.forward_no_alloc(x, wg, None, w1, w2, d["k"], d["first"], d["L"], outs[0], *outs[1:])

    check_replays(call, outs, None, "forward_no_alloc decode T=32 H=1024 I=2048")
