"""The five MoE workloads and how their synthetic inputs are drawn.

Each workload fixes the layer shape, the top-k, the expert share and the
value distributions; ``layer_inputs`` draws the tensors from the seeded
streams in ``synth``. Only the local experts' weights are drawn, each from
its own stream, so share 0 of a split layer holds exactly the same weight
bytes as experts 0..L-1 of the whole layer.
"""
import numpy as np

from . import BIAS, LOGITS, W1, W2, WG, X, fp8_rows, normal_bf16, normal_f32, tie_levels_f32

# name -> shape. S/s: number of shares and the share this GPU runs; first/L: the
# share's expert range as the workload states it (the partition rule itself is
# part of the method and lives in the oracle and the library, not here).
WORKLOADS = {
    # Tiny layer: T16 H128 I256 E8 top-2.
    "tiny": dict(T=16, H=128, I=256, E=8, k=2, S=1, s=0, first=0, L=8, bias=False, seed=1000),
    # Decode-shaped, weight-bandwidth bound: T32 H4096 I14336 E8 top-2.
    "decode": dict(T=32, H=4096, I=14336, E=8, k=2, S=1, s=0, first=0, L=8, bias=False,
                   seed=1001),
    # Fine-grained experts with a per-expert router bias: T512 H7168 I2048 E256 top-8.
    "fine": dict(T=512, H=7168, I=2048, E=256, k=8, S=1, s=0, first=0, L=256, bias=True,
                 seed=1002),
    # Share 0 of 384 experts split over 5 shares (77/77/77/77/76), prefill shape:
    # T4096 H7168 I2048 top-8; this share holds experts 0..76.
    "share0": dict(T=4096, H=7168, I=2048, E=384, k=8, S=5, s=0, first=0, L=77, bias=False,
                   seed=1004),
}

# Routing-only stress: fp32 logits [T, 1024] ~ N(0,1), top-8, T in {1, 64, 4096},
# plus a tie-heavy variant quantised to eight levels.
ROUTING = dict(E=1024, k=8, T=(1, 64, 4096), seed=1003)

SIGMA_X, SIGMA_WG, SIGMA_W, SIGMA_BIAS, SIGMA_LOGITS = 1.0, 0.1, 0.02, 1.0, 1.0


def layer_inputs(cfg, T=None, H=None, I=None, seed=None, first=None, L=None, weights=True):
    """Draw x, W_g, bias, W1, W2 for a workload, optionally at reduced sizes.

    Returns a dict of numpy arrays: x [T,H] bf16 bits, wg [E,H] fp32,
    bias [E] fp32 or None, w1 [L,2I,H] bf16 bits (rows [0,I) gate, [I,2I) up),
    w2 [L,H,I] bf16 bits, plus the scalar shape fields. weights=False leaves
    w1 and w2 out (None): x, W_g and the bias do not depend on them, so a
    larger token batch can reuse expert weights drawn earlier.
    """
    c = dict(cfg)
    if T is not None:
        c["T"] = T
    if H is not None:
        c["H"] = H
    if I is not None:
        c["I"] = I
    if seed is not None:
        c["seed"] = seed
    if first is not None:
        c["first"], c["L"] = first, L
    T, H, I, E, k, sd = c["T"], c["H"], c["I"], c["E"], c["k"], c["seed"]
    first, L = c["first"], c["L"]
    out = dict(c)
    out["x"] = normal_bf16(sd, X, (T, H), SIGMA_X)
    out["wg"] = normal_f32(sd, WG, (E, H), SIGMA_WG)
    out["bias"] = normal_f32(sd, BIAS, (E,), SIGMA_BIAS) if c.get("bias") else None
    out["w1"] = normal_bf16(sd, W1, (L, 2 * I, H), SIGMA_W, first_expert=first) if weights else None
    out["w2"] = normal_bf16(sd, W2, (L, H, I), SIGMA_W, first_expert=first) if weights else None
    return out


def fp8_weights(d):
    """FP8 E4M3 expert weights with per-row scales for the layer drawn by
    layer_inputs (the same normals its bf16 W1 / W2 round): returns
    (w1q [L,2I,H] uint8, w1s [L,2I] fp32, w2q [L,H,I] uint8, w2s [L,H] fp32)."""
    sd, H, I, first, L = d["seed"], d["H"], d["I"], d["first"], d["L"]
    w1q, w1s = fp8_rows(sd, W1, (L, 2 * I, H), SIGMA_W, first_expert=first)
    w2q, w2s = fp8_rows(sd, W2, (L, H, I), SIGMA_W, first_expert=first)
    return w1q, w1s, w2q, w2s


def routing_logits(T, E=ROUTING["E"], seed=ROUTING["seed"], ties=False):
    if ties:
        return tie_levels_f32(seed, LOGITS + 100, (T, E))
    return normal_f32(seed, LOGITS, (T, E), SIGMA_LOGITS)


def algorithmic_bytes(cfg, counts=None):
    """Bytes the layer must move: touched experts' W1 and W2, W_g, bias, x, y
    and the routing outputs. counts: per-local-expert entry counts (None =
    every local expert touched)."""
    T, H, I, E, k, L = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["L"]
    touched = L if counts is None else int(np.count_nonzero(np.asarray(counts)))
    w = touched * (3 * I * H) * 2
    return w + E * H * 4 + (E * 4 if cfg.get("bias") else 0) + T * H * 2 * 2 + T * k * 8
