"""The seeded input generator: determinism, distributions, bf16 rounding."""
import numpy as np

import synth
from synth import configs


def test_deterministic_and_split_invariant():
    a = synth.normal_bf16(42, synth.W1, (3, 50, 70), 0.02)
    b = synth.normal_bf16(42, synth.W1, (3, 50, 70), 0.02)
    assert np.array_equal(a, b)
    # expert 2 alone equals block 2 of the stacked draw
    c = synth.normal_bf16(42, synth.W1, (1, 50, 70), 0.02, first_expert=2)
    assert np.array_equal(c[0], a[2])
    assert not np.array_equal(a[0], a[1])


def test_moments():
    x = synth.normal_f32(1, synth.X, (400000,), 1.0).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    w = synth.bf16_to_f32(synth.normal_bf16(1, synth.W2, (1, 400000), 0.02)).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.0005


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, -0.0], np.float32)
    b = synth.f32_to_bf16(f)
    back = synth.bf16_to_f32(b)
    assert list(back) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, -0.0]


def test_tie_levels():
    lg = configs.routing_logits(64, ties=True)
    lv = set(np.unique(lg).tolist())
    assert lv <= {(l - 3.5) * 0.5 for l in range(8)} and len(lv) >= 6


def test_topk_ids_distinct():
    ids = synth.topk_ids(3, synth.IDS, 500, 40, 8)
    assert ids.min() >= 0 and ids.max() < 40
    assert all(len(set(r)) == 8 for r in ids.tolist())


def test_workload_share_matches_full_layer():
    full = configs.layer_inputs(configs.WORKLOADS["tiny"], first=0, L=8)
    part = configs.layer_inputs(configs.WORKLOADS["tiny"], first=3, L=2)
    assert np.array_equal(full["w1"][3:5], part["w1"]) and np.array_equal(full["w2"][3:5], part["w2"])


def test_fp8_rows_nearest_code_and_scale():
    """The FP8 weight generator: scale = max|w| / 448 per row, and every code
    is the nearest E4M3 value to w / scale (ties to the even code), checked by
    brute force over all codes against torch's float8_e4m3fn decoding."""
    import torch
    R, C = 6, 200
    q, s = synth.fp8_rows(21, synth.W2, (2, R, C), 0.02, first_expert=3)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    finite = ~np.isnan(vals)
    codes = np.arange(256)[finite]
    for e in range(2):
        w = synth.normal_f32(21, synth.W2, (R * C,), 0.02, expert=3 + e).reshape(R, C)
        for r in range(R):
            amax = np.float32(np.abs(w[r]).max())
            assert s[e, r] == np.float32(amax / np.float32(448.0))
            y = (w[r] / s[e, r]).astype(np.float64)
            for c in range(C):
                d = np.abs(vals[finite] - y[c])
                best = codes[d == d.min()]
                if len(best) > 1:  # a tie: the even code (equal magnitudes share parity)
                    best = best[best % 2 == 0]
                    best = best[np.sign(vals[best]) == np.sign(y[c])] if y[c] != 0 else best
                assert q[e, r, c] in best, (e, r, c, y[c], q[e, r, c], best)
            assert np.abs(vals[q[e, r]]).max() == 448.0
