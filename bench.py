#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

A step is one pass of the whole layer -- router logits, routing, histogram /
scan / permutation, grouped expert FFN, combine -- over one batch of the
decode-shaped workload (T=32 tokens, H=4096, I=14336, 8 experts, top-2,
bf16 weights). The step issues the five library calls in the order
moe_forward issues them, so that HIP events can bracket the grouped-FFN call
(the kernels that stream the expert weights) on the stream the library
launches on; moe_forward itself is timed over the same number of steps as a
check. Inputs are synthetic (seeded), resident in HBM before timing starts.

Prints one JSON line: tokens/s of the whole step, the grouped-FFN roofline
(algorithmic bytes / measured duration against 8 TB/s, and against the read
rate a plain streaming probe reaches on the same part), the oracle timed on
the host cores as a CPU baseline, and routing microseconds at 1024 experts.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_decode_pmc_traffic.md")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "fine", "share0"])
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-routing", action="store_true", help="skip the routing-only timings")
    ap.add_argument("--weights", default="bf16", choices=["bf16", "fp8"],
                    help="expert weight format: bf16 (the headline), or FP8 E4M3 codes with "
                         "per-row fp32 scales (moe_grouped_ffn_fp8; x stays bf16)")
    ap.add_argument("--routing-sweep", action="store_true",
                    help="instead of the layer step: route + permute microseconds over "
                         "T in {1, 64, 4096} x E in {8 .. 4096}, k = 8 (k = E below 8), warm and "
                         "with the caches flushed before each call; one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one elementwise kernel that reads 256 MiB and writes 256 MiB "
                         "(calibrates the HBM byte counters)")
    return ap.parse_args()


def ffn_source_digest():
    """Digest of the grouped-FFN code (ffn.hip, ffn_sk.hip, device.h) with
    line comments, trailing blanks and empty lines removed, so that editing a
    comment does not retire the committed counter summary."""
    h = hashlib.sha256()
    for name in ("ffn.hip", "ffn_sk.hip", "device.h"):
        with open(os.path.join(ROOT, "routing_grouped_expert_amd", "csrc", name)) as f:
            for line in f:
                code = re.sub(r"//.*$", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per grouped-FFN call from the committed rocprofv3 counter
    summary, or None when it is missing, for another workload, or was taken
    on a different FFN source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = dict(re.findall(r"^(\w+)\s*=\s*(\S+)\s*$", open(TRAFFIC_FILE).read(), re.M))
    if kv.get("workload") != workload or kv.get("ffn_source_sha256") != ffn_source_digest():
        return None
    return float(kv["hbm_bytes_per_call"])


def routing_sweep():
    """Cost table of the routing steps (route + permute) over token counts and
    expert counts: median microseconds per call, warm (inputs cached) and cold
    (a 512 MiB buffer written between calls, so logits and ids come from HBM)."""
    import torch

    import routing_grouped_expert_amd as moe
    from synth import configs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    table = []
    for E in (8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096):
        k = min(8, E)
        for T in (1, 64, 4096):
            lg = torch.from_numpy(configs.routing_logits(T, E=E)).to(dev)
            ids = torch.empty((T, k), dtype=torch.int32, device=dev)
            wts = torch.empty((T, k), dtype=torch.float32, device=dev)
            cnt = torch.empty((E,), dtype=torch.int32, device=dev)
            off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
            perm = torch.empty((T * k,), dtype=torch.int32, device=dev)
            e2p = torch.empty((T * k,), dtype=torch.int32, device=dev)
            ws = moe.alloc_workspace(T, 128, 128, E, k, E)

            def call():
                moe.route(lg, k, ids, wts, stream)
                moe.permute(ids, E, 0, E, cnt, off, perm, e2p, ws, stream)

            res = {}
            for mode in ("warm", "cold"):
                for _ in range(5):
                    call()
                times = []
                for _ in range(50):
                    if mode == "cold":
                        flush.fill_(1)
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    call()
                    b.record(stream)
                    times.append((a, b))
                torch.cuda.synchronize()
                us = sorted(a.elapsed_time(b) * 1e3 for a, b in times)
                res[mode] = {"median": round(us[25], 2), "p10": round(us[5], 2), "p90": round(us[45], 2)}
            table.append({"E": E, "T": T, "k": k, **res})
            print(f"E {E:5d} T {T:5d} k {k}: warm {res['warm']['median']:7.2f} us  "
                  f"cold {res['cold']['median']:7.2f} us", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "route + permute microseconds per call", "unit": "us",
                      "higher_is_better": False, "data": "synthetic (seeded N(0,1) logits)",
                      "table": table}))


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "expert-parallel path is not built.", file=sys.stderr)
        sys.exit(2)
    if args.routing_sweep:
        routing_sweep()
        return

    import torch

    import routing_grouped_expert_amd as moe
    from synth import configs

    dev = torch.device("cuda:0")
    cfg = configs.WORKLOADS[args.workload]
    d = configs.layer_inputs(cfg)
    T, H, I, E, k, first, L = (d[n] for n in ("T", "H", "I", "E", "k", "first", "L"))

    def to_dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    x, wg = to_dev(d["x"]), to_dev(d["wg"])
    bias = None if d["bias"] is None else to_dev(d["bias"])
    fp8 = args.weights == "fp8"
    if fp8:
        w1q, w1s, w2q, w2s = (to_dev(a) for a in configs.fp8_weights(d))
        w1 = w2 = None
    else:
        w1, w2 = to_dev(d["w1"]), to_dev(d["w2"])
    y = torch.empty((T, H), dtype=torch.int16, device=dev)
    ws = moe.alloc_workspace(T, H, I, E, k, L)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((L + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((T * k,), dtype=torch.int32, device=dev)
    e2p = torch.empty((T * k,), dtype=torch.int32, device=dev)
    eo = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    del d

    def step(ev0=None, ev1=None):
        moe.router_logits(x, wg, bias, logits, ws, stream)
        moe.route(logits, k, ids, wts, stream)
        moe.permute(ids, E, first, L, counts, offsets, perm, e2p, ws, stream)
        if ev0 is not None:
            ev0.record(stream)
        if fp8:
            moe.grouped_ffn_fp8(x, perm, offsets, k, w1q, w1s, w2q, w2s, eo, ws, stream)
        else:
            moe.grouped_ffn(x, perm, offsets, k, w1, w2, eo, ws, stream)
        if ev1 is not None:
            ev1.record(stream)
        moe.combine(eo, e2p, wts, y, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        step(e0, e1)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ffn_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs)

    # moe_forward over the same number of steps (same kernels in one call)
    def forward():
        if fp8:
            moe.forward_fp8(x, wg, bias, w1q, w1s, w2q, w2s, k, first, L, y, ws, stream=stream)
        else:
            moe.forward(x, wg, bias, w1, w2, k, first, L, y, ws, stream=stream)

    for _ in range(2):
        forward()
    torch.cuda.synchronize()
    f0 = time.perf_counter()
    for _ in range(args.steps):
        forward()
    torch.cuda.synchronize()
    forward_ms = (time.perf_counter() - f0) / args.steps * 1e3

    cnt = counts.cpu().numpy()[first:first + L]
    n_local = int(cnt.sum())
    touched = int(np.count_nonzero(cnt))
    # Algorithmic bytes of one grouped-FFN call: each touched expert's W1 and W2
    # once (3*I*H bf16, or 3*I*H FP8 codes plus 3 row scales per I or H rows),
    # each local entry's gathered row (H bf16) and its fp32 output row (H fp32).
    wbytes = 3 * I * H + (2 * I + H) * 4 if fp8 else 3 * I * H * 2
    ffn_bytes = touched * wbytes + n_local * H * 2 + n_local * H * 4
    achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
    layer_bytes = configs.algorithmic_bytes(cfg, cnt) - (touched * 3 * I * H * 2 - touched * wbytes)
    yv = y.cpu().numpy().view(np.uint16)
    assert np.isfinite((yv.astype(np.uint32) << 16).view(np.float32)).all()

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()

    # Achievable HBM read rate on this part: the probe library streams 2 GiB once.
    probe_gbs = None
    probe_path = os.path.join(ROOT, "routing_grouped_expert_amd", "libhbmprobe.so")
    if os.path.exists(probe_path):
        import ctypes
        plib = ctypes.CDLL(probe_path)
        plib.hbm_read_probe.restype = ctypes.c_int
        plib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p]
        nbytes = 2 << 30
        pbuf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        sh = ctypes.c_void_p(stream.cuda_stream)
        rc = plib.hbm_read_probe(pbuf.data_ptr(), nbytes, sink.data_ptr(), sh)
        if rc == 0:
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            for _ in range(5):
                rc |= plib.hbm_read_probe(pbuf.data_ptr(), nbytes, sink.data_ptr(), sh)
            p1.record(stream)
            torch.cuda.synchronize()
            if rc == 0:
                probe_gbs = nbytes / (p0.elapsed_time(p1) / 5 * 1e-3) / 1e9
        del pbuf, sink

    routing = None
    if not args.no_routing:
        routing = {}
        for Tr in configs.ROUTING["T"]:
            lg = to_dev(configs.routing_logits(Tr))
            Er, kr = configs.ROUTING["E"], configs.ROUTING["k"]
            ri = torch.empty((Tr, kr), dtype=torch.int32, device=dev)
            rw = torch.empty((Tr, kr), dtype=torch.float32, device=dev)
            rc = torch.empty((Er,), dtype=torch.int32, device=dev)
            ro = torch.empty((Er + 1,), dtype=torch.int32, device=dev)
            rp = torch.empty((Tr * kr,), dtype=torch.int32, device=dev)
            re_ = torch.empty((Tr * kr,), dtype=torch.int32, device=dev)
            rws = moe.alloc_workspace(Tr, 128, 128, Er, kr, Er)
            n_it = 200
            for _ in range(10):
                moe.route(lg, kr, ri, rw, stream)
                moe.permute(ri, Er, 0, Er, rc, ro, rp, re_, rws, stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n_it):
                moe.route(lg, kr, ri, rw, stream)
                moe.permute(ri, Er, 0, Er, rc, ro, rp, re_, rws, stream)
            b.record(stream)
            torch.cuda.synchronize()
            routing[f"T{Tr}"] = round(a.elapsed_time(b) / n_it * 1e3, 2)

    cpu = None
    if not args.no_cpu_baseline and not fp8:  # the oracle baseline is reported for the bf16 layer
        import oracle
        d = configs.layer_inputs(cfg)
        n_tok = min(T, 32)
        sample = np.arange(n_tok, dtype=np.int32)
        oracle.default()
        # Repeat the sampled forward until about 10 s of host time have passed.
        reps = 0
        c0 = time.perf_counter()
        while True:
            oracle.forward(d["x"], d["wg"], d["w1"], d["w2"], k, first, L, d["bias"], sample)
            reps += 1
            if time.perf_counter() - c0 >= 10.0:
                break
        c1 = time.perf_counter()
        cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        cpu = {"value": round(reps * n_tok / (c1 - c0), 3), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{n_tok} of {T} tokens of the {args.workload} workload, {reps} times: "
                         f"fp64 router for all tokens, routing, and the expert FFN + combine "
                         f"of the sampled tokens; {c1 - c0:.2f} s wall"}

    out = {
        "metric": "MoE layer tokens/s + % of HBM/MFMA roofline; routing us at 1024 experts",
        "value": round(T * args.steps / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not fp8 else "bf16 activations, fp8-e4m3 weights (per-row fp32 scales)",
        "data": "synthetic (seeded normal inputs; random-init weights of the stated shapes)",
        "config": {"workload": f"{args.workload}: T={T} H={H} I={I} E={E} top-{k}"
                               + (f" share {cfg['s']} of {cfg['S']} (experts {first}..{first + L - 1})"
                                  if cfg["S"] > 1 else ""),
                   "tokens": T, "hidden": H, "intermediate": I, "experts": E, "top_k": k,
                   "local_experts": L},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if fp8 else committed_traffic(args.workload),
                     "kernel": "grouped-FFN call (plan, W1 + SwiGLU, W2 kernels)",
                     "kernel_ms": round(ffn_ms, 4), "algorithmic_bytes": ffn_bytes,
                     "hbm_read_probe_gbs": None if probe_gbs is None else round(probe_gbs, 1),
                     "frac_of_probe": None if probe_gbs is None else round(achieved / probe_gbs, 4)},
        "cpu_baseline": cpu,
        "forward_ms_per_step": None if forward_ms is None else round(forward_ms, 4),
        "layer_hbm_frac": round(layer_bytes / (elapsed / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
        "routing_us_1024_experts": routing,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
