#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

A step is one call of moe_forward -- router logits, routing, histogram /
scan / permutation, grouped expert FFN, combine -- over one batch of the
fine-grained workload (T=512 tokens, H=7168, I=2048, 256 experts, top-8,
router bias, bf16 weights: the largest of the layer workloads by bytes and
time). Inputs are synthetic (seeded) and resident in HBM before timing
starts; ``value`` is tokens / wall time over the timed steps.

The same run also measures:
  - the per-call breakdown (the five library calls in moe_forward's order,
    HIP events around each call on the library's stream): the grouped-FFN
    call is the dominant work, and ``roofline`` relates its algorithmic bytes
    to its measured duration (against 8 TB/s, and against the read rate of a
    plain streaming probe on the same part);
  - the share-0 prefill layer (E=384 over 5 shares, experts 0..76, T=4096)
    and the decode layer (T=32, H=4096, I=14336, E=8, top-2) as extra keys;
  - the same layers and the headline one with FP8 E4M3 expert weights
    (moe_forward_fp8: per-row fp32 scales, bf16 activations) as the
    ``*_fp8`` keys;
  - an MFMA-bound probe: the share-0 expert weights with T=32768 tokens, the
    grouped FFN's useful bf16 TFLOP/s against the 2.5 PFLOP/s dense peak;
  - routing microseconds at 1024 experts (route + permute, T = 1 / 64 / 4096),
    replayed from a captured graph (and issued call by call from Python, and
    as single calls warm and cold, the Infinity Cache flushed before each);
  - the tiny layer (T=16, E=8, top-2) as single moe_forward calls, warm and
    cold;
  - the oracle timed on the host cores as a CPU baseline (headline layer).
Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROBE_TOKENS = 32768
# A GPU spin (~0.5 ms) queued before each single timed call, so that the call
# waits behind running work and its events hold no host launch latency.
SPIN_CYCLES = 1000000


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fine", choices=["tiny", "decode", "fine", "share0"])
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the share-0 / decode / FP8 extra keys and the MFMA probe")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-routing", action="store_true", help="skip the routing-only timings")
    ap.add_argument("--weights", default="bf16", choices=["bf16", "fp8"],
                    help="expert weight format: bf16 (the headline), or FP8 E4M3 codes with "
                         "per-row fp32 scales (moe_forward_fp8; x stays bf16)")
    ap.add_argument("--routing-sweep", action="store_true",
                    help="instead of the layer step: the routing variants' microseconds per "
                         "call over T in {1, 4, .., 4096} x E in {8 .. 4096}, k = --routing-k "
                         "(k = E below it), from replayed graphs; one JSON line")
    ap.add_argument("--routing-k", type=int, default=8,
                    help="selections per token of the routing sweep (default 8)")
    ap.add_argument("--routing-only", action="store_true",
                    help="only the routing timings at 1024 experts (one JSON line)")
    ap.add_argument("--probe-only", action="store_true",
                    help="only the MFMA probe (share-0 weights, T=32768), for counter runs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one elementwise kernel that reads 256 MiB and writes 256 MiB "
                         "(calibrates the HBM byte counters)")
    return ap.parse_args()


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def ffn_source_digest():
    """Digest of the grouped-FFN code (ffn.hip, ffn_sk.hip, ffn_dense.hip,
    plan.h, device.h) with line comments, trailing blanks and empty lines
    removed, so that editing a comment does not retire a committed counter
    summary."""
    h = hashlib.sha256()
    for name in ("ffn.hip", "ffn_sk.hip", "ffn_dense.hip", "plan.h", "device.h"):
        with open(os.path.join(ROOT, "routing_grouped_expert_amd", "csrc", name)) as f:
            for line in f:
                code = re.sub(r"//.*$", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per grouped-FFN call from the committed rocprofv3 counter
    summary of this workload (profiles/ffn_<workload>_pmc_traffic.md), or None
    when it is missing or was taken on a different FFN source."""
    path = os.path.join(ROOT, "profiles", f"ffn_{workload}_pmc_traffic.md")
    if not os.path.exists(path):
        return None
    kv = dict(re.findall(r"^(\w+)\s*=\s*(\S+)\s*$", open(path).read(), re.M))
    if kv.get("workload") != workload or kv.get("ffn_source_sha256") != ffn_source_digest():
        return None
    return float(kv["hbm_bytes_per_call"])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def pct(v, q):
    return float(np.percentile(np.asarray(v), q))


class Layer:
    """One workload's inputs, outputs and workspace on cuda:0."""

    def __init__(self, name, fp8=False, T=None, weights_from=None):
        import torch

        from synth import configs
        self.torch = torch
        self.name = name
        self.cfg = dict(configs.WORKLOADS[name])
        if T is not None:
            self.cfg["T"] = T
        t0 = time.perf_counter()
        d = configs.layer_inputs(self.cfg, weights=weights_from is None)
        self.T, self.H, self.I, self.E, self.k = (d[n] for n in ("T", "H", "I", "E", "k"))
        self.first, self.L = d["first"], d["L"]
        self.fp8 = fp8
        dev = torch.device("cuda:0")
        self.x, self.wg = self.to_dev(d["x"]), self.to_dev(d["wg"])
        self.bias = None if d["bias"] is None else self.to_dev(d["bias"])
        if weights_from is not None:
            self.w1, self.w2 = weights_from.w1, weights_from.w2
            self.wq = weights_from.wq
        elif fp8:
            self.wq = tuple(self.to_dev(a) for a in configs.fp8_weights(d))
            self.w1 = self.w2 = None
        else:
            self.w1, self.w2 = self.to_dev(d["w1"]), self.to_dev(d["w2"])
            self.wq = None
        self.host = d if name == "fine" and T is None and not fp8 else None  # kept for the oracle
        del d
        T, H, E, k, L = self.T, self.H, self.E, self.k, self.L
        import routing_grouped_expert_amd as moe
        self.moe = moe
        self.y = torch.empty((T, H), dtype=torch.int16, device=dev)
        self.ws = moe.alloc_workspace(T, H, self.I, E, k, L)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.wts = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), dtype=torch.int32, device=dev)
        self.offsets = torch.empty((L + 1,), dtype=torch.int32, device=dev)
        self.perm = torch.empty((T * k,), dtype=torch.int32, device=dev)
        self.e2p = torch.empty((T * k,), dtype=torch.int32, device=dev)
        self.eo = torch.empty((T * k, H), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        log(f"{name} T={T}: inputs ready in {time.perf_counter() - t0:.1f} s")

    def to_dev(self, a):
        a = np.ascontiguousarray(a)
        return self.torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda:0")

    def describe(self):
        c = self.cfg
        s = (f"{self.name}: T={self.T} H={self.H} I={self.I} E={self.E} top-{self.k}"
             + (", router bias" if c.get("bias") else ""))
        if c["S"] > 1:
            s += f", share {c['s']} of {c['S']} (experts {self.first}..{self.first + self.L - 1})"
        return s

    def forward(self):
        m = self.moe
        if self.fp8:
            w1q, w1s, w2q, w2s = self.wq
            m.forward_fp8(self.x, self.wg, self.bias, w1q, w1s, w2q, w2s, self.k, self.first,
                          self.L, self.y, self.ws, stream=self.stream)
        else:
            m.forward(self.x, self.wg, self.bias, self.w1, self.w2, self.k, self.first, self.L,
                      self.y, self.ws, stream=self.stream)

    def calls(self):
        """The five library calls of moe_forward, in its order."""
        m, s = self.moe, self.stream

        def router():
            m.router_logits(self.x, self.wg, self.bias, self.logits, self.ws, s)

        def route():
            m.route(self.logits, self.k, self.ids, self.wts, s)

        def permute():
            m.permute(self.ids, self.E, self.first, self.L, self.counts, self.offsets, self.perm,
                      self.e2p, self.ws, s)

        def ffn():
            if self.fp8:
                w1q, w1s, w2q, w2s = self.wq
                m.grouped_ffn_fp8(self.x, self.perm, self.offsets, self.k, w1q, w1s, w2q, w2s,
                                  self.eo, self.ws, s)
            else:
                m.grouped_ffn(self.x, self.perm, self.offsets, self.k, self.w1, self.w2, self.eo,
                              self.ws, s)

        def combine():
            m.combine(self.eo, self.e2p, self.wts, self.y, s)

        return [("router", router), ("route", route), ("permute", permute), ("ffn", ffn),
                ("combine", combine)]

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def time_forward(self, steps, warmup):
        """Wall time of `steps` back-to-back moe_forward calls (synchronised on
        both sides), then each call's event duration on the stream over another
        `steps` calls (the timed loop itself issues nothing but the calls)."""
        torch = self.torch
        for _ in range(warmup):
            self.forward()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.forward()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        evs = [(self.ev(), self.ev()) for _ in range(steps)]
        for a, b in evs:
            a.record(self.stream)
            self.forward()
            b.record(self.stream)
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) for a, b in evs]
        return elapsed, per

    def time_forward_graph(self, steps):
        """(ms per step, outputs equal) for `steps` moe_forward calls captured
        in one HIP graph and replayed: the median of 3 replays (events around
        each replay), and whether every replay's output equals the eager
        calls' (reported, not asserted: the GPU tests check replays)."""
        torch = self.torch
        torch.cuda.synchronize()
        ref = self.y.clone()
        g = torch.cuda.CUDAGraph()
        saved = self.stream
        with torch.cuda.graph(g):
            self.stream = torch.cuda.current_stream()  # the capture stream
            try:
                for _ in range(steps):
                    self.forward()
            finally:
                self.stream = saved
        torch.cuda.synchronize()
        reps, same = [], True
        for _ in range(3):
            self.y.fill_(7)
            a, b = self.ev(), self.ev()
            a.record(self.stream)
            g.replay()
            b.record(self.stream)
            torch.cuda.synchronize()
            reps.append(a.elapsed_time(b) / steps)
            same = same and torch.equal(self.y, ref)
        del g
        if not same:
            log(f"{self.name}: graph replay output differs from the eager calls")
        return float(np.median(reps)), same

    def time_calls(self, steps):
        """Mean event duration (ms) of each of the five calls over `steps`
        back-to-back layer passes."""
        torch = self.torch
        calls = self.calls()
        for _ in range(2):
            for _, f in calls:
                f()
        torch.cuda.synchronize()
        evs = [[(self.ev(), self.ev()) for _ in calls] for _ in range(steps)]
        for row in evs:
            for (a, b), (_, f) in zip(row, calls):
                a.record(self.stream)
                f()
                b.record(self.stream)
        torch.cuda.synchronize()
        out = {}
        for i, (n, _) in enumerate(calls):
            out[n] = float(np.mean([row[i][0].elapsed_time(row[i][1]) for row in evs]))
        return out

    def ffn_counts(self):
        """(algorithmic bytes, useful flops, local entries, touched experts) of
        one grouped-FFN call, from the expert counts of the last pass."""
        cnt = self.counts.cpu().numpy()[self.first:self.first + self.L]
        n_local = int(cnt.sum())
        touched = int(np.count_nonzero(cnt))
        H, I = self.H, self.I
        # each touched expert's W1 and W2 once (3 I H bf16, or 3 I H FP8 codes
        # plus one fp32 scale per row), each local entry's gathered bf16 row in
        # and fp32 output row out
        wbytes = 3 * I * H + (2 * I + H) * 4 if self.fp8 else 3 * I * H * 2
        nbytes = touched * wbytes + n_local * H * 2 + n_local * H * 4
        flops = 6.0 * H * I * n_local
        return nbytes, flops, n_local, touched, cnt

    def layer_bytes(self, cnt):
        from synth import configs
        b = configs.algorithmic_bytes(self.cfg, cnt)
        if self.fp8:
            touched = int(np.count_nonzero(cnt))
            b += touched * ((3 * self.I * self.H + (2 * self.I + self.H) * 4)
                            - 3 * self.I * self.H * 2)
        return b

    def check_output(self):
        yv = self.y.cpu().numpy().view(np.uint16)
        assert np.isfinite((yv.astype(np.uint32) << 16).view(np.float32)).all(), "non-finite y"


def summarize(layer, steps, warmup):
    """Layer timing, per-call breakdown and the grouped-FFN roofline figures."""
    elapsed, per = layer.time_forward(steps, warmup)
    graph_ms, graph_same = layer.time_forward_graph(steps)
    calls = layer.time_calls(steps)
    layer.check_output()
    fbytes, fflops, n_local, touched, cnt = layer.ffn_counts()
    ffn_ms = calls["ffn"]
    ms = elapsed / steps * 1e3
    lbytes = layer.layer_bytes(cnt)
    return {
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(layer.T / (ms * 1e-3), 1),
        "step_ms_median": round(pct(per, 50), 4), "step_ms_p10": round(pct(per, 10), 4),
        "step_ms_p90": round(pct(per, 90), 4),
        "ms_per_step_graph": round(graph_ms, 4),
        "graph_replay_matches_eager": graph_same,
        "layer_hbm_frac": round(lbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "call_ms": {n: round(v, 4) for n, v in calls.items()},
        "ffn_ms": round(ffn_ms, 4),
        "ffn_bytes": fbytes,
        "ffn_gbs": round(fbytes / (ffn_ms * 1e-3) / 1e9, 1),
        "ffn_hbm_frac": round(fbytes / (ffn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "ffn_useful_tflops": round(fflops / (ffn_ms * 1e-3) / 1e12, 1),
        "ffn_mfma_frac": round(fflops / (ffn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "local_entries": n_local, "touched_experts": touched,
    }


def hbm_probe(torch, stream):
    """Read rate (GB/s) of a plain streaming kernel over 2 GiB (probe library,
    not part of the MoE path), or None when the probe library is absent."""
    probe_path = os.path.join(ROOT, "routing_grouped_expert_amd", "libhbmprobe.so")
    if not os.path.exists(probe_path):
        return None
    import ctypes
    plib = ctypes.CDLL(probe_path)
    plib.hbm_read_probe.restype = ctypes.c_int
    plib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p]
    nbytes = 2 << 30
    pbuf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    sh = ctypes.c_void_p(stream.cuda_stream)
    rc = plib.hbm_read_probe(pbuf.data_ptr(), nbytes, sink.data_ptr(), sh)
    if rc != 0:
        return None
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(5):
        rc |= plib.hbm_read_probe(pbuf.data_ptr(), nbytes, sink.data_ptr(), sh)
    p1.record(stream)
    torch.cuda.synchronize()
    return None if rc != 0 else nbytes / (p0.elapsed_time(p1) / 5 * 1e-3) / 1e9


def routing_timings(torch):
    """Routing (selection, weights, histogram, scan, permutation) at E = 1024,
    k = 8, T = 1 / 64 / 4096 through moe_route_permute, microseconds per call:
    `graph` replays 200 captured calls (each replay checked against the eager
    outputs), `eager` issues 200 calls from Python back to back, `separate`
    replays 200 captured moe_route + moe_permute pairs, `cold` times single
    calls (median of 30, HIP events around the call) each issued after a kernel
    that writes a 512 MiB buffer (the 256 MB Infinity Cache then holds none of
    the routing's inputs or outputs) and `warm_single` the same single calls
    without that write; both queue a GPU spin of ~0.5 ms before the call, so
    the call waits behind running work and no host launch latency is timed."""
    import routing_grouped_expert_amd as moe
    from synth import configs

    Er, kr = configs.ROUTING["E"], configs.ROUTING["k"]
    out = {"graph": {}, "eager": {}, "separate": {}, "cold": {}, "warm_single": {}}
    n_it = 200
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    for Tr in configs.ROUTING["T"]:
        lg = torch.from_numpy(configs.routing_logits(Tr)).to("cuda:0")
        bufs = dict(ri=torch.empty((Tr, kr), dtype=torch.int32, device="cuda:0"),
                    rw=torch.empty((Tr, kr), dtype=torch.float32, device="cuda:0"),
                    rc=torch.empty((Er,), dtype=torch.int32, device="cuda:0"),
                    ro=torch.empty((Er + 1,), dtype=torch.int32, device="cuda:0"),
                    rp=torch.empty((Tr * kr,), dtype=torch.int32, device="cuda:0"),
                    re=torch.empty((Tr * kr,), dtype=torch.int32, device="cuda:0"))
        rws = moe.alloc_workspace(Tr, 128, 128, Er, kr, Er)

        def pair(s=None, b=bufs):
            moe.route_permute(lg, kr, 0, Er, b["ri"], b["rw"], b["rc"], b["ro"], b["rp"], b["re"],
                              rws, s)

        def separate(s=None, b=bufs):
            moe.route(lg, kr, b["ri"], b["rw"], s)
            moe.permute(b["ri"], Er, 0, Er, b["rc"], b["ro"], b["rp"], b["re"], rws, s)

        stream = torch.cuda.current_stream()
        for _ in range(10):
            pair(stream)
        torch.cuda.synchronize()
        ref = {n: t.clone() for n, t in bufs.items()}
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_it):
            pair(stream)
        b.record(stream)
        torch.cuda.synchronize()
        out["eager"][f"T{Tr}"] = round(a.elapsed_time(b) / n_it * 1e3, 2)

        for key, cold in (("cold", True), ("warm_single", False)):
            one = []
            for i in range(30):
                if cold:
                    flush.fill_(i & 0xFF)
                torch.cuda._sleep(SPIN_CYCLES)
                a.record(stream)
                pair(stream)
                b.record(stream)
                torch.cuda.synchronize()
                one.append(a.elapsed_time(b) * 1e3)
            out[key][f"T{Tr}"] = round(float(np.median(one)), 2)

        for key, fn in (("graph", pair), ("separate", separate)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(n_it):
                    fn(None)
            reps = []
            for _ in range(3):
                for t in bufs.values():
                    t.fill_(-7)
                torch.cuda.synchronize()
                a.record(stream)
                g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                reps.append(a.elapsed_time(b) / n_it * 1e3)
                for n, t in bufs.items():
                    if n == "rp":  # positions past the local entries are not written
                        nl = int(ref["ro"][-1])
                        ok = torch.equal(t[:nl], ref[n][:nl])
                    else:
                        ok = torch.equal(t, ref[n])
                    assert ok, f"graph replay of routing T={Tr} ({key}): {n} differs from eager"
            out[key][f"T{Tr}"] = round(float(np.median(reps)), 2)
            del g
    return out


def tiny_layer_us(torch):
    """The tiny layer (T=16 H=128 I=256 E=8 top-2) through moe_forward: the
    median of 50 single calls (HIP events around each call) warm, and cold,
    each issued after a kernel that writes a 512 MiB buffer (so the Infinity
    Cache holds none of the layer's 1.6 MB); both queue a GPU spin of ~0.5 ms
    before the call (no host launch latency is timed). Its bytes and flops take
    well under a microsecond at the roofs: the figure is the kernels' latency
    chain."""
    lay = Layer("tiny")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    for _ in range(5):
        lay.forward()
    torch.cuda.synchronize()
    res = {"workload": lay.describe()}
    for key, cold in (("warm_us", False), ("cold_us", True)):
        one = []
        for i in range(50):
            if cold:
                flush.fill_(i & 0xFF)
            torch.cuda._sleep(SPIN_CYCLES)
            a, b = lay.ev(), lay.ev()
            a.record(lay.stream)
            lay.forward()
            b.record(lay.stream)
            torch.cuda.synchronize()
            one.append(a.elapsed_time(b) * 1e3)
        res[key] = round(float(np.median(one)), 2)
    lay.check_output()
    del flush
    return res


def cpu_baseline(layer, n_tok=32):
    """The oracle (C, OpenMP over the host threads) on the headline layer:
    fp64 router and routing for all T tokens, timed once, and the expert FFN +
    combine of n_tok sampled tokens, repeated for ~10 s; scaled to the whole
    layer as T / (router time + T x per-token FFN time)."""
    import oracle
    d = layer.host
    T = layer.T
    oracle.default()
    one = np.array([0], np.int32)
    sample = np.linspace(0, T - 1, n_tok).astype(np.int32)
    args = (d["x"], d["wg"], d["w1"], d["w2"], layer.k, layer.first, layer.L, d["bias"])
    r0 = time.perf_counter()
    oracle.forward(*args, one)
    t_route = time.perf_counter() - r0  # router + routing for all T, one token's FFN
    reps, c0 = 0, time.perf_counter()
    while True:
        oracle.forward(*args, sample)
        reps += 1
        if time.perf_counter() - c0 >= 10.0:
            break
    wall = time.perf_counter() - c0
    per_tok = max((wall / reps - t_route) / (n_tok - 1), 1e-9)
    tok_s = T / (t_route + T * per_tok)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": round(tok_s, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"{layer.name} layer: fp64 router + routing of all {T} tokens "
                       f"({t_route:.2f} s), then the expert FFN + combine of {n_tok} sampled "
                       f"tokens {reps} times ({per_tok * 1e3:.1f} ms per token); "
                       f"{wall + t_route:.1f} s wall, tokens/s = T / (router + T x per-token)")}


def mfma_probe(torch, base, steps):
    """The share-0 expert weights with T=32768 tokens (about 683 entries per
    local expert, above the 312 flop/byte ridge): the grouped FFN's useful
    bf16 TFLOP/s and its fraction of the dense peak."""
    layer = Layer("share0", T=PROBE_TOKENS, weights_from=base)
    layer.forward()
    calls = layer.time_calls(max(3, min(steps, 10)))
    layer.check_output()
    fbytes, fflops, n_local, touched, _ = layer.ffn_counts()
    ms = calls["ffn"]
    res = {"workload": f"share-0 experts (E=384 / 5 shares, 77 local), T={PROBE_TOKENS} "
                       f"H={layer.H} I={layer.I} top-{layer.k}",
           "local_entries": n_local, "ffn_ms": round(ms, 4),
           "useful_tflops": round(fflops / (ms * 1e-3) / 1e12, 1),
           "mfma_frac": round(fflops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "weight_gbs": round(fbytes / (ms * 1e-3) / 1e9, 1),
           "layer_ms": round(sum(calls.values()), 4)}
    del layer
    torch.cuda.empty_cache()
    return res


def routing_sweep(k_sweep=8):
    """Cost table of the routing variants (selection + permutation through
    moe_route_permute_variant) over token counts and expert counts:
    microseconds per call from a replayed graph of 50 back-to-back calls
    (median of 3 replays), for every variant that applies to the cell, the
    outputs of all variants checked equal, and the variant the plan picks."""
    import torch

    import routing_grouped_expert_amd as moe
    from synth import configs

    dev = torch.device("cuda:0")
    table = []
    n_it = 50
    for E in (8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096):
        k = min(k_sweep, E)
        for T in (1, 4, 16, 64, 256, 1024, 4096):
            lg = torch.from_numpy(configs.routing_logits(T, E=E)).to(dev)
            bufs = [torch.empty((T, k), dtype=torch.int32, device=dev),
                    torch.empty((T, k), dtype=torch.float32, device=dev),
                    torch.empty((E,), dtype=torch.int32, device=dev),
                    torch.empty((E + 1,), dtype=torch.int32, device=dev),
                    torch.empty((T * k,), dtype=torch.int32, device=dev),
                    torch.empty((T * k,), dtype=torch.int32, device=dev)]
            ws = moe.alloc_workspace(T, 128, 128, E, k, E)
            row = {"E": E, "T": T, "k": k, "plan": moe.routing_plan(T, E, k, E), "us": {}}
            ref = None
            for v in ("one_block", "two_kernels", "tiled"):
                try:
                    moe.route_permute(lg, k, 0, E, *bufs, ws, variant=v)
                except moe.MoeError as exc:
                    if exc.status != 2:
                        raise
                    continue
                torch.cuda.synchronize()
                out = [b.clone() for b in bufs]
                nl = int(out[3][-1])
                out[4] = out[4][:nl]
                if ref is None:
                    ref = out
                else:
                    assert all(torch.equal(a, b) for a, b in zip(out, ref)), (E, T, v)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(n_it):
                        moe.route_permute(lg, k, 0, E, *bufs, ws, variant=v)
                reps = []
                for _ in range(3):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    g.replay()
                    b.record()
                    torch.cuda.synchronize()
                    reps.append(a.elapsed_time(b) / n_it * 1e3)
                del g
                row["us"][v] = round(float(np.median(reps)), 2)
            row["best"] = min(row["us"], key=row["us"].get)
            table.append(row)
            print(f"E {E:5d} T {T:5d}: " + "  ".join(f"{v} {u:7.2f}" for v, u in row["us"].items())
                  + f"   plan {row['plan']}", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "routing (selection + permutation) microseconds per call",
                      "unit": "us", "higher_is_better": False,
                      "data": "synthetic (seeded N(0,1) logits)", "table": table}))


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "expert-parallel path is not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    # Everything runs on one created stream (default priority), as a serving
    # loop would, not on the legacy null stream: the fine-grained layer ran
    # 3.568 against 3.582 ms per step there.
    with torch.cuda.stream(torch.cuda.Stream()):
        run(args, torch)


def run(args, torch):
    if args.routing_sweep:
        routing_sweep(args.routing_k)
        return

    fp8 = args.weights == "fp8"
    if args.routing_only:
        r = routing_timings(torch)
        print(json.dumps({"routing_us_1024_experts": r["graph"],
                          "routing_us_1024_experts_eager": r["eager"],
                          "routing_us_1024_experts_separate_calls": r["separate"],
                          "routing_us_1024_experts_cold": r["cold"],
                          "routing_us_1024_experts_warm_single": r["warm_single"]}))
        return
    if args.probe_only:
        base = Layer("share0", fp8=False)
        print(json.dumps({"mfma_probe": mfma_probe(torch, base, args.steps)}))
        return

    extras = {}
    probe = None
    if not args.no_extras:
        extras["tiny"] = tiny_layer_us(torch)
        log(f"tiny: {extras['tiny']['warm_us']} us warm, {extras['tiny']['cold_us']} us cold")
        for name in ("share0", "decode"):
            if name == args.workload:
                continue
            lay = Layer(name, fp8=fp8)
            extras[name] = dict(workload=lay.describe(), **summarize(lay, args.steps, args.warmup))
            log(f"{name}: {extras[name]['ms_per_step']} ms/step")
            if name == "share0" and not fp8:
                probe = mfma_probe(torch, lay, args.steps)
                log(f"mfma probe: {probe['useful_tflops']} TFLOP/s")
            del lay
            torch.cuda.empty_cache()
        if not fp8:
            # the FP8 E4M3 weight path (moe_forward_fp8) on the same workloads
            for name in ("decode", "share0", args.workload):
                lay = Layer(name, fp8=True)
                extras[f"{name}_fp8"] = dict(
                    workload=lay.describe() + ", FP8 E4M3 weights with per-row fp32 scales",
                    **summarize(lay, args.steps, args.warmup))
                log(f"{name} fp8: {extras[name + '_fp8']['ms_per_step']} ms/step")
                del lay
                torch.cuda.empty_cache()

    layer = Layer(args.workload, fp8=fp8)
    head = summarize(layer, args.steps, args.warmup)
    log(f"{args.workload}: {head['ms_per_step']} ms/step")

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst

    probe_gbs = hbm_probe(torch, layer.stream)
    routing = None if args.no_routing else routing_timings(torch)
    cpu = None
    if not args.no_cpu_baseline and layer.host is not None:
        cpu = cpu_baseline(layer)

    achieved = head["ffn_gbs"]
    out = {
        "metric": "MoE layer tokens/s + % of HBM/MFMA roofline; routing us at 1024 experts",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not fp8 else "bf16 activations, fp8-e4m3 weights (per-row fp32 scales)",
        "data": "synthetic (seeded normal inputs; random-init weights of the stated shapes)",
        "config": {"workload": layer.describe(), "tokens": layer.T, "hidden": layer.H,
                   "intermediate": layer.I, "experts": layer.E, "top_k": layer.k,
                   "local_experts": layer.L},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if fp8 else committed_traffic(args.workload),
                     "kernel": "grouped-FFN call (plan, W1 + SwiGLU, W2 kernels)",
                     "kernel_ms": head["ffn_ms"], "algorithmic_bytes": head["ffn_bytes"],
                     "mfma_useful_tflops": head["ffn_useful_tflops"],
                     "mfma_frac": head["ffn_mfma_frac"],
                     "hbm_read_probe_gbs": None if probe_gbs is None else round(probe_gbs, 1),
                     "frac_of_probe": None if probe_gbs is None else round(achieved / probe_gbs, 4)},
        "cpu_baseline": cpu,
        "step_ms": {"median": head["step_ms_median"], "p10": head["step_ms_p10"],
                    "p90": head["step_ms_p90"]},
        "ms_per_step_graph": head["ms_per_step_graph"],
        "graph_replay_matches_eager": head["graph_replay_matches_eager"],
        "layer_hbm_frac": head["layer_hbm_frac"],
        "call_ms": head["call_ms"],
        "routing_us_1024_experts": None if routing is None else routing["graph"],
        "routing_us_1024_experts_eager": None if routing is None else routing["eager"],
        "routing_us_1024_experts_separate_calls": None if routing is None else routing["separate"],
        "routing_us_1024_experts_cold": None if routing is None else routing["cold"],
        "routing_us_1024_experts_warm_single": None if routing is None else routing["warm_single"],
    }
    for name, e in extras.items():
        out[name] = e
    if probe is not None:
        out["mfma_probe"] = probe
    print(json.dumps(out))


if __name__ == "__main__":
    main()
