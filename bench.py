"""Benchmark of the W4A16 decode path on one MI355X.

One step = one pass of the vocabulary-head workload: the batch-1 W4A16 GEMV of a
262144 x 1536 packed table (4-bit codes, group 32, bf16 steps) with a bf16
activation vector, plus the 4-bit row gather of 64 token ids from the same
table (the table serves both the output layer and the input lookup, as on the
dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch", section "Step 2 - Keep
the Vocabulary Tables in 4-Bit").  Three copies of the table are rotated so that
the 256 MB Infinity Cache cannot hold the working set.

`value` = algorithmic HBM bytes of one step / measured step time (GB/s, 1e9 B).
A step is one launch (w4_gemv_gather: the product and the gather together),
the steps launched back to back; the same step replayed as one HIP graph per
step, and as two launches (product, then gather) in one graph, are reported
beside it.
Printed as ONE JSON line, with the dominant kernel's roofline, the CPU oracle's
time on a bounded sample of the same workload, and (under "extra") the other
workloads of this path: the single 2048 x 1536 GEMV, the 35-layer decode-step
sweep, the small-batch products and the expert-indexed layers.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth

V, K, NIDS = 262144, 1536, 64
COPIES = 3
SWEEP_SHAPES = [(2560, 1536), (1536, 2048), (16384, 1536), (1536, 8192)]
SWEEP_LAYERS = 35


def gbps(nbytes: float, seconds: float) -> float:
    """Effective bandwidth in GB/s (GB = 1e9 B): bytes moved / time."""
    return nbytes / seconds / 1e9


def w4_bytes(n: int, k: int) -> int:
    """Packed bytes of an n x k W4 matrix: codes (k/2 per row) + bf16 steps."""
    return n * (k // 2) + n * (k // 32) * 2


def gemv_bytes(n: int, k: int) -> int:
    """Algorithmic bytes of one GEMV: packed weights + 16-bit x + fp32 y."""
    return w4_bytes(n, k) + 2 * k + 4 * n


def gather_bytes(n_ids: int, k: int) -> int:
    """Algorithmic bytes of a row gather: the packed rows, the ids, bf16 out."""
    return w4_bytes(n_ids, k) + 4 * n_ids + 2 * n_ids * k


STEP_BYTES = gemv_bytes(V, K) + gather_bytes(NIDS, K)


GEMV_SOURCES = ["bit_weight_only_02_amd/csrc/w4_gemv.hip", "bit_weight_only_02_amd/csrc/w4_device.h",
                "bit_weight_only_02_amd/csrc/w4_gather.h"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemv_gather_vocab_head_step_traffic.json")


def kernel_source_digest() -> str:
    """sha256 over the sources of the GEMV kernel (to tell whether a stored
    counter measurement still describes the kernel that runs)."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """(HBM bytes per launch, kernel instance) of the decode step's launch (the
    vocabulary-head product with the gather workgroups) from the stored
    rocprofv3 FETCH_SIZE/WRITE_SIZE runs; (None, None) if the kernel's sources
    have changed since they were taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, None
    if rec.get("source_digest") != kernel_source_digest():
        return None, None
    name = rec.get("kernel", "")
    return rec.get("traffic_bytes_per_launch"), name.split("(")[0].replace("void ", "")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _median_rate(nbytes: float, fn, groups: int = 3, min_seconds: float = 2.0) -> float:
    """Median over `groups` timed groups (each repeating fn for >= min_seconds)
    of nbytes / (seconds per call), in GB/s."""
    rates = []
    for _ in range(groups):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
        rates.append(gbps(nbytes, el / reps))
    return sorted(rates)[len(rates) // 2]


def cpu_baseline(codes, steps, x, ids):
    """The oracle, as it stands, on the headline workload: all cores (OpenMP
    over rows) on full steps (the 262144x1536 GEMV plus the 64-row gather), and
    one core on a 16384-row sample of the GEMV plus the gather; each the median
    of 3 timed groups of >= 2 s."""
    import oracle
    import synth
    full = lambda: (oracle.gemv(codes, steps, V, K, x, synth.BF16, threads=True),  # noqa: E731
                    oracle.gather(codes, steps, V, K, ids))
    rows = 16384
    one = lambda: (oracle.gemv(codes, steps, V, K, x, synth.BF16, rows=(0, rows)),  # noqa: E731
                   oracle.gather(codes, steps, V, K, ids))
    all_cores = _median_rate(STEP_BYTES, full)
    single = _median_rate(gemv_bytes(rows, K) + gather_bytes(NIDS, K), one)
    return {"value": round(all_cores, 3), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "full steps (262144x1536 GEMV + 64-row gather), median of 3 groups of >= 2 s",
            "single_thread": {"value": round(single, 3), "unit": "GB/s",
                              "sample": f"{rows}-row GEMV sample + 64-row gather, median of 3 groups of >= 2 s"},
            "cpu_model": cpu_model()}


def cpu_baselines(np, synth):
    """The oracle on a bounded sample of every configuration, one core and (where
    the oracle has a threaded form) all cores, each the median of 3 timed
    groups, in the configuration's own unit."""
    import oracle
    rng = np.random.default_rng(7)
    out = {"cpu_model": cpu_model(), "threads_all_cores": oracle.num_threads()}

    def done(name):
        print(f"cpu baseline: {name} timed", file=sys.stderr, flush=True)

    def gemv_rates(N, Kx, rows_one):
        c, st = synth.w4_matrix(rng, N, Kx)
        xv = synth.activations(rng, Kx, synth.F16)
        allc = _median_rate(gemv_bytes(N, Kx), lambda: oracle.gemv(c, st, N, Kx, xv, synth.F16, threads=True))
        one = _median_rate(gemv_bytes(rows_one, Kx),
                           lambda: oracle.gemv(c, st, N, Kx, xv, synth.F16, rows=(0, rows_one)))
        done(f"{N}x{Kx} product")
        return one, allc
    # single GEMV 2048x1536 (GB/s)
    one, allc = gemv_rates(2048, 1536, 2048)
    out["single_gemv_2048x1536"] = {"unit": "GB/s", "one_core": round(one, 3), "all_cores": round(allc, 3),
                                    "sample": "whole product"}
    # 35-layer decode sweep (us per sweep): one layer's four products, times 35
    shapes = [(2560, 1536), (1536, 2048), (16384, 1536), (1536, 8192)]
    t_one = t_all = 0.0
    for N, Kx in shapes:
        one, allc = gemv_rates(N, Kx, min(N, 2048))
        t_one += gemv_bytes(N, Kx) / (one * 1e9)
        t_all += gemv_bytes(N, Kx) / (allc * 1e9)
    out["decode_sweep_35_layers"] = {"unit": "us per sweep", "one_core": round(35 * t_one * 1e6, 1),
                                     "all_cores": round(35 * t_all * 1e6, 1),
                                     "sample": "one layer's four products (one core: up to 2048 rows of each), x35"}
    # small-M products at M = 16 (us per set of the four shapes; the oracle's
    # product of M rows has no threaded form): 256 rows of each shape
    t = 0.0
    for N, Kx in shapes:
        c, st = synth.w4_matrix(rng, 256, Kx)
        X = synth.activations(rng, (16, Kx), synth.F16)
        r = _median_rate(w4_bytes(256, Kx), lambda: oracle.gemm(c, st, 256, Kx, X, synth.F16, 16), min_seconds=1.0)
        t += w4_bytes(N, Kx) / (r * 1e9)
        done(f"small-M {N}x{Kx}")
    out["small_m_M16_set"] = {"unit": "us per set", "one_core": round(t * 1e6, 1), "all_cores": None,
                              "sample": "256 rows of each of the four shapes at M = 16, scaled by rows"}
    # expert layer, one token (us per token): 8 experts' gate/up and down with
    # the routed sum, one layer, times 30 (the oracle's expert product has no
    # threaded form)
    E = 8
    ids = np.arange(E, dtype=np.int32).reshape(1, E)
    route = np.full((1, E), 1.0 / E, dtype=np.float32)
    gc, gs = synth.w4_matrix(rng, E * 1408, 2816)
    dc, ds = synth.w4_matrix(rng, E * 2816, 704)
    x0 = synth.activations(rng, (1, 2816), synth.BF16)
    G = synth.activations(rng, (E, 1408), synth.BF16)

    def layer():
        oracle.moe(gc, gs, 1408 * 2816 // 8, 1408 * 2816 // 32, 1408, 2816, x0, synth.BF16, 0, ids, E,
                   n_experts=E)
        oracle.moe(dc, ds, 2816 * 704 // 8, 2816 * 704 // 32, 2816, 704, G, synth.BF16, 1, ids, E,
                   n_experts=E, route_w=route, ldx=1408)
    lb = E * (w4_bytes(1408, 2816) + w4_bytes(2816, 704))
    r = _median_rate(lb, layer, min_seconds=1.0)
    done("expert layer")
    out["moe_30_layers_top8_T1"] = {"unit": "us per token", "one_core": round(30 * lb / (r * 1e9) * 1e6, 1),
                                    "all_cores": None, "sample": "one layer of 8 experts, x30"}
    return out


class Timer:
    """HIP events on torch's current stream (the stream every call runs on)."""

    def __init__(self, torch):
        self.torch = torch

    def per_call(self, fn, n: int, warmup: int = 2) -> float:
        """Seconds per call of fn(i) over n back-to-back calls."""
        t = self.torch
        for i in range(warmup):
            fn(i)
        t.cuda.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    def graph_per_call(self, fn, n: int, replays: int = 5) -> float:
        """Seconds per call when n calls are captured in one HIP graph."""
        t = self.torch
        fn(0)
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        s = t.cuda.Stream()
        with t.cuda.stream(s):
            with t.cuda.graph(g, stream=s):
                for i in range(n):
                    fn(i)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / replays / n


def probe_ceiling(w4, torch, reps: int = 10) -> dict:
    """Plain streaming-read ceiling of this device (GB/s): per launch over a
    4 GiB buffer, and the steady rate from the slope between 1 GiB and 4 GiB
    reads (which takes out each launch's fixed ramp-up and drain)."""
    big = 4 << 30
    buf = torch.ones(big // 4, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    small = buf[: (1 << 30) // 4]
    t_big = Timer(torch).per_call(lambda i: w4.w4_probe_stream(buf, out), reps)
    t_small = Timer(torch).per_call(lambda i: w4.w4_probe_stream(small, out), reps)
    del buf, small
    torch.cuda.empty_cache()
    return {"per_launch_4GiB": gbps(big, t_big),
            "steady": gbps(big - (1 << 30), max(t_big - t_small, 1e-9))}


def dev_matrix(torch, np, codes, steps):
    return (torch.from_numpy(codes.view(np.int32)).cuda(),
            torch.from_numpy(steps.view(np.int16)).cuda().view(torch.bfloat16))


def extra_single_gemv(w4, torch, np, synth, timer):
    """Single W4A16 GEMV 2048 x 1536, fp16 x, seed 0: back-to-back calls over
    300 rotated copies (534 MB, beyond the Infinity Cache), eager and in one
    HIP graph."""
    rng = np.random.default_rng(0)
    N, Kc = 2048, 1536
    codes, steps = synth.w4_matrix(rng, N, Kc)
    x = synth.activations(rng, Kc, synth.F16)
    c0, s0 = dev_matrix(torch, np, codes, steps)
    copies = 300
    cs = [c0] + [c0.clone() for _ in range(copies - 1)]
    ss = [s0] + [s0.clone() for _ in range(copies - 1)]
    dx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
    y = torch.empty(N, device="cuda")

    def call(i):
        w4.w4_gemv(cs[i % copies], ss[i % copies], dx, y)
    eager = timer.per_call(call, copies)
    graph = timer.graph_per_call(call, copies)
    wb = w4_bytes(N, Kc)
    out = {"us_per_call_eager": round(eager * 1e6, 3), "us_per_call_graph": round(graph * 1e6, 3),
           "weight_GBps_graph": round(gbps(wb, graph), 1),
           "frac_of_peak_graph": round(gbps(wb, graph) / HBM_PEAK_GBPS, 4)}
    del cs, ss
    torch.cuda.empty_cache()
    # Steady state in one multi-matrix launch: 128 independent copies of the
    # matrix stacked like an expert table and run by the expert-indexed entry
    # point (ids 0..127, one activation row per matrix); two such tables of
    # 227 MB each, alternated, so that no launch finds its weights in the
    # Infinity Cache.
    per_launch = 128
    tabs = [(c0.repeat(per_launch, 1).contiguous(), s0.repeat(per_launch, 1).contiguous()) for _ in range(2)]
    ids = torch.arange(per_launch, dtype=torch.int32, device="cuda").view(4, per_launch // 4)
    X = dx.view(1, Kc).repeat(per_launch, 1).contiguous()
    Y = torch.empty((per_launch, N), device="cuda")

    def multi(i):
        tc, ts = tabs[i % 2]
        w4.w4_moe_gemv_ids(tc, ts, N * Kc // 8, N * Kc // 32, N, Kc, X, ids, x_per_pair=True,
                           n_experts=per_launch, Y=Y)
    mg = timer.graph_per_call(multi, 20)
    per_gemv = mg / per_launch
    out["multi_matrix_launch"] = {"matrices_per_launch": per_launch, "us_per_launch_graph": round(mg * 1e6, 2),
                                  "us_per_gemv": round(per_gemv * 1e6, 3),
                                  "weight_GBps": round(gbps(wb, per_gemv), 1),
                                  "frac_of_peak": round(gbps(wb, per_gemv) / HBM_PEAK_GBPS, 4)}
    del tabs
    torch.cuda.empty_cache()
    return out


def extra_sweep(w4, torch, np, synth, timer, reps: int = 20):
    """Decode-step weight sweep: 35 layers x {2560x1536, 1536x2048, 16384x1536,
    1536x8192}, fp16 x ~ N(0,1), outputs renormalised between matrices: one
    persistent chain launch, and for reference the same 140 products as
    separate launches (eager and in one HIP graph)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    shapes = SWEEP_SHAPES * SWEEP_LAYERS
    mats = []
    for N, Kc in shapes:
        c, s = synth.w4_matrix_torch(g, N, Kc, "cuda")
        mats.append((c[0], s[0].view(torch.bfloat16)))
    ys = [torch.empty(N, device="cuda") for N, _ in shapes]
    xs = [torch.empty(Kc, dtype=torch.float16, device="cuda") for _, Kc in shapes]
    x0 = torch.from_numpy(synth.activations(np.random.default_rng(0), 1536, synth.F16).view(np.int16)
                          ).cuda().view(torch.float16)
    desc = w4.w4_chain_desc(mats, ys)
    sync = w4.w4_chain_sync(len(shapes))
    # The chain (a cooperative launch) runs on a stream of its own: on the
    # default stream of a process that had used four other streams it measured
    # 692 against 622 us per sweep (a plain launch of the same kernel: 603 us
    # on either).
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        chain = timer.per_call(lambda i: w4.w4_gemv_chain(desc, x0, sync), reps)
    torch.cuda.synchronize()
    err = int(sync[2].item())

    def separate(i):
        for j, ((c, s), y) in enumerate(zip(mats, ys)):
            if j == 0:
                w4.w4_gemv(c, s, x0, y)
            else:
                w4.w4_rms_renorm(ys[j - 1], shapes[j][1], out=xs[j])
                w4.w4_gemv(c, s, xs[j], y)
    eager = timer.per_call(separate, 3, warmup=1)
    graph = timer.graph_per_call(separate, 1, replays=reps)
    wb = sum(w4_bytes(N, Kc) for N, Kc in shapes)
    out = {"us_per_sweep_chain": round(chain * 1e6, 2),
           "weight_GBps_chain": round(gbps(wb, chain), 1),
           "frac_of_peak_chain": round(gbps(wb, chain) / HBM_PEAK_GBPS, 4),
           "us_per_sweep_separate_eager": round(eager * 1e6, 1),
           "us_per_sweep_separate_graph": round(graph * 1e6, 1),
           "sweep_weight_bytes": wb, "chain_error_word": err}
    del mats, ys, xs
    torch.cuda.empty_cache()
    return out


def extra_small_m(w4, torch, np, synth, timer, reps: int = 20):
    """Small-batch products on the four sweep shapes, M in {2, 4, 8, 16} bf16
    rows; copies rotated to exceed the Infinity Cache."""
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    copies = 24  # 24 x 25.2 MB per set
    sets = []
    for _ in range(copies):
        mats = []
        for N, Kc in SWEEP_SHAPES:
            c, s = synth.w4_matrix_torch(g, N, Kc, "cuda")
            mats.append((c[0], s[0].view(torch.bfloat16)))
        sets.append(mats)
    set_bytes = sum(w4_bytes(N, Kc) for N, Kc in SWEEP_SHAPES)
    ws = w4.new_workspace(max(w4.w4_gemm_smallM_workspace_bytes(N, Kc, M)
                              for N, Kc in SWEEP_SHAPES for M in (2, 4, 8, 16)))
    out = {}
    for M in (2, 4, 8, 16):
        X = [torch.randn((M, Kc), generator=g, device="cuda").to(torch.bfloat16) for _, Kc in SWEEP_SHAPES]
        Y = [torch.empty((M, N), device="cuda") for N, _ in SWEEP_SHAPES]
        per_shape = {}
        for si, (N, Kc) in enumerate(SWEEP_SHAPES):
            t = timer.per_call(lambda i: w4.w4_gemm_smallM(*sets[i % copies][si], X[si], Y[si], workspace=ws),
                               reps)
            per_shape[f"{N}x{Kc}"] = round(t * 1e6, 2)

        def one_set(i):
            for si in range(4):
                w4.w4_gemm_smallM(*sets[i % copies][si], X[si], Y[si], workspace=ws)
        tset = timer.graph_per_call(one_set, copies)
        bytes_set = set_bytes + sum(2 * M * Kc + 4 * M * N for N, Kc in SWEEP_SHAPES)
        out[f"M{M}"] = {"us_per_shape_eager": per_shape, "us_per_set_graph": round(tset * 1e6, 2),
                        "GBps_set_graph": round(gbps(bytes_set, tset), 1),
                        "frac_of_peak_set_graph": round(gbps(bytes_set, tset) / HBM_PEAK_GBPS, 4)}
    del sets
    torch.cuda.empty_cache()
    return out


def extra_moe(w4, torch, np, synth, timer, reps: int = 5):
    """Expert layers: 30 layers x 128 experts, gate/up 1408x2816 and down
    2816x704 (group 32, bf16 steps), top-8 of 128 per token, router weights
    softmax of N(0,1); T = 1 and 4 tokens; direct addressing and a 32-slot pool
    (the two must agree bit for bit)."""
    E, topk, S, L = 128, 8, 32, 30
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    layers = []
    for _ in range(L):
        gu_c, gu_s = synth.w4_matrix_torch(g, 1408, 2816, "cuda", count=E)
        dn_c, dn_s = synth.w4_matrix_torch(g, 2816, 704, "cuda", count=E)
        layers.append((gu_c.view(-1, 2816 // 8), gu_s.view(-1, 2816 // 32).view(torch.bfloat16),
                       dn_c.view(-1, 704 // 8), dn_s.view(-1, 704 // 32).view(torch.bfloat16)))
    per_expert = w4_bytes(1408, 2816) + w4_bytes(2816, 704)
    out = {}
    for T in (1, 4):
        rng = np.random.default_rng(T)
        picks = [synth.expert_choice(rng, T, E, topk) for _ in range(L)]
        ids = [torch.from_numpy(p[0]).cuda() for p in picks]
        route = [torch.from_numpy(p[1]).cuda() for p in picks]
        x0 = torch.randn((T, 2816), generator=g, device="cuda").to(torch.bfloat16)
        G = torch.empty((T * topk, 1408), device="cuda")
        ws = w4.new_workspace(max(w4.w4_moe_gemv_ids_workspace_bytes(1408, 2816, T, topk, w4.W4_F32_RMS, False, False),
                                  w4.w4_moe_gemv_ids_workspace_bytes(2816, 704, T, topk, w4.W4_F32_RMS, True, True)))
        Dn = [torch.empty((T, 2816), device="cuda") for _ in range(2)]

        # Each product renormalises its fp32 input rows on load (the gate half
        # of each choice's gate/up row; the previous layer's routed sum)
        def token(i, slot=None, pools=None):
            x = x0
            for li, (gc, gs, dc, ds) in enumerate(layers):
                kw = {}
                if pools is not None:
                    gc, gs, dc, ds = pools[li]
                    kw = dict(slot_of=slot[li], n_slots=S)
                w4.w4_moe_gemv_ids(gc, gs, 1408 * 2816 // 8, 1408 * 2816 // 32, 1408, 2816, x, ids[li],
                                   n_experts=E, Y=G, workspace=ws, **kw)
                w4.w4_moe_gemv_ids(dc, ds, 2816 * 704 // 8, 2816 * 704 // 32, 2816, 704, G, ids[li],
                                   x_per_pair=True, n_experts=E, route_w=route[li], Y=Dn[li & 1],
                                   workspace=ws, **kw)
                x = Dn[li & 1]
        eager = timer.per_call(token, reps, warmup=1)
        graph = timer.graph_per_call(token, 1, replays=reps)
        # unique expert bytes read per token step (each distinct expert once per layer)
        distinct = sum(len(np.unique(p[0])) for p in picks)
        nbytes = distinct * per_expert
        # 32-slot pools holding each layer's chosen experts
        slots, pools = [], []
        for li, p in enumerate(picks):
            slot_of, used = synth.slot_map(np.random.default_rng(100 + li), p[0], E, S)
            gc, gs, dc, ds = layers[li]
            sel = torch.from_numpy(used).cuda().long()
            dst = torch.from_numpy(slot_of[used]).cuda().long()

            def pool(t, rows):
                pt = torch.zeros((S * rows, t.shape[1]), dtype=t.dtype, device="cuda")
                pt.view(S, rows, -1)[dst] = t.view(E, rows, -1)[sel]
                return pt
            pools.append((pool(gc, 1408), pool(gs, 1408), pool(dc, 2816), pool(ds, 2816)))
            slots.append(torch.from_numpy(slot_of).cuda())
        token(0)
        last = Dn[(L - 1) & 1]
        ref = last.clone()
        token(0, slot=slots, pools=pools)
        torch.cuda.synchronize()
        identical = bool(torch.equal(ref.view(torch.int32), last.view(torch.int32)))
        pool_graph = timer.graph_per_call(lambda i: token(i, slots, pools), 1, replays=reps)
        out[f"T{T}"] = {"us_per_token_eager": round(eager * 1e6, 1),
                        "us_per_token_graph": round(graph * 1e6, 1),
                        "us_per_token_pool_graph": round(pool_graph * 1e6, 1),
                        "expert_GBps_graph": round(gbps(nbytes, graph), 1),
                        "frac_of_peak_graph": round(gbps(nbytes, graph) / HBM_PEAK_GBPS, 4),
                        "expert_bytes_per_token": nbytes,
                        "pool_bitwise_identical_to_direct": identical}
        del pools
    out["streaming_T1"] = moe_streaming(w4, torch, np, synth, layers, E, topk, S)
    del layers
    torch.cuda.empty_cache()
    return out


def moe_streaming(w4, torch, np, synth, layers, E, topk, S, steps: int = 6):
    """Expert streaming through 32-slot pools (the anyesh.me page's design, on
    this box's PCIe link): the 30 layers' experts sit in a pinned host store;
    per layer and token the LFU pool takes the misses by asynchronous copies on
    a second stream while a shared dense FFN (gate/up 2x2816x2816, down
    2816x2816, W4) runs on the compute stream, then one join.  The host reads
    each layer's routing only after the previous layer has finished, as a
    router's choice would be.  Two managers with pools of their own run the
    same tokens, one joining before the dense FFN (overlap off) and one after
    it (overlap on), token by token in alternation so that drift of the link
    falls on both.  Reported: the medians of us per token with the overlap on
    and off and with every expert resident (direct addressing), bytes streamed
    per token, the copy stream's GB/s, the overlap fraction (the median of the
    per-token time saved over the overlap possible, min(copy, dense FFN) per
    token), and bitwise identity of the last layer's output against direct
    addressing."""
    L, T = len(layers), 1
    KG, NG, KD, ND, DF = 2816, 1408, 704, 2816, 2816
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    parts = [[gc.view(E, -1), gs.view(torch.int16).view(E, -1), dc.view(E, -1), ds.view(torch.int16).view(E, -1)]
             for gc, gs, dc, ds in layers]
    part_bytes = [p[0].numel() * p.element_size() for p in parts[0]]
    host = [[p.view(torch.uint8).cpu().pin_memory() for p in lp] for lp in parts]
    dense = []
    for _ in range(L):
        a = synth.w4_matrix_torch(g, 2 * DF, DF, "cuda")
        b = synth.w4_matrix_torch(g, DF, 2 * DF // 2, "cuda")
        dense.append((a[0], a[1][0].view(torch.bfloat16), b[0][0], b[1][0].view(torch.bfloat16)))
    rng = np.random.default_rng(7)
    tokens = [[synth.expert_choice(rng, T, E, topk) for _ in range(L)] for _ in range(steps + 1)]
    dev = [[(torch.from_numpy(i).cuda(), torch.from_numpy(r).cuda()) for i, r in tk] for tk in tokens]
    x0 = torch.randn((T, KG), generator=g, device="cuda").to(torch.bfloat16)
    Gb = torch.empty((T * topk, NG), device="cuda")
    Db = [torch.empty((T, ND), device="cuda") for _ in range(2)]
    Hd = torch.empty(2 * DF, device="cuda")
    Yd = torch.empty(DF, device="cuda")
    ws = w4.new_workspace(w4.w4_moe_gemv_ids_workspace_bytes(ND, KD, T, topk, w4.W4_F32_RMS, True, True))
    xd = torch.empty(DF, dtype=torch.float16, device="cuda")
    copy_stream = torch.cuda.Stream()

    def dense_ffn(li, x):
        ga, gs_, da, ds_ = dense[li]
        w4.w4_rms_renorm(x, DF, out=xd)
        w4.w4_gemv(ga[0], gs_, xd, Hd)
        w4.w4_rms_renorm(Hd, DF, out=xd)
        w4.w4_gemv(da, ds_, xd, Yd)

    def new_state():
        """A fresh manager with empty pools of its own."""
        return {"pool": w4.w4_pool_create(L, E, S, part_bytes),
                "pools": [[torch.empty((S, p.shape[1]), dtype=p.dtype, device="cuda") for p in lp] for lp in parts],
                "slots": [torch.full((E,), -1, dtype=torch.int32, device="cuda") for _ in range(L)]}

    def token(k, st=None, overlap=True):
        """One token; st None: every expert resident (direct addressing)."""
        x = x0
        for li in range(L):
            (gc, gs, dc, ds) = layers[li]
            ids_dev, route = dev[k][li]
            kw = {}
            if st is not None:
                # the router's choice is read on the host once the previous
                # layer's output exists (the page's callback on the top-k
                # node): a host wait, then the copies are requested
                pool, pools, slots = st["pool"], st["pools"], st["slots"]
                torch.cuda.current_stream().synchronize()
                w4.w4_pool_prepare(pool, li, tokens[k][li][0], host[li], pools[li], slots[li], copy_stream)
                if not overlap:
                    w4.w4_pool_join(pool, li)
                dense_ffn(li, Db[(li + 1) & 1] if li else torch.zeros(DF, device="cuda"))
                if overlap:
                    w4.w4_pool_join(pool, li)
                gc, gs, dc, ds = (pools[li][0].view(-1, KG // 8), pools[li][1].view(torch.bfloat16).view(-1, KG // 32),
                                  pools[li][2].view(-1, KD // 8), pools[li][3].view(torch.bfloat16).view(-1, KD // 32))
                kw = dict(slot_of=slots[li], n_slots=S)
            else:
                dense_ffn(li, Db[(li + 1) & 1] if li else torch.zeros(DF, device="cuda"))
            w4.w4_moe_gemv_ids(gc, gs, NG * KG // 8, NG * KG // 32, NG, KG, x, ids_dev, n_experts=E, Y=Gb,
                               workspace=ws, **kw)
            w4.w4_moe_gemv_ids(dc, ds, ND * KD // 8, ND * KD // 32, ND, KD, Gb, ids_dev, x_per_pair=True,
                               n_experts=E, route_w=route, Y=Db[li & 1], workspace=ws, **kw)
            if st is not None:
                w4.w4_pool_release(st["pool"], li)
            x = Db[li & 1]
        return x

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # the two managers see the same requests (so the same copies), token by
    # token in alternation; token 0 warms each up
    st_off, st_on = new_state(), new_state()
    token(0, st_off, overlap=False)
    token(0, st_on, overlap=True)
    h0, m0, b0 = w4.w4_pool_stats(st_on["pool"])
    t_off, t_on = [], []
    for k in range(1, steps + 1):
        t_off.append(timed(lambda: token(k, st_off, overlap=False)))
        t_on.append(timed(lambda: token(k, st_on, overlap=True)))
    h1, m1, b1 = w4.w4_pool_stats(st_on["pool"])
    hits, misses, per_tok = (h1 - h0) / steps, (m1 - m0) / steps, (b1 - b0) / steps
    t_res = [timed(lambda k=k: token(k)) for k in range(1, steps + 1)]
    # identity: the last token's output through the pools (as they stand)
    # against direct addressing of the resident experts
    y_on = token(steps, st_on).clone()
    y_off = token(steps).clone()
    torch.cuda.synchronize()
    identical = bool(torch.equal(y_on.view(torch.int32), y_off.view(torch.int32)))
    w4.w4_pool_destroy(st_off["pool"])
    w4.w4_pool_destroy(st_on["pool"])
    # the copy stream alone: pinned host to device, 64 MB copies into scratch
    src = host[0][0].view(-1)[:64 << 20]
    dst = torch.empty(src.numel(), dtype=torch.uint8, device="cuda")
    n = max(1, int(per_tok // src.numel()))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(copy_stream):
        e0.record()
        for _ in range(n):
            dst.copy_(src, non_blocking=True)
        e1.record()
    torch.cuda.synchronize()
    copy_gbps = n * src.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    t_dense = sum(timed(lambda li=li: dense_ffn(li, Db[0])) for li in range(L))
    t_copy = per_tok / (copy_gbps * 1e9)
    med = lambda v: float(np.median(v))
    saved = med([a - b for a, b in zip(t_off, t_on)])
    res = {"us_per_token_overlap_on": round(med(t_on) * 1e6, 1), "us_per_token_overlap_off": round(med(t_off) * 1e6, 1),
           "us_per_token_all_resident": round(med(t_res) * 1e6, 1),
           "tokens_timed_per_mode": steps,
           "expert_bytes_streamed_per_token": int(per_tok),
           "misses_per_token": round(misses, 2), "hits_per_token": round(hits, 2),
           "copy_GBps": round(copy_gbps, 1),
           "overlap_fraction": round(saved / max(1e-9, min(t_copy, t_dense)), 3),
           "us_dense_ffn_per_token": round(t_dense * 1e6, 1),
           "streamed_bitwise_identical_to_resident": identical}
    del host, st_off, st_on, dense
    return res


def extra_gather_per_layer(w4, torch, np, synth, timer, reps: int = 200):
    """Row gather from the per-layer 4-bit table at its own width, 262144 x 8960
    (1.32 GB packed): 64 ids per call, fresh ids each call, in one HIP graph."""
    Vp, Kp, n = 262144, 8960, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    dc, ds = synth.w4_matrix_torch(g, Vp, Kp, "cuda")
    dc, ds = dc.view(Vp, Kp // 8), ds.view(Vp, Kp // 32).view(torch.bfloat16)
    ids = [torch.from_numpy(synth.token_ids(np.random.default_rng(10 + i), n, Vp)).cuda() for i in range(reps)]
    out = torch.empty((n, Kp), dtype=torch.bfloat16, device="cuda")
    t = timer.graph_per_call(lambda i: w4.w4_embed_gather(dc, ds, ids[i % reps], out), reps)
    nbytes = gather_bytes(n, Kp)
    res = {"us_per_call_graph": round(t * 1e6, 3), "bytes_per_call": nbytes,
           "GBps_graph": round(gbps(nbytes, t), 1), "frac_of_peak_graph": round(gbps(nbytes, t) / HBM_PEAK_GBPS, 4)}
    del dc, ds
    torch.cuda.empty_cache()
    return res


def extra_grid_pack(w4, torch, np, synth, timer, reps: int = 20):
    """Grid packing of a 262144 x 1536 bf16 table into codes and steps (805 MB
    read, 226 MB written per call), two table copies rotated."""
    Vt, Kt, copies = 262144, 1536, 2
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    tabs = [(torch.randn((Vt, Kt), generator=g, device="cuda") * 0.03).to(torch.bfloat16) for _ in range(copies)]
    codes = torch.empty((Vt, Kt // 8), dtype=torch.int32, device="cuda")
    steps = torch.empty((Vt, Kt // 32), dtype=torch.bfloat16, device="cuda")
    t = timer.per_call(lambda i: w4.w4_grid_to_codes(tabs[i % copies], codes, steps), reps, warmup=2)
    nbytes = 2 * Vt * Kt + w4_bytes(Vt, Kt)
    res = {"us_per_call": round(t * 1e6, 2), "bytes_per_call": nbytes, "GBps": round(gbps(nbytes, t), 1),
           "frac_of_peak": round(gbps(nbytes, t) / HBM_PEAK_GBPS, 4), "table": "arbitrary bf16 N(0, 0.03)"}
    # a table on a 4-bit grid, as the page's trained tables are: codes uniform
    # in 0..15, one positive step per group with a 5-bit significand (so every
    # (c - 8) * step is a bf16 value), the values exact in bf16
    del tabs
    torch.cuda.empty_cache()
    G = Kt // 32
    tabs = []
    for _ in range(copies):
        c = torch.randint(0, 16, (Vt, Kt), generator=g, device="cuda", dtype=torch.int32)
        e = torch.randint(100, 140, (Vt, G), generator=g, device="cuda", dtype=torch.int32)
        mnt = torch.randint(0, 16, (Vt, G), generator=g, device="cuda", dtype=torch.int32) * 8
        st = ((e * 128 + mnt).to(torch.int16)).view(torch.bfloat16).float()
        tabs.append(((c - 8).float().view(Vt, G, 32) * st.view(Vt, G, 1)).view(Vt, Kt).to(torch.bfloat16))
        del c, e, mnt, st
    t = timer.per_call(lambda i: w4.w4_grid_to_codes(tabs[i % copies], codes, steps), reps, warmup=2)
    res["grid_table"] = {"us_per_call": round(t * 1e6, 2), "GBps": round(gbps(nbytes, t), 1),
                         "frac_of_peak": round(gbps(nbytes, t) / HBM_PEAK_GBPS, 4),
                         "table": "on a 4-bit grid: codes uniform, 5-bit-significand steps"}
    del tabs
    torch.cuda.empty_cache()
    return res


def extra_attention(w4, torch, np, synth, timer, reps: int = 20):
    """Decode attention of one token, 8 query heads over one key/value head of
    width 512: the full 131072-position cache (268 MB of keys and values, two
    copies rotated) and a 512-slot ring (64 copies), each call's two launches
    replayed from a HIP graph (and timed eagerly beside it)."""
    H, D = 8, 512
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    q = torch.randn((H, D), generator=g, device="cuda").to(torch.bfloat16)
    out = {}
    for name, L, copies in (("full_131072", 131072, 2), ("ring_512", 512, 64)):
        ks = [torch.randn((L, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(copies)]
        vs = [torch.randn((L, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(copies)]
        o = torch.empty((H, D), device="cuda")
        ws = w4.new_workspace(w4.w4_decode_attention_workspace_bytes(H, D, L))
        call = lambda i: w4.w4_decode_attention(q, ks[i % copies], vs[i % copies], 0.0442, o,  # noqa: E731
                                                workspace=ws)
        te = timer.per_call(call, reps, warmup=2)
        t = timer.graph_per_call(call, reps)
        nbytes = 2 * L * D * 2
        out[name] = {"us_per_call": round(t * 1e6, 2), "us_per_call_eager": round(te * 1e6, 2), "kv_bytes": nbytes,
                     "GBps": round(gbps(nbytes, t), 1), "frac_of_peak": round(gbps(nbytes, t) / HBM_PEAK_GBPS, 4)}
        del ks, vs
    torch.cuda.empty_cache()
    return out


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak


def extra_prompt(w4, torch, np, synth, timer, reps: int = 64):
    """Prompt-chunk product [256, 1536] x [1536, 24576] on the matrix cores
    (the product the dev.to page quotes in TFLOP/s for 256-token prompt
    chunks): 16 weight copies rotated (340 MB, beyond the 256 MB MALL), bf16
    and fp16 activations; two launches per call (activation and step staging,
    then the product)."""
    M, K, N, copies = 256, 1536, 24576, 16
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    mats = []
    for _ in range(copies):
        c, s = synth.w4_matrix_torch(g, N, K, "cuda")
        mats.append((c.view(N, K // 8), s.view(N, K // 32).view(torch.bfloat16)))
    flops = 2.0 * M * N * K
    out = {"flop_per_call": flops, "weight_copies_rotated": copies}
    ws = w4.new_workspace(w4.w4_gemm_prompt_workspace_bytes(N, K, M))
    for name, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        X = torch.randn((M, K), generator=g, device="cuda").to(dt)
        Y = torch.empty((M, N), device="cuda")
        t = timer.per_call(lambda i: w4.w4_gemm_prompt(mats[i % copies][0], mats[i % copies][1], X, Y,
                                                       workspace=ws), reps, warmup=copies)
        tf = flops / t / 1e12
        out[name] = {"us_per_call": round(t * 1e6, 2), "TFLOPs": round(tf, 1),
                     "frac_of_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
    del mats
    torch.cuda.empty_cache()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="time the CPU oracle on a sample of every configuration and print its JSON")
    ap.add_argument("--no-extra", action="store_true", help="only the vocabulary-head step")
    ap.add_argument("--only", choices=["single", "sweep", "small_m", "moe", "prompt", "gather8960", "grid", "attention"],
                    help="run one secondary workload alone (kernel traces) and print its JSON")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this path runs on one MI355X; see the design notes on sharding)", file=sys.stderr)
        return 2

    import numpy as np

    if args.cpu_baselines:
        import synth
        print(json.dumps({"cpu_baselines": cpu_baselines(np, synth)}), flush=True)
        return 0

    import torch

    import bit_weight_only_02_amd as w4
    import synth

    torch.cuda.set_device(0)
    timer = Timer(torch)
    if args.only:
        run = {"single": extra_single_gemv, "sweep": extra_sweep, "small_m": extra_small_m,
               "moe": extra_moe, "prompt": extra_prompt, "gather8960": extra_gather_per_layer, "grid": extra_grid_pack, "attention": extra_attention}[args.only]
        print(json.dumps({"workload": args.only, "result": run(w4, torch, np, synth, timer)}), flush=True)
        return 0
    rng = np.random.default_rng(0)
    codes, steps = synth.w4_matrix(rng, V, K)
    x = synth.activations(rng, K, synth.BF16)
    ids = synth.token_ids(rng, NIDS, V)

    c0, s0 = dev_matrix(torch, np, codes, steps)
    dcodes = [c0] + [c0.clone() for _ in range(COPIES - 1)]
    dsteps = [s0] + [s0.clone() for _ in range(COPIES - 1)]
    dx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    dids = torch.from_numpy(ids).cuda()
    y = torch.empty(V, dtype=torch.float32, device="cuda")
    gout = torch.empty((NIDS, K), dtype=torch.bfloat16, device="cuda")

    def step(i):
        # the product and the gather of the same table, one launch
        c = i % COPIES
        w4.w4_gemv_gather(dcodes[c], dsteps[c], dx, dids, y, gout)

    def step_two_launches(i):
        c = i % COPIES
        w4.w4_gemv(dcodes[c], dsteps[c], dx, y)
        w4.w4_embed_gather(dcodes[c], dsteps[c], dids, gout)

    # One decode step is replayed as one HIP graph (as the dev.to page does per
    # decode step); one graph per table copy, replayed in rotation.
    side = torch.cuda.Stream()

    def step_graphs(fn):
        gs = []
        for c in range(COPIES):
            fn(c)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    fn(c)
            gs.append(g)
        torch.cuda.synchronize()
        return gs
    # The step is one launch: W untimed steps, then K steps launched back to
    # back on the stream, bracketed by synchronisations (this is also the
    # dominant kernel's duration: a rocprofv3 trace of this command agrees).
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_s = timer.per_call(step, args.steps, warmup=0)
    wall = time.perf_counter() - t0
    # the same step replayed as one HIP graph per step (the page replays a graph
    # per decode step; with one launch it only adds the replay's overhead)
    graphs = step_graphs(step)
    step_graph_s = timer.per_call(lambda i: graphs[i % COPIES].replay(), args.steps, warmup=2)
    # for comparison: the product alone, the gather alone, and the step as two
    # launches in one graph
    gemv_call = lambda i: w4.w4_gemv(dcodes[i % COPIES], dsteps[i % COPIES], dx, y)  # noqa: E731
    gemv_s = timer.per_call(gemv_call, args.steps, warmup=2)
    gemv_graph_s = timer.graph_per_call(gemv_call, args.steps)
    gather_s = timer.graph_per_call(lambda i: w4.w4_embed_gather(dcodes[i % COPIES], dsteps[i % COPIES],
                                                                  dids, gout), args.steps)
    graphs2 = step_graphs(step_two_launches)
    step2_s = timer.per_call(lambda i: graphs2[i % COPIES].replay(), args.steps, warmup=2)
    del graphs2
    ceiling = probe_ceiling(w4, torch)
    achieved = gbps(STEP_BYTES, step_s)
    traffic, kname = measured_traffic()
    result = {
        "metric": "achieved HBM GB/s (% of peak) for W4A16 GEMV; us per 35-layer decode sweep",
        "value": round(gbps(STEP_BYTES, step_s), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; codes uniform 0..15, steps bf16(|N(0,0.02)|+1e-4), x ~ N(0,1))",
        "config": {"workload": "vocabulary-head W4A16 GEMV 262144x1536 (bf16 x, batch 1) + "
                               "4-bit row gather of 64 ids from the same table",
                   "table_copies_rotated": COPIES, "step_bytes": STEP_BYTES},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": (kname or "w4::gemv_kernel") + " (product and gather workgroups, one launch)",
                     "bytes_per_launch": STEP_BYTES,
                     "avg_launch_us": round(step_s * 1e6, 3)},
        "extra": {"ms_per_step_graph": round(step_graph_s * 1e3, 5),
                  "ms_per_step_two_launches_graph": round(step2_s * 1e3, 5),
                  "gemv_alone_us": round(gemv_s * 1e6, 3),
                  "gemv_alone_us_graph": round(gemv_graph_s * 1e6, 3),
                  "gemv_alone_GBps": round(gbps(gemv_bytes(V, K), gemv_s), 2),
                  "gemv_alone_weight_GBps": round(gbps(w4_bytes(V, K), gemv_s), 2),
                  "gather_alone_us_graph": round(gather_s * 1e6, 3),
                  "probe_read_ceiling_GBps": {k: round(v, 1) for k, v in ceiling.items()},
                  "step_frac_of_probe": round(achieved / max(ceiling.values()), 4),
                  "timed_wall_s": round(wall, 4)},
    }
    del dcodes, dsteps, graphs
    torch.cuda.empty_cache()
    if not args.no_extra:
        ex = result["extra"]
        ex["single_gemv_2048x1536_f16"] = extra_single_gemv(w4, torch, np, synth, timer)
        ex["decode_sweep_35_layers"] = extra_sweep(w4, torch, np, synth, timer)
        ex["small_m_sweep_shapes_bf16"] = extra_small_m(w4, torch, np, synth, timer)
        ex["moe_30_layers_top8_of_128"] = extra_moe(w4, torch, np, synth, timer)
        ex["prompt_chunk_256x1536x24576"] = extra_prompt(w4, torch, np, synth, timer)
        ex["gather_per_layer_table_262144x8960"] = extra_gather_per_layer(w4, torch, np, synth, timer)
        ex["grid_pack_262144x1536"] = extra_grid_pack(w4, torch, np, synth, timer)
        ex["decode_attention_8x512"] = extra_attention(w4, torch, np, synth, timer)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(codes, steps, x, ids)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
