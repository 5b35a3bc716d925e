"""Benchmark of y = x . dequant(W) on one MI355X.

A step is one pass of the whole product path over one batch: the LLaMA-7B
decode layer set (fused QKV 4096x12288, o_proj 4096x4096, fused gate+up
4096x22016, down 11008x4096), int4 with fp16 zero-points, group 128, fp16
activations, M = 1, each layer through wq_gemv.  The headline value is the
weight bytes (codes + scales + zero-points) streamed per second.

Weights are resident in HBM before timing starts.  Each step uses the next of
R distinct copies of the layer set (R * 107.5 MB > 1 GiB), so the 256 MB
last-level cache cannot serve a step from an earlier one: every step streams
its weights from HBM, as a multi-layer decode does.  The R steps of one
rotation are captured once in a HIP graph (through torch.cuda.CUDAGraph) and
replayed, so host-side launch cost does not starve the GPU; the eager
(launch-by-launch) rate is reported beside it.

Also reported:
  decode_other_m the same layer set at M = 4 and 16 (graph-replayed);
  other_m1_layers  the single 4096 x 4096 layer and the largest (405B-width)
                layer at M = 1, against HBM peak and the streaming-read ceiling;
  roofline      the dominant kernel (the gate+up GEMV, the largest layer)
                against HBM bandwidth: its launches back to back over the
                rotated copies, captured in a HIP graph and timed between HIP
                events on its stream;
  gemm          the prefill layer set at M = 2048 (symmetric int4, group -1 and
                128) through wq_gemm, as TFLOP/s against dense fp16 MFMA peak
                (each layer's launches graph-replayed; eager steps beside it);
  fused_gate_up the gate+up layer at M = 1 and 2048: plain product, plain
                product + torch SiLU/multiply, and the fused SiLU(gate)*up
                entry points;
  hadamard      the online rotation of the activations alone and followed by
                the product, on the QKV layer at M = 1 and 2048;
  fine_zero_groups  2-bit layers with per-column scales and a zero-point per
                8 rows, decode layer set shapes at M = 1 and 2048;
  layer_stack   tokens per second through 32 LLaMA-7B-shaped decoder layers
                (quantised products vs dense fp16 torch matmuls on weights
                dequantised at load time), one HIP graph per token;
  cpu_baseline  the CPU oracle on a bounded sample of the same step.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s
METRIC = "weight GB/s (GEMV, M=1) & TFLOP/s (GEMM, M=2048) as % of HBM/MFMA roofline"
KERNEL_SOURCES = ["wq_gemv.hip", "wq_decode.hpp", "wq_layout.hpp"]  # the dominant (GEMV) kernel's sources
ALL_SOURCES = ["wq_api.hip", "wq_common.hpp", "wq_decode.hpp", "wq_gemm.hip", "wq_gemv.hip", "wq_hadamard.hip",
               "wq_layout.hpp"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--gemm-steps", type=int, default=20)
    p.add_argument("--no-gemm", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-fused", action="store_true")
    p.add_argument("--no-hadamard", action="store_true")
    p.add_argument("--no-fine", action="store_true")
    p.add_argument("--stack-layers", type=int, default=32,
                   help="decoder layers in the token-by-token stack benchmark (0: skip it)")
    p.add_argument("--stack-tokens", type=int, default=50)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain device copy of known size (counter calibration)")
    p.add_argument("--points", action="store_true",
                   help="instead of the step: time every configuration point (all shapes, M, bits and "
                        "groups of the workloads) against its roofline, plus context numbers")
    p.add_argument("--points-configs", default="1,2,3,4,5,6",
                   help="configurations for --points (comma-separated ids)")
    p.add_argument("--points-only", nargs="*", default=[],
                   help="restrict --points to cases cid/layer/bits/M-list ('*' matches any), "
                        "e.g. 5/wide/4/1,2 4/up/*/1")
    p.add_argument("--no-read-ceiling", action="store_true",
                   help="--points: skip the streaming-read ceiling of each M=1 point")
    p.add_argument("--profile-case", nargs="*", default=[],
                   help="instead of the step: launch only these products back to back, each "
                        "cid/layer/bits/group/M (e.g. 5/wide/4/32/1), for rocprofv3 runs; 'copy' "
                        "adds a 256 MiB device copy (counter calibration)")
    p.add_argument("--profile-reps", type=int, default=40)
    return p.parse_args()


def kernel_hash(files=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "weight_only_quantized_w4a16_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(khash):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "gemv_gate_up_m1_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != khash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Dev:
    """Moves seeded workload arrays to cuda:0 and repacks layers (no timing)."""

    def __init__(self):
        import torch

        import weight_only_quantized_w4a16_amd as wq

        self.torch, self.wq = torch, wq
        self.dev = torch.device("cuda:0")

    def t(self, a, dtype):
        import numpy as np
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return self.torch.from_numpy(a.view(np.int16)).view(dtype).to(self.dev)
        return self.torch.from_numpy(a.view(np.int32)).to(self.dev)

    def repack(self, L, copies=1, fn=None):
        import workloads as wl
        torch, wq = self.torch, self.wq
        fn = fn or wq.wq_repack
        q = self.t(L.qweight, torch.int32)
        sc = self.t(L.scales, torch.float16)
        z = None
        if L.mode == wl.ZERO_F16 or L.mode in wl.FINE_ZERO_GROUP:
            z = self.t(L.zeros, torch.float16)
        elif L.mode == wl.ZERO_PACKED:
            z = self.t(L.zeros, torch.int32)
        lut = self.t(L.lut, torch.float16) if L.lut is not None else None
        out = [fn(q, sc, z, L.mode, L.g_idx, L.K, L.N, L.bits, L.group_size, lut=lut) for _ in range(copies)]
        del q, sc, z
        return out


WARM_MS = 100.0  # GPU time spent on the measured work itself before any timing


def warm_up(stream, replay, ms=WARM_MS):
    """Run replay() (work on `stream`) until `ms` milliseconds of GPU time have
    passed.  The GPU's clocks ramp up over tens of milliseconds after an idle
    spell (host-side set-up, repacking): without this the first point timed
    after a set-up measured up to 25 % slower than the same point timed later
    in the same process."""
    import torch
    spent = 0.0
    while spent < ms:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        replay()
        e1.record(stream)
        torch.cuda.synchronize()
        spent += max(e0.elapsed_time(e1), 0.01)


def graph_time(stream, fn, n, replays=5):
    """fn(i) launches call i on `stream`; n calls captured in one HIP graph;
    after warm_up(), the median over `replays` replays of the GPU time per
    call, in us."""
    import statistics

    import torch
    with torch.cuda.stream(stream):
        for i in range(n):
            fn(i)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
    torch.cuda.synchronize()

    def replay():
        with torch.cuda.stream(stream):
            g.replay()
    warm_up(stream, replay)
    ts = []
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / n * 1e3)
    del g
    return statistics.median(ts)


_probe = None


def probe_lib():
    """libwq_probe.so (the streaming-read probe, include/wq_probe.h)."""
    global _probe
    if _probe is None:
        import ctypes

        from weight_only_quantized_w4a16_amd import build as wq_build
        if not os.path.exists(wq_build.PROBE_LIB):
            raise RuntimeError(f"{wq_build.PROBE_LIB} is not built")
        L = ctypes.CDLL(wq_build.PROBE_LIB)
        L.wq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p]
        L.wq_probe_stream_read.restype = ctypes.c_int
        _probe = L
    return _probe


def read_ceiling(stream, bufs, nbytes, n):
    """The fastest one launch reads `nbytes` bytes: the streaming-read probe
    over the rotated buffers `bufs` (same protocol as the product: n launches
    per graph replay, median of 5), best over a sweep of workgroup counts and
    loads in flight.  Returns (us per launch, GB/s, best launch shape)."""
    import torch
    L = probe_lib()
    nbytes = nbytes // 16 * 16
    sink = torch.zeros(4, dtype=torch.uint8, device=bufs[0].device)
    best = None
    for wgs in (512, 1024, 2048, 4096, 8192):
        for u in (4, 8):
            def call(i):
                rc = L.wq_probe_stream_read(bufs[i % len(bufs)].data_ptr(), nbytes, wgs, u, sink.data_ptr(),
                                            stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"wq_probe_stream_read failed ({rc})")
            us = graph_time(stream, call, n)
            if best is None or us < best[0]:
                best = (us, wgs, u)
    us, wgs, u = best
    return us, nbytes / us / 1e3, {"workgroups": wgs, "loads_in_flight": u}


def run_profile_cases(args):
    """Only the named products (and an optional device copy of known size),
    each warmed up (warm_up) and then launched --profile-reps times back to
    back over rotated copies of its layer: the workload of the committed
    rocprofv3 summaries, one process per counter pass, so every dispatch of a
    kernel in the run belongs to one case (the summaries keep the last
    --profile-reps dispatches of each kernel)."""
    import torch

    import workloads as wl
    d = Dev()
    wq = d.wq
    wq.lib()
    torch.cuda.set_device(d.dev)
    stream = torch.cuda.current_stream()
    for spec in args.profile_case:
        if spec == "copy":
            src = torch.empty(1 << 28, dtype=torch.uint8, device=d.dev).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(5):
                dst.copy_(src)
            torch.cuda.synchronize()
            print(json.dumps({"case": "copy", "bytes": 1 << 28, "calls": 5}), flush=True)
            del src, dst
            continue
        cid, lname, bits, gs, M = spec.split("/")
        cfg = wl.CONFIGS[int(cid)]
        L = cfg.layer(lname, int(bits), int(gs))
        M = int(M)
        wb = L.weight_bytes()
        R = max(2, -(-(1 << 30) // wb))
        copies = d.repack(L, R)
        tdt = torch.float16 if cfg.dtype == wl.F16 else torch.bfloat16
        x = d.t(cfg.x(M, L.K), tdt)
        y = torch.empty((M, L.N), dtype=tdt, device=d.dev)
        ws = torch.empty(max(wq.wq_workspace_bytes(M, L.N, L.K, L.bits, copies[0].perm is not None), 16),
                         dtype=torch.uint8, device=d.dev)
        for i in range(R):
            wq.linear(x, copies[i], out=y, ws=ws, stream=stream)
        torch.cuda.synchronize()
        # clocks up first; the summaries keep the last --profile-reps dispatches
        warm_up(stream, lambda: [wq.linear(x, copies[i], out=y, ws=ws, stream=stream) for i in range(R)])
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.profile_reps):
            wq.linear(x, copies[i % R], out=y, ws=ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        print(json.dumps({"case": spec, "path": "gemv" if wq.use_gemv(M, copies[0]) else "gemm",
                          "calls": args.profile_reps, "rotated_copies": R, "weight_bytes": wb,
                          "us_per_call_event_timed": round(e0.elapsed_time(e1) / args.profile_reps * 1e3, 3)}),
              flush=True)
        del copies, x, y, ws
        torch.cuda.empty_cache()


def _match(spec, cid, lname, bits, M):
    f = spec.split("/") + ["*"] * 4
    return ((f[0] in ("*", str(cid))) and (f[1] in ("*", lname)) and (f[2] in ("*", str(bits)))
            and (f[3] == "*" or str(M) in f[3].split(",")))


def run_points(args):
    """Every configuration point (layer shape x M x code width x group) through
    the product entry point a caller uses (linear(): the GEMV for decode-sized M,
    the GEMM above), timed as back-to-back launches over R rotated copies of the
    layer (R x weight bytes > 1 GiB) captured in a HIP graph and replayed; the
    median of 5 replays.  Each point is set against t_ideal = max(algorithmic
    bytes / 8 TB/s, 2MNK / 2.5 PFLOP/s), and each M = 1 point against the
    streaming-read ceiling of its weight bytes (the probe kernel reading the
    same rotated buffers under the same protocol).  Context: single-call latency
    with a cold last-level cache (512 MB written in between), torch's own
    streaming read and copy over 2 GiB, and torch.matmul in fp16 on weights
    dequantised at load time (wq_dequant_debug) at the prefill shapes."""
    import statistics

    import torch

    import workloads as wl

    d = Dev()
    wq = d.wq
    wq.lib()
    dev = d.dev
    torch.cuda.set_device(dev)
    s = torch.cuda.Stream()

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    points, cold = [], []
    want = {int(c) for c in args.points_configs.split(",")}
    only = args.points_only
    for cid, cfg in wl.CONFIGS.items():
        if cid not in want:
            continue
        tdt = torch.float16 if cfg.dtype == wl.F16 else torch.bfloat16
        for (lname, K, N) in cfg.layers:
            for bits in cfg.bits:
                Ms = [M for M in cfg.Ms if not only or any(_match(sp, cid, lname, bits, M) for sp in only)]
                if not Ms:
                    continue
                for gs in cfg.groups:
                    L = cfg.layer(lname, bits, gs)
                    wb = L.weight_bytes()
                    R = max(2, -(-(1 << 30) // wb))
                    copies = d.repack(L, R)
                    n = R * max(1, -(-8 // R))
                    ceiling = None
                    if 1 in Ms and not args.no_read_ceiling:
                        nbytes = min(wb, copies[0].packed.numel())
                        r_us, r_gbs, shape = read_ceiling(s, [c.packed for c in copies], nbytes, n)
                        ceiling = {"read_us": round(r_us, 2), "read_GBps": round(r_gbs, 1), "bytes": nbytes,
                                   "shape": shape}
                    for M in Ms:
                        x = d.t(cfg.x(M, K), tdt)
                        y = torch.empty((M, N), dtype=tdt, device=dev)
                        has_perm = copies[0].perm is not None
                        ws = torch.empty(max(wq.wq_workspace_bytes(M, N, K, bits, has_perm), 16),
                                         dtype=torch.uint8, device=dev)
                        path = "gemv" if wq.use_gemv(M, copies[0]) else "gemm"
                        us = graph_time(s, lambda i: wq.linear(x, copies[i % R], out=y, ws=ws, stream=s), n)
                        flops = 2.0 * M * N * K
                        alg = wb + 2 * M * K + 2 * M * N + (4 * K if has_perm else 0)
                        t_ideal = max(alg / (HBM_PEAK_GBS * 1e3), flops / (MFMA_F16_PEAK_TFLOPS * 1e6))
                        pt = {"config": cfg.name, "layer": f"{lname} {K}x{N}", "bits": bits, "group": gs, "M": M,
                              "path": path, "us": round(us, 2), "weight_GBps": round(wb / us / 1e3, 1),
                              "tflops": round(flops / us / 1e6, 1), "t_ideal_us": round(t_ideal, 2),
                              "frac_of_ideal": round(t_ideal / us, 3)}
                        if M == 1 and ceiling is not None:
                            pt["read_ceiling"] = ceiling
                            pt["frac_of_read_ceiling"] = round(ceiling["read_us"] / us, 3)
                        points.append(pt)
                        print(f"[points] {points[-1]}", file=sys.stderr, flush=True)
                        if M == 1 and cid in (1, 2):
                            # one call after 512 MB of writes (the last-level cache holds none of it)
                            ts = []
                            for r in range(5):
                                with torch.cuda.stream(s):
                                    scratch.fill_(r)
                                e0 = torch.cuda.Event(enable_timing=True)
                                e1 = torch.cuda.Event(enable_timing=True)
                                e0.record(s)
                                wq.linear(x, copies[r % R], out=y, ws=ws, stream=s)
                                e1.record(s)
                                torch.cuda.synchronize()
                                ts.append(e0.elapsed_time(e1) * 1e3)
                            cold.append({"config": cfg.name, "layer": f"{lname} {K}x{N}", "M": 1,
                                         "us": round(statistics.median(ts), 2)})
                        del x, y, ws
                    del copies
                    torch.cuda.empty_cache()
    del scratch
    ctx = {}
    if not only:
        # torch's own streaming kernels over 2 GiB (context for what a read can reach)
        big = torch.empty(1 << 31, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(big)
        v = big.view(torch.float32)  # 0x01010101: a normal float
        read_us = graph_time(s, lambda i: v.sum(), 4)
        copy_us = graph_time(s, lambda i: dst.copy_(big), 4)
        probe_us, probe_gbs, shape = read_ceiling(s, [big], 1 << 31, 4)
        del big, dst, v
        torch.cuda.empty_cache()
        ctx = {"bytes": 1 << 31, "torch_f32_sum_read_GBps": round((1 << 31) / read_us / 1e3, 1),
               "torch_copy_read_plus_write_GBps": round(2 * (1 << 31) / copy_us / 1e3, 1),
               "probe_read_GBps": round(probe_gbs, 1), "probe_shape": shape}
    # dense fp16 comparator: torch.matmul on weights dequantised at load time
    dense = []
    if 3 in want and not only:
        c3 = wl.CONFIGS[3]
        for (lname, K, N) in c3.layers:
            layer = d.repack(c3.layer(lname, 4, -1))[0]
            W = wq.wq_dequant_debug(layer, torch.float16)
            del layer
            for M in c3.Ms:
                x = d.t(c3.x(M, K), torch.float16)
                y = torch.empty((M, N), dtype=torch.float16, device=dev)
                us = graph_time(s, lambda i: torch.matmul(x, W, out=y), 4)
                dense.append({"layer": f"{lname} {K}x{N}", "M": M, "us": round(us, 2),
                              "tflops": round(2.0 * M * N * K / us / 1e6, 1)})
            del W
            torch.cuda.empty_cache()
    print(json.dumps({"points": points, "cold_single_call": cold, "stream_2GiB": ctx,
                      "dense_fp16_torch_matmul": dense}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the product path runs on a single GPU (asked for "
              f"--gpus {args.gpus}); how it would shard over several is a design note only.",
              file=sys.stderr)
        sys.exit(2)
    if args.points:
        run_points(args)
        return
    if args.profile_case:
        run_profile_cases(args)
        return

    import numpy as np
    import torch

    import weight_only_quantized_w4a16_amd as wq
    import workloads as wl

    if not os.path.exists(wq.LIB_PATH):
        from weight_only_quantized_w4a16_amd import build as wq_build
        wq_build.build()
    wq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def to_dev(a, dtype):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(dtype).to(dev)
        return torch.from_numpy(a.view(np.int32)).to(dev)

    def repack_copies(L, copies, repack=None):
        repack = repack or wq.wq_repack
        q = to_dev(L.qweight, torch.int32)
        s = to_dev(L.scales, torch.float16)
        z = None
        if L.mode == wl.ZERO_F16 or L.mode in wl.FINE_ZERO_GROUP:
            z = to_dev(L.zeros, torch.float16)
        elif L.mode == wl.ZERO_PACKED:
            z = to_dev(L.zeros, torch.int32)
        lut = to_dev(L.lut, torch.float16) if L.lut is not None else None
        out = [repack(q, s, z, L.mode, L.g_idx, L.K, L.N, L.bits, L.group_size, lut=lut)
               for _ in range(copies)]
        del q, s, z
        return out

    # ---------------- decode layer set (the step) ----------------
    cfg = wl.CONFIGS[2]
    M = 1
    layers = [cfg.layer(name) for (name, _, _) in cfg.layers]
    set_bytes = sum(L.weight_bytes() for L in layers)
    R = max(2, -(-(1 << 30) // set_bytes))
    packed = [repack_copies(L, R) for L in layers]
    xs = [to_dev(cfg.x(M, L.K), torch.float16) for L in layers]
    ys = [torch.empty((M, L.N), dtype=torch.float16, device=dev) for L in layers]
    torch.cuda.synchronize()

    def step(i, events=None):
        r = i % R
        for j, L in enumerate(layers):
            if events is not None:
                events[j][0].record(stream)
            wq.wq_gemv(xs[j], packed[j][r], out=ys[j], stream=stream)
            if events is not None:
                events[j][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    warm_up(stream, lambda: [step(i) for i in range(R)])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms_per_step = e0.elapsed_time(e1) / args.steps

    # One rotation (R steps) captured as a graph; the timed region replays it.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(R):
                for j in range(len(layers)):
                    wq.wq_gemv(xs[j], packed[j][i], out=ys[j], stream=cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    replays = max(1, -(-args.steps // R))
    for _ in range(max(1, args.warmup // R)):
        graph.replay()
    torch.cuda.synchronize()
    warm_up(stream, graph.replay)
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    timed_steps = replays * R
    ms_per_step = e0.elapsed_time(e1) / timed_steps
    value = set_bytes / (ms_per_step * 1e-3) / 1e9

    # per-kernel breakdown: HIP events around every launch (informational; an
    # event pair adds its own gap to each launch)
    nev = min(args.steps, 100)
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in layers] for _ in range(nev)]
    for i in range(nev):
        step(i, evs[i])
    torch.cuda.synchronize()
    kernel_us = []
    for j, L in enumerate(layers):
        t = sum(evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(nev)) / nev * 1e3
        kernel_us.append(t)
    dom = int(np.argmax([L.weight_bytes() for L in layers]))
    Ld = layers[dom]

    # dominant kernel (the largest layer): nd launches back to back over the
    # rotated copies, captured in a HIP graph on stream s1 and replayed between
    # two HIP events recorded on s1 -> average launch time (median of 5 replays)
    nd = max(args.steps, 4 * R)
    s1 = torch.cuda.Stream()
    dom_us = graph_time(s1, lambda i: wq.wq_gemv(xs[dom], packed[dom][i % R], out=ys[dom], stream=s1), nd)
    alg_bytes = Ld.weight_bytes() + 2 * M * Ld.K + 2 * M * Ld.N
    achieved = alg_bytes / (dom_us * 1e-6) / 1e9
    khash = kernel_hash()
    traffic = read_traffic(khash)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": f"wq_gemv {Ld.name} M={M}", "algorithmic_bytes_per_launch": alg_bytes,
                "avg_launch_us": round(dom_us, 3), "launches_timed": nd}
    # the same layer set at the other decode batch sizes of the configuration
    decode_m = {}
    for Mx in (4, 16):
        xm = [to_dev(cfg.x(Mx, L.K), torch.float16) for L in layers]
        ym = [torch.empty((Mx, L.N), dtype=torch.float16, device=dev) for L in layers]
        gm = torch.cuda.CUDAGraph()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for i in range(R):
                for j in range(len(layers)):
                    wq.wq_gemv(xm[j], packed[j][i], out=ym[j], stream=cap)
            with torch.cuda.graph(gm, stream=cap):
                for i in range(R):
                    for j in range(len(layers)):
                        wq.wq_gemv(xm[j], packed[j][i], out=ym[j], stream=cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        gm.replay()
        torch.cuda.synchronize()
        warm_up(stream, gm.replay)
        e0.record(stream)
        for _ in range(replays):
            gm.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (replays * R)
        decode_m[f"M{Mx}"] = {"ms_per_step": round(ms, 5), "weight_GBps": round(set_bytes / (ms * 1e-3) / 1e9, 1)}
        del gm, xm, ym
    per_kernel = {L.name.split("/")[-1]: {"us_with_events": round(t, 3),
                                          "weight_GBps": round(L.weight_bytes() / (t * 1e-6) / 1e9, 1)}
                  for L, t in zip(layers, kernel_us)}
    del packed, xs, ys
    torch.cuda.empty_cache()

    # ---------------- the other M = 1 layers of the workloads ----------------
    # The single 4096 x 4096 layer (c1: int4 symmetric, group 128, fp16) and
    # the largest layer (c5: the 405B-width 16384 x 53248 act-order layer,
    # bf16, packed zero-points, group 32), each through wq_gemv launched back
    # to back over rotated copies in a HIP graph, against HBM peak and against
    # the streaming-read ceiling of the same bytes (the probe kernel reading the
    # same buffers under the same protocol).
    extra_m1 = {}
    s2 = torch.cuda.Stream()
    for key, cid, lname in (("c1_4096x4096", 1, "layer"), ("c5_wide_16384x53248", 5, "wide")):
        cx = wl.CONFIGS[cid]
        Lx = cx.layer(lname)
        wbx = Lx.weight_bytes()
        Rx = max(2, -(-(1 << 30) // wbx))
        cps = repack_copies(Lx, Rx)
        tdt = torch.float16 if cx.dtype == wl.F16 else torch.bfloat16
        xx = to_dev(cx.x(1, Lx.K), tdt)
        yx = torch.empty((1, Lx.N), dtype=tdt, device=dev)
        has_perm = cps[0].perm is not None
        wsx = torch.empty(max(wq.wq_workspace_bytes(1, Lx.N, Lx.K, Lx.bits, has_perm), 16), dtype=torch.uint8,
                          device=dev)
        nx = Rx * max(1, -(-8 // Rx))
        us = graph_time(s2, lambda i: wq.wq_gemv(xx, cps[i % Rx], out=yx, ws=wsx, stream=s2), nx, replays=7)
        r_us, _, shape = read_ceiling(s2, [c.packed for c in cps], min(wbx, cps[0].packed.numel()), nx)
        algx = wbx + 2 * Lx.K + 2 * Lx.N + (4 * Lx.K if has_perm else 0)
        extra_m1[key] = {"config": cx.name, "layer": f"{lname} {Lx.K}x{Lx.N}", "M": 1, "bits": Lx.bits,
                         "group": Lx.group_size, "us": round(us, 2), "weight_GBps": round(wbx / us / 1e3, 1),
                         "algorithmic_bytes": algx, "frac_of_hbm_peak": round(algx / us / 1e3 / HBM_PEAK_GBS, 4),
                         "read_ceiling_us": round(r_us, 2), "frac_of_read_ceiling": round(r_us / us, 3),
                         "rotated_copies": Rx}
        del cps, xx, yx, wsx
        torch.cuda.empty_cache()

    # ---------------- prefill GEMM at M = 2048 ----------------
    gemm = None
    if not args.no_gemm:
        c3 = wl.CONFIGS[3]
        Mg = 2048
        gemm = {}
        for gs in (-1, 128):
            gl = [c3.layer(name, 4, gs) for (name, _, _) in c3.layers]
            gp = [repack_copies(L, 2) for L in gl]
            gx = [to_dev(c3.x(Mg, L.K), torch.float16) for L in gl]
            gy = [torch.empty((Mg, L.N), dtype=torch.float16, device=dev) for L in gl]
            flops = sum(2.0 * Mg * L.N * L.K for L in gl)

            def gstep(i):
                for j in range(len(gl)):
                    wq.wq_gemm(gx[j], gp[j][i % 2], out=gy[j], stream=stream)

            for i in range(3):
                gstep(i)
            torch.cuda.synchronize()
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for i in range(args.gemm_steps):
                gstep(i)
            a1.record(stream)
            torch.cuda.synchronize()
            eager_ms = a0.elapsed_time(a1) / args.gemm_steps
            # each layer's launches (alternating copies) captured in a graph and
            # replayed: GPU time per launch, median of 5 replays
            layer_us = []
            for j in range(len(gl)):
                n = 2 * max(1, args.gemm_steps // 2)
                gg = torch.cuda.CUDAGraph()
                cap.wait_stream(stream)
                with torch.cuda.stream(cap):
                    with torch.cuda.graph(gg, stream=cap):
                        for i in range(n):
                            wq.wq_gemm(gx[j], gp[j][i % 2], out=gy[j], stream=cap)
                    gg.replay()
                stream.wait_stream(cap)
                torch.cuda.synchronize()

                def gg_replay():
                    with torch.cuda.stream(cap):
                        gg.replay()
                warm_up(cap, gg_replay)
                ts = []
                for _ in range(5):
                    with torch.cuda.stream(cap):
                        a0.record(cap)
                        gg.replay()
                        a1.record(cap)
                    torch.cuda.synchronize()
                    ts.append(a0.elapsed_time(a1) / n * 1e3)
                layer_us.append(sorted(ts)[2])
                del gg
            gms = sum(layer_us) * 1e-3
            tflops = flops / (gms * 1e-3) / 1e12
            gemm[f"group_{gs}"] = {
                "M": Mg, "ms_per_step": round(gms, 4), "tflops": round(tflops, 1),
                "peak_tflops": MFMA_F16_PEAK_TFLOPS, "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                "eager_ms_per_step": round(eager_ms, 4),
                "per_layer_tflops": {L.name.split("/")[-1]: round(2.0 * Mg * L.N * L.K / (layer_us[j] * 1e-6) / 1e12, 1)
                                     for j, L in enumerate(gl)}}
            del gp, gx, gy
            torch.cuda.empty_cache()

    # ---------------- activation-fused gate+up ----------------
    # The gate+up layer three ways, each over rotated copies, launches back to
    # back between events: the plain product (y = [gate | up], no activation),
    # the plain product followed by torch's SiLU and multiply (two more
    # launches, y written and read back), and the fused product writing
    # h = SiLU(gate) * up.
    fused = None
    if not args.no_fused:
        Lg = cfg.layer("gate_up")
        I = Lg.N // 2
        Rg = max(2, -(-(1 << 30) // Lg.weight_bytes()))
        fused = {"layer": f"gate_up {Lg.K}x{Lg.N}", "rotated_copies": Rg}
        sg = torch.cuda.Stream()
        plain = repack_copies(Lg, Rg)
        fpack = repack_copies(Lg, Rg, wq.wq_repack_gate_up)
        for Mf, fn, ffn in ((1, wq.wq_gemv, wq.wq_gemv_gate_up), (2048, wq.wq_gemm, wq.wq_gemm_gate_up)):
            xf = to_dev(cfg.x(Mf, Lg.K), torch.float16)
            yf = torch.empty((Mf, Lg.N), dtype=torch.float16, device=dev)
            hf = torch.empty((Mf, I), dtype=torch.float16, device=dev)
            n = max(4 * Rg, 40) if Mf == 1 else 2 * Rg

            def plain_call(i):
                fn(xf, plain[i % Rg], out=yf, stream=sg)

            def unfused_call(i):
                fn(xf, plain[i % Rg], out=yf, stream=sg)
                torch.mul(torch.nn.functional.silu(yf[:, :I]), yf[:, I:], out=hf)

            def fused_call(i):
                ffn(xf, fpack[i % Rg], out=hf, stream=sg)

            res = {}
            for name, call in (("plain_us", plain_call), ("unfused_torch_silu_us", unfused_call),
                               ("fused_us", fused_call)):
                res[name] = round(graph_time(sg, call, n), 3)
            if Mf == 1:
                res["fused_weight_GBps"] = round(Lg.weight_bytes() / (res["fused_us"] * 1e-6) / 1e9, 1)
            else:
                res["fused_tflops"] = round(2.0 * Mf * Lg.N * Lg.K / (res["fused_us"] * 1e-6) / 1e12, 1)
            fused[f"M{Mf}"] = res
            del xf, yf, hf
        del plain, fpack
        torch.cuda.empty_cache()

    # ---------------- online Hadamard rotation ----------------
    # The rotation alone (2 * M * K bytes moved) and the rotated product
    # (rotation, then the plain product on the rotated rows) against the plain
    # product, on the QKV layer (K = 4096, block 128), launches back to back.
    had = None
    if not args.no_hadamard:
        Lq = cfg.layer("qkv")
        Rq = max(2, -(-(1 << 30) // Lq.weight_bytes()))
        qp = repack_copies(Lq, Rq)
        had = {"layer": f"qkv {Lq.K}x{Lq.N}", "block": 128, "rotated_copies": Rq}
        sh = torch.cuda.Stream()
        for Mh, fn in ((1, wq.wq_gemv), (2048, wq.wq_gemm)):
            xh = to_dev(cfg.x(Mh, Lq.K), torch.float16)
            xr = torch.empty_like(xh)
            yh = torch.empty((Mh, Lq.N), dtype=torch.float16, device=dev)
            n = max(4 * Rq, 40) if Mh == 1 else 2 * Rq

            def rot(i):
                wq.wq_hadamard(xh, 128, out=xr, stream=sh)

            def prod(i):
                fn(xh, qp[i % Rq], out=yh, stream=sh)

            def rot_prod(i):
                wq.wq_hadamard(xh, 128, out=xr, stream=sh)
                fn(xr, qp[i % Rq], out=yh, stream=sh)

            res = {}
            for name, call in (("rotate_us", rot), ("product_us", prod), ("rotate_then_product_us", rot_prod)):
                res[name] = round(graph_time(sh, call, n), 3)
            res["rotate_GBps"] = round(4.0 * Mh * Lq.K / (res["rotate_us"] * 1e-6) / 1e9, 1)
            had[f"M{Mh}"] = res
            del xh, xr, yh
        del qp
        torch.cuda.empty_cache()

    # ---------------- zero-points with their own group ----------------
    # 2-bit codes, one scale per column and an fp16 zero-point every 8 rows
    # (the zero-point granularity experiment of the Marlin zero-point issue),
    # on the decode layer set's shapes: each layer at M = 1 (weight GB/s) and
    # M = 2048 (TFLOP/s), launches back to back over rotated copies.
    fine = None
    if not args.no_fine:
        fine = {"bits": 2, "group_size": -1, "zero_group": 8, "layers": {}}
        sfz = torch.cuda.Stream()
        for (name, K, N) in wl.LLAMA7B:
            Lf = wl.make_layer(K, N, 2, -1, wl.ZERO_F16_G8, 8100 + K + N, scale_range=(0.002, 0.01),
                               name=f"fine/{name}")
            Rf = max(2, -(-(1 << 30) // Lf.weight_bytes()))
            fp = repack_copies(Lf, Rf)
            res = {"weight_bytes": Lf.weight_bytes()}
            for Mf, fn in ((1, wq.wq_gemv), (2048, wq.wq_gemm)):
                xf = to_dev(wl.make_x(Mf, K, wl.F16, 5), torch.float16)
                yf = torch.empty((Mf, N), dtype=torch.float16, device=dev)
                n = max(4 * Rf, 40) if Mf == 1 else Rf
                us = graph_time(sfz, lambda i: fn(xf, fp[i % Rf], out=yf, stream=sfz), n)
                if Mf == 1:
                    res["M1_us"] = round(us, 3)
                    res["M1_weight_GBps"] = round(Lf.weight_bytes() / (us * 1e-6) / 1e9, 1)
                else:
                    res["M2048_us"] = round(us, 1)
                    res["M2048_tflops"] = round(2.0 * Mf * N * K / (us * 1e-6) / 1e12, 1)
                del xf, yf
            fine["layers"][name] = res
            del fp
        torch.cuda.empty_cache()

    # ---------------- decode layer stack (tokens per second) ----------------
    # A token through L LLaMA-7B-shaped decoder layers (fused QKV, o_proj,
    # activation-fused gate+up, down; every layer its own weights, 107.5 MB
    # per layer), captured as one HIP graph per token, against the same chain
    # on weights dequantised at load time to dense fp16 and multiplied by
    # torch (the exllama discussion's "dequantise at load" comparator).
    stack = None
    if args.stack_layers > 0:
        from weight_only_quantized_w4a16_amd.stack import DecodeStack, DecoderWeights
        nl = args.stack_layers
        t_setup = time.perf_counter()
        dec, dense = [], []
        qbytes = 0
        for li in range(nl):
            ws = {}
            dw = {}
            for (name, _, _) in wl.LLAMA7B:
                L = wl.stack_layer(li, name)
                qbytes += L.weight_bytes()
                pl = repack_copies(L, 1)[0]
                dw[name] = wq.wq_dequant_debug(pl, torch.float16)
                if name == "gate_up":
                    pl = repack_copies(L, 1, wq.wq_repack_gate_up)[0]
                ws[name] = pl
            dec.append(DecoderWeights(ws["qkv"], ws["o_proj"], ws["gate_up"], ws["down"]))
            dense.append(dw)
        torch.cuda.synchronize()
        setup_s = time.perf_counter() - t_setup
        Ms = 1
        st = DecodeStack(dec, Ms, torch.float16, dev)
        dim, inter = st.dim, st.inter
        x0 = to_dev(wl.make_x(Ms, dim, wl.F16, 4242), torch.float16)

        def dense_step(x):
            for dw in dense:
                qkv = torch.matmul(x, dw["qkv"])
                o = torch.matmul(qkv[:, :dim], dw["o_proj"])
                gu = torch.matmul(o, dw["gate_up"])
                h = torch.nn.functional.silu(gu[:, :inter]) * gu[:, inter:]
                x = torch.matmul(h, dw["down"])
            return x

        def stack_time(fn):
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                for _ in range(2):
                    fn()
            cap.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    fn()
            stream.wait_stream(cap)
            torch.cuda.synchronize()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            warm_up(stream, g.replay)
            reps = max(5, args.stack_tokens)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps, reps

        q_ms, reps = stack_time(lambda: st.step(x0, stream=torch.cuda.current_stream()))
        d_ms, _ = stack_time(lambda: dense_step(x0))
        dbytes = sum(sum(t.numel() * 2 for t in dw.values()) for dw in dense)
        stack = {"layers": nl, "M": Ms, "tokens_timed": reps, "setup_s": round(setup_s, 1),
                 "quantized": {"ms_per_token": round(q_ms, 4), "tokens_per_s": round(1e3 / q_ms, 1),
                               "weight_bytes_per_token": qbytes,
                               "weight_GBps": round(qbytes / (q_ms * 1e-3) / 1e9, 1)},
                 "dense_fp16_torch": {"ms_per_token": round(d_ms, 4), "tokens_per_s": round(1e3 / d_ms, 1),
                                      "weight_bytes_per_token": dbytes,
                                      "weight_GBps": round(dbytes / (d_ms * 1e-3) / 1e9, 1)},
                 "speedup_vs_dense": round(d_ms / q_ms, 2)}
        del dec, dense, st
        torch.cuda.empty_cache()

    # ---------------- plain copy (counter calibration) ----------------
    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu:
        import oracle
        xs_h = [cfg.x(M, L.K) for L in layers]
        reps = 0
        t0 = time.perf_counter()
        while True:
            for L, xh in zip(layers, xs_h):
                oracle.linear(xh, cfg.dtype, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, L.N, L.K,
                              L.bits, L.group_size)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds or reps >= 50:
                break
        dt = time.perf_counter() - t0
        model = ""
        try:
            with open("/proc/cpuinfo") as fh:
                model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
        except OSError:
            pass
        cpu = {"value": round(reps * set_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "cpu_model": model, "kind": "oracle",
               "sample": f"{reps} full passes of the decode layer set (M=1, all columns) in {dt:.1f} s"}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": timed_steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "llama7b_decode_layer_set_int4_zero_f16_g128_M1",
                   "layers": [f"{L.name.split('/')[-1]} {L.K}x{L.N}" for L in layers], "M": M,
                   "weight_bytes_per_step": set_bytes, "rotated_copies": R},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "eager": {"ms_per_step": round(eager_ms_per_step, 5),
                  "value": round(set_bytes / (eager_ms_per_step * 1e-3) / 1e9, 1)},
        "roofline": roofline, "per_kernel": per_kernel, "decode_other_m": decode_m, "other_m1_layers": extra_m1,
        "gemm_m2048": gemm,
        "fused_gate_up": fused, "hadamard": had, "fine_zero_groups": fine, "layer_stack": stack, "cpu_baseline": cpu,
        "kernel_sources_sha256_16": khash,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
