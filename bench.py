"""Benchmark of the fused packed-int4 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the hot path over one batch of synthetic input:
  decode   the W4A16 GEMV at M=1, N=13312, K=2048, G=128 (the gate_up
           shape) over a rotating pool of distinct weight copies larger
           than twice the 256 MB Infinity Cache, so every call streams its
           14.06 MB of packed weights and scales from HBM;
  prefill  the dynamic W4A8 linear at M=2048, N=13312, K=2048, G=128: the
           activation quantizer, then the GEMM, each launched PRE_REPS
           times over the same batch so that a graph launch's fixed cost
           does not enter the per-launch average.
Each leg is captured once in a HIP graph and replayed; HIP events on the
launch stream bracket every replay, giving per-kernel average durations.
The timed region runs the K decode legs back to back and then the K
prefill legs, so that no decode leg pays for the write-back of the
prefill's 104 MiB output (its cold reads would evict those dirty lines
from the Infinity Cache).
HBM traffic per launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
recorded in TRAFFIC (scaled by the factor a plain copy of known size
reads); it is reported only while the kernel's sources hash to the ones
those counters were taken on.

Before the warmup steps, untimed steps run for --settle-seconds so that the
shader clock has left its idle state (the first hundred milliseconds of
work run measurably slower).

After the timed steps:
  ceilings      a plain streaming read of each cold decode weight copy
                (libq4_probe, several launch shapes, the fastest kept) and the
                int8 matrix-core rate with the shader clock it ran at; the
                decode and prefill rooflines are also given against these;
  decode sweep  the decode GEMV over N = 2048 .. 65536 on cold pools, beside
                the same streaming read;
  microdecoder  the frame (35 per-channel W4A8 linears at M=1, 15 passes)
                hot (one stack copy) and cold (four copies in rotation), with
                one launch per linear, one launch per pass
                (q4_linear_w4a8_dynamic_multi) and one launch per group of
                linears a layer can run together ({q,k,v}, {o}, {gate,up},
                {down}), with the first pass after a cache flush timed
                against the passes that follow it;
  and the other layouts' legs (zero points, int8 weights, W4A16 at M = 4
  and 8, per-channel W4A8 at M = 4, W4A32, the dequantize-then-GEMM
  comparator).

Headline value: effective weight GB/s of the decode GEMV (packed + scale
bytes / average kernel duration).  The prefill TOPS (2*M*N*K / GEMM
duration) is reported beside it with its own roofline.  The oracle (CPU,
float64 / exact integer) is timed on a bounded sample on the host cores,
with every BLAS thread and with one, beside the CPU model and BLAS library.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, TOP/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s

DEC_N, DEC_K, DEC_G = 13312, 2048, 128
PRE_M, PRE_N, PRE_K, PRE_G = 2048, 13312, 2048, 128
POOL_BYTES_MIN = 512 << 20      # >= 2x the 256 MB Infinity Cache
PRE_REPS = 8                    # prefill launches per leg per step

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "int4_dequantize_matmul_amd", "csrc")
# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the bench's
# kernels (one launch per call for each);
# FETCH_SIZE reads half the bytes of a plain 256 MiB copy and WRITE_SIZE all
# of them, hence the scales.  "sources" are hashed together.
TRAFFIC = {
    "decode": {"sources": ["gemv_stream.hip", "q4_device.hpp"],
               "sha256": "a1bc4f0dc27dc178823aa83c99c842ca981097173327d620d23e7d754e7908c2",
               "fetch_kib": 6918.56, "write_kib": 104.00, "fetch_scale": 2.0, "write_scale": 1.0,
               "profile": "profiles/gemv_w4a16_m1_n13312_k2048_traffic.md"},
    "prefill": {"sources": ["gemm_tiled.hip", "q4_device.hpp", "q4_lds_dma.hpp"],
                "sha256": "624d1024415de1166ceb80144e2b1292f8951a7c506188cd5bb682fd6c09efb6",
                "fetch_kib": 23791.85, "write_kib": 106496.08, "fetch_scale": 2.0, "write_scale": 1.0,
                "profile": "profiles/tiled_w4a8_m2048_n13312_k2048_g128_traffic.md"},
}


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(kind):
    """HBM bytes per launch from the recorded counters, or None when the
    kernel's sources changed since they were taken (or none were taken)."""
    t = TRAFFIC[kind]
    if t["sha256"] is None or t["fetch_kib"] is None or sources_sha256(t["sources"]) != t["sha256"]:
        return None
    return int(round((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024))


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="budget of the oracle timing on the host (0 disables it)")
    p.add_argument("--no-graph", action="store_true", help="eager launches instead of graph replay")
    p.add_argument("--no-microdecoder", action="store_true", help="skip the microdecoder frame measurement")
    p.add_argument("--no-comparator", action="store_true",
                   help="skip the dequantize-then-GEMM comparator (torch bf16 / int8 GEMM)")
    p.add_argument("--no-zero-points", action="store_true",
                   help="skip the per-group zero-point layouts (decode and prefill)")
    p.add_argument("--no-w8", action="store_true", help="skip the int8-weight float-activation decode (W8A16, W8A32)")
    p.add_argument("--no-w4a32", action="store_true", help="skip the W4A32 GEMV (N = K = 2048, G = 32) and its f32 GEMV")
    p.add_argument("--no-channel", action="store_true", help="skip the per-channel W4A8 linear at M=4, N=3072, K=1023")
    p.add_argument("--no-decode-batch", action="store_true", help="skip the W4A16 decode GEMV at M = 4 and 8")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured ceilings (streaming-read probe, int8 MFMA rate, shader clock)")
    p.add_argument("--no-sweep", action="store_true", help="skip the decode GEMV size sweep over N")
    p.add_argument("--settle-seconds", type=float, default=0.3,
                   help="untimed steps run before the warmup so that the clocks settle")
    p.add_argument("--route-sweep", action="store_true",
                   help="time every route over the batch size instead (one JSON line per N and M) and exit")
    p.add_argument("--route-n", type=str, default=str(DEC_N),
                   help="comma-separated shapes for --route-sweep: N, or NxK (K defaults to 2048)")
    p.add_argument("--route-m", type=str, default="",
                   help="comma-separated batch sizes for --route-sweep (default 1..256)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="after timing, one plain device copy of this many MiB (calibrates byte counters)")
    return p.parse_args()


def decode_bytes(N=DEC_N, K=DEC_K, G=DEC_G):
    """Algorithmic bytes of one decode call: packed weights + bf16 scales."""
    return N * (K // 2) + N * (K // G) * 2


def prefill_ops(M=PRE_M, N=PRE_N, K=PRE_K):
    return 2 * M * N * K


def microdecoder_leg(q4, WL, dev, timed_replays=5, eager=False):
    """The microdecoder stack: 5 layers x {q, k, v, o, gate, up, down}, W4A8
    per channel at M=1, each linear quantizing its own bf16 input row (inside
    the decode kernel), the 35 linears run 15 times per frame.  Hot: one copy
    of the stack (128 MB packed, resident in the Infinity Cache after the
    first pass).  Cold: pass p reads copy p % 4 (515 MB in all, so every pass
    streams from HBM).

    Three ways to run a pass: one q4_linear_w4a8_dynamic call per linear (35
    launches); one q4_linear_w4a8_dynamic_multi call for all 35 (one launch,
    as if the linears were independent); and one multi call per group of
    linears a layer can run together, {q, k, v}, {o}, {gate, up}, {down}
    (20 launches, the order a real layer's dependencies allow).  For each: hot and cold frame times, and the first pass after
    the cache has been flushed (by passes over the other copies) against
    the 14 passes that follow it."""
    import torch

    lin = WL.microdecoder_linears()
    lib = q4.raw()
    copies, per_linear = 4, []
    packed_bytes = scale_bytes = 0
    for i, (_l, _name, N, K) in enumerate(lin):
        d = WL.microdecoder_linear(i)
        packed, sw = q4.q4_quantize_matrix(d["W"])
        packed_bytes += packed.nbytes
        scale_bytes += sw.nbytes
        wq = [torch.from_numpy(packed).to(dev) for _ in range(copies)]
        x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).view(torch.bfloat16).to(dev)
        ws = torch.empty(q4.q4_w4a8_dynamic_workspace(1, K), dtype=torch.uint8, device=dev)
        per_linear.append(dict(N=N, K=K, wq=wq, sw=torch.from_numpy(sw).to(dev), x=x, ws=ws,
                               y=torch.empty((1, N), dtype=torch.float32, device=dev)))
    x0 = per_linear[0]["x"]
    arrs = [q4.w4a8_problems([(c["x"], c["wq"][k], c["sw"], c["y"]) for c in per_linear]) for k in range(copies)]
    # launches that respect a layer's dependencies: {q, k, v}, {o}, {gate, up},
    # {down}, i.e. four per layer and twenty per pass
    groups = []
    for base in range(0, len(per_linear), len(WL.LAYER_LINEARS)):
        groups += [[base, base + 1, base + 2], [base + 3], [base + 4, base + 5], [base + 6]]
    garrs = [[(q4.w4a8_problems([(per_linear[i]["x"], per_linear[i]["wq"][k], per_linear[i]["sw"],
                                  per_linear[i]["y"]) for i in grp]), len(grp)) for grp in groups]
             for k in range(copies)]
    pass_bytes = packed_bytes + scale_bytes

    # the stream is looked up at each call: inside a capture it is the
    # capturing stream
    def pass_each(copy):
        stream = q4._stream(x0)
        for c in per_linear:
            st = lib.q4_linear_w4a8_dynamic(q4._ptr(c["x"]), q4.DT["bf16"], q4._ptr(c["wq"][copy]),
                                            q4._ptr(c["sw"]), q4._ptr(c["y"]), 1, c["N"], c["K"], 0,
                                            q4.ENC["excess8"], q4._ptr(c["ws"]), c["ws"].numel(), stream)
            assert st == 0, st

    def pass_multi(copy):
        stream = q4._stream(x0)
        st = lib.q4_linear_w4a8_dynamic_multi(arrs[copy], len(per_linear), q4.DT["bf16"], 1, stream)
        assert st == 0, st

    def pass_grouped(copy):
        stream = q4._stream(x0)
        for arr, n in garrs[copy]:
            st = lib.q4_linear_w4a8_dynamic_multi(arr, n, q4.DT["bf16"], 1, stream)
            assert st == 0, st

    class Eager:                      # --no-graph: the same sequence, launched directly
        def __init__(self, fn, seq):
            self.fn, self.seq = fn, seq

        def replay(self):
            for k in self.seq:
                self.fn(k)

    def graph_of(fn, copies_seq):
        for k in copies_seq:          # warm (and route) outside the capture
            fn(k)
        if eager:
            return Eager(fn, list(copies_seq))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in copies_seq:
                fn(k)
        g.replay()
        torch.cuda.synchronize()
        return g

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    out = {"linears": len(lin), "passes_per_frame": 15, "calls_per_frame": 15 * len(lin),
           "bytes_per_pass": pass_bytes, "stack_copies_cold": copies}
    for tag, fn in (("", pass_each), ("multi_", pass_multi), ("grouped_", pass_grouped)):
        for cold in (False, True):
            g = graph_of(fn, [p % copies if cold else 0 for p in range(15)])
            if tag == "":
                out["path"] = q4.q4_last_path()
            e0 = ev()
            for _ in range(timed_replays):
                g.replay()
            e1 = ev()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / timed_replays
            key = "cold" if cold else "hot"
            out[f"{tag}{key}_frame_us"] = round(us, 2)
            out[f"{tag}{key}_effective_gbs"] = round(15 * pass_bytes / (us * 1e-6) / 1e9, 1)
        # residency: the first pass over copy 0 after passes over copies 1..3
        # (387 MB, more than the 256 MB cache) against the 14 that follow.
        # Taken as differences between graphs that share the flush, so that
        # the launch cost of a graph cancels out.
        seqs = ([1, 2, 3], [1, 2, 3, 0], [1, 2, 3] + [0] * 15)
        graphs = [graph_of(fn, q) for q in seqs]
        t = [[], [], []]
        for _ in range(timed_replays):
            for i, g in enumerate(graphs):
                torch.cuda.synchronize()
                e0 = ev()
                g.replay()
                e1 = ev()
                torch.cuda.synchronize()
                t[i].append(e0.elapsed_time(e1) * 1e3)
        med = [float(np.median(v)) for v in t]
        out[f"{tag}first_pass_us"] = round(med[1] - med[0], 2)
        out[f"{tag}later_pass_us"] = round((med[2] - med[1]) / 14, 2)
    # per-channel decode quantizes inside the GEMV: one kernel per call there
    out["launches_per_frame"] = out["calls_per_frame"] * (1 if out["path"] == "gemv" else 2)
    out["multi_launches_per_frame"] = 15
    out["grouped_launches_per_frame"] = 15 * len(groups)
    return out


def zero_point_leg(q4, lib, pool, s_dec, x_dec, xq_pre, sx_pre, w_pre, s_pre, dev):
    """The asymmetric layouts at the workload shapes, with seeded 4-bit zero
    points per row and group: the W4A16 decode at M=1 over the same cold
    pool of weight copies, and the grouped W4A8 prefill at M=2048.  HIP
    events around graph replays."""
    import torch

    rng = np.random.default_rng(1006)
    z_dec = torch.from_numpy(rng.integers(0, 16, (DEC_N, DEC_K // DEC_G), dtype=np.uint8)).to(dev)
    z_pre = torch.from_numpy(rng.integers(0, 16, (PRE_N, PRE_K // PRE_G), dtype=np.uint8)).to(dev)
    yb = torch.empty((1, DEC_N), dtype=torch.bfloat16, device=dev)
    y = torch.empty((PRE_M, PRE_N), dtype=torch.float32, device=dev)

    def dec(w):
        st = lib.q4_linear_w4a16_zp(q4._ptr(x_dec), q4._ptr(w), q4._ptr(s_dec), q4._ptr(z_dec), q4._ptr(yb),
                                    None, 1, DEC_N, DEC_K, DEC_G, q4._stream(x_dec))
        assert st == 0, st

    def pre():
        st = lib.q4_linear_w4a8_zp(q4._ptr(xq_pre), q4._ptr(sx_pre), q4._ptr(w_pre), q4._ptr(s_pre),
                                   q4._ptr(z_pre), q4._ptr(y), PRE_M, PRE_N, PRE_K, PRE_G, q4._stream(xq_pre))
        assert st == 0, st

    def timed(fn, calls, replays=5):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * calls)

    dec(pool[0])
    dec_path = q4.q4_last_path()
    us_d = timed(lambda: [dec(w) for w in pool], len(pool))
    pre()
    pre_path = q4.q4_last_path()
    us_p = timed(lambda: [pre() for _ in range(PRE_REPS)], PRE_REPS)
    zbytes = decode_bytes() + DEC_N * (DEC_K // DEC_G)     # + one zero-point byte per group
    return {"decode_path": dec_path, "decode_avg_us": round(us_d, 3),
            "decode_gbs": round(zbytes / (us_d * 1e-6) / 1e9, 1), "decode_bytes_per_call": zbytes,
            "prefill_path": pre_path, "prefill_avg_us": round(us_p, 3),
            "prefill_tops": round(prefill_ops() / (us_p * 1e-6) / 1e12, 1)}


def w4a32_leg(q4, lib, WL, dev, replays=5):
    """W4A32 GEMV at M=1, N=K=2048, G=32 (f32 x, f16 group scales,
    two's-complement nibbles): 2.36 MB per call, over a cold pool of 256
    weight copies (604 MB) and hot.  Beside it an f32 GEMV of the same shape
    (torch.mv on a 16.8 MB f32 matrix, hipBLAS) over its own cold pool: the
    speed-up of the int4 GEMV over f32 is the pages' own figure for this
    shape.  HIP events around graph replays."""
    import torch

    d = WL.w4a32_gemv()
    N, K, G = d["N"], d["K"], d["G"]
    x = torch.from_numpy(d["x"]).to(dev)
    w0 = torch.from_numpy(d["qweight"]).to(dev)
    s0 = torch.from_numpy(d["scales_f16"].view(np.int16)).to(dev)
    pool = [(w0.clone(), s0.clone()) for _ in range(256)]
    y = torch.empty((1, N), dtype=torch.float32, device=dev)

    def q4call(ws):
        assert lib.q4_linear_w4a32(q4._ptr(x), q4._ptr(ws[0]), q4._ptr(ws[1]), q4._ptr(y), 1, N, K, G,
                                   q4.ENC["twos"], q4._stream(x)) == 0

    w32 = torch.randn((N, K), dtype=torch.float32, device=dev)
    fpool = [w32.clone() for _ in range(max(2, -(-POOL_BYTES_MIN // (N * K * 4))))]
    yf = torch.empty(N, dtype=torch.float32, device=dev)
    xv = x.view(-1)

    def f32call(w):
        torch.mv(w, xv, out=yf)

    def timed(fn, items):
        fn(items[0])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for it in items:
                fn(it)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * len(items))

    nbytes = N * K // 2 + N * (K // G) * 2
    out = {"workload": f"W4A32 GEMV M=1 N={N} K={K} G={G}", "bytes_per_call": nbytes, "copies": len(pool)}
    cold = timed(q4call, pool)
    out["path"] = q4.q4_last_path()
    hot = timed(q4call, [pool[0]] * len(pool))
    f_cold = timed(f32call, fpool)
    f_hot = timed(f32call, [fpool[0]] * len(fpool))
    out.update(cold_us=round(cold, 3), hot_us=round(hot, 3), cold_gbs=round(nbytes / (cold * 1e-6) / 1e9, 1),
               f32_copies=len(fpool), f32_cold_us=round(f_cold, 3), f32_hot_us=round(f_hot, 3),
               speedup_over_f32_cold=round(f_cold / cold, 2), speedup_over_f32_hot=round(f_hot / hot, 2))
    del pool, fpool
    torch.cuda.empty_cache()
    return out


def decode_batch_leg(q4, lib, WL, pool, s_dec, dev, Ms=(4, 8), replays=5):
    """The W4A16 decode GEMV at the other batch sizes of its workload
    (M = 4 and 8; N = 13312, K = 2048, G = 128), over the same cold pool as
    the M = 1 headline, on the default route (the streaming kernel, whose
    rows do not depend on M) and on the matrix-core route; HIP events around
    graph replays."""
    import torch

    d = WL.w4a16_gemv()   # the workload's own activation rows for M = 1, 4, 8
    out = {}
    runs = [(M, r) for M in Ms for r in ("auto", "gemv_mc")]
    for M, route in runs:
        q4.q4_set_path(route)
        x = torch.from_numpy(np.ascontiguousarray(d["x"][M]).view(np.int16)).view(torch.bfloat16).to(dev)
        yb = torch.empty((M, DEC_N), dtype=torch.bfloat16, device=dev)

        def call(w):
            assert lib.q4_linear_w4a16(q4._ptr(x), q4._ptr(w), q4._ptr(s_dec), q4._ptr(yb), None, M, DEC_N,
                                       DEC_K, DEC_G, q4.ENC["excess8"], q4._stream(x)) == 0

        call(pool[0])
        path = q4.q4_last_path()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for w in pool:
                call(w)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (replays * len(pool))
        out[f"m{M}_{route}"] = {"path": path, "avg_us": round(us, 3),
                                "weight_gbs": round(decode_bytes() / (us * 1e-6) / 1e9, 1)}
    q4.q4_set_path("auto")
    return out


def channel_leg(q4, lib, WL, dev, replays=5):
    """Per-channel W4A8 at M=4, N=3072, K=1023 (odd K, pad nibble): the
    dynamic call (f32 rows quantized, then the linear) and the linear on
    given codes, each over a cold pool of weight copies (>= 512 MiB) and hot;
    HIP events around graph replays."""
    import torch

    d = WL.w4a8_channel()
    M, N, K = d["M"], d["N"], d["K"]
    packed, sw = q4.q4_quantize_matrix(d["W"])
    w0 = torch.from_numpy(packed).to(dev)
    pool = [w0.clone() for _ in range(max(2, -(-POOL_BYTES_MIN // w0.numel())))]
    swd = torch.from_numpy(sw).to(dev)
    x = torch.from_numpy(d["x"]).to(dev)
    ws = torch.empty(q4.q4_w4a8_dynamic_workspace(M, K), dtype=torch.uint8, device=dev)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    assert lib.q8_quantize_rows(q4._ptr(x), q4.DT["f32"], M, K, q4._ptr(xq), q4._ptr(sx), q4._stream(x)) == 0
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def dyn(w):
        assert lib.q4_linear_w4a8_dynamic(q4._ptr(x), q4.DT["f32"], q4._ptr(w), q4._ptr(swd), q4._ptr(y), M, N, K,
                                          0, q4.ENC["excess8"], q4._ptr(ws), ws.numel(), q4._stream(x)) == 0

    def codes(w):
        assert lib.q4_linear_w4a8(q4._ptr(xq), q4._ptr(sx), q4._ptr(w), q4._ptr(swd), q4._ptr(y), M, N, K, 0,
                                  q4.ENC["excess8"], q4._stream(xq)) == 0

    def timed(fn, items):
        fn(items[0])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for it in items:
                fn(it)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * len(items))

    nbytes = packed.nbytes + sw.nbytes
    out = {"workload": f"W4A8 per channel M={M} N={N} K={K}", "bytes_per_call": nbytes, "copies": len(pool)}
    for name, fn in (("dynamic", dyn), ("codes", codes)):
        cold = timed(fn, pool)
        out[f"{name}_path"] = q4.q4_last_path()
        hot = timed(fn, [pool[0]] * len(pool))
        out[f"{name}_cold_us"] = round(cold, 3)
        out[f"{name}_hot_us"] = round(hot, 3)
        out[f"{name}_cold_gbs"] = round(nbytes / (cold * 1e-6) / 1e9, 1)
    del pool
    torch.cuda.empty_cache()
    return out


def w8_leg(q4, lib, x_dec, dev):
    """int8 weights with one scale per row (W8A16 and W8A32) at the decode
    shape, M=1, N=13312, K=2048, over a cold pool of distinct weight copies
    (>= 512 MiB); HIP events around graph replays."""
    import torch

    rng = np.random.default_rng(1007)
    w0 = torch.from_numpy(rng.integers(-128, 128, (DEC_N, DEC_K), dtype=np.int8)).to(dev)
    copies = max(2, -(-POOL_BYTES_MIN // w0.numel()))
    pool = [w0.clone() for _ in range(copies)]
    sw = torch.from_numpy(rng.uniform(0.001, 0.05, DEC_N).astype(np.float32)).to(dev)
    x32 = x_dec.float().contiguous()
    yb = torch.empty((1, DEC_N), dtype=torch.bfloat16, device=dev)
    y = torch.empty((1, DEC_N), dtype=torch.float32, device=dev)

    def a16(w):
        assert lib.q8_linear_w8a16(q4._ptr(x_dec), q4._ptr(w), q4._ptr(sw), q4._ptr(yb), None, 1, DEC_N, DEC_K,
                                   q4._stream(x_dec)) == 0

    def a32(w):
        assert lib.q8_linear_w8a32(q4._ptr(x32), q4._ptr(w), q4._ptr(sw), q4._ptr(y), 1, DEC_N, DEC_K,
                                   q4._stream(x32)) == 0

    nbytes = DEC_N * DEC_K + DEC_N * 4
    out = {"copies": copies, "bytes_per_call": nbytes}
    for name, fn in (("w8a16", a16), ("w8a32", a32)):
        fn(pool[0])
        out[f"{name}_path"] = q4.q4_last_path()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for w in pool:
                fn(w)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (5 * copies)
        out[f"{name}_avg_us"] = round(us, 3)
        out[f"{name}_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    del pool
    torch.cuda.empty_cache()
    return out


def comparator_leg(q4, lib, p, x_pre, w_pre, xq_pre, dev, reps=PRE_REPS):
    """Dequantize-then-GEMM, the comparator for the fused prefill kernels
    (not part of the library, which never writes weights in float): the
    prefill weights unpacked once into bf16 in HBM (torch elementwise ops;
    bf16 rounds q * s, so this path is not bit-exact), then torch's dense
    bf16 GEMM (hipBLASLt) at M=2048; torch's int8 GEMM on the quantized
    activations against the int8 codes; and the per-call cost of the unpack
    itself.  Beside them, the library's fused W4A16 prefill on the same
    bf16 activations, packed weights and (bf16-valued) scales, bf16 output
    like the GEMM's.  Times are HIP events around graph replays."""
    import torch

    N, K, G = PRE_N, PRE_K, PRE_G
    s = torch.from_numpy(p["scales"]).to(dev)

    def dequant():
        u = torch.stack([w_pre & 15, w_pre >> 4], dim=-1).reshape(N, K).to(torch.int16) - 8
        return (u.to(torch.float32).view(N, K // G, G) * s.view(N, K // G, 1)).reshape(N, K).to(torch.bfloat16)

    wf = dequant()
    wf_t = wf.t().contiguous()                       # [K, N]: no transposed view into the GEMM
    q8_t = (torch.stack([w_pre & 15, w_pre >> 4], dim=-1).reshape(N, K).to(torch.int16) - 8).to(torch.int8)
    q8_t = q8_t.t().contiguous()                     # [K, N] int8
    out = {"weights_bf16_bytes": wf.numel() * 2}

    def time_leg(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (3 * reps)

    x_bf = x_pre.view(torch.bfloat16)
    us = time_leg(lambda: torch.mm(x_bf, wf_t))
    out["bf16_gemm_us"] = round(us, 2)
    out["bf16_gemm_tflops"] = round(prefill_ops() / (us * 1e-6) / 1e12, 1)
    out["dequant_us"] = round(time_leg(dequant), 2)
    try:
        us8 = time_leg(lambda: torch._int_mm(xq_pre, q8_t))
        out["int8_gemm_us"] = round(us8, 2)
        out["int8_gemm_tops"] = round(prefill_ops() / (us8 * 1e-6) / 1e12, 1)
    except RuntimeError as e:                        # int8 GEMM not offered by this torch build
        out["int8_gemm_us"] = None
        out["int8_gemm_error"] = str(e)[:120]
    s_bf = s.to(torch.bfloat16)                      # exact: the scales are bf16 values
    yb = torch.empty((PRE_M, N), dtype=torch.bfloat16, device=dev)

    def w4a16():
        st = lib.q4_linear_w4a16(q4._ptr(x_bf), q4._ptr(w_pre), q4._ptr(s_bf), q4._ptr(yb), None, PRE_M, N, K, G,
                                 q4.ENC["excess8"], q4._stream(x_bf))
        assert st == 0, st

    us16 = time_leg(w4a16)
    out["w4a16_fused_path"] = q4.q4_last_path()
    out["w4a16_fused_us"] = round(us16, 2)
    out["w4a16_fused_tflops"] = round(prefill_ops() / (us16 * 1e-6) / 1e12, 1)
    out["w4a16_fused_frac_of_bf16_peak"] = round(prefill_ops() / (us16 * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
    del wf, wf_t, q8_t, yb
    torch.cuda.empty_cache()
    return out


def route_sweep(q4, dev, shapes=((DEC_N, DEC_K),), Ms=(1, 2, 4, 8, 12, 16, 17, 20, 24, 32, 40, 48, 64, 96, 128, 256)):
    """Decode route against the tiled route at each batch size, per (N, K)
    shape, hot weights (one graph of 20 calls), G = 128: one JSON line per M."""
    for N, K in shapes:
        _route_sweep_n(q4, dev, N, K, Ms)


def _route_sweep_n(q4, dev, N, K, Ms):
    import torch

    G = DEC_G
    rng = np.random.default_rng(3)
    w = torch.from_numpy(rng.integers(0, 256, (N, K // 2), dtype=np.uint8)).to(dev)
    sb = (rng.uniform(0.002, 0.03, (N, K // G)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    s_bf = torch.from_numpy(sb.view(np.int16)).view(torch.bfloat16).to(dev)
    s_g = torch.from_numpy(rng.uniform(0.002, 0.03, (N, K // G)).astype(np.float32)).to(dev)
    s_c = torch.from_numpy(rng.uniform(0.002, 0.03, N).astype(np.float32)).to(dev)
    lib = q4.raw()
    paths = {"gemv": 2, "tiled": 3, "gemv_mc": 4, "auto": 0}

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (5 * reps)

    for M in Ms:
        x = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(dev).to(torch.bfloat16)
        xq = torch.from_numpy(rng.integers(-127, 128, (M, K), dtype=np.int8)).to(dev)
        sx = torch.from_numpy(rng.uniform(0.001, 0.02, M).astype(np.float32)).to(dev)
        yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        calls = {
            "w4a16": lambda: lib.q4_linear_w4a16(q4._ptr(x), q4._ptr(w), q4._ptr(s_bf), q4._ptr(yb), None,
                                                 M, N, K, G, 1, q4._stream(x)),
            "w4a8_grouped": lambda: lib.q4_linear_w4a8(q4._ptr(xq), q4._ptr(sx), q4._ptr(w), q4._ptr(s_g),
                                                       q4._ptr(y), M, N, K, G, 1, q4._stream(x)),
            "w4a8_channel": lambda: lib.q4_linear_w4a8(q4._ptr(xq), q4._ptr(sx), q4._ptr(w), q4._ptr(s_c),
                                                       q4._ptr(y), M, N, K, 0, 1, q4._stream(x)),
        }
        line = {"M": M, "N": N, "K": K, "G": G}
        for op, fn in calls.items():
            for pn, pv in paths.items():
                if pn == "gemv_mc" and op != "w4a16":
                    continue
                lib.q4_set_path(pv)
                assert fn() == 0
                line[f"{op}:{pn}"] = {"us": round(timed(fn), 2), "kernel": q4.q4_last_path()}
        lib.q4_set_path(0)
        print(json.dumps(line), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds: float):
    """Time the oracle on bounded samples of the two legs on the host cores,
    with every BLAS thread and with one."""
    import threadpoolctl

    import oracle.formats as F
    import oracle.linear as L
    import oracle.quantize as Q
    from int4_dequantize_matmul_amd import workloads as WL

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
            | {"library": os.path.basename(i.get("filepath", ""))} for i in info]
    d = WL.w4a16_gemv(Ms=(1,))
    x1, w, s = d["x"][1], d["qweight"], d["scales_bf16"]
    p = WL.w4a8_prefill()
    rows = 16
    xq, sx = Q.quantize_q8_rows(p["x"][:rows], "bf16")

    def run(budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            L.linear_w4a16(x1, w, s, DEC_G, F.EXCESS8)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 200:
                break
        t1 = time.perf_counter()
        L.linear_w4a8(xq, sx, p["qweight"], p["scales"], PRE_G, F.EXCESS8)
        el_p = time.perf_counter() - t1
        return reps, el, el_p

    reps, el, el_p = run(seconds * 0.4)
    with threadpoolctl.threadpool_limits(limits=1):
        reps1, el1, el_p1 = run(seconds * 0.2)
    dec = decode_bytes() * reps / el / 1e9
    pre = prefill_ops(rows) / el_p / 1e12
    return {
        "value": round(dec, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"oracle W4A16 decode (float64 factored sum) at M=1, N={DEC_N}, K={DEC_K}, G={DEC_G}, "
                  f"{reps} calls in {el:.2f} s",
        "prefill": {"value": round(pre, 6), "unit": "TOPS",
                    "sample": f"oracle grouped W4A8 (exact int + f32 epilogue) on {rows} of {PRE_M} "
                              f"activation rows, {el_p:.2f} s"},
        "one_thread": {"value": round(decode_bytes() * reps1 / el1 / 1e9, 4), "unit": "GB/s",
                       "sample": f"{reps1} decode calls in {el1:.2f} s",
                       "prefill_tops": round(prefill_ops(rows) / el_p1 / 1e12, 6)},
        "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(), "blas": blas,
        "note": "an exact reference (numpy float64 / exact integers), not a tuned CPU kernel",
    }


def ceilings_leg(q4, probe, pool, dev, dec_us, gemm_us, cu_count, replays=5):
    """Measured ceilings on this device: a plain streaming read of each cold
    decode weight copy (the bytes the decode GEMV must fetch from memory;
    several launch shapes, the fastest kept), and the int8 matrix-core rate
    with the shader clock it ran at."""
    import torch

    nbytes = pool[0].numel()
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    shapes = [(1024, 256), (2048, 256), (4096, 256), (8192, 128), (3328, 64), (6656, 64)]
    best = None
    per_shape = {}
    for blocks, threads in shapes:
        def leg():
            for w in pool:
                probe.q4_probe_read(w, sink, blocks, threads)
        leg()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            leg()
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (replays * len(pool))
        per_shape[f"{blocks}x{threads}"] = round(us, 3)
        best = us if best is None else min(best, us)
    # int8 MFMA: four workgroups of four waves per CU, 200 rounds of 16 MFMAs each
    blocks, iters = 4 * cu_count, 200
    out = torch.zeros(8 * blocks, dtype=torch.int64, device=dev)
    probe.q4_probe_mfma_i8(out, blocks, iters)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        probe.q4_probe_mfma_i8(out, blocks, iters)
    e1.record()
    torch.cuda.synchronize()
    mfma_us = e0.elapsed_time(e1) * 1e3 / replays
    ops = 2 * 32768 * 16 * iters * 4 * blocks
    o = out.cpu().numpy().reshape(-1, 2)
    clock_ghz = float(np.median(o[:, 0] / np.maximum(o[:, 1], 1)) * 0.1)
    tops = ops / (mfma_us * 1e-6) / 1e12
    return {
        "read_probe_us": round(best, 3), "read_probe_bytes": nbytes,
        "read_probe_gbs": round(nbytes / (best * 1e-6) / 1e9, 1), "read_probe_shapes_us": per_shape,
        "decode_frac_of_probe": round(best / dec_us, 4),
        "mfma_i8_probe_tops": round(tops, 1), "mfma_i8_probe_us": round(mfma_us, 2),
        "shader_clock_ghz": round(clock_ghz, 3),
        "int8_peak_at_clock_tops": round(INT8_PEAK_TOPS * clock_ghz / 2.4, 1),
        "prefill_frac_of_mfma_probe": round(prefill_ops() / (gemm_us * 1e-6) / 1e12 / tops, 4),
    }


def decode_sweep_leg(q4, probe, WL, dev, Ns=(2048, 4096, 8192, 13312, 26624, 53248, 65536), replays=5):
    """The W4A16 decode GEMV at M=1, K=2048, G=128 over N, each on a cold pool
    of weight copies totalling >= 512 MB, beside a plain streaming read of
    the same copies."""
    import torch

    lib = q4.raw()
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    out = {}
    for N in Ns:
        d = WL.small_float_case(7000 + N, 1, N, DEC_K, DEC_G)
        w = torch.from_numpy(d["qweight"]).to(dev)
        s = torch.from_numpy(d["scales_bf16"].view(np.int16)).view(torch.bfloat16).to(dev)
        x = torch.from_numpy(d["x_bf16"].view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        n = max(2, -(-POOL_BYTES_MIN // w.numel()))
        pool = [w.clone() for _ in range(n)]

        def dec():
            for wc in pool:
                assert lib.q4_linear_w4a16(q4._ptr(x), q4._ptr(wc), q4._ptr(s), q4._ptr(y), None, 1, N, DEC_K,
                                           DEC_G, q4.ENC["excess8"], q4._stream(x)) == 0

        def rd():
            for wc in pool:
                probe.q4_probe_read(wc, sink, 2048, 256)

        res = {}
        for name, fn in (("gemv", dec), ("read", rd)):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / (replays * n)
        b = decode_bytes(N)
        out[str(N)] = {"bytes": b, "copies": n, "gemv_us": round(res["gemv"], 3),
                       "gemv_gbs": round(b / (res["gemv"] * 1e-6) / 1e9, 1),
                       "read_us": round(res["read"], 3),
                       "frac_of_hbm_peak": round(b / (res["gemv"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "frac_of_read": round(res["read"] / res["gemv"], 4)}
        del pool
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the linear runs on a single GPU; splitting N across GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import int4_dequantize_matmul_amd as q4
    from int4_dequantize_matmul_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.route_sweep:
        shapes = tuple((int(v.split("x")[0]), int(v.split("x")[1]) if "x" in v else DEC_K)
                       for v in args.route_n.split(","))
        kw = {"Ms": tuple(int(v) for v in args.route_m.split(","))} if args.route_m else {}
        route_sweep(q4, dev, shapes=shapes, **kw)
        return

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # ---- decode inputs: one weight matrix copied into a rotating pool ----
    d = WL.w4a16_gemv(Ms=(1,))
    w_host = T(d["qweight"])
    per_copy = w_host.numel()
    pool_n = max(2, -(-POOL_BYTES_MIN // per_copy))
    pool = [w_host.clone() for _ in range(pool_n)]
    s_dec = T(d["scales_bf16"])
    x_dec = T(d["x"][1])
    yb_dec = torch.empty((1, DEC_N), dtype=torch.bfloat16, device=dev)

    # ---- prefill inputs ----
    p = WL.w4a8_prefill()
    x_pre = T(p["x"])
    w_pre = T(p["qweight"])
    s_pre = T(p["scales"])
    ws = torch.empty(q4.q4_w4a8_dynamic_workspace(PRE_M, PRE_K), dtype=torch.uint8, device=dev)
    xq_pre = ws[: PRE_M * PRE_K].view(torch.int8).view(PRE_M, PRE_K)
    sx_off = (PRE_M * PRE_K + 255) // 256 * 256
    sx_pre = ws[sx_off: sx_off + 4 * PRE_M].view(torch.float32)
    y_pre = torch.empty((PRE_M, PRE_N), dtype=torch.float32, device=dev)
    lib = q4.raw()

    def dec_call(w):
        st = lib.q4_linear_w4a16(q4._ptr(x_dec), q4._ptr(w), q4._ptr(s_dec), q4._ptr(yb_dec), None,
                                 1, DEC_N, DEC_K, DEC_G, q4.ENC["excess8"], q4._stream(x_dec))
        assert st == 0, st

    def quant_call():
        st = lib.q8_quantize_rows(q4._ptr(x_pre), q4.DT["bf16"], PRE_M, PRE_K, q4._ptr(xq_pre),
                                  q4._ptr(sx_pre), q4._stream(x_pre))
        assert st == 0, st

    def gemm_call():
        st = lib.q4_linear_w4a8(q4._ptr(xq_pre), q4._ptr(sx_pre), q4._ptr(w_pre), q4._ptr(s_pre),
                                q4._ptr(y_pre), PRE_M, PRE_N, PRE_K, PRE_G, q4.ENC["excess8"],
                                q4._stream(xq_pre))
        assert st == 0, st

    def quant_leg():
        for _ in range(PRE_REPS):
            quant_call()

    def gemm_leg():
        for _ in range(PRE_REPS):
            gemm_call()

    def decode_leg():
        for w in pool:
            dec_call(w)

    # warm the libraries (device probe, code objects) before any capture
    decode_leg()
    quant_call()
    gemm_call()
    torch.cuda.synchronize()
    dec_path, gemm_path = None, None
    dec_call(pool[0]); dec_path = q4.q4_last_path()
    gemm_call(); gemm_path = q4.q4_last_path()
    torch.cuda.synchronize()

    if args.no_graph:
        legs = [decode_leg, quant_leg, gemm_leg]
    else:
        graphs = []
        for fn in (decode_leg, quant_leg, gemm_leg):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs.append(g)
        legs = [g.replay for g in graphs]

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]

    def step():
        for leg in legs:
            leg()

    # untimed steps until the clocks have settled, then the warmup steps
    t_settle, settle_steps = time.perf_counter(), 0
    while time.perf_counter() - t_settle < args.settle_seconds:
        step()
        torch.cuda.synchronize()
        settle_steps += 1
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The K decode legs run back to back, then the K prefill legs (quantizer
    # and GEMM): a decode leg right after a prefill leg would pay for the
    # write-back of the prefill's 104 MiB output as the decode's cold reads
    # evict it from the Infinity Cache.
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        legs[0]()
        ev[i][1].record()
    for i in range(args.steps):
        ev[i][2].record()
        legs[1]()
        ev[i][3].record()
        legs[2]()
        ev[i][4].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dec_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    quant_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps / PRE_REPS
    gemm_ms = sum(e[3].elapsed_time(e[4]) for e in ev) / args.steps / PRE_REPS
    dec_us_per_call = dec_ms * 1e3 / pool_n
    dec_gbs = decode_bytes() / (dec_us_per_call * 1e-6) / 1e9
    gemm_tops = prefill_ops() / (gemm_ms * 1e-3) / 1e12
    e2e_tops = prefill_ops() / ((quant_ms + gemm_ms) * 1e-3) / 1e12

    # hot reference: the same weight buffer every call (Infinity Cache resident)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.no_graph:
        hot = lambda: [dec_call(pool[0]) for _ in range(pool_n)]  # noqa: E731
    else:
        gh = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gh):
            for _ in range(pool_n):
                dec_call(pool[0])
        hot = gh.replay
    hot()
    e0.record()
    for _ in range(5):
        hot()
    e1.record()
    torch.cuda.synchronize()
    hot_us = e0.elapsed_time(e1) * 1e3 / (5 * pool_n)

    out = {
        "metric": "int4 GEMV effective weight GB/s (% HBM peak) at M=1; prefill W4A8 TOPS (% MFMA)",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"W4A16 decode GEMV M=1 N={DEC_N} K={DEC_K} G={DEC_G} over {pool_n} weight "
                        f"copies ({pool_n * per_copy / 2**20:.0f} MiB) + W4A8 prefill M={PRE_M} "
                        f"N={PRE_N} K={PRE_K} G={PRE_G}",
            "decode_path": dec_path, "prefill_path": gemm_path,
            "timing": "HIP events around graph replays" if not args.no_graph else "HIP events, eager",
            "prefill_launches_per_leg": PRE_REPS,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_bytes("decode"),
            "traffic_unit": "bytes per launch",
            "kernel": "decode GEMV (W4A16, gemv_stream_w4a16)", "bytes_per_launch": decode_bytes(),
            "avg_us": round(dec_us_per_call, 3), "hot_avg_us": round(hot_us, 3),
            "hot_gbs": round(decode_bytes() / (hot_us * 1e-6) / 1e9, 1),
        },
        "prefill": {
            "value": round(gemm_tops, 2), "unit": "TOPS", "dtype": "int8",
            "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                         "traffic": traffic_bytes("prefill"), "traffic_unit": "bytes per launch",
                         "ops_per_launch": prefill_ops(), "avg_us": round(gemm_ms * 1e3, 3)},
            "quantize_avg_us": round(quant_ms * 1e3, 3),
            "end_to_end_tops": round(e2e_tops, 2),
        },
    }
    out["config"]["settle_steps"] = settle_steps
    if not args.no_ceilings or not args.no_sweep:
        from int4_dequantize_matmul_amd import probe
    if not args.no_ceilings:
        cu = torch.cuda.get_device_properties(dev).multi_processor_count
        c = ceilings_leg(q4, probe, pool, dev, dec_us_per_call, gemm_ms * 1e3, cu)
        out["ceilings"] = c
        out["roofline"]["probe_us"] = c["read_probe_us"]
        out["roofline"]["frac_of_probe"] = c["decode_frac_of_probe"]
        out["roofline"]["peak_at_clock"] = round(HBM_PEAK_GBS, 1)
        pr = out["prefill"]["roofline"]
        pr["peak_at_clock"] = c["int8_peak_at_clock_tops"]
        pr["frac_at_clock"] = round(pr["achieved"] / c["int8_peak_at_clock_tops"], 4)
        pr["mfma_probe_tops"] = c["mfma_i8_probe_tops"]
        pr["frac_of_mfma_probe"] = c["prefill_frac_of_mfma_probe"]
    if not args.no_sweep:
        out["decode_sweep"] = decode_sweep_leg(q4, probe, WL, dev)
    if not args.no_microdecoder:
        out["microdecoder"] = microdecoder_leg(q4, WL, dev, eager=args.no_graph)
    if not args.no_zero_points:
        out["zero_points"] = zero_point_leg(q4, lib, pool, s_dec, x_dec, xq_pre, sx_pre, w_pre, s_pre, dev)
    if not args.no_w8:
        out["w8"] = w8_leg(q4, lib, x_dec, dev)
    if not args.no_decode_batch:
        out["decode_batch"] = decode_batch_leg(q4, lib, WL, pool, s_dec, dev)
    if not args.no_w4a32:
        out["w4a32"] = w4a32_leg(q4, lib, WL, dev)
    if not args.no_channel:
        out["w4a8_channel"] = channel_leg(q4, lib, WL, dev)
    if not args.no_comparator:
        out["comparator"] = comparator_leg(q4, lib, p, x_pre, w_pre, xq_pre, dev)
    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = args.copy_mib << 20
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
