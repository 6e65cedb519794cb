#!/usr/bin/env python3
"""Throughput of the tiled GEMM / GEMV library on one MI355X.

Default run: the headline workload, a bf16 GEMM C = A . B with
M = N = K = 4096 (NN, fp32 output, no bias), timed over --steps launches
after --warmup untimed ones, with the inputs resident in HBM and rotated over
several copies so consecutive launches do not hit in the 256 MiB MALL.  One
JSON line is printed with:
  value      TFLOP/s = 2 M N K / t  (the metric of the "GEMM to FlashAttention"
             page's benchmark listing and roofline section),
  roofline   achieved vs the dense bf16 MFMA peak (2516.6 TFLOP/s),
  gemv       the M = 1 decode GEMV (W 4096 x 4096 bf16, + bias, bf16 y) in
             GB/s of algorithmic bytes vs 8 TB/s HBM, rotated over 20 copies
             of W (640 MiB > MALL),
  cpu_baseline  the fp64 oracle on the host cores over a bounded row sample
             of the same product (the sample's GPU rows are also compared).

--workload picks another workload (linear layers, attention products, fp8,
ragged shapes, fp32) and prints its line in the same form; --gpus > 1 is not
supported (one GPU per process, nothing is sharded here).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (2MNK/t) bf16 4096³ and % of MFMA peak; GEMV GB/s % HBM peak"

# MI355X published peaks (dense, no sparsity).
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
BYTES = {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1}


# ---------------------------------------------------------------- algorithmic work


def gemm_flops(M, N, K, batch=1):
    """2 M N K per problem: one multiply and one add per term of every sum."""
    return 2.0 * M * N * K * batch


def gemm_bytes(M, N, K, in_bytes, out_bytes, batch=1, bias=False):
    """Compulsory traffic: read A and B once, write C once (+ the fp32 bias)."""
    return float(batch * ((M * K + K * N) * in_bytes + M * N * out_bytes) + (4 * N if bias else 0))


def intensity(M, N, K, in_bytes, out_bytes=None):
    """FLOP per compulsory byte (the arithmetic intensity of the roofline model)."""
    out_bytes = in_bytes if out_bytes is None else out_bytes
    return gemm_flops(M, N, K) / gemm_bytes(M, N, K, in_bytes, out_bytes)


def tile_count(M, N, bm, bn):
    """Output tiles of an M x N result cut into bm x bn tiles (partial edge tiles count)."""
    return -(-M // bm) * -(-N // bn)


def roofline_time(flops, nbytes, peak_tflops, peak_gbs=PEAK_HBM_GBS):
    """Lower bound on time: min(peak, bandwidth x intensity) turned into seconds."""
    return max(flops / (peak_tflops * 1e12), nbytes / (peak_gbs * 1e9))


# ---------------------------------------------------------------- workloads

WORKLOADS = {
    # name: (M, N, K, batch, in, out, trans_b, bias)
    "square_bf16": (4096, 4096, 4096, 1, "bf16", "f32", False, False),
    "qkv": (8192, 12288, 4096, 1, "bf16", "bf16", True, True),
    "ffn_up": (8192, 14336, 4096, 1, "bf16", "bf16", True, True),
    "ffn_down": (8192, 4096, 14336, 1, "bf16", "bf16", True, True),
    "attn_scores": (2048, 2048, 128, 128, "f16", "f16", True, False),
    "attn_output": (2048, 128, 2048, 128, "f16", "f16", False, False),
    "fp8_square": (8192, 8192, 8192, 1, "e4m3", "bf16", False, False),
    "ragged_1000x3000x777": (1000, 3000, 777, 1, "bf16", "bf16", False, False),
    "ragged_4097x511x1023": (4097, 511, 1023, 1, "bf16", "bf16", False, False),
    "f32_256": (256, 256, 256, 1, "f32", "f32", False, False),
    "gemv": (1, 4096, 4096, 1, "bf16", "bf16", True, True),
    # skinny M: batched decode through one 4096 x 4096 linear layer (the GEMM
    # page's batch-size table), fp16 as there, + bias
    "skinny_m4": (4, 4096, 4096, 1, "f16", "f16", True, True),
    "skinny_m16": (16, 4096, 4096, 1, "f16", "f16", True, True),
    "skinny_m64": (64, 4096, 4096, 1, "f16", "f16", True, True),
    "skinny_m256": (256, 4096, 4096, 1, "f16", "f16", True, True),
    # the same layer through tmm_gemm_splitk (K in 4 slices, workspace
    # allocated outside the timed region); slices in SPLITK below
    "skinny_m256_splitk": (256, 4096, 4096, 1, "f16", "f16", True, True),
    # full BLAS form (tmm_gemm_ex), options in FULL_FORM below
    "ffn_up_relu": (8192, 14336, 4096, 1, "bf16", "bf16", True, True),
    "ffn_down_residual": (8192, 4096, 14336, 1, "bf16", "bf16", True, True),
    "wgrad_qkv": (4096, 12288, 8192, 1, "bf16", "f32", False, False),
    # fused convolution as an implicit GEMM: (GEMM rows = pixels, filters,
    # R S C, 1, in, out, -, -); the full shape is in CONV below
    "conv_listing": (8 * 64 * 64, 64, 9 * 32, 1, "bf16", "f32", True, True),
    "conv_large": (64 * 64 * 64, 128, 9 * 64, 1, "bf16", "bf16", True, True),
    # fused attention: (Nq queries, Nk keys, D head size, batch x heads, in, out, -, -)
    "attn_fused": (2048, 2048, 128, 128, "f16", "f16", True, False),
}

ATTENTION = ("attn_fused",)

# Split-K workloads: K slices of tmm_gemm_splitk.
SPLITK = {"skinny_m256_splitk": 4}

# Fused stride-1 convolutions (NHWC): the conv_fused listing's problem of the
# Lecture 27 notes (batch 8, 64 x 64, 32 -> 64 channels, 3 x 3, one-pixel
# halo, scale 1 + 0.01 f, bias 0.5, ReLU, 2 x 2 max pool; bf16 inputs, fp32
# output as there) and the same layer at batch 64 with 64 -> 128 channels.
CONV = {
    "conv_listing": dict(N=8, H=64, W=64, C=32, K=64, R=3, S=3, pad=1, pool=2),
    "conv_large": dict(N=64, H=64, W=64, C=64, K=128, R=3, S=3, pad=1, pool=2),
}

# Full-form options: a linear layer with a fused ReLU; FFN-down adding its
# output onto the residual stream (beta = 1, C read); the weight gradient of
# the QKV projection, dW = X^T . dY with X (tokens x in) stored as is
# (trans_a), fp32 gradient.
FULL_FORM = {
    "ffn_up_relu": {"relu": True},
    "ffn_down_residual": {"beta": 1.0},
    "wgrad_qkv": {"trans_a": True},
}


def attention_flops(Nq, Nk, D, batch=1):
    """Two products per head, S = Q K^T and O = P V: 2 Nq Nk D each."""
    return 4.0 * Nq * Nk * D * batch


def attention_bytes(Nq, Nk, D, in_bytes, out_bytes, batch=1):
    """Compulsory traffic: read Q, K and V once, write O once."""
    return float(batch * ((Nq + 2 * Nk) * D * in_bytes + Nq * D * out_bytes))


def work(name):
    """(algorithmic flops, algorithmic bytes) of one launch of a workload."""
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    if name in ATTENTION:
        return attention_flops(M, N, K, Z), attention_bytes(M, N, K, BYTES[fin], BYTES[fout], Z)
    if name in CONV:
        c = CONV[name]
        OH = (c["H"] + 2 * c["pad"] - c["R"] + 1) // c["pool"]
        OW = (c["W"] + 2 * c["pad"] - c["S"] + 1) // c["pool"]
        nbytes = (c["N"] * c["H"] * c["W"] * c["C"] + c["K"] * c["R"] * c["S"] * c["C"]) * BYTES[fin] \
            + c["N"] * OH * OW * c["K"] * BYTES[fout] + 8 * c["K"]
        return gemm_flops(M, N, K), float(nbytes)
    nbytes = gemm_bytes(M, N, K, BYTES[fin], BYTES[fout], Z, bias)
    if FULL_FORM.get(name, {}).get("beta"):
        nbytes += float(Z * M * N * BYTES[fout])   # the old C is read
    return gemm_flops(M, N, K, Z), nbytes


def describe(name):
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    lay = "NT" if tb else "NN"
    b = f"batch {Z} x " if Z > 1 else ""
    if name == "gemv":
        return f"{fin} GEMV y = W.x + bias, W {N}x{K}, {fout} y"
    if name in CONV:
        c = CONV[name]
        return (f"{fin} fused conv NHWC {c['N']}x{c['H']}x{c['W']}x{c['C']} -> {c['K']}, "
                f"{c['R']}x{c['S']} pad {c['pad']}, scale+bias+ReLU+{c['pool']}x{c['pool']} max pool, {fout} out")
    if name in FULL_FORM:
        o = FULL_FORM[name]
        lay = ("T" if o.get("trans_a") else "N") + ("T" if tb else "N")
        extra = (", ReLU" if o.get("relu") else "") + (f", + {o['beta']} C" if o.get("beta") else "")
        return f"{fin} GEMM {M}x{N}x{K} {lay}, {fout} out{', fp32 bias' if bias else ''}{extra}"
    if name in ATTENTION:
        return (f"{fin} fused attention softmax(Q K^T/sqrt(D)) V, batch x heads {Z}, "
                f"{M} queries x {N} keys, head size {K}, {fout} out")
    sk = f", split-K {SPLITK[name]}" if name in SPLITK else ""
    return f"{fin} GEMM {b}{M}x{N}x{K} {lay}, {fout} out{', fp32 bias' if bias else ''}{sk}"


def make_inputs(name, copies, dev):
    """Seeded synthetic operands of a workload, `copies` distinct device copies."""
    import torch

    import synthetic as syn
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    if name in ATTENTION:
        # N(0,1) Q, K, V of batch x heads independent heads (the attention shapes)
        Q, Kt, V = (syn.to_bits(syn.normal(shape, syn.seed_of(6, t)), fin)
                    for t, shape in (("A", (Z, M, K)), ("B", (Z, N, K)), ("V", (Z, N, K))))
        hQ, hK, hV = (syn.as_torch(X, fin) for X in (Q, Kt, V))
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[fout]
        sets = [(hQ.to(dev), hK.to(dev), hV.to(dev), torch.empty((Z, M, K), dtype=tdt, device=dev))
                for _ in range(copies)]
        return sets, None, (Q, Kt, V, 1.0, 1.0)
    if name in CONV:
        c = CONV[name]
        x = syn.to_bits(syn.uniform((c["N"], c["H"], c["W"], c["C"]), syn.seed_of(9, "A")), fin)
        w = syn.to_bits(syn.uniform((c["K"], c["R"], c["S"], c["C"]), syn.seed_of(9, "B")), fin)
        sc = (1.0 + 0.01 * np.arange(c["K"])).astype(np.float32)
        bi = np.full(c["K"], 0.5, dtype=np.float32)
        OH = (c["H"] + 2 * c["pad"] - c["R"] + 1) // c["pool"]
        OW = (c["W"] + 2 * c["pad"] - c["S"] + 1) // c["pool"]
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[fout]
        hx, hw = syn.as_torch(x, fin), syn.as_torch(w, fin)
        sets = [(hx.to(dev), hw.to(dev), torch.empty((c["N"], OH, OW, c["K"]), dtype=tdt, device=dev))
                for _ in range(copies)]
        return sets, (torch.from_numpy(sc).to(dev), torch.from_numpy(bi).to(dev)), (x, w, (sc, bi), 1.0, 1.0)
    if name in FULL_FORM and FULL_FORM[name].get("trans_a"):
        xa = syn.normal((K, M), syn.seed_of(8, "A"))   # stored K x M (tokens x in)
        xb = syn.normal((K, N), syn.seed_of(8, "B"))
        A, B = syn.to_bits(xa, fin), syn.to_bits(xb, fin)
        hA, hB = syn.as_torch(A, fin), syn.as_torch(B, fin)
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[fout]
        sets = [(hA.to(dev), hB.to(dev), torch.empty((M, N), dtype=tdt, device=dev)) for _ in range(copies)]
        return sets, None, (A, B, None, 1.0, 1.0)
    cfg = {"square_bf16": 2, "qkv": 3, "ffn_up": 3, "ffn_down": 3, "gemv": 3, "attn_scores": 4,
           "attn_output": 4, "fp8_square": 5}.get(name, 7 if name.startswith("skinny") else 5)
    ashape = (Z, M, K) if Z > 1 else (M, K)
    bshape = ((Z, N, K) if tb else (Z, K, N)) if Z > 1 else ((N, K) if tb else (K, N))
    sa = sb = 1.0
    if name == "attn_output":
        A = syn.softmax_rows_f16(Z, M, syn.seed_of(4, "logits"))
        B = syn.to_bits(syn.normal(bshape, syn.seed_of(4, "V")), fin)
    elif fin == "e4m3":
        xa = syn.normal(ashape, syn.seed_of(cfg, "A"))
        xb = syn.normal(bshape, syn.seed_of(cfg, "B"))
        sa, sb = syn.e4m3_scale(xa), syn.e4m3_scale(xb)
        A, B = syn.quantize_e4m3(xa, sa), syn.quantize_e4m3(xb, sb)
    else:
        wstd = 0.02 if tb and Z == 1 else 1.0   # linear-layer weights ~ N(0, 0.02^2)
        xa = syn.normal(ashape, syn.seed_of(cfg, "A"))
        xb = syn.normal(bshape, syn.seed_of(cfg, "B"), std=wstd)
        A, B = syn.to_bits(xa, fin), syn.to_bits(xb, fin)
    bvec = syn.normal((N,), syn.seed_of(cfg, "bias"), 0.02) if bias else None
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[fout]
    sets = []
    hA, hB = syn.as_torch(A, fin), syn.as_torch(B, fin)
    for _ in range(copies):
        dA, dB = hA.to(dev), hB.to(dev)
        dC = torch.empty((Z, M, N) if Z > 1 else (M, N), dtype=tdt, device=dev)
        sets.append((dA, dB, dC))
    dbias = torch.from_numpy(bvec).to(dev) if bvec is not None else None
    if FULL_FORM.get(name, {}).get("beta"):
        for _, _, dC in sets:   # an old C to add onto (the residual stream)
            dC.copy_(torch.randn(dC.shape, device=dev).to(dC.dtype))
    return sets, dbias, (A, B, bvec, float(sa), float(sb))


def launcher(name, sets, dbias, sa, sb):
    import tiled_matrix_multiplication_amd as tmm
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    if name in CONV:
        c = CONV[name]
        sc, bi = dbias

        def run(i):
            x, w, out = sets[i % len(sets)]
            tmm.tmm_conv2d_fused(x, w, out, c["pad"], scale=sc, bias=bi, relu=True, pool=c["pool"])
        return run
    if name in FULL_FORM:
        o = FULL_FORM[name]

        def run(i):
            A, B, C = sets[i % len(sets)]
            tmm.tmm_gemm_ex(A, B, C, bias=dbias, trans_a=o.get("trans_a", False), trans_b=tb,
                            beta=o.get("beta", 0.0), relu=o.get("relu", False))
        return run
    if name in ATTENTION:
        scale = float(K) ** -0.5

        def run(i):
            Q, Kt, V, O = sets[i % len(sets)]
            tmm.tmm_attention_fwd(Q, Kt, V, O, scale=scale)
    elif name == "gemv":
        def run(i):
            W, x, y = sets[i % len(sets)]
            tmm.tmm_gemv(W, x.view(-1)[:K], y.view(-1), bias=dbias)
    elif name in SPLITK:
        import torch
        S = SPLITK[name]
        ws = torch.empty(tmm.splitk_workspace_bytes(M, N, S) // 4, dtype=torch.float32,
                         device=sets[0][0].device)

        def run(i):
            A, B, C = sets[i % len(sets)]
            tmm.tmm_gemm_splitk(A, B, C, bias=dbias, trans_b=tb, splits=S, workspace=ws)
    elif Z > 1:
        def run(i):
            A, B, C = sets[i % len(sets)]
            tmm.tmm_gemm_strided_batched(A, B, C, bias=dbias, trans_b=tb)
    else:
        def run(i):
            A, B, C = sets[i % len(sets)]
            tmm.tmm_gemm(A, B, C, bias=dbias, trans_b=tb, scale_a=sa, scale_b=sb)
    return run


SETTLE_S = 0.15


def settle(run):
    """Keep the GPU busy for SETTLE_S seconds of wall time before anything is
    timed: from idle, the chip's clock ramps up over the first ~30 ms of
    sustained load (4096^3 bf16: 155 us per launch at first, 125 us after
    ~30 ms), so a short warmup would time the ramp rather than the kernel."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < SETTLE_S and i < 100000:
        for _ in range(8):
            run(i)
            i += 1
        torch.cuda.synchronize()
    return i


def time_steps(run, steps, warmup):
    """Average ms per launch from HIP events on the launching (current) stream,
    after the clock has settled and `warmup` untimed launches."""
    import torch
    settle(run)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        run(warmup + i)
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


# Launches per captured graph: a replay has a fixed cost of its own, spread
# over the launches it holds (1000 against 100 took the decode GEMV from
# 7.42 to 7.34 us per launch).
GRAPH_LAUNCHES = 1000

# Workloads whose kernel runs for less than the host cost of an eager call
# (~20-30 us from Python through ctypes): timed as graph replays, so that
# the figure is the kernel's and not the launch loop's.
GRAPH_TIMED = {"gemv", "conv_listing", "ragged_1000x3000x777", "ragged_4097x511x1023", "f32_256"}


def time_graph(run, launches, replays, warmup):
    """Average ms per launch of `launches` calls captured once in a HIP graph and
    replayed `replays` times (HIP events on the replaying stream).  Removes the
    host cost of each eager call (Python, ctypes, stream query), which for a
    ~10 us kernel is as long as the kernel itself."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        settle(run)
        for i in range(warmup):
            run(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(launches):
            run(i)
    graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    end.record()
    end.synchronize()
    ms = start.elapsed_time(end) / (replays * launches)
    del graph
    return ms


def _smi_handle(amdsmi):
    """The amdsmi handle of cuda:0 (matched by PCI address where torch
    reports it, else the first GPU amdsmi lists)."""
    import torch
    handles = amdsmi.amdsmi_get_processor_handles()
    try:
        pr = torch.cuda.get_device_properties(0)
        want = (int(pr.pci_domain_id), int(pr.pci_bus_id), int(pr.pci_device_id))
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
            dom, bus, rest = bdf.split(":")
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                return h
    except Exception:  # noqa: BLE001 (older torch without PCI fields)
        pass
    return handles[0]


def gpu_state_under_load(run, seconds=1.0):
    """GFX clock of each XCD and the socket power while `run` keeps the GPU
    busy back to back (after the timed region), read in this process through
    the amdsmi library (no other program is started), or None where it is
    missing or fails.  Under sustained load the clock may settle below its
    2.4 GHz maximum, which the MFMA roofline's peak assumes."""
    import threading

    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = _smi_handle(amdsmi)
    except Exception:  # noqa: BLE001 (any failure: report nothing)
        return None
    got = {}

    def sample():
        time.sleep(seconds / 2)
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            got["clocks"] = [int(c) for c in m["current_gfxclks"] if isinstance(c, int) and 0 < c < 65535]
            got["power"] = m.get("current_socket_power")
        except Exception as e:  # noqa: BLE001
            got["err"] = repr(e)

    th = threading.Thread(target=sample)
    th.start()
    t0 = time.perf_counter()
    i = 0
    while th.is_alive() and time.perf_counter() - t0 < seconds + 20:
        for _ in range(8):
            run(i)
            i += 1
        torch.cuda.synchronize()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    if not got.get("clocks"):
        return None
    power = got.get("power")
    return {"gfx_clock_mhz": got["clocks"],
            "socket_power_w": power if isinstance(power, int) and 0 < power < 65535 else None,
            "source": "amdsmi GPU metrics (in process), read once while the timed kernel ran back to back"}


def read_ceiling(rows=4096, row_bytes=8192, copies=18, waves=(4, 8, 16)):
    """The GEMV's weight stream alone (include/tmm_probes.h, tmmp_stream_read):
    W's bytes read once with the GEMV's launch shape and access pattern and
    no arithmetic, over `copies` rotated buffers, timed like the GEMV (launches
    in a HIP graph).  For each waves-per-workgroup setting: microseconds per
    launch and GB/s; the best is the measured ceiling the GEMV is set against."""
    import torch

    import synthetic as syn
    import tiled_matrix_multiplication_amd.probes as probes
    n = rows * row_bytes // 2
    base = syn.as_torch(syn.to_bits(syn.normal((rows, row_bytes // 2), 7001, 0.02), "bf16"), "bf16").to("cuda:0")
    bufs = [base.clone().view(-1) for _ in range(copies)]
    assert bufs[0].numel() == n
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    out = {}
    for w in waves:
        def run(i, w=w):
            probes.stream_read(bufs[i % copies], rows, row_bytes, w, sink)
        ms = time_graph(run, GRAPH_LAUNCHES, 5, 20)
        out[w] = {"us_per_launch": round(ms * 1e3, 3), "GB/s": round(rows * row_bytes / (ms * 1e-3) / 1e9, 1)}
    best = min(out, key=lambda w: out[w]["us_per_launch"])
    del bufs, base
    return {"bytes_per_launch": rows * row_bytes, "copies_rotated": copies,
            "timing": f"{GRAPH_LAUNCHES} launches captured in one HIP graph, replayed",
            "by_waves_per_group": {str(w): out[w] for w in waves}, "best_waves_per_group": best,
            "us_per_launch": out[best]["us_per_launch"], "achieved": out[best]["GB/s"], "unit": "GB/s",
            "frac_of_peak": round(out[best]["GB/s"] / PEAK_HBM_GBS, 4)}


def mfma_ceiling(flops=2.0 * 4096 ** 3):
    """The matrix cores alone (include/tmm_probes.h, tmmp_mfma_loop): the
    headline's flops as matrix instructions on register-resident operands
    (no loads, no LDS, no stores), 256 workgroups of 8 waves, for each
    instruction shape: bf16 N(0,1) and zeros, fp8 e4m3 from N(0, 16^2).
    Random operands draw more power than zeros, and the chip lowers its
    clock to stay within its power limit, so this is the rate a GEMM on such
    data can approach, below the published peak."""
    import torch

    import tiled_matrix_multiplication_amd.probes as probes
    groups = 256
    iters = int(round(flops / (groups * 8 * (1 << 20))))
    iters -= iters % 4
    g = torch.Generator(device="cuda:0")
    g.manual_seed(7002)
    ops = torch.randn(1 << 25, device="cuda:0", generator=g).to(torch.bfloat16)
    zeros = torch.zeros_like(ops)
    ops8 = (torch.randn(1 << 26, device="cuda:0", generator=g) * 16).to(torch.float8_e4m3fn)
    sink = torch.empty(groups * 512, dtype=torch.float32, device="cuda:0")
    out = {}
    cases = (("random", ops, 1, "16x16x32", "bf16"), ("random", ops, 0, "32x32x16", "bf16"),
             ("zeros", zeros, 1, "16x16x32", "bf16"), ("zeros", zeros, 0, "32x32x16", "bf16"),
             ("random_fp8", ops8, 3, "16x16x128", "e4m3"), ("random_fp8", ops8, 2, "32x32x64", "e4m3"))
    for label, data, shape, name, fmt in cases:
        def run(i, shape=shape, data=data):
            probes.mfma_loop(data, shape, groups, iters, sink)
        ms, _ = time_steps(run, 50, 5)
        tf = groups * 8 * iters * (1 << 20) / (ms * 1e-3) / 1e12
        out[f"{label}_{name}"] = {"us_per_launch": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                                  "frac_of_peak": round(tf / PEAK_TFLOPS[fmt], 4)}
    del ops, zeros, ops8
    return out


def copies_for(name):
    """Enough distinct input copies that a launch finds its operands out of the MALL."""
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    per = work(name)[1] if (name in ATTENTION or name in CONV) \
        else Z * ((M * K + K * N) * BYTES[fin] + M * N * BYTES[fout])
    return int(max(1, min(20, np.ceil(600e6 / per))))


def measure(name, steps, warmup, dev):
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    copies = copies_for(name)
    if name == "gemv":
        import torch

        import synthetic as syn
        W = syn.to_bits(syn.normal((N, K), syn.seed_of(3, "B"), 0.02), fin)
        x = syn.to_bits(syn.normal((1, K), syn.seed_of(3, "A")), fin)
        hW, hx = syn.as_torch(W, fin), syn.as_torch(x, fin)
        sets = [(hW.to(dev), hx.to(dev), torch.empty((N,), dtype=torch.bfloat16, device=dev))
                for _ in range(copies)]
        dbias = torch.from_numpy(syn.normal((N,), syn.seed_of(3, "bias"), 0.02)).to(dev)
        host = (x, W, None, 1.0, 1.0)
        sa = sb = 1.0
    else:
        sets, dbias, host = make_inputs(name, copies, dev)
        sa, sb = host[3], host[4]
    run = launcher(name, sets, dbias, sa, sb)
    ms, wall = time_steps(run, steps, warmup)
    flops, nbytes = work(name)
    out = {"ms": ms, "wall": wall, "flops": flops, "bytes": nbytes, "copies": copies,
           "sets": sets, "host": host}
    if name in GRAPH_TIMED or name.startswith("skinny"):
        # the eager call is host-bound at this size: time the kernel in a graph
        out["ms_eager"] = ms
        out["ms"] = time_graph(run, GRAPH_LAUNCHES, max(2, steps // 500), warmup)
    return out


def roofline_entry(name, r):
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    t = r["ms"] * 1e-3
    ai = r["flops"] / r["bytes"]
    ridge = PEAK_TFLOPS[fin] * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = traffic_from_profile(name)
    if ai >= ridge:
        ach = r["flops"] / t / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_TFLOPS[fin], "unit": "TFLOP/s",
                "frac": round(ach / PEAK_TFLOPS[fin], 4), "traffic": traffic}
    ach = r["bytes"] / t / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}


# ---------------------------------------------------------------- HBM traffic

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "tiled_matrix_multiplication_amd", "csrc")


# Sources that define each workload's dominant kernel (the host dispatch and
# the shared parameter header are not part of it).
KERNEL_SOURCES = {
    "gemm": ["gemm_mfma.h", "gemm_ring.h", "gemm_quad.h", "gemm_quad8.h", "load_words.h", "gemm_f32.hip",
             "gemm_bf16.hip", "gemm_f16.hip", "gemm_f8.hip", "gemm_ring_ta.hip"],
    "shortk": ["gemm_mfma.h", "gemm_ring.h", "gemm_short_k.hip"],
    "gemv": ["gemv.hip"],
    "skinny": ["gemm_skinny.hip"],
    "attention": ["attention.hip"],
    "conv": ["conv_implicit.hip", "conv_quad.h", "gemm_quad.h", "gemm_ring.h", "gemm_mfma.h"],
    "splitk": ["gemm_mfma.h", "gemm_ring.h", "gemm_quad.h", "gemm_quad8.h", "load_words.h", "gemm_f32.hip",
               "gemm_bf16.hip", "gemm_f16.hip", "gemm_f8.hip", "gemm_ring_ta.hip", "splitk.hip"],
    "f32small": ["gemm_f32_small.hip"],
}


# Largest M the library sends to its several-row GEMV (gemv.hip) rather than
# the skinny MFMA kernel; the traffic hash and the counter filter follow it.
GEMV_MULTI_MAX_M = 4


def kernel_family(name):
    if name == "gemv":
        return "gemv"
    if name in ATTENTION:
        return "attention"
    if name in SPLITK:
        return "splitk"
    if name.startswith("skinny"):
        return "gemv" if WORKLOADS[name][0] <= GEMV_MULTI_MAX_M else "skinny"
    if name in CONV:
        return "conv"
    if name == "f32_256":
        return "f32small"   # fp32 256^3: the small-product kernel (gemm_f32_small.hip)
    if name == "attn_scores":
        return "shortk"     # Q.K^T over whole 256x256 tiles: the persistent short-K kernel
    return "gemm"


def code_without_comments(text):
    """C++ source with // and /* */ comments and blank runs removed (string
    literals in these sources hold no comment markers), so that an edit to a
    comment does not count as a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(name):
    """Hash of the code (comments aside) of the workload's kernel sources:
    counter-derived traffic is only reported for the kernel code it was
    measured on."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_family(name)]:
        h.update(f.encode())
        h.update(code_without_comments(open(os.path.join(CSRC, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def traffic_path(name):
    return os.path.join(PROFILES, f"traffic_{name}.json")


def traffic_from_profile(name):
    """HBM bytes per launch from profiles/traffic_<name>.json, or None when
    absent or measured on other kernel sources."""
    path = traffic_path(name)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    return d["bytes_per_launch"] if d.get("source_hash") == kernel_source_hash(name) else None


def _counter_per_dispatch(csv_path, counter, kernel_substr):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"{csv_path}: no {counter} rows for kernels matching {kernel_substr!r}")
    return sum(vals) / len(vals), len(vals)


def summarize_pmc(name, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes,
                  kernel_substr="gemm_", copy_substr="copy"):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the workload's kernel by
    what the same counters read for a plain copy of `copy_bytes` bytes."""
    if kernel_family(name) == "gemv":
        kernel_substr = "gemv"
    elif name in ATTENTION:
        kernel_substr = "attn_fwd"
    elif name in SPLITK:
        kernel_substr = "gemm_"   # the partial products; the sum kernel is added below
    elif name.startswith("skinny"):
        kernel_substr = "gemm_skinny"
    elif name in CONV:
        kernel_substr = "conv_"   # conv_implicit_kernel or conv_quad_kernel
    f_k, nf = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel_substr)
    w_k, nw = _counter_per_dispatch(write_csv, "WRITE_SIZE", kernel_substr)
    if name in SPLITK:   # one call = the partial-product kernel + the sum kernel
        f_k += _counter_per_dispatch(fetch_csv, "FETCH_SIZE", "splitk_reduce")[0]
        w_k += _counter_per_dispatch(write_csv, "WRITE_SIZE", "splitk_reduce")[0]
    f_c, _ = _counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", copy_substr)
    w_c, _ = _counter_per_dispatch(copy_write_csv, "WRITE_SIZE", copy_substr)
    fetch_scale = copy_bytes / f_c     # bytes per counter unit, from the copy's reads
    write_scale = copy_bytes / w_c
    out = {"workload": describe(name), "source_hash": kernel_source_hash(name),
           "hash_covers": KERNEL_SOURCES[kernel_family(name)],
           "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k, "dispatches": [nf, nw],
           "copy_bytes": copy_bytes, "copy_fetch_kib": f_c, "copy_write_kib": w_c,
           "fetch_bytes": f_k * fetch_scale, "write_bytes": w_k * write_scale,
           "bytes_per_launch": f_k * fetch_scale + w_k * write_scale}
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    out["algorithmic_bytes"] = work(name)[1]
    os.makedirs(PROFILES, exist_ok=True)
    json.dump(out, open(traffic_path(name), "w"), indent=1)
    print(json.dumps(out))


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of `nbytes` (torch's copy kernel), for
    calibrating the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": steps}))


# ---------------------------------------------------------------- CPU baseline


def compare_rows(C, idx, o):
    """Relative Frobenius difference of GPU output rows `idx` from oracle rows `o`."""
    import torch
    g = C[torch.as_tensor(idx, device=C.device)].float().cpu().numpy().astype(np.float64)
    den = float(np.linalg.norm(o))
    return float(np.linalg.norm(g - o) / den) if den > 0 else float(np.linalg.norm(g - o))


def cpu_baseline(name, r, target_s=20.0):
    """The oracle, as it stands, on a row sample of the workload's first problem.

    Times it on the host cores (OpenMP threads), scales to the metric's unit,
    and compares the sampled GPU rows against it."""
    import oracle
    if name in ATTENTION:
        return cpu_baseline_attention(name, r, target_s)
    if name in FULL_FORM:
        return cpu_baseline_full(name, r, target_s)
    if name in CONV:
        return cpu_baseline_conv(name, r, target_s)
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    A, B, bvec, sa, sb = r["host"]
    if Z > 1:
        A, B = A[0], B[0]
    rng = np.random.default_rng(12345)

    def run_rows(rows):
        idx = np.sort(rng.choice(M, size=rows, replace=False)) if rows < M else np.arange(M)
        t0 = time.perf_counter()
        o = oracle.gemm(fin, np.ascontiguousarray(A[idx]), B, trans_b=tb, bias=bvec, scale_a=sa, scale_b=sb)
        return idx, o, time.perf_counter() - t0

    # two small runs separate the fixed cost (decoding B) from the per-row cost
    idx, o, t8 = run_rows(min(M, 8))
    if M > 8:
        idx, o, t64 = run_rows(min(M, 64))
        per_row = max((t64 - t8) / max(min(M, 64) - 8, 1), 1e-6)
        rows = int(min(M, max(64, (target_s - t8) / per_row)))
        if rows > len(idx):
            idx, o, t = run_rows(rows)
        else:
            t = t64
    else:
        t = t8
    flops = gemm_flops(len(idx), N, K)
    C = r["sets"][0][2]
    C0 = C[0] if Z > 1 else C
    err = compare_rows(C0, idx, o)
    line = {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds": round(t, 2),
            "sample": (f"{len(idx)} of {M} rows" if len(idx) < M else f"all {M} rows") +
                      f" of the {describe(name)} product ({len(idx)}x{N}x{K}, fp64 triple loop; "
                      f"time includes decoding the inputs)",
            "sample_rel_fro_vs_gpu": err, **host_cpus()}
    if name == "square_bf16":
        line["single_core"] = single_core_1024()
        line["page_context"] = page_cpu_figures()
    return line


def host_cpus():
    """CPUs of the host: all of them, and those this process may run on."""
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:  # noqa: BLE001
        usable = os.cpu_count()
    return {"nproc": usable, "host_cpus": os.cpu_count()}


def single_core_1024():
    """The oracle on one thread for a 1024^3 bf16 product (the same inputs'
    recipe as the square workload), and that time times 64 -- the 4096^3
    product has 64 times the multiply-adds -- as the one-core estimate."""
    import oracle
    import synthetic as syn
    n = 1024
    A = syn.to_bits(syn.normal((n, n), syn.seed_of(2, "A")), "bf16")
    B = syn.to_bits(syn.normal((n, n), syn.seed_of(2, "B")), "bf16")
    before = oracle.threads()
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.gemm("bf16", A, B)
        t = time.perf_counter() - t0
    finally:
        oracle.set_threads(before)
    return {"seconds_1024": round(t, 3), "tflops": round(gemm_flops(n, n, n) / t / 1e12, 6), "threads": 1,
            "extrapolated_4096_seconds": round(64 * t, 1),
            "note": "4096^3 has 64x the multiply-adds of 1024^3"}


def page_cpu_figures():
    """The pages' CPU FP32 times for N = 4096 (context only)."""
    try:
        with open(os.path.join(ROOT, "tests", "golden", "page_figures.json")) as f:
            d = json.load(f)["cpu_fp32_4096_seconds"]
        return {"seconds": d["printed"], "source": d["source"].split(":")[0]}
    except Exception:  # noqa: BLE001
        return None


def cpu_baseline_full(name, r, target_s=20.0):
    """The oracle's full form on a row sample (rows of op(A)).  The sample is
    compared with the GPU rows unless beta != 0 (the timed launches kept
    adding onto C, so the GPU's C is not one launch's result)."""
    import oracle
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    o = FULL_FORM[name]
    A, B, bvec, sa, sb = r["host"]
    ta = o.get("trans_a", False)
    rng = np.random.default_rng(12345)

    def run_rows(rows):
        idx = np.sort(rng.choice(M, size=rows, replace=False))
        a = np.ascontiguousarray(A[:, idx] if ta else A[idx])
        cin = np.zeros((rows, N)) if o.get("beta") else None
        t0 = time.perf_counter()
        out = oracle.gemm_ex(fin, a, B, ta, tb, 1.0, o.get("beta", 0.0), cin, bvec, o.get("relu", False))
        return idx, out, time.perf_counter() - t0

    idx, out, t8 = run_rows(8)
    idx, out, t64 = run_rows(64)
    per_row = max((t64 - t8) / 56, 1e-6)
    rows = int(min(M, max(64, (target_s - t8) / per_row)))
    t = t64
    if rows > len(idx):
        idx, out, t = run_rows(rows)
    err = None if o.get("beta") else compare_rows(r["sets"][0][2], idx, out)
    return {"value": round(gemm_flops(len(idx), N, K) / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.threads(), "kind": "oracle", "seconds": round(t, 2),
            "sample": f"{len(idx)} of {M} rows of the {describe(name)} product (fp64; time includes "
                      f"decoding the inputs)",
            "sample_rel_fro_vs_gpu": err}


def cpu_baseline_conv(name, r, target_s=20.0):
    """The oracle's direct convolution on whole images (1, 2, 4, ... until
    about target_s seconds), compared with the GPU's output for them."""
    import oracle
    c = CONV[name]
    x, w, (sc, bi), _, _ = r["host"]
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]
    n, t, out = 1, 0.0, None
    while True:
        t0 = time.perf_counter()
        out = oracle.conv2d(fin, x[:n], w, c["pad"], sc, bi, True, c["pool"])
        t = time.perf_counter() - t0
        if t * 2 > target_s or n * 2 > c["N"]:
            break
        n *= 2
    g = r["sets"][0][2][:n].float().cpu().numpy().astype(np.float64)
    den = float(np.linalg.norm(out))
    err = float(np.linalg.norm(g - out) / den) if den > 0 else float(np.linalg.norm(g - out))
    per_img = gemm_flops(M // c["N"], N, K)
    return {"value": round(per_img * n / t / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds": round(t, 2),
            "sample": f"{n} of {c['N']} images of the {describe(name)} workload (fp64 direct "
                      f"convolution; time includes decoding)",
            "sample_rel_fro_vs_gpu": err}


def cpu_baseline_attention(name, r, target_s=20.0):
    """The oracle's attention on whole heads (every query, key and value of
    heads 0, 1, ...): one head is timed first, then as many heads as fill
    about target_s seconds; scaled to TFLOP/s like the GPU figure."""
    import oracle
    Nq, Nk, D, Z, fin, fout, tb, bias = WORKLOADS[name]
    Q, Kt, V, _, _ = r["host"]
    scale = float(D) ** -0.5

    def run_heads(n):
        t0 = time.perf_counter()
        outs = [oracle.attention(fin, Q[z], Kt[z], V[z], scale) for z in range(n)]
        return outs, time.perf_counter() - t0

    outs, t1 = run_heads(1)
    n = int(min(Z, max(1, target_s // max(t1, 1e-3))))
    t = t1
    if n > 1:
        outs, t = run_heads(n)
    O = r["sets"][0][3]
    errs = [compare_rows(O[z], np.arange(Nq), outs[z]) for z in range(n)]
    return {"value": round(attention_flops(Nq, Nk, D, n) / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.threads(), "kind": "oracle", "seconds": round(t, 2),
            "sample": (f"{n} of {Z} heads of the {describe(name)} workload, every query, key and "
                       f"value of each (fp64, max-subtracted softmax; time includes decoding)"),
            "sample_rel_fro_vs_gpu": max(errs)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="square_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-gemv", action="store_true", help="skip the GEMV side measurement")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (matrix cores alone, the GEMV's read stream alone)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES, --steps times (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE/WRITE_SIZE outputs of --workload and of "
                         "--copy-calib into profiles/traffic_<workload>.json")
    ap.add_argument("--copy-bytes", type=int, default=0, help="bytes of the calibration copy")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc, copy_bytes=args.copy_bytes)
        return 0
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this library runs on one GPU per "
              "process and shards nothing (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calib:
        copy_calibration(args.copy_calib, args.steps)
        return 0
    import tiled_matrix_multiplication_amd  # noqa: F401  (fails loudly without libtmm.so)
    dev = "cuda:0"
    name = args.workload
    M, N, K, Z, fin, fout, tb, bias = WORKLOADS[name]

    r = measure(name, args.steps, args.warmup, dev)
    roof = roofline_entry(name, r)
    value = r["flops"] / (r["ms"] * 1e-3) / 1e12
    per = "4 Nq Nk D batch / t" if name in ATTENTION else "2MNK/t"
    line = {
        "metric": METRIC if name == "square_bf16" else f"{describe(name)}: TFLOP/s ({per})",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fin,
        "data": "synthetic",
        "config": {"workload": describe(name), "M": M, "N": N, "K": K, "batch": Z,
                   "layout": ("T" if FULL_FORM.get(name, {}).get("trans_a") else "N") + ("T" if tb else "N"),
                   "out": fout, "bias": bias,
                   "input_copies_rotated": r["copies"]},
        "roofline": roof,
    }
    if "ms_eager" in r:
        line["timing"] = {"kind": f"{GRAPH_LAUNCHES} launches captured in one HIP graph, replayed",
                          "ms_per_eager_call": round(r["ms_eager"], 5)}
    if name in CONV:
        line["metric"] = f"{describe(name)}: TFLOP/s (2 pixels K R S C / t)"
        line["config"] = dict(workload=describe(name), **CONV[name], input_copies_rotated=r["copies"])
    if name in ATTENTION:
        line["config"] = {"workload": describe(name), "Nq": M, "Nk": N, "D": K, "batch_heads": Z,
                          "out": fout, "scale": "1/sqrt(D)", "input_copies_rotated": r["copies"]}
    if name == "square_bf16" and not args.no_gemv:
        g = measure("gemv", max(1000, args.steps), max(20, args.warmup), dev)
        gbs = g["bytes"] / (g["ms"] * 1e-3) / 1e9
        line["gemv"] = {"workload": describe("gemv"), "us_per_launch": round(g["ms"] * 1e3, 3),
                        "timing": f"{GRAPH_LAUNCHES} launches captured in one HIP graph, replayed",
                        "us_per_eager_call": round(g["ms_eager"] * 1e3, 3),
                        "bytes_per_launch": int(g["bytes"]), "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "weight_copies_rotated": g["copies"], "traffic": traffic_from_profile("gemv")}
        del g
    if name == "square_bf16":
        line["gpu_state"] = gpu_state_under_load(launcher(name, r["sets"], None, 1.0, 1.0))
    if name == "square_bf16" and not args.no_ceilings:
        c = mfma_ceiling()
        best = max(v["TFLOP/s"] for k, v in c.items() if k.startswith("random_") and "fp8" not in k)
        line["mfma_ceiling"] = dict(c, note="bf16 matrix instructions alone on register-resident operands, the "
                                            "headline's flops; the chip's clock falls under random data",
                                    headline_frac_of_random_ceiling=round(value / best, 4))
        if "gemv" in line:
            rc = read_ceiling()
            line["gemv"]["read_ceiling"] = rc
            line["gemv"]["frac_of_read_ceiling"] = round(line["gemv"]["achieved"] / rc["achieved"], 4)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(name, r)
    line["wall_s_timed"] = round(r["wall"], 4)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
