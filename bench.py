#!/usr/bin/env python3
"""Benchmark of the activation-sparse expert FFN on one MI355X.

Workload: one Mixtral-8x7B-shaped SwiGLU expert (d=4096, f=14336), fp16 gate /
down rows, INT2 group-64 up weights, thresholds calibrated to 90% activation
sparsity, one token per call (decode).  A step is one call of
moe_expert_forward_sparse on one token: the fused kernel (INT2 up GEMV, mask,
compaction, gate/down row gathers, fused SiLU, partial rows) and the small
kernel that sums the partial rows into y.  Steps rotate over R distinct expert
instances (32 by default: between two visits to one instance the other 31
calls touch about 1.3 GB, five times the 256 MB Infinity Cache) and 16 tokens,
so the weights come from HBM, as they would when 32 layers x 8 experts are
resident.  Inputs are resident in HBM before the timed region starts; the K
launches are captured once in a HIP graph and replayed, so the host's launch
overhead is not what is measured.

Prints one JSON line.  --gpus above 1 is refused: the path runs on one GPU.
Besides the headline, the line carries "more" (the same expert at batch 4;
decode steps through the 32-layer Mixtral-shaped stack at 1 and 16 tokens and
through the fine-grained 64+2 layer at 1 and 64 tokens, router included) and
"batched" (the Mixtral-8x22B-shaped layer at 256 tokens on the dense MFMA path,
with MFMA utilisation, and on the sparse path); --no-layers / --no-batched skip
them.

``roofline.achieved`` is the algorithmic bytes of a call (INT2 up codes, fp16
scales and zeros, x, y, and the gate and down rows of the channels the mask
selects, counted from an identical untimed pass) divided by the event-timed
duration of the whole call, i.e. of both of its kernels.  ``roofline.traffic``
is the HBM traffic per call that rocprofv3 counted (FETCH_SIZE + WRITE_SIZE of
both kernels, each scaled by what the same counter reads for an elementwise
kernel of known size, ``--copy-probe``); it is read from the committed
counter summary and reported only while the kernel sources it was taken on
are unchanged (their SHA-256 is recorded there), else null.

``cpu_baseline`` is the fp64 oracle on the host cores (one thread, then N
threads of independent calls) on the headline workload; ``cpu_baseline.more``
times it the same way on the fine-grained layer and on one layer of the
32-layer stack (host copies of the device-built layers; the decode step of
the stack is extrapolated from that layer), and on the small d=256 expert.
"""
from __future__ import annotations

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

METRIC = "expert-FFN tokens/s + achieved HBM GB/s (d=4096,f=14336, 90% sparse, batch 1)"
HBM_PEAK_GBS = 8000.0
D, F = 4096, 14336
NTOK = 16
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_expert_sparse_mixtral_b1_s90.md")
KERNEL_SOURCES = ["expert_sparse.hpp", "expert_sparse_f16.hip", "reduce.hip", "internal.hpp",
                  "device.hpp", "route_common.hpp", "api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_instances(R, sparsity, dev):
    import torch
    import activation_sparse_expert_amd as moe
    import synth
    cfg = synth.CFG_MIXTRAL
    xs = synth.CONFIGS[cfg]["x_scale"]
    experts = []
    for i in range(R):
        g = synth.device_normal(synth.seed_of(cfg, 0, i, synth.T_GATE), (F, D), 0.02, dev, torch.float16)
        dn = synth.device_normal(synth.seed_of(cfg, 0, i, synth.T_DOWN), (F, D), 0.02, dev, torch.float16)
        u = synth.device_normal(synth.seed_of(cfg, 0, i, synth.T_UP), (F, D), 0.02, dev)
        q, sz = moe.pack_up_int2(u)
        del u
        ex = moe.Expert(q, sz, g, dn, float("inf"))
        # calibration: |v| of the 64 seeded calibration vectors, from the library
        xc = torch.from_numpy(synth.calibration_f32(cfg, D, xs, 0, i)).half().to(dev)
        v = torch.empty((64, F), dtype=torch.float32, device=dev)
        moe.expert_forward_sparse(ex, xc, v_out=v)
        torch.cuda.synchronize()
        ex.threshold = float(np.float32(np.quantile(np.abs(v.cpu().numpy()).ravel(), sparsity)))
        experts.append(ex)
        log(f"instance {i + 1}/{R} ready")
    return experts


def kernel_sources_sha():
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "activation_sparse_expert_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic():
    """HBM bytes per call from the committed counter summary, or None when
    there is none or the kernels changed since it was taken."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_call:\s*([0-9]+)", text)
    if not sha or not val or sha.group(1) != kernel_sources_sha():
        return None
    return int(val.group(1))


def copy_probe(mib):
    """Elementwise kernel of known size for scaling FETCH_SIZE / WRITE_SIZE:
    out = -src over `mib` MiB of fp32 (reads and writes exactly that much)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "kernel": "neg (elementwise)", "launches": 10}), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def batched_measure(reps=10, T=256, dense_only=False):
    """The batched layer: 8 experts (d=6144, f=16384, bf16), top-2, T tokens.
    Times moe_layer_forward on the dense bf16 MFMA path and on the 70%-sparse
    path (HIP events around `reps` calls each, after warm-up).  dense_only:
    the new dense path alone, 3 calls at T and at 2048 tokens (for profiling)."""
    import torch
    import activation_sparse_expert_amd as moe
    import synth
    cfg = synth.CFG_WIDE
    c = synth.CONFIGS[cfg]
    d, f, E, k = c["d"], c["f"], c["E"], c["k"]
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    gate = torch.empty((E, f, d), dtype=bf, device=dev)
    down = torch.empty((E, f, d), dtype=bf, device=dev)
    up_q = torch.empty((E, f, d // 4), dtype=torch.uint8, device=dev)
    up_sz = torch.empty((E, f, d // 64, 2), dtype=torch.int16, device=dev)
    up_dense = torch.empty((E, f, d), dtype=bf, device=dev)
    thr = torch.empty(E, dtype=torch.float32, device=dev)
    for e in range(E):
        gate[e].copy_(synth.device_normal(synth.seed_of(cfg, 0, e, synth.T_GATE), (f, d), 0.02, dev, bf))
        down[e].copy_(synth.device_normal(synth.seed_of(cfg, 0, e, synth.T_DOWN), (f, d), 0.02, dev, bf))
        u = synth.device_normal(synth.seed_of(cfg, 0, e, synth.T_UP), (f, d), 0.02, dev)
        moe.pack_up_int2(u, up_q=up_q[e], up_sz=up_sz[e])
        del u
        moe.materialize_up_bf16(up_q[e], up_sz[e], d, out=up_dense[e])
        ex = moe.Expert(up_q[e], up_sz[e], gate[e], down[e], float("inf"))
        xc = torch.from_numpy(synth.calibration_f32(cfg, d, c["x_scale"], 0, e)).to(bf).to(dev)
        v = torch.empty((64, f), dtype=torch.float32, device=dev)
        moe.expert_forward_sparse(ex, xc, v_out=v)
        torch.cuda.synchronize()
        thr[e] = float(np.quantile(np.abs(v.cpu().numpy()).ravel(), c["sparsity"]))
    R = torch.from_numpy(synth.router_f32(cfg, 0, E, d)).to(bf).to(dev)
    down_dense = moe.transpose_down(down)
    L = moe.Layer(d=d, f=f, E=E, S=0, k=k, renormalize=True, router_w=R, up_q=up_q, up_sz=up_sz,
                  gate_t=gate, down=down, thresholds=thr, up_dense=up_dense, down_dense=down_dense)
    L_rowmajor = moe.Layer(d=d, f=f, E=E, S=0, k=k, renormalize=True, router_w=R, up_q=up_q,
                           up_sz=up_sz, gate_t=gate, down=down, thresholds=thr, up_dense=up_dense)
    x = torch.from_numpy(synth.tokens_f32(cfg, T, d, c["x_scale"])).to(bf).to(dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    ws = moe.new_workspace(L.workspace_bytes(T), dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    out = {}
    L.density = 1.0 - c["sparsity"]          # union-density input of the AUTO / MIXED rules
    legs = (("dense_mfma", moe.PATH_DENSE, L),
            ("dense_mfma_rowmajor_down", moe.PATH_DENSE, L_rowmajor),
            ("sparse", moe.PATH_SPARSE, L),
            ("auto", moe.PATH_AUTO, L))
    if dense_only:
        legs, reps = legs[:1], 3
    for name, path, LL in legs:
        for _ in range(3):
            moe.layer_forward(LL, x, path=path, y=y, ws=ws, trace={"expert_count": cnt})
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            moe.layer_forward(LL, x, path=path, y=y, ws=ws)
        e1.record()
        e1.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / reps
        used = int((cnt.cpu().numpy() > 0).sum())
        flops = 2.0 * 3 * T * k * d * f                      # three products per (token, slot)
        wbytes = used * 3 * d * f * 2                         # bf16 weights of the experts used
        out[name] = {"ms_per_layer": sec * 1e3, "tokens_per_s": T / sec,
                     "tflops": flops / sec / 1e12}
        if name == "dense_mfma_rowmajor_down":
            out[name]["what"] = ("the older bf16 kernels (64/128-token passes, W^down read "
                                 "row-major), for comparison")
        if name == "auto":
            flags = torch.zeros(E, dtype=torch.uint8, device=dev)
            moe.layer_forward(LL, x, path=path, y=y, ws=ws, trace={"expert_dense": flags})
            out[name]["what"] = (f"per call: {'dense' if LL.auto_dense_min(T) else 'sparse'} "
                                 f"(expected bytes of both paths, density {LL.density:.2f})")
            out[name]["dense_experts"] = int(flags.sum().item())
        if path == moe.PATH_DENSE:
            out[name]["mfma_util"] = flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS
            out[name]["weight_gbs"] = wbytes / sec / 1e9
            out[name]["hbm_frac"] = wbytes / sec / 1e9 / HBM_PEAK_GBS
            # roofline-attainable MFMA share at this intensity (flop per weight byte)
            out[name]["mfma_attainable"] = min(1.0, flops / wbytes * HBM_PEAK_GBS / 1e3
                                               / MFMA_BF16_PEAK_TFLOPS)
    out["workload"] = (f"Mixtral-8x22B-shaped layer, 8 experts d={d} f={f} bf16, top-2, "
                       f"{T} tokens; dense = threshold off on bf16 MFMA (256 x 256 tiles, "
                       f"W^down transposed once), sparse = 70% thresholds")
    # extra point: the same layer at a micro-batch of 2048 tokens (about 512 per
    # expert, 512 flop per weight byte, above the 312.5 flop/B ridge), where the
    # dense path is a real contraction and MFMA utilisation is the measure
    T2 = 2048
    x2 = torch.from_numpy(synth.tokens_f32(cfg, T2, d, c["x_scale"])).to(bf).to(dev)
    y2 = torch.empty((T2, d), dtype=torch.float32, device=dev)
    ws2 = moe.new_workspace(L.workspace_bytes(T2), dev)
    legs2 = (("dense_mfma_T2048", L), ("dense_mfma_rowmajor_down_T2048", L_rowmajor))
    for key, LL in (legs2[:1] if dense_only else legs2):
        for _ in range(2):
            moe.layer_forward(LL, x2, path=moe.PATH_DENSE, y=y2, ws=ws2, trace={"expert_count": cnt})
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        n2 = 3 if dense_only else 5
        for _ in range(n2):
            moe.layer_forward(LL, x2, path=moe.PATH_DENSE, y=y2, ws=ws2)
        e1.record()
        e1.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / n2
        flops = 2.0 * 3 * T2 * k * d * f
        wbytes = int((cnt.cpu().numpy() > 0).sum()) * 3 * d * f * 2
        out[key] = {
            "workload": f"same layer, micro-batch {T2} tokens, dense bf16 MFMA path"
                        + ("" if LL is L else " (older kernels, for comparison)"),
            "ms_per_layer": sec * 1e3, "tokens_per_s": T2 / sec, "tflops": flops / sec / 1e12,
            "mfma_util": flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "flop_per_weight_byte": flops / wbytes,
            "mfma_attainable": min(1.0, flops / wbytes * HBM_PEAK_GBS / 1e3 / MFMA_BF16_PEAK_TFLOPS)}
    del x2, y2, ws2
    del L, L_rowmajor, gate, down, down_dense, up_q, up_sz, up_dense
    torch.cuda.empty_cache()
    return out


def device_layer(cfg, layer, E, S, k, d, f, wdt, xscale, sparsity, bias=None, router_std=0.02):
    """A layer drawn on the device: E routed + S shared experts, INT2 up packed
    by the library, thresholds at the `sparsity` quantile of |v| over the 64
    seeded calibration vectors (v from the library)."""
    import torch
    import activation_sparse_expert_amd as moe
    import synth
    dev = torch.device("cuda:0")
    dt = torch.float16 if wdt == "f16" else torch.bfloat16
    n = E + S
    gate = torch.empty((n, f, d), dtype=dt, device=dev)
    down = torch.empty((n, f, d), dtype=dt, device=dev)
    up_q = torch.empty((n, f, d // 4), dtype=torch.uint8, device=dev)
    up_sz = torch.empty((n, f, d // 64, 2), dtype=torch.int16, device=dev)
    thr = torch.empty(n, dtype=torch.float32, device=dev)
    v = torch.empty((64, f), dtype=torch.float32, device=dev)
    for e in range(n):
        gate[e].copy_(synth.device_normal(synth.seed_of(cfg, layer, e, synth.T_GATE), (f, d), 0.02, dev, dt))
        down[e].copy_(synth.device_normal(synth.seed_of(cfg, layer, e, synth.T_DOWN), (f, d), 0.02, dev, dt))
        u = synth.device_normal(synth.seed_of(cfg, layer, e, synth.T_UP), (f, d), 0.02, dev)
        moe.pack_up_int2(u, up_q=up_q[e], up_sz=up_sz[e])
        del u
        xc = torch.from_numpy(synth.calibration_f32(cfg, d, xscale, layer, e)).to(dt).to(dev)
        moe.expert_forward_sparse(moe.Expert(up_q[e], up_sz[e], gate[e], down[e], float("inf")), xc,
                                  v_out=v)
        thr[e] = torch.quantile(v.abs().flatten()[: 1 << 24].double(), sparsity).float()
    R = torch.from_numpy(synth.router_f32(cfg, layer, E, d, router_std)).to(dt).to(dev)
    return moe.Layer(d=d, f=f, E=E, S=S, k=k, renormalize=True, router_w=R, up_q=up_q, up_sz=up_sz,
                     gate_t=gate, down=down, thresholds=thr,
                     router_bias=None if bias is None else torch.from_numpy(bias).to(dev))


def layer_bytes(L, masks, idx, dense=None):
    """Algorithmic bytes of one layer call: router rows, and for every expert
    touched its INT2 codes, scales and the gate and down rows of the union of
    its tokens' masks; x in and y out.  dense [E+S] (0/1): those experts read
    their three 16-bit weight matrices whole instead."""
    T = masks.shape[0]
    d, f, E, k = L.d, L.f, L.E, L.k
    b = E * d * 2 + T * d * 2 + T * d * 4
    for e in range(E + L.S):
        if e < E:
            sel = np.argwhere(idx == e)
            if len(sel) == 0:
                continue
        if dense is not None and dense[e]:
            b += 3 * d * f * 2
            continue
        if e < E:
            union = np.zeros(f, dtype=bool)
            for t, s_ in sel:
                union |= masks[t, s_].astype(bool)
        else:
            union = masks[:, k + (e - E)].astype(bool).any(axis=0)
        b += d * f // 4 + 4 * f * (d // 64) + 2 * int(union.sum()) * d * 2
    return b


def time_graph(fn, reps, inner):
    """Capture `inner` calls of fn() in a HIP graph, replay `reps` times after
    one untimed replay; returns seconds per call."""
    import torch
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(2):
            fn()
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(inner):
            fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        stream.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (reps * inner)


def layer_workload(layers, xs_by_layer, label, path=None):
    """Decode step through `layers` (one moe_layer_forward each, captured in a
    graph): tokens/s and algorithmic GB/s.  path: MOE_PATH_SPARSE (default),
    MOE_PATH_AUTO or MOE_PATH_MIXED, whose per-expert paths are read back and
    priced (dense experts at their three 16-bit matrices)."""
    import torch
    import activation_sparse_expert_amd as moe
    dev = torch.device("cuda:0")
    path = moe.PATH_SPARSE if path is None else path
    T = xs_by_layer[0].shape[0]
    ys = [torch.empty((T, L.d), dtype=torch.float32, device=dev) for L in layers]
    wss = [moe.new_workspace(L.workspace_bytes(T), dev) for L in layers]
    total_b = 0
    n_dense = 0
    for L, x, y, ws in zip(layers, xs_by_layer, ys, wss):
        tr = dict(topk_idx=torch.empty((T, L.k), dtype=torch.int32, device=dev),
                  masks=torch.empty((T, L.k + L.S, L.f), dtype=torch.uint8, device=dev))
        moe.layer_forward(L, x, y=y, ws=ws, trace=tr)
        dense = None
        if path in (moe.PATH_AUTO, moe.PATH_MIXED):
            flags = torch.zeros(L.E, dtype=torch.uint8, device=dev)
            moe.layer_forward(L, x, path=path, y=y, ws=ws, trace=dict(expert_dense=flags))
            # the shared experts are dense from n* tokens (AUTO: n* = 1 on a dense call)
            nstar = L.auto_dense_min(T) if path == moe.PATH_AUTO else L.mixed_dense_min(T)
            dense = np.concatenate([flags.cpu().numpy(),
                                    np.full(L.S, 1 if 0 < nstar <= T else 0, np.uint8)])
            n_dense += int(dense.sum())
        torch.cuda.synchronize()
        total_b += layer_bytes(L, tr["masks"].cpu().numpy(), tr["topk_idx"].cpu().numpy(), dense)

    def step():
        for L, x, y, ws in zip(layers, xs_by_layer, ys, wss):
            moe.layer_forward(L, x, path=path, y=y, ws=ws)
    sec = time_graph(step, reps=5, inner=4)
    out = {"workload": label, "tokens": T, "ms_per_step": sec * 1e3, "tokens_per_s": T / sec,
           "bytes_per_step": total_b, "achieved_gbs": total_b / sec / 1e9,
           "hbm_frac": total_b / sec / 1e9 / HBM_PEAK_GBS}
    if path in (moe.PATH_AUTO, moe.PATH_MIXED):
        out["dense_experts"] = n_dense
    return out


# oracle timings of the layer workloads, filled by layers_measure(cpu=True)
ORACLE_LAYERS = {}


def oracle_layer_rate(L, x_bits, budget_s, label, per_step_layers=1):
    """The fp64 oracle's layer_forward, as it stands, on a host copy of the
    device layer L (same weights, codes, thresholds and router): single-token
    calls over the tokens x_bits (uint16 [n][d]) on one host thread, then on N
    threads with independent calls (the oracle's C code runs outside the GIL),
    each leg about budget_s / 2 and at least one call per thread.  A decode
    step of per_step_layers such layers is extrapolated from the per-layer
    time (labelled as such)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    h = lambda t: t.detach().cpu().numpy()
    wdt = "bf16" if L.gate_t.dtype == __import__("torch").bfloat16 else "f16"
    up_q, up_sz = h(L.up_q), h(L.up_sz).view(np.uint16)
    g, dn = h(L.gate_t).view(np.uint16), h(L.down).view(np.uint16)
    rw = h(L.router_w).view(np.uint16)
    bias = None if L.router_bias is None else h(L.router_bias).astype(np.float32)
    thr = h(L.thresholds).astype(np.float32)

    def worker(first, leg_s):
        n, t0 = 0, time.perf_counter()
        while n == 0 or time.perf_counter() - t0 < leg_s:
            t = (first + n) % len(x_bits)
            oracle.layer_forward(x_bits[t:t + 1], wdt, rw, wdt, bias, L.E, L.k, L.S, L.renormalize,
                                 up_q, up_sz, g, dn, wdt, thr)
            n += 1
        return n, time.perf_counter() - t0

    n1, el1 = worker(0, budget_s / 2)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(lambda i: worker(i, budget_s / 2), range(threads)))
    eln = time.perf_counter() - t0
    nn = sum(r[0] for r in res)
    r = {"workload": label, "unit": "tokens/s", "kind": "oracle",
         "value": nn / eln / per_step_layers, "cores": threads,
         "single_thread": n1 / el1 / per_step_layers,
         "sample": f"{n1} single-token layer calls on one thread in {el1:.1f} s, {nn} on "
                   f"{threads} threads in {eln:.1f} s"}
    if per_step_layers > 1:
        r["extrapolated"] = (f"one of the {per_step_layers} layers timed; tokens/s of a decode "
                             f"step = layer calls/s / {per_step_layers}")
    return r


def oracle_tiny_rate(budget_s):
    """The oracle's expert_forward on the small d=256, f=704 expert (host-drawn,
    50% threshold from its 64 calibration vectors), single tokens, one thread."""
    import oracle
    import synth
    cfg = synth.CFG_TINY
    c = synth.CONFIGS[cfg]
    d, f = c["d"], c["f"]
    g, u, dn = synth.expert_weights_f32(cfg, 0, 0, d, f)
    q, sz = oracle.pack_up_int2(u)
    W = oracle.dequant_up(q, sz, d)
    xc = synth.to_f16_bits(synth.calibration_f32(cfg, d, c["x_scale"], 0, 0))
    thr = oracle.calibrate_threshold(np.abs(xc.view(np.float16).astype(np.float64) @ W.T), 0.5)
    toks = synth.to_f16_bits(synth.tokens_f32(cfg, NTOK, d, c["x_scale"]))
    gb, db = synth.to_f16_bits(g), synth.to_f16_bits(dn)
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget_s:
        oracle.expert_forward(toks[n % NTOK:n % NTOK + 1], "f16", q, sz, gb, db, "f16", thr)
        n += 1
    el = time.perf_counter() - t0
    return {"workload": f"one expert d={d} f={f}, 50% threshold, batch 1", "unit": "tokens/s",
            "kind": "oracle", "value": n / el, "cores": 1,
            "sample": f"{n} single-token calls on one thread in {el:.1f} s"}


def layers_measure(fine_only=False, stack_only=False, cpu=False):
    """The 32-layer Mixtral stack (T = 1, 16) and the fine-grained 64+2 layer
    (T = 1, 64), each as tokens/s of a decode step, router included; the fine
    layer again with dense copies under MOE_PATH_AUTO and MOE_PATH_MIXED
    (T = 64, 256)."""
    import torch
    import activation_sparse_expert_amd as moe
    import synth
    dev = torch.device("cuda:0")
    out = {}
    if stack_only:
        return stack_measure(out, cpu)
    c = synth.CONFIGS[synth.CFG_FINE]
    bias = synth.zipf_bias(synth.CFG_FINE, 0, c["E"], c["zipf_s"])
    fine = device_layer(synth.CFG_FINE, 0, c["E"], c["S"], c["k"], c["d"], c["f"], c["wdt"],
                        c["x_scale"], c["sparsity"], bias=bias)
    for T in (1, 64):
        x = torch.from_numpy(synth.tokens_f32(synth.CFG_FINE, T, c["d"], c["x_scale"])).half().to(dev)
        out[f"fine_T{T}"] = layer_workload(
            [fine], [x], f"DeepSeek-V2-Lite-shaped layer, 64 routed (top-6) + 2 shared experts, "
                         f"d=2048 f=1408, Zipf router bias, 70% sparsity, {T} tokens")
    if cpu:
        log("timing the oracle on the fine-grained layer")
        xb = synth.to_f16_bits(synth.tokens_f32(synth.CFG_FINE, NTOK, c["d"], c["x_scale"]))
        ORACLE_LAYERS["fine_T1"] = oracle_layer_rate(
            fine, xb, 6.0, "the fine-grained layer (64 routed top-6 + 2 shared, d=2048 f=1408, "
                           "70% sparsity), 1 token per call, router included")
    # the same layer with dense fp16 copies (up materialised, W^down transposed)
    # under MOE_PATH_AUTO (one path per call, from the expected bytes of both)
    # and MOE_PATH_MIXED (per expert: dense from n* tokens)
    n = c["E"] + c["S"]
    fine.up_dense = torch.empty((n, c["f"], c["d"]), dtype=torch.float16, device=dev)
    for e in range(n):
        moe.materialize_up(fine.up_q[e], fine.up_sz[e], c["d"], torch.float16, out=fine.up_dense[e])
    fine.down_dense = moe.transpose_down(fine.down)
    fine.density = 1.0 - c["sparsity"]
    for T in (64, 256):
        x = torch.from_numpy(synth.tokens_f32(synth.CFG_FINE, T, c["d"], c["x_scale"])).half().to(dev)
        choice = "dense MFMA" if fine.auto_dense_min(T) else "sparse"
        r = layer_workload(
            [fine], [x], f"the same layer with dense fp16 copies, MOE_PATH_AUTO (per call: "
                         f"{choice}), {T} tokens", path=moe.PATH_AUTO)
        out[f"fine_T{T}_auto"] = r
        out[f"fine_T{T}_mixed"] = layer_workload(
            [fine], [x], f"the same layer, MOE_PATH_MIXED (per expert: dense MFMA at >= "
                         f"{fine.mixed_dense_min(T)} tokens, the others sparse, the GEMMs on a "
                         f"second stream), {T} tokens", path=moe.PATH_MIXED)
        if T == 256:
            out["fine_T256"] = layer_workload(
                [fine], [x], f"the same layer, sparse path for every expert, {T} tokens")
    del fine
    torch.cuda.empty_cache()
    if fine_only:
        return out
    return stack_measure(out, cpu)


def stack_measure(out, cpu=False):
    """The 32-layer Mixtral stack, T = 1 and 16, into `out`."""
    import torch
    import synth
    dev = torch.device("cuda:0")
    c = synth.CONFIGS[synth.CFG_STACK]
    log("drawing the 32-layer stack (64.9 GB)")
    stack = [device_layer(synth.CFG_STACK, l, c["E"], 0, c["k"], c["d"], c["f"], c["wdt"], c["x_scale"],
                          c["sparsity"]) for l in range(c["L"])]
    for T in (1, 16):
        xs = synth.hidden_stream_f32(synth.CFG_STACK, c["L"], T, c["d"], c["x_scale"])
        xl = [torch.from_numpy(xs[l]).half().to(dev) for l in range(c["L"])]
        out[f"stack_T{T}"] = layer_workload(
            stack, xl, f"32 Mixtral-8x7B-shaped layers x 8 experts (d=4096 f=14336), top-2, "
                       f"80% sparsity, {T} tokens per decode step through all layers")
    if cpu:
        log("timing the oracle on layer 0 of the stack")
        xs0 = synth.hidden_stream_f32(synth.CFG_STACK, 1, NTOK, c["d"], c["x_scale"])[0]
        ORACLE_LAYERS["stack_T1"] = oracle_layer_rate(
            stack[0], synth.to_f16_bits(xs0), 8.0,
            "decode step through the 32-layer Mixtral-shaped stack (8 experts per layer, top-2, "
            "80% sparsity), 1 token", per_step_layers=c["L"])
    del stack
    torch.cuda.empty_cache()
    return out


def bits_measure(sparsity=0.9):
    """One Mixtral-8x7B-shaped expert with the up codes at 8, 4, 2 and 1 bits,
    one token per call, 90% sparsity: time per call and algorithmic bytes
    (codes d f bits/8, scales f d/16, gate + down rows of the active channels,
    x) per call."""
    import torch
    import activation_sparse_expert_amd as moe
    import synth
    d, f = D, F
    dev = torch.device("cuda:0")
    g = synth.device_normal(synth.seed_of(2, 0, 0, synth.T_GATE), (f, d), 0.02, dev, torch.float16)
    dn = synth.device_normal(synth.seed_of(2, 0, 0, synth.T_DOWN), (f, d), 0.02, dev, torch.float16)
    u = synth.device_normal(synth.seed_of(2, 0, 0, synth.T_UP), (f, d), 0.02, dev)
    xs = synth.device_normal(synth.seed_of(2, 0, 0, synth.T_X), (64, d), 1 / 64, dev, torch.float16)
    res = {}
    for bits in (8, 4, 2, 1):
        up_q, up_sz = moe.pack_up_bits(u, bits)
        ex = moe.Expert(up_q, up_sz, g, dn, 0.0)
        v = torch.empty((64, f), dtype=torch.float32, device=dev)
        ws = moe.new_workspace(moe.workspace_size(moe.OP_EXPERT_BITS, 1, d, f), dev)
        y = torch.empty((1, d), dtype=torch.float32, device=dev)
        ex.threshold = -1.0
        for t in range(64):
            moe.expert_forward_sparse_bits(ex, bits, xs[t:t + 1], y=y, v_out=v[t:t + 1], ws=ws)
        torch.cuda.synchronize()
        ex.threshold = float(torch.quantile(v.abs().flatten()[:1 << 24].float(), sparsity))
        m = torch.empty((1, f), dtype=torch.uint8, device=dev)
        act = 0
        for t in range(64):
            moe.expert_forward_sparse_bits(ex, bits, xs[t:t + 1], y=y, mask_out=m, ws=ws)
            act += int(m.sum().item())
        act /= 64
        ci = [0]

        def call():
            t = ci[0] % 64
            ci[0] += 1
            moe.expert_forward_sparse_bits(ex, bits, xs[t:t + 1], y=y, ws=ws)
        sec = time_graph(call, reps=10, inner=64)
        nbytes = d * f * bits / 8 + f * (d // 64) * 4 + 2 * act * d * 2 + d * 2
        # four tokens per call (x staged in LDS); rows of the union of the masks
        y4 = torch.empty((4, d), dtype=torch.float32, device=dev)
        ws4 = moe.new_workspace(moe.workspace_size(moe.OP_EXPERT_BITS, 4, d, f), dev)
        m4 = torch.empty((4, f), dtype=torch.uint8, device=dev)
        uni = 0
        for t in range(0, 64, 4):
            moe.expert_forward_sparse_bits(ex, bits, xs[t:t + 4], y=y4, mask_out=m4, ws=ws4)
            uni += int(m4.any(dim=0).sum().item())
        uni /= 16

        def call4():
            t = (ci[0] % 16) * 4
            ci[0] += 1
            moe.expert_forward_sparse_bits(ex, bits, xs[t:t + 4], y=y4, ws=ws4)
        sec4 = time_graph(call4, reps=10, inner=32)
        res[f"int{bits}"] = {"us_per_call": sec * 1e6, "tokens_per_s": 1 / sec,
                             "active_channels": act, "bytes_per_call": nbytes,
                             "achieved_gbs": nbytes / sec / 1e9,
                             "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                             "batch4_us_per_call": sec4 * 1e6,
                             "batch4_tokens_per_s": 4 / sec4,
                             "batch4_union_channels": uni}
        del up_q, up_sz, ex
    res["workload"] = ("one Mixtral-8x7B-shaped expert (d=4096, f=14336), up codes at 8/4/2/1 bits "
                       "(2 bits: the INT2 format, for comparison on the same schedule), "
                       "90% sparsity, batch 1 and 4")
    return res


def eamc_measure():
    """Nearest stored request-level EAM (cosine distance) over a collection:
    per call n stored EAMs of L x E int32 counts are read once."""
    import torch
    import activation_sparse_expert_amd as moe
    import synth
    res = {}
    for name, n, L, E, k in (("mixtral_32x8_n1000", 1000, 32, 8, 2),
                             ("arctic_35x128_n4096", 4096, 35, 128, 2)):
        a = torch.from_numpy(synth.eam_collection(7, n, L, E, k)).cuda()
        b, q = a[:n].contiguous(), a[n].contiguous()
        idx = torch.empty(1, dtype=torch.int32, device=a.device)
        dist = torch.empty(n, dtype=torch.float64, device=a.device)
        sec = time_graph(lambda: moe.eamc_match(b, q, idx=idx, dist=dist), reps=20, inner=50)
        nbytes = n * L * E * 4 + L * E * 4 + n * 8
        res[name] = {"workload": f"{n} stored EAMs of {L} layers x {E} experts, one query",
                     "us_per_call": sec * 1e6, "bytes_per_call": nbytes,
                     "achieved_gbs": nbytes / sec / 1e9,
                     "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS}
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sparsity, budget_s):
    """The fp64 oracle, as it stands, on instance 0 and the same tokens: once on
    one host thread, then on N threads that each run independent single-token
    calls (the oracle's C code runs outside the GIL), N = the cores this
    process may use (at most 16).  Each leg runs for about budget_s / 2."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import synth
    cfg = synth.CFG_MIXTRAL
    xs = synth.CONFIGS[cfg]["x_scale"]
    g, u, dn = synth.expert_weights_f32(cfg, 0, 0, D, F)
    q, sz = oracle.pack_up_int2(u)
    gb, db = synth.to_f16_bits(g), synth.to_f16_bits(dn)
    W = oracle.dequant_up(q, sz, D)
    xc = synth.to_f16_bits(synth.calibration_f32(cfg, D, xs, 0, 0))
    vcal = xc.view(np.float16).astype(np.float64) @ W.T
    del W
    thr = oracle.calibrate_threshold(np.abs(vcal), sparsity)
    toks = synth.to_f16_bits(synth.tokens_f32(cfg, NTOK, D, xs))

    def worker(first, leg_s):
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < leg_s:
            t = (first + n) % NTOK
            oracle.expert_forward(toks[t:t + 1], "f16", q, sz, gb, db, "f16", thr)
            n += 1
        return n, time.perf_counter() - t0

    n1, el1 = worker(0, budget_s / 2)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(lambda i: worker(i, budget_s / 2), range(threads)))
    eln = time.perf_counter() - t0
    nn = sum(r[0] for r in res)
    model = cpu_model()
    return dict(value=nn / eln, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{nn} single-token calls of the fp64 oracle on expert instance 0 "
                       f"(d={D}, f={F}, {int(sparsity * 100)}% threshold) on {threads} threads "
                       f"in {eln:.1f} s, {model}",
                cpu_model=model,
                single_thread={"value": n1 / el1, "unit": "tokens/s", "cores": 1,
                               "sample": f"{n1} calls on one thread in {el1:.1f} s"})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--instances", type=int, default=32)
    ap.add_argument("--sparsity", type=float, default=0.9)
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--dist-replays", type=int, default=15,
                    help="further timed replays of the K-step graph for the median and p10/p90")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--batched-only", action="store_true",
                    help="only the batched-layer measurement (for profiling)")
    ap.add_argument("--dense-only", action="store_true",
                    help="only the dense MFMA path of the batched layer, at 256 and 2048 tokens, "
                         "three calls each (for profiling)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline expert call (no batch-4, layer, batched or CPU legs; "
                         "for counter passes)")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the layer workloads (32-layer stack, fine-grained layer)")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the batched-layer (dense MFMA vs sparse) measurement")
    ap.add_argument("--fine-only", action="store_true",
                    help="only the fine-grained layer workloads (sparse, AUTO, MIXED)")
    ap.add_argument("--stack-only", action="store_true",
                    help="only the 32-layer stack workloads (T = 1, 16)")
    ap.add_argument("--variants-only", action="store_true",
                    help="only the 8/4/1-bit expert and EAMC measurements (for profiling)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run the known-size elementwise kernel (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the expert path here runs on a single MI355X "
              "and has no multi-GPU mode (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.batched_only or args.dense_only:
        print(json.dumps({"batched": batched_measure(dense_only=args.dense_only)}), flush=True)
        return
    if args.fine_only:
        print(json.dumps({"more": layers_measure(fine_only=True)}), flush=True)
        return
    if args.stack_only:
        print(json.dumps({"more": layers_measure(stack_only=True)}), flush=True)
        return
    if args.variants_only:
        print(json.dumps({"expert_up_bits": bits_measure(), "eamc_match": eamc_measure()}),
              flush=True)
        return

    import torch
    import activation_sparse_expert_amd as moe
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"building {args.instances} expert instances d={D} f={F}")
    experts = build_instances(args.instances, args.sparsity, dev)
    cfg = synth.CFG_MIXTRAL
    x_all = torch.from_numpy(synth.tokens_f32(cfg, NTOK, D, synth.CONFIGS[cfg]["x_scale"])).half().to(dev)
    xs = [x_all[i:i + 1] for i in range(NTOK)]
    y = torch.empty((1, D), dtype=torch.float32, device=dev)
    ws = moe.new_workspace(moe.workspace_size(moe.OP_EXPERT, 1, D, F), dev)

    # untimed pass: realised active rows per (instance, token) -> algorithmic bytes
    R = len(experts)
    nnz = np.zeros((R, NTOK))
    m = torch.empty((1, F), dtype=torch.uint8, device=dev)
    for r in range(R):
        for t in range(NTOK):
            moe.expert_forward_sparse(experts[r], xs[t], y=y, ws=ws, mask_out=m)
            nnz[r, t] = float(m.sum().item())
        log(f"masks of instance {r + 1}/{R} counted")
    fixed = D * F // 4 + F * (D // 64) * 4 + D * 2 + D * 4     # INT2 up + scales + x + y
    per_call = fixed + 2 * nnz * D * 2                            # + gate and down rows
    sched = [(i % R, (i // R) % NTOK) for i in range(args.steps)]
    bytes_timed = float(sum(per_call[r, t] for r, t in sched))

    stream = torch.cuda.Stream()
    log(f"timing {args.steps} steps")
    # warmup (eager), then capture the K steps in one graph
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            r, t = i % R, (i // R) % NTOK
            moe.expert_forward_sparse(experts[r], xs[t], y=y, ws=ws)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for r, t in sched:
            moe.expert_forward_sparse(experts[r], xs[t], y=y, ws=ws)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):     # replay runs on the current stream
        graph.replay()                  # one untimed replay
        stream.synchronize()
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    sec = ms / 1e3
    K = args.steps
    # the spread: the same K-step graph replayed again, each replay timed
    per_step = []
    with torch.cuda.stream(stream):
        for _ in range(args.dist_replays):
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            graph.replay()
            a1.record(stream)
            a1.synchronize()
            per_step.append(a0.elapsed_time(a1) / K)
    per_step = np.array(per_step)
    avg_launch_s = sec / K
    achieved = bytes_timed / K / avg_launch_s / 1e9
    out = {
        "metric": METRIC,
        "value": K * 1 / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "one Mixtral-8x7B-shaped SwiGLU expert, INT2 up + fp16 gate/down, "
                        "90% activation sparsity, batch 1 (decode)",
            "d": D, "f": F, "tokens_per_step": 1, "sparsity_target": args.sparsity,
            "sparsity_realised": float(1 - nnz.mean() / F), "instances": R,
            "bytes_per_step_mean": bytes_timed / K,
        },
        "dist": {
            "replays": int(len(per_step)),
            "ms_per_step_median": float(np.median(per_step)) if len(per_step) else None,
            "ms_per_step_p10": float(np.percentile(per_step, 10)) if len(per_step) else None,
            "ms_per_step_p90": float(np.percentile(per_step, 90)) if len(per_step) else None,
            "what": "each further replay of the same K-step graph timed on its own",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": counted_traffic(),
        },
    }
    if args.headline_only:
        print(json.dumps(out), flush=True)
        return
    # the same expert call at batch 4 (Mixtral shape, 90% sparsity)
    x4 = [x_all[i:i + 4] for i in range(0, NTOK, 4)]
    y4 = torch.empty((4, D), dtype=torch.float32, device=dev)
    ws4 = moe.new_workspace(moe.workspace_size(moe.OP_EXPERT, 4, D, F), dev)
    m4 = torch.empty((4, F), dtype=torch.uint8, device=dev)
    b4 = 0.0
    for r in range(R):
        for t in range(len(x4)):
            moe.expert_forward_sparse(experts[r], x4[t], y=y4, ws=ws4, mask_out=m4)
            u = int(m4.any(dim=0).sum().item())
            b4 += D * F // 4 + F * (D // 64) * 4 + 4 * D * (2 + 4) + 2 * u * D * 2
        log(f"batch-4 masks of instance {r + 1}/{R} counted")
    b4 /= R * len(x4)
    calls = [(experts[i % R], x4[(i // R) % len(x4)]) for i in range(R * len(x4))]
    ci = [0]

    def call4():
        e_, x_ = calls[ci[0] % len(calls)]
        ci[0] += 1
        moe.expert_forward_sparse(e_, x_, y=y4, ws=ws4)
    sec4 = time_graph(call4, reps=5, inner=len(calls) * 8)
    out["more"] = {"expert_b4": {
        "workload": "one Mixtral-8x7B-shaped expert, 90% sparsity, batch 4 (union of the 4 masks read once)",
        "ms_per_call": sec4 * 1e3, "tokens_per_s": 4 / sec4, "bytes_per_call": b4,
        "achieved_gbs": b4 / sec4 / 1e9, "hbm_frac": b4 / sec4 / 1e9 / HBM_PEAK_GBS}}
    del experts, calls
    torch.cuda.empty_cache()
    if not args.no_layers:
        log("measuring the layer workloads")
        out["more"].update(layers_measure(cpu=not args.no_cpu))
        log("measuring the 8/4/1-bit up variants")
        out["more"]["expert_up_bits"] = bits_measure()
        log("measuring the EAMC match")
        out["more"]["eamc_match"] = eamc_measure()
    if not args.no_batched:
        log("measuring the batched layer (dense MFMA and sparse paths)")
        out["batched"] = batched_measure()
    if not args.no_cpu:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(args.sparsity, args.cpu_budget)
        more = dict(ORACLE_LAYERS)
        more["tiny_T1"] = oracle_tiny_rate(2.0)
        out["cpu_baseline"]["more"] = more
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
