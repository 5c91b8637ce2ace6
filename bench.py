#!/usr/bin/env python3
"""Throughput of exact tiled masked softmax attention on one MI355X.

One step = one pass of the whole hot path over one batch: attn_fwd followed by
the three backward launches (prepass, dK/dV, dQ) on the same stream.  Inputs
are seeded synthetic tensors already resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --copy-probe     # plain device copy of known size, for scaling HBM counters
    python bench.py --issue-probe    # MFMA rate with 0..12 independent FMAs per MFMA, 1 and 2 waves/SIMD
    python bench.py --atomic-probe   # fp32 atomic-add rate in the sparse dKV scatter's pattern
    python bench.py --lds-probe      # LDS read bandwidth with 4, 8 and 16 waves per compute unit

The roofline object's "traffic" (HBM bytes per launch of the dominant kernel)
comes from profiles/<kernel>_<workload>_traffic.md, written from rocprofv3
FETCH_SIZE / WRITE_SIZE runs scaled by what the same counters read for the
copy probe; it is reported only while the kernel's sources still hash to the
value recorded there, else null.

Flops are algorithmic: only allowed (query, key) pairs count.  Per pair the
forward does 2d + 2dv flops (S = c Q K^T, then P V) and the backward 6d + 4dv
(S recompute, dP = G V^T, dV, dK, dQ).  The dK/dV kernel accounts for
4d + 4dv of them and the dQ kernel for 2d (its S and dP recomputations are
redundant work, not counted).
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

KERNEL_SOURCES = {
    "fwd": ["exact_tiled_softmax_amd/csrc/dense_fwd.hip", "exact_tiled_softmax_amd/csrc/device.hpp"],
    "bwd_dkdv": ["exact_tiled_softmax_amd/csrc/dense_dkdv.hip", "exact_tiled_softmax_amd/csrc/device.hpp"],
    "bwd_dq": ["exact_tiled_softmax_amd/csrc/dense_dq.hip", "exact_tiled_softmax_amd/csrc/device.hpp"],
    "sparse_fwd": ["exact_tiled_softmax_amd/csrc/sparse.hip", "exact_tiled_softmax_amd/csrc/device.hpp"],
    "sparse_dkv": ["exact_tiled_softmax_amd/csrc/sparse.hip", "exact_tiled_softmax_amd/csrc/device.hpp"],
}
RIDGE = 2500.0e12 / 8000.0e9  # flop per byte where the bf16 MFMA and HBM roofs meet
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # dense MFMA peaks (fp32: vector)
PEAK_HBM_GBS = 8000.0
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
METRIC = "attention fwd+bwd TFLOP/s and % bf16 MFMA peak (causal, seq 2048, d=128)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cores_and_model():
    """(threads the oracle's BLAS uses, CPU model name from /proc/cpuinfo)."""
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return int(cores), model


def dense_algorithmic_bytes(w, gam_bytes=0):
    """Compulsory HBM bytes per launch of each dense kernel: every input read
    once, every output written once (dtype-sized tensors, fp32 LSE / D rows).
    With the stored-gamma backward (gam_bytes of gamma tiles), the dK/dV
    kernel also writes the tiles and the dQ kernel reads K and the tiles and
    writes dQ."""
    esz = 4 if w.dtype == "f32" else 2
    q = w.B * w.H * w.n * w.d * esz            # Q, dQ
    g = w.B * w.H * w.n * w.dv * esz           # G, Y
    k = w.B * w.H_kv * w.n * w.d * esz         # K, dK
    v = w.B * w.H_kv * w.n * w.dv * esz        # V, dV
    row = w.B * w.H * w.n * 4                  # one fp32 per query row (LSE, D, LSE2)
    return {"fwd": q + k + v + g + row,        # Q, K, V read; Y, LSE written
            "bwd_prep": 2 * g + row + 2 * row,  # G, Y, LSE read; D, LSE2 written
            "bwd_dkdv": q + g + k + v + 2 * row + k + v + gam_bytes,  # Q, G, K, V, LSE2, D read; dK, dV (gamma) written
            "bwd_dq": (k + gam_bytes + q) if gam_bytes else (q + g + k + v + 2 * row + q)}  # inputs read; dQ written


def stored_gamma_bytes(w):
    """Bytes of the gamma tiles the stored-gamma backward writes and reads:
    16 KiB per (64-key, 128-query) tile that a causal / window mask reaches,
    per (batch, head)."""
    tiles = 0
    for qt in range((w.n + 127) // 128):
        q0 = qt * 128
        hi = (w.n - 1) // 64
        if w.causal:
            hi = min(hi, (min(q0 + 128, w.n) - 1) // 64)
        lo = max(0, int((q0 - w.window + 1) / 64)) if w.window > 0 else 0
        tiles += max(0, hi - lo + 1)
    return w.B * w.H * tiles * 64 * 128 * 2


def sources_sha256(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch (fetch + write) recorded for this kernel and
    workload, or None when absent or taken from different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    try:
        if vals["source_sha256"] != sources_sha256(kernel):
            return None
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe():
    """Copies 256 MiB device to device five times (torch's copy kernel): the
    known traffic per dispatch (256 MiB read, 256 MiB written) scales the
    FETCH_SIZE / WRITE_SIZE counters of the attention kernels."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "dispatches": 5}), flush=True)


def issue_probe():
    """MFMA rate this device sustains with K independent fp32 FMAs, or K
    independent base-2 exponentials, issued after every MFMA (K = 0 .. 12), at
    one and two waves per SIMD: how much vector work hides under the matrix
    instructions.  One JSON line per setting."""
    import torch
    import exact_tiled_softmax_amd as ets
    sink = torch.empty(4096, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for trans, kind in ((0, "fma"), (1, "exp")):
        for wps in (1, 2):
            for k in (0, 2, 4, 6, 8, 12):
                ets.attn_issue_probe(wps, k, trans, 64, sink, sink.numel(), stream=stream)  # warm-up
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                n = ets.attn_issue_probe(wps, k, trans, 2048, sink, sink.numel(), stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                tf = n * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12
                print(json.dumps({"probe": "issue", "waves_per_simd": wps, "kind": kind, "per_mfma": k,
                                  "mfma_TFLOP/s": tf}), flush=True)


def atomic_probe():
    """fp32 atomic adds per second into rows of a [rows x 576] table, checked
    against the expected counts: random rows of a 16384-row table (the sparse
    dKV accumulator's shape, 37.7 MB), random rows of 1024- and 64-row tables
    (2.4 MB and 147 KB, small enough to stay in one XCD's 4 MB L2), and the
    16384 rows in order (the pattern of a contiguous accumulator such as a
    dQ tile)."""
    import torch
    import exact_tiled_softmax_amd as ets
    n_idx, blocks, gpw = 1 << 20, 4096, 64
    stream = torch.cuda.current_stream()
    for name, rows, order in (("random", 16384, "random"), ("random", 1024, "random"), ("random", 64, "random"),
                              ("sequential", 16384, "sequential")):
        g = torch.Generator(device="cpu").manual_seed(0)
        if order == "random":
            idx_h = torch.randint(0, rows, (n_idx,), generator=g, dtype=torch.int32)
        else:
            idx_h = (torch.arange(n_idx, dtype=torch.int32) % rows).to(torch.int32)
        idx = idx_h.cuda()
        table = torch.zeros(rows, 576, dtype=torch.float32, device="cuda")
        ets.attn_atomic_probe(table, rows, idx, n_idx, 64, 1, stream=stream)  # warm-up
        table.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        n = ets.attn_atomic_probe(table, rows, idx, n_idx, blocks, gpw, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        visits = blocks * 4 * gpw * 4
        want = torch.bincount(idx_h[torch.arange(visits) % n_idx].long(), minlength=rows).float()
        exact = bool(torch.equal(table.cpu(), want[:, None].expand(rows, 576)))
        print(json.dumps({"probe": "atomic", "rows": rows, "order": order, "table_MB": rows * 576 * 4 / 1e6,
                          "adds": n, "ms": ms, "G_adds/s": n / (ms * 1e-3) / 1e9, "counts_exact": exact}),
              flush=True)


def lds_probe():
    """LDS read bytes per second and per compute unit, 4 / 8 / 16 waves per CU."""
    import torch
    import exact_tiled_softmax_amd as ets
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for waves in (4, 8, 16):
        ets.attn_lds_probe(waves, 16, sink, sink.numel(), stream=stream)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        n = ets.attn_lds_probe(waves, 4096, sink, sink.numel(), stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        print(json.dumps({"probe": "lds", "waves_per_cu": waves, "bytes": n, "ms": ms,
                          "TB/s": n / (ms * 1e-3) / 1e12, "GB/s_per_cu": n / (ms * 1e-3) / 1e9 / cus}), flush=True)


def mfma_microbench(waves_per_simd=2, iters=4096):
    """Dense bf16 MFMA rate this device sustains (no memory traffic), TFLOP/s."""
    import torch
    import exact_tiled_softmax_amd as ets
    sink = torch.empty(4096, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ets.attn_mfma_probe(waves_per_simd, 64, sink, sink.numel(), stream=stream)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    n = ets.attn_mfma_probe(waves_per_simd, iters, sink, sink.numel(), stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    tf = n * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"TFLOP/s": tf, "frac_of_datasheet": tf / PEAK_TFLOPS["bf16"], "waves_per_simd": waves_per_simd}


def dense_pairs(w, block_mask):
    """|A| = number of allowed (query, key) pairs per (batch, head) lane, counted on the host."""
    n = w.n
    i = np.arange(n)[:, None]
    total = 0
    step = max(1, (1 << 22) // n)
    for r0 in range(0, n, step):
        ii = i[r0:r0 + step]
        j = np.arange(n)[None, :]
        a = np.ones((ii.shape[0], n), bool)
        if w.causal:
            a &= j <= ii
        if w.window > 0:
            a &= (ii - j) < w.window
        if block_mask is not None:
            a &= block_mask[ii // w.mask_tile, j // w.mask_tile] != 0
        total += int(a.sum())
    return total


def cpu_baseline_dense(w, arr, block_mask, budget_s=12.0):
    """The fp64 oracle, untouched, timed on the host on a bounded sample of
    (batch, head) lanes of the same workload."""
    from oracle import dense
    cores, model = host_cores_and_model()
    allowed = dense.Allowed(w.n, w.n, causal=w.causal, window=w.window, block_mask=block_mask,
                            block_q=w.mask_tile, block_k=w.mask_tile)
    drop = dense.Dropout(float(np.float32(w.rho)), seed=w.drop_seed) if w.rho > 0 else None
    per_pair = (2 * w.d + 2 * w.dv) + (6 * w.d + 4 * w.dv)
    pairs_lane = dense_pairs(w, block_mask)
    lanes, t_total = 0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            t0 = time.perf_counter()
            dense.forward_rows(arr["Q64"], arr["K64"], arr["V64"], allowed, w.c, b, h, np.arange(w.n), drop)
            dense.vjp_lane(arr["Q64"], arr["K64"], arr["V64"], allowed, w.c, arr["G64"], b, h, drop)
            t_total += time.perf_counter() - t0
            lanes += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    tflops = lanes * pairs_lane * per_pair / t_total / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": cores, "cpu_model": model, "kind": "oracle",
            "sample": f"fp64 forward + VJP of {lanes} of {w.B * w.H} (batch, head) lanes "
                      f"({lanes * pairs_lane} allowed pairs) in {t_total:.1f} s"}


def bench_dense(w, args):
    import torch
    import exact_tiled_softmax_amd as ets
    from workloads import device as gh

    if args.no_dropout and w.rho > 0:
        import dataclasses
        w = dataclasses.replace(w, rho=0.0)
    arr = workloads.dense_arrays(w)
    block_mask = arr["block_mask"]
    dt = DTYPE_CODE[w.dtype]
    Q, K, V, G = (gh.to_dev(arr[k], w.dtype) for k in ("Q", "K", "V", "G"))
    Y = gh.empty((w.B, w.H, w.n, w.dv), w.dtype)
    LSE = torch.empty((w.B, w.H, w.n), dtype=torch.float32, device="cuda")
    dQ, dK, dV = gh.empty(Q.shape, w.dtype), gh.empty(K.shape, w.dtype), gh.empty(V.shape, w.dtype)
    mask = {"causal": int(w.causal), "window": w.window, "block_q": w.mask_tile, "block_k": w.mask_tile}
    if block_mask is not None:
        mask["block_mask"] = gh.to_dev(block_mask, "u8")
    drop = (w.rho, w.drop_seed) if w.rho > 0 else None
    # the workspace of the backward's fastest form for this mask and dropout
    # (the stored-gamma form with dropout and a causal / window mask;
    # --recompute-dq: the minimal workspace, the dQ kernel recomputes)
    ws_size = ets.attn_bwd_workspace_size if args.recompute_dq else (
        lambda *s: ets.attn_bwd_workspace_size_fast(*s, mask, drop))
    ws_bytes = ws_size(dt, w.B, w.H, w.H_kv, w.n, w.n, w.d, w.dv)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    shape = (dt, w.B, w.H, w.H_kv, w.n, w.n, w.d, w.dv)
    stream = torch.cuda.current_stream()

    def fwd():
        ets.attn_fwd(*shape, Q, K, V, mask, w.c, w.block_b, drop, Y, LSE, stream=stream)

    def bwd(phase):
        ets.attn_bwd_phase(phase, *shape, Q, K, V, Y, LSE, G, mask, w.c, w.block_b, drop, dQ, dK, dV, ws,
                           ws_bytes, stream=stream)

    names = ["fwd", "bwd_prep", "bwd_dkdv", "bwd_dq"]
    calls = [fwd, lambda: bwd(1), lambda: bwd(2), lambda: bwd(4)]

    def run_steps(n, timed_kernels):
        """n steps; HIP events on the stream around the kernels listed."""
        evs = []
        for _ in range(n):
            row = {}
            for k, c in enumerate(calls):
                if k in timed_kernels:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    c()
                    e1.record(stream)
                    row[k] = (e0, e1)
                else:
                    c()
            evs.append(row)
        return evs

    def mean_ms(evs, k):
        return float(np.mean([r[k][0].elapsed_time(r[k][1]) for r in evs]))

    # The warm-up steps carry events on every kernel and name the dominant one;
    # the timed steps bracket only that kernel (every event record costs the
    # step a few microseconds); an untimed pass afterwards gives the
    # per-kernel breakdown.
    wu = run_steps(args.warmup, range(len(calls)))
    torch.cuda.synchronize()
    cand = ["fwd", "bwd_dkdv", "bwd_dq"]
    # (the fastest warm-up launch of each: a kernel's first launch also loads it)
    dom = max(cand, key=lambda n: min(r[names.index(n)][0].elapsed_time(r[names.index(n)][1]) for r in wu)) \
        if args.warmup > 0 else "bwd_dkdv"
    t0 = time.perf_counter()
    tev = run_steps(args.steps, {names.index(dom)})
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    dom_ms = mean_ms(tev, names.index(dom))
    bev = run_steps(args.steps, range(len(calls)))
    torch.cuda.synchronize()
    kern_ms = {n: mean_ms(bev, k) for k, n in enumerate(names)}

    pairs = dense_pairs(w, block_mask) * w.B * w.H
    d, dv = w.d, w.dv
    flops = {"fwd": pairs * (2 * d + 2 * dv), "bwd_dkdv": pairs * (4 * d + 4 * dv), "bwd_dq": pairs * 2 * d}
    f_fwd, f_bwd = flops["fwd"], flops["bwd_dkdv"] + flops["bwd_dq"]
    peak = PEAK_TFLOPS[w.dtype]
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    gam_bytes = stored_gamma_bytes(w) if ws_bytes > ets.attn_bwd_workspace_size(*shape) else 0
    nbytes = dense_algorithmic_bytes(w, gam_bytes)
    kernels = {}
    for n in names:
        gbs = nbytes[n] / (kern_ms[n] * 1e-3) / 1e9
        kernels[n] = {"ms": kern_ms[n], "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
                      "algorithmic_bytes": nbytes[n]}
        if n != "bwd_prep":
            tf = flops[n] / (kern_ms[n] * 1e-3) / 1e12
            kernels[n].update({"TFLOP/s": tf, "frac_peak": tf / peak})
    # the roof that binds: MFMA when the step's flops per compulsory byte
    # exceed the ridge point, else HBM; the dominant kernel's duration is its
    # HIP-event average over the timed steps
    intensity = (f_fwd + f_bwd) / sum(nbytes.values())
    if intensity >= RIDGE or w.dtype == "f32":
        ach = flops[dom] / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                    "frac": ach / peak, "flops_per_launch": flops[dom]}
    else:
        ach = nbytes[dom] / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": ach / PEAK_HBM_GBS, "bytes_per_launch": nbytes[dom]}
    roofline.update({"traffic": recorded_traffic(dom, w.name), "kernel": dom, "kernel_ms": dom_ms,
                     "flop_per_byte": intensity, "ridge_flop_per_byte": RIDGE})
    fwd_tf = f_fwd / (kern_ms["fwd"] * 1e-3) / 1e12
    bwd_ms = kern_ms["bwd_prep"] + kern_ms["bwd_dkdv"] + kern_ms["bwd_dq"]
    bwd_tf = f_bwd / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1), workloads module)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "kv_heads": w.H_kv, "seq_len": w.n,
                   "head_dim": w.d, "causal": w.causal, "window": w.window,
                   "tile_mask_p": w.block_mask_p, "dropout": w.rho, "allowed_pairs": pairs,
                   "dq_form": ("stored_gamma" if ws_bytes > ets.attn_bwd_workspace_size(*shape) else "recompute"),
                   "workspace_bytes": ws_bytes},
        "frac_peak": value / peak,
        "fwd": {"ms": kern_ms["fwd"], "TFLOP/s": fwd_tf, "frac_peak": fwd_tf / peak},
        "bwd": {"ms": bwd_ms, "TFLOP/s": bwd_tf, "frac_peak": bwd_tf / peak},
        "kernels": kernels,
        "roofline": roofline,
        "mfma_microbench": mfma_microbench(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_dense(w, arr, block_mask)
    return out


def cpu_baseline_sparse(w, a, budget_s=12.0):
    """The fp64 oracle timed on a bounded sample of tokens of the sparse workload."""
    from oracle import sparse
    cores, model = host_cores_and_model()
    sink = a["sink"].astype(np.float64)
    per_pair = w.H * ((2 * w.dqk + 2 * w.dv) + (6 * w.dqk + 4 * w.dv))
    toks, pairs, t_total = [], 0, 0.0
    for t in range(w.Tq - 1, -1, -97):  # spread over the length mix
        t0 = time.perf_counter()
        sparse.forward(a["Q64"], a["KV64"], a["idx"], a["length"], sink, w.alpha, w.dv, tokens=[t])
        sparse.vjp(a["Q64"], a["KV64"], a["idx"], a["length"], sink, w.alpha, w.dv, a["dO64"], tokens=[t])
        t_total += time.perf_counter() - t0
        toks.append(t)
        pairs += int(a["length"][t])
        if t_total >= budget_s:
            break
    return {"value": pairs * per_pair / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu_model": model,
            "kind": "oracle",
            "sample": f"fp64 forward + VJP of {len(toks)} of {w.Tq} tokens ({pairs} valid slots) in {t_total:.1f} s"}


def bench_sparse(w, args):
    import torch
    import exact_tiled_softmax_amd as ets
    from workloads import device as gh

    a = workloads.sparse_arrays(w)
    dt = DTYPE_CODE[w.dtype]
    Q, KV, dO = gh.to_dev(a["Q"], w.dtype), gh.to_dev(a["KV"], w.dtype), gh.to_dev(a["dO"], w.dtype)
    idx = torch.from_numpy(a["idx"]).cuda()
    length = torch.from_numpy(a["length"]).cuda()
    sink = torch.from_numpy(a["sink"]).cuda()
    O = gh.empty((w.Tq, w.H, w.dv), w.dtype)
    LSE = torch.empty((w.Tq, w.H), dtype=torch.float32, device="cuda")
    dQ, dKV = gh.empty(Q.shape, w.dtype), gh.empty(KV.shape, w.dtype)
    dSink = torch.empty(w.H, dtype=torch.float32, device="cuda")
    det = bool(args.deterministic)
    nb = (ets.attn_sparse_bwd_det_workspace_size if det else ets.attn_sparse_bwd_workspace_size)(
        w.Tq, w.H, w.Tkv, w.dqk, w.dv, w.topk)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    shape = (dt, w.Tq, w.H, w.Tkv, w.dqk, w.dv, w.topk)
    stream = torch.cuda.current_stream()

    def fwd():
        ets.attn_sparse_fwd(*shape, Q, KV, idx, length, sink, w.alpha, O, LSE, stream=stream)

    def bwd():
        if det:
            ets.attn_sparse_bwd_det(ets.ATTN_LSE_TOTAL, *shape, Q, KV, idx, length, sink, w.alpha, O, LSE, dO, dQ,
                                    dKV, dSink, ws, nb, stream=stream)
        else:
            ets.attn_sparse_bwd(*shape, Q, KV, idx, length, sink, w.alpha, O, LSE, dO, dQ, dKV, dSink, ws, nb,
                                stream=stream)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        fwd()
        ev[s][1].record(stream)
        bwd()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    pairs = int(a["length"].sum())
    fl_f = pairs * w.H * (2 * w.dqk + 2 * w.dv)
    fl_b = pairs * w.H * (6 * w.dqk + 4 * w.dv)
    gathered = pairs * w.dqk * 2                      # bytes of selected rows read per pass
    fwd_gbs = gathered / (f_ms * 1e-3) / 1e9
    out = {
        "metric": "sparse attention fwd+bwd TFLOP/s and gathered GB/s", "value": (fl_f + fl_b) / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), workloads module)",
        "config": {"workload": w.name, "tokens": w.Tq, "heads": w.H, "kv_rows": w.Tkv, "d_qk": w.dqk, "d_v": w.dv,
                   "topk": w.topk, "valid_pairs": pairs, "deterministic_dkv": det},
        "fwd": {"ms": f_ms, "TFLOP/s": fl_f / (f_ms * 1e-3) / 1e12, "gathered_GB/s": fwd_gbs},
        "bwd": {"ms": b_ms, "TFLOP/s": fl_b / (b_ms * 1e-3) / 1e12,
                "gathered_GB/s": 2 * gathered / (b_ms * 1e-3) / 1e9},
        "roofline": {"bound": "hbm", "achieved": fwd_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": fwd_gbs / PEAK_HBM_GBS, "traffic": recorded_traffic("sparse_fwd", w.name),
                     "kernel": "sparse_fwd",
                     "bytes_per_launch": gathered},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_sparse(w, a)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_causal_bf16_b4h16_n2048_d128", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true", help="run only the reference copy (counter scaling)")
    ap.add_argument("--issue-probe", action="store_true", help="run only the MFMA + VALU issue probe")
    ap.add_argument("--atomic-probe", action="store_true", help="run only the fp32 atomic-rate probe")
    ap.add_argument("--lds-probe", action="store_true", help="run only the LDS read-bandwidth probe")
    ap.add_argument("--no-dropout", action="store_true", help="dense workloads: run the same shape with rate 0")
    ap.add_argument("--recompute-dq", action="store_true",
                    help="dense workloads with dropout: the minimal backward workspace (the dQ kernel recomputes)")
    ap.add_argument("--deterministic", action="store_true",
                    help="sparse workload: the bit-reproducible dKV backward (attn_sparse_bwd_det)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the (batch, head) lanes shard with no exchange, so N GPUs would each run this "
              "same per-GPU workload)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a visible GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    if args.issue_probe:
        issue_probe()
        return
    if args.atomic_probe:
        atomic_probe()
        return
    if args.lds_probe:
        lds_probe()
        return
    w = workloads.WORKLOADS[args.workload]
    if isinstance(w, workloads.DenseWorkload):
        out = bench_dense(w, args)
    else:
        out = bench_sparse(w, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
