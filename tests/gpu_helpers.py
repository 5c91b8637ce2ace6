"""Device plumbing for the GPU tests: torch for memory, the C ABI for compute.

Inputs come from ``workloads`` (seeded, rounded to the storage dtype); the
oracle receives the same values widened to float64.
"""

import numpy as np
import pytest

import workloads
from workloads import device

DT = {"f32": 0, "f16": 1, "bf16": 2}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    return torch


def to_dev(storage, dtype):
    torch_cuda()
    return device.to_dev(storage, dtype)


def empty(shape, dtype):
    torch_cuda()
    return device.empty(shape, dtype)


def from_dev(t, dtype):
    return device.from_dev(t, dtype)


def rel_fro(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def lse_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(x) & np.isneginf(ref)
    if np.any(np.isneginf(x) != np.isneginf(ref)):
        return float("inf")
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, x - ref)
    return float(np.max(np.abs(diff), initial=0.0))


def mask_arg(causal=False, window=0, block_mask=None, block_q=64, block_k=64, dense_mask=None):
    """attn_mask_t fields as a dict of device objects (kept alive by the caller)."""
    d = {"causal": int(causal), "window": int(window), "block_q": block_q, "block_k": block_k}
    if block_mask is not None:
        d["block_mask"] = to_dev(np.asarray(block_mask, np.uint8), "u8")
    if dense_mask is not None:
        d["dense_mask"] = to_dev(np.asarray(dense_mask, np.uint8), "u8")
    return d


def dense_run(dtype, Q, K, V, G, mask, scale, block_b=0, dropout=None, backward=True, ws_form="fast"):
    """Run attn_fwd (and attn_bwd) on storage arrays; return float64 results.
    ws_form "fast": a workspace of attn_bwd_workspace_size_fast bytes (the
    stored-gamma backward where the call has one: dropout with a causal /
    window mask), "min": the minimal one (the dQ kernel recomputes)."""
    import exact_tiled_softmax_amd as ets
    torch = torch_cuda()
    B, H, n_q, d = Q.shape
    H_kv, n_k, dv = K.shape[1], K.shape[2], V.shape[3]
    dq, dk, dvv = to_dev(Q, dtype), to_dev(K, dtype), to_dev(V, dtype)
    Y = empty((B, H, n_q, dv), dtype)
    LSE = torch.zeros((B, H, n_q), dtype=torch.float32, device="cuda")
    dt = DT[dtype]
    ets.attn_fwd(dt, B, H, H_kv, n_q, n_k, d, dv, dq, dk, dvv, mask, scale, block_b, dropout, Y, LSE)
    out = {"Y": Y, "LSE": LSE}
    if backward:
        dg = to_dev(G, dtype)
        dQ, dK, dV = empty(Q.shape, dtype), empty(K.shape, dtype), empty(V.shape, dtype)
        if ws_form == "fast":
            ws_bytes = ets.attn_bwd_workspace_size_fast(dt, B, H, H_kv, n_q, n_k, d, dv, mask, dropout)
        else:
            ws_bytes = ets.attn_bwd_workspace_size(dt, B, H, H_kv, n_q, n_k, d, dv)
        # all-ones bytes (NaN as bf16 / fp16 / fp32): a workspace entry read
        # before it is written turns the gradients into NaN
        ws = torch.full((ws_bytes,), 255, dtype=torch.uint8, device="cuda")
        ets.attn_bwd(dt, B, H, H_kv, n_q, n_k, d, dv, dq, dk, dvv, Y, LSE, dg, mask, scale, block_b,
                     dropout, dQ, dK, dV, ws, ws_bytes)
        out.update(dQ=dQ, dK=dK, dV=dV)
    torch.cuda.synchronize()
    res = {k: (from_dev(v, dtype) if k != "LSE" else v.cpu().numpy().astype(np.float64)) for k, v in out.items()}
    res["_dev"] = out
    return res


def sparse_run(dtype, Q, KV, idx, length, sink, scale, dO=None, lse_kind=None, det=False):
    """Run attn_sparse_fwd (and attn_sparse_bwd when dO is given); with
    lse_kind, the _lse entry points in that LSE convention; with det, the
    deterministic backward."""
    import exact_tiled_softmax_amd as ets
    torch = torch_cuda()
    Tq, H, dqk = Q.shape
    Tkv = KV.shape[0]
    dv = 512 if dO is None else dO.shape[2]
    topk = idx.shape[1]
    dt = DT[dtype]
    q, kv = to_dev(Q, dtype), to_dev(KV, dtype)
    di = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    dl = None if length is None else torch.from_numpy(np.ascontiguousarray(length, np.int32)).cuda()
    ds = None if sink is None else torch.from_numpy(np.ascontiguousarray(sink, np.float32)).cuda()
    O = empty((Tq, H, dv), dtype)
    LSE = torch.zeros((Tq, H), dtype=torch.float32, device="cuda")
    if lse_kind is None:
        ets.attn_sparse_fwd(dt, Tq, H, Tkv, dqk, dv, topk, q, kv, di, dl, ds, scale, O, LSE)
    else:
        ets.attn_sparse_fwd_lse(lse_kind, dt, Tq, H, Tkv, dqk, dv, topk, q, kv, di, dl, ds, scale, O, LSE)
    out = {"O": O, "LSE": LSE}
    if dO is not None:
        g = to_dev(dO, dtype)
        dQ, dKV = empty(Q.shape, dtype), empty(KV.shape, dtype)
        dSink = torch.zeros(H, dtype=torch.float32, device="cuda") if sink is not None else None
        nb = (ets.attn_sparse_bwd_det_workspace_size if det else ets.attn_sparse_bwd_workspace_size)(
            Tq, H, Tkv, dqk, dv, topk)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        if det:
            ets.attn_sparse_bwd_det(ets.ATTN_LSE_TOTAL if lse_kind is None else lse_kind, dt, Tq, H, Tkv, dqk, dv,
                                    topk, q, kv, di, dl, ds, scale, O, LSE, g, dQ, dKV, dSink, ws, nb)
        elif lse_kind is None:
            ets.attn_sparse_bwd(dt, Tq, H, Tkv, dqk, dv, topk, q, kv, di, dl, ds, scale, O, LSE, g, dQ, dKV, dSink,
                                ws, nb)
        else:
            ets.attn_sparse_bwd_lse(lse_kind, dt, Tq, H, Tkv, dqk, dv, topk, q, kv, di, dl, ds, scale, O, LSE, g,
                                    dQ, dKV, dSink, ws, nb)
        out.update(dQ=dQ, dKV=dKV)
        if dSink is not None:
            out["dSink"] = dSink
    torch.cuda.synchronize()
    res = {}
    for k, v in out.items():
        res[k] = v.cpu().numpy().astype(np.float64) if k in ("LSE", "dSink") else from_dev(v, dtype)
    res["_dev"] = out
    return res
