"""Full-size workloads in the launch configuration bench.py times, checked
against the fp64 oracle on outputs it can compute one by one:

  * whole (batch, head) lanes (every Y, LSE, dQ, dK, dV of the lane), and
  * the last query rows of a lane with the keys only they can see (with a
    causal mask, keys j >= i0 receive gradient only from rows i >= i0), and
  * for the sparse workload, sampled tokens (O, LSE, dQ) and the KV rows only
    the last tokens can select (their dKV), plus a property for dSink, whose
    every term needs every token: dSink_h = -sum_t exp(z_h - LSE_th) dO_th.O_th
    evaluated in fp64 from the kernel's own O and LSE.

Tolerances as in the small parity tests (bf16/fp16: relative Frobenius
<= 1e-2, LSE max abs <= 1e-3).
"""

import math

import numpy as np
import pytest

import workloads
from oracle import dense, sparse
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

REL_TOL = 1e-2
LSE_TOL = 1e-3


def _dense_full(name):
    w = workloads.WORKLOADS[name]
    a = workloads.dense_arrays(w)
    m = gh.mask_arg(causal=w.causal, window=w.window, block_mask=a["block_mask"], block_q=w.mask_tile,
                    block_k=w.mask_tile)
    drop = (w.rho, w.drop_seed) if w.rho > 0 else None
    r = gh.dense_run(w.dtype, a["Q"], a["K"], a["V"], a["G"], m, w.c, block_b=w.block_b, dropout=drop)
    allowed = dense.Allowed(w.n, w.n, causal=w.causal, window=w.window, block_mask=a["block_mask"],
                            block_q=w.mask_tile, block_k=w.mask_tile)
    odrop = dense.Dropout(float(np.float32(w.rho)), seed=w.drop_seed) if w.rho > 0 else None
    return w, a, r, allowed, odrop


def _check_lane(w, a, r, allowed, odrop, b, h, rows=None):
    rows = np.arange(w.n) if rows is None else rows
    Y, LSE = dense.forward_rows(a["Q64"], a["K64"], a["V64"], allowed, w.c, b, h, rows, odrop)
    dQ, dK, dV = dense.vjp_lane(a["Q64"], a["K64"], a["V64"], allowed, w.c, a["G64"], b, h, odrop, rows=rows)
    assert gh.rel_fro(r["Y"][b, h, rows], Y) <= REL_TOL
    assert gh.lse_err(r["LSE"][b, h, rows], LSE) <= LSE_TOL
    assert gh.rel_fro(r["dQ"][b, h, rows], dQ) <= REL_TOL
    # keys that only these rows can see (all keys for a whole lane)
    k0 = int(rows[0]) if w.causal else 0
    assert w.H == w.H_kv
    assert gh.rel_fro(r["dK"][b, h, k0:], dK[k0:]) <= REL_TOL
    assert gh.rel_fro(r["dV"][b, h, k0:], dV[k0:]) <= REL_TOL


def test_dense_causal_bf16_b4h16_n2048_d128():
    w, a, r, allowed, odrop = _dense_full("dense_causal_bf16_b4h16_n2048_d128")
    for b, h in ((0, 0), (3, 15), (2, 7)):
        _check_lane(w, a, r, allowed, odrop, b, h)
    rng = np.random.default_rng(0)
    for _ in range(16):  # random rows of every other lane
        b, h = rng.integers(0, w.B), rng.integers(0, w.H)
        rows = np.sort(rng.choice(w.n, 8, replace=False))
        Y, LSE = dense.forward_rows(a["Q64"], a["K64"], a["V64"], allowed, w.c, b, h, rows)
        assert gh.rel_fro(r["Y"][b, h, rows], Y) <= REL_TOL
        assert gh.lse_err(r["LSE"][b, h, rows], LSE) <= LSE_TOL


def test_masked_window256_tiles64_f16_b2h32_n4096_d64():
    w, a, r, allowed, odrop = _dense_full("masked_window256_tiles64_f16_b2h32_n4096_d64")
    for b, h in ((0, 0), (1, 31)):
        _check_lane(w, a, r, allowed, odrop, b, h)


def test_dropout_causal_bf16_b1h16_n8192_d128():
    w, a, r, allowed, odrop = _dense_full("dropout_causal_bf16_b1h16_n8192_d128")
    tail = np.arange(w.n - 192, w.n)
    for h in (0, 9, 15):
        _check_lane(w, a, r, allowed, odrop, 0, h, rows=tail)
    rng = np.random.default_rng(1)
    for h in (3, 12):
        rows = np.sort(rng.choice(w.n, 24, replace=False))
        Y, LSE = dense.forward_rows(a["Q64"], a["K64"], a["V64"], allowed, w.c, 0, h, rows, odrop)
        assert gh.rel_fro(r["Y"][0, h, rows], Y) <= REL_TOL
        assert gh.lse_err(r["LSE"][0, h, rows], LSE) <= LSE_TOL


def test_sparse_topk2048_sink_bf16_tq4096_h64_tkv16384_d576():
    w = workloads.WORKLOADS["sparse_topk2048_sink_bf16_tq4096_h64_tkv16384_d576"]
    a = workloads.sparse_arrays(w)
    r = gh.sparse_run(w.dtype, a["Q"], a["KV"], a["idx"], a["length"], a["sink"], w.alpha, dO=a["dO"])
    sink64 = a["sink"].astype(np.float64)
    # sampled tokens: padded ones (short prefixes) and full ones
    toks = [0, 1, 100, 510, 511, 1500, 2900, 4095]
    O, LSE = sparse.forward(a["Q64"], a["KV64"], a["idx"], a["length"], sink64, w.alpha, w.dv, tokens=toks)
    dQ, _, _ = sparse.vjp(a["Q64"], a["KV64"], a["idx"], a["length"], sink64, w.alpha, w.dv, a["dO64"], tokens=toks)
    assert gh.rel_fro(r["O"][toks], O[toks]) <= REL_TOL
    assert gh.lse_err(r["LSE"][toks], LSE[toks]) <= LSE_TOL
    assert gh.rel_fro(r["dQ"][toks], dQ[toks]) <= REL_TOL
    # KV rows only the last 24 tokens can select
    t0 = w.Tq - 24
    j0 = workloads.causal_prefix_end(t0 - 1, w.Tq, w.Tkv) + 1
    late = list(range(t0, w.Tq))
    _, dKV, _ = sparse.vjp(a["Q64"], a["KV64"], a["idx"], a["length"], sink64, w.alpha, w.dv, a["dO64"], tokens=late)
    assert gh.rel_fro(r["dKV"][j0:], dKV[j0:]) <= REL_TOL
    # dSink from the kernel's own O and LSE (fp64 on the host)
    D = np.einsum("thv,thv->th", a["dO64"], r["O"])
    want = -(np.exp(sink64[None, :] - r["LSE"]) * D).sum(axis=0)
    assert gh.rel_fro(r["dSink"], want) <= REL_TOL
