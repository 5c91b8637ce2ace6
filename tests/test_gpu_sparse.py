"""Parity of the HIP sparse (shared-KV top-k with sink) path with the fp64
oracle, through the C ABI.  bf16/fp16: relative Frobenius error <= 1e-2 on O,
dQ, dKV and dSink, LSE max abs error <= 1e-3."""

import math

import numpy as np
import pytest

import workloads
from oracle import sparse
from tests import gpu_helpers as gh
from tests.conftest import golden

pytestmark = pytest.mark.gpu

H, DQK, DV = 64, 576, 512
REL_TOL = 1e-2
LSE_TOL = 1e-3


def _case(Tq, Tkv, topk, dtype, seed, lengths="random", sink=True, dup=False):
    rng = np.random.default_rng(seed)
    Q, Q64 = workloads.round_to(rng.standard_normal((Tq, H, DQK)), dtype)
    KV, KV64 = workloads.round_to(rng.standard_normal((Tkv, DQK)), dtype)
    dO, dO64 = workloads.round_to(rng.standard_normal((Tq, H, DV)), dtype)
    z = rng.standard_normal(H).astype(np.float32) if sink else None
    idx = np.full((Tq, topk), -1, np.int32)
    if lengths == "random":
        L = rng.integers(0, topk + 1, Tq).astype(np.int32)
        L[0], L[-1] = 0, topk
    else:
        L = np.full(Tq, topk, np.int32)
    for t in range(Tq):
        idx[t, :L[t]] = rng.choice(Tkv, L[t], replace=dup)
    return dict(Q=Q, Q64=Q64, KV=KV, KV64=KV64, dO=dO, dO64=dO64, sink=z, idx=idx, L=L)


def _check(c, dtype, alpha, use_length=True):
    length = c["L"] if use_length else None
    r = gh.sparse_run(dtype, c["Q"], c["KV"], c["idx"], length, c["sink"], alpha, dO=c["dO"])
    sink64 = None if c["sink"] is None else c["sink"].astype(np.float64)
    O, LSE = sparse.forward(c["Q64"], c["KV64"], c["idx"], length, sink64, alpha, DV)
    dQ, dKV, dSink = sparse.vjp(c["Q64"], c["KV64"], c["idx"], length, sink64, alpha, DV, c["dO64"])
    assert gh.rel_fro(r["O"], O) <= REL_TOL
    assert gh.lse_err(r["LSE"], LSE) <= LSE_TOL
    assert gh.rel_fro(r["dQ"], dQ) <= REL_TOL
    assert gh.rel_fro(r["dKV"], dKV) <= REL_TOL
    if sink64 is not None:
        assert gh.rel_fro(r["dSink"], dSink) <= REL_TOL
    # KV rows no token selected get exactly zero
    used = set()
    for t in range(c["idx"].shape[0]):
        used |= set(c["idx"][t, :(c["L"][t] if use_length else c["idx"].shape[1])].tolist())
    unused = sorted(set(range(c["KV"].shape[0])) - used)
    assert np.all(r["dKV"][unused] == 0)
    return r


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_sparse_ragged_lengths_with_sink(dtype):
    c = _case(24, 300, 100, dtype, 1)
    r = _check(c, dtype, 1.0 / 24.0)
    # the token with no selected row: O = 0 and LSE = its sink logit
    assert np.all(r["O"][0] == 0)
    np.testing.assert_allclose(r["LSE"][0], c["sink"], atol=1e-6)


def test_sparse_without_sink_and_without_lengths():
    c = _case(16, 200, 64, "bf16", 2, lengths="full", sink=False)
    _check(c, "bf16", 1.0 / 24.0, use_length=False)


def test_sparse_duplicate_indices():
    c = _case(12, 50, 70, "bf16", 3, dup=True)
    _check(c, "bf16", 1.0 / 24.0)


def test_sparse_page_example_embedded():
    # the tiny example of the DSA page, embedded in the 576/512 tied row:
    # value column 0 holds v, key column 575 holds ln p, q = e_575, alpha = 1
    g = golden("dsa_tiny.json")
    pr = g["printed"]
    Q = np.zeros((1, H, DQK))
    Q[0, :, 575] = 1.0
    KV = np.zeros((2, DQK))
    KV[:, 0] = pr["v"]
    KV[:, 575] = np.log(pr["p"])
    dO = np.zeros((1, H, DV))
    dO[0, :, 0] = pr["g"]
    sink = np.full(H, math.log(pr["p_sink"]), np.float32)
    idx = np.array([[0, 1]], np.int32)
    Qs, Q64 = workloads.round_to(Q, "f16")
    KVs, KV64 = workloads.round_to(KV, "f16")
    dOs, _ = workloads.round_to(dO, "f16")
    r = gh.sparse_run("f16", Qs, KVs, idx, None, sink, 1.0, dO=dOs)
    np.testing.assert_allclose(r["O"][0, :, 0], pr["o"], atol=2e-3)
    np.testing.assert_allclose(r["LSE"][0], 0.0, atol=2e-3)
    # dKV rows are (p_u g, ..., sum over heads of dS_u) ; dSink sums -p_sink D over the one token
    np.testing.assert_allclose(r["dKV"][:, 0], H * np.asarray(pr["p"]) * pr["g"], rtol=2e-3)
    np.testing.assert_allclose(r["dKV"][:, 575], H * np.asarray(pr["dS"]), rtol=5e-3)
    np.testing.assert_allclose(r["dSink"], pr["dz"], atol=2e-3)


@pytest.mark.parametrize("sink", [True, False])
def test_sparse_kv_only_lse_export_and_backward(sink):
    # [P5] section 7.2: the KV-only LSE leaves the sink out; the backward given
    # it normalises with logaddexp(LSE_kv, z) and must reach the same gradients
    import exact_tiled_softmax_amd as ets
    c = _case(20, 260, 90, "bf16", 5, sink=sink)
    alpha = 1.0 / 24.0
    sink64 = None if c["sink"] is None else c["sink"].astype(np.float64)
    ref = gh.sparse_run("bf16", c["Q"], c["KV"], c["idx"], c["L"], c["sink"], alpha, dO=c["dO"])
    r = gh.sparse_run("bf16", c["Q"], c["KV"], c["idx"], c["L"], c["sink"], alpha, dO=c["dO"],
                      lse_kind=ets.ATTN_LSE_KV)
    assert np.array_equal(r["O"], ref["O"])  # the output does not depend on the convention
    want = sparse.lse_kv(c["Q64"], c["KV64"], c["idx"], c["L"], alpha)
    assert gh.lse_err(r["LSE"], want) <= LSE_TOL
    assert np.all(np.isneginf(r["LSE"][0]))  # token 0 selects no row
    dQ, dKV, dSink = sparse.vjp(c["Q64"], c["KV64"], c["idx"], c["L"], sink64, alpha, DV, c["dO64"])
    assert gh.rel_fro(r["dQ"], dQ) <= REL_TOL
    assert gh.rel_fro(r["dKV"], dKV) <= REL_TOL
    assert gh.rel_fro(r["dQ"], ref["dQ"]) <= 1e-3
    if sink:
        assert gh.rel_fro(r["dSink"], dSink) <= REL_TOL
    else:
        assert np.array_equal(r["LSE"], ref["LSE"])  # without a sink the conventions coincide
        assert np.array_equal(r["dQ"], ref["dQ"])


def test_sparse_deterministic_dkv_is_bit_reproducible():
    # [P5] section 9: fp32 atomics make dKV depend on the order of the adds; the
    # deterministic mode sums fixed-point integers, so two runs agree bit for bit
    c = _case(40, 300, 120, "bf16", 6, dup=True)
    alpha = 1.0 / 24.0
    sink64 = c["sink"].astype(np.float64)
    r1 = gh.sparse_run("bf16", c["Q"], c["KV"], c["idx"], c["L"], c["sink"], alpha, dO=c["dO"], det=True)
    r2 = gh.sparse_run("bf16", c["Q"], c["KV"], c["idx"], c["L"], c["sink"], alpha, dO=c["dO"], det=True)
    ref = gh.sparse_run("bf16", c["Q"], c["KV"], c["idx"], c["L"], c["sink"], alpha, dO=c["dO"])
    assert np.array_equal(r1["dKV"], r2["dKV"])
    assert np.array_equal(r1["dQ"], ref["dQ"]) and np.array_equal(r1["dSink"], ref["dSink"])
    _, dKV, _ = sparse.vjp(c["Q64"], c["KV64"], c["idx"], c["L"], sink64, alpha, DV, c["dO64"])
    assert gh.rel_fro(r1["dKV"], dKV) <= REL_TOL
    assert gh.rel_fro(r1["dKV"], ref["dKV"]) <= 1e-2


@pytest.mark.parametrize("log2_scale", [-20, -30])
def test_sparse_deterministic_dkv_absolute_error_bound(log2_scale):
    # The fixed-point mode rounds each per-token contribution to dKV to a
    # multiple of 2^-32, so its absolute error is at most (selections of the
    # row) * 2^-33 beyond the fp32 path; at small gradient scales that bound is
    # what limits it.  dO is scaled by a power of two, which is exact in bf16.
    c = _case(40, 300, 120, "bf16", 9, dup=True)
    alpha = 1.0 / 24.0
    s = 2.0 ** log2_scale
    dO, dO64 = workloads.round_to(c["dO64"] * s, "bf16")
    assert np.array_equal(dO64, c["dO64"] * s)
    det = gh.sparse_run("bf16", c["Q"], c["KV"], c["idx"], c["L"], c["sink"], alpha, dO=dO, det=True)
    ref = gh.sparse_run("bf16", c["Q"], c["KV"], c["idx"], c["L"], c["sink"], alpha, dO=dO)
    cnt = np.zeros(c["KV"].shape[0])
    for t in range(c["idx"].shape[0]):
        np.add.at(cnt, c["idx"][t, :c["L"][t]], 1.0)
    a, b = det["dKV"], ref["dKV"]
    # one bf16 ulp (2^-7 relative) for the two final roundings, a small
    # allowance for the order-dependent fp32 sums of the atomic path, plus the
    # fixed-point bound of the row
    tol = (2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 2.0 ** -16 * np.abs(b).max()
           + cnt[:, None] * 2.0 ** -33)
    assert np.all(np.abs(a - b) <= tol)
    assert np.all(a[cnt == 0] == 0)
    if log2_scale == -20:
        sink64 = c["sink"].astype(np.float64)
        _, dKV, _ = sparse.vjp(c["Q64"], c["KV64"], c["idx"], c["L"], sink64, alpha, DV, dO64)
        assert gh.rel_fro(det["dKV"], dKV) <= REL_TOL
