"""Debug checks of the C ABI (environment variable ATTN_DEBUG) and the
behaviour of bad index data without them.

With ATTN_DEBUG set, index and length arrays are validated on the device
before any attention kernel runs (ATTN_ERR_INVALID_ARG, outputs untouched)
and outputs are scanned for NaN / infinity afterwards (ATTN_ERR_NONFINITE):
the course refuses non-finite results (intale.github.io ch. 19, closing
paragraph of "Rescale earlier mass before adding a new tile").  Without it,
an out-of-range top-k index reads as an all-zero row and never touches memory
outside the KV tensor.
"""

import numpy as np
import pytest

import workloads
from oracle import sparse
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

H, DQK, DV = 64, 576, 512


def _sparse_case(Tq=6, Tkv=80, topk=40, seed=5):
    rng = np.random.default_rng(seed)
    Q, Q64 = workloads.round_to(rng.standard_normal((Tq, H, DQK)), "bf16")
    KV, KV64 = workloads.round_to(rng.standard_normal((Tkv, DQK)), "bf16")
    dO, dO64 = workloads.round_to(rng.standard_normal((Tq, H, DV)), "bf16")
    idx = np.stack([rng.choice(Tkv, topk, replace=False) for _ in range(Tq)]).astype(np.int32)
    L = np.full(Tq, topk, np.int32)
    sink = rng.standard_normal(H).astype(np.float32)
    return dict(Q=Q, Q64=Q64, KV=KV, KV64=KV64, dO=dO, dO64=dO64, idx=idx, L=L, sink=sink)


def _sparse_call(c, idx, L, backward=False):
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    Tq, Tkv, topk = c["Q"].shape[0], c["KV"].shape[0], idx.shape[1]
    q, kv = gh.to_dev(c["Q"], "bf16"), gh.to_dev(c["KV"], "bf16")
    di = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    dl = torch.from_numpy(np.ascontiguousarray(L, np.int32)).cuda()
    ds = torch.from_numpy(c["sink"]).cuda()
    O = torch.full((Tq, H, DV), 321, dtype=torch.int16, device="cuda")
    LSE = torch.full((Tq, H), 7.0, device="cuda")
    st = ets.attn_sparse_fwd(ets.ATTN_BF16, Tq, H, Tkv, DQK, DV, topk, q, kv, di, dl, ds, 1 / 24, O, LSE,
                             raise_on_error=False)
    if not backward:
        torch.cuda.synchronize()
        return st, O, LSE
    g = gh.to_dev(c["dO"], "bf16")
    dQ = torch.full((Tq, H, DQK), 321, dtype=torch.int16, device="cuda")
    dKV = torch.full((Tkv, DQK), 321, dtype=torch.int16, device="cuda")
    dSink = torch.zeros(H, device="cuda")
    nb = ets.attn_sparse_bwd_workspace_size(Tq, H, Tkv, DQK, DV, topk)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    st2 = ets.attn_sparse_bwd(ets.ATTN_BF16, Tq, H, Tkv, DQK, DV, topk, q, kv, di, dl, ds, 1 / 24, O, LSE, g, dQ,
                              dKV, dSink, ws, nb, raise_on_error=False)
    torch.cuda.synchronize()
    return st, st2, dQ, dKV


@pytest.mark.parametrize("what", ["index_negative", "index_past_end", "length_above_topk", "length_negative"])
def test_debug_rejects_bad_topk_data_before_launch(monkeypatch, what):
    import exact_tiled_softmax_amd as ets
    monkeypatch.setenv("ATTN_DEBUG", "1")
    c = _sparse_case()
    idx, L = c["idx"].copy(), c["L"].copy()
    if what == "index_negative":
        idx[2, 5] = -1
    elif what == "index_past_end":
        idx[4, 39] = c["KV"].shape[0]
    elif what == "length_above_topk":
        L[1] = idx.shape[1] + 1
    else:
        L[3] = -2
    st, O, LSE = _sparse_call(c, idx, L)
    assert st == ets.ATTN_ERR_INVALID_ARG
    assert bool((O == 321).all()) and bool((LSE == 7.0).all())  # nothing launched
    st, st2, dQ, dKV = _sparse_call(c, idx, L, backward=True)
    assert st == st2 == ets.ATTN_ERR_INVALID_ARG
    assert bool((dQ == 321).all()) and bool((dKV == 321).all())


def test_debug_accepts_valid_data_and_ignores_padding(monkeypatch):
    import exact_tiled_softmax_amd as ets
    monkeypatch.setenv("ATTN_DEBUG", "1")
    c = _sparse_case()
    idx, L = c["idx"].copy(), c["L"].copy()
    L[0] = 10
    idx[0, 10:] = -1          # padding past the length is never read
    st, st2, _, _ = _sparse_call(c, idx, L, backward=True)
    assert st == st2 == ets.ATTN_OK


def test_out_of_range_index_reads_as_zero_row_without_debug(monkeypatch):
    # no debug checks: bad indices inside the valid slots read as an all-zero
    # KV row (score 0, value 0) and their dKV contributions are dropped
    monkeypatch.delenv("ATTN_DEBUG", raising=False)
    import exact_tiled_softmax_amd as ets
    c = _sparse_case(seed=6)
    Tkv = c["KV"].shape[0]
    idx = c["idx"].copy()
    idx[1, 3], idx[2, 0], idx[5, 39] = -3, Tkv + 11, -(2 ** 31)
    st, st2, dQ, dKV = _sparse_call(c, idx, c["L"], backward=True)
    assert st == st2 == ets.ATTN_OK
    # the oracle on KV with one extra all-zero row that the bad indices name
    KV64z = np.concatenate([c["KV64"], np.zeros((1, DQK))])
    idxz = np.where((idx < 0) | (idx >= Tkv), Tkv, idx).astype(np.int32)
    sink64 = c["sink"].astype(np.float64)
    rdQ, rdKV, _ = sparse.vjp(c["Q64"], KV64z, idxz, c["L"], sink64, 1 / 24, DV, c["dO64"])
    assert gh.rel_fro(gh.from_dev(dQ, "bf16"), rdQ) <= 1e-2
    assert gh.rel_fro(gh.from_dev(dKV, "bf16"), rdKV[:Tkv]) <= 1e-2


def test_debug_lengths_check_and_nonfinite_scan(monkeypatch):
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    monkeypatch.setenv("ATTN_DEBUG", "1")
    n, d = 64, 64
    w = workloads.DenseWorkload("t", B=2, H=1, H_kv=1, n=n, d=d, dv=d, dtype="bf16", c=0.125, seed=3)
    a = workloads.dense_arrays(w)
    Q, K, V = gh.to_dev(a["Q"], "bf16"), gh.to_dev(a["K"], "bf16"), gh.to_dev(a["V"], "bf16")
    Y = torch.full((2, 1, n, d), 123, dtype=torch.int16, device="cuda")
    LSE = torch.full((2, 1, n), 5.0, device="cuda")
    bad_len = torch.tensor([n, n + 1], dtype=torch.int32, device="cuda")
    m = {"causal": 1, "lengths": bad_len}
    st = ets.attn_fwd(ets.ATTN_BF16, 2, 1, 1, n, n, d, d, Q, K, V, m, 0.125, 0, None, Y, LSE, raise_on_error=False)
    assert st == ets.ATTN_ERR_INVALID_ARG
    assert bool((Y == 123).all())
    ok_len = torch.tensor([n, 0], dtype=torch.int32, device="cuda")
    st = ets.attn_fwd(ets.ATTN_BF16, 2, 1, 1, n, n, d, d, Q, K, V, {"causal": 1, "lengths": ok_len}, 0.125, 0,
                      None, Y, LSE, raise_on_error=False)
    assert st == ets.ATTN_OK  # empty rows' LSE = -inf is allowed
    # a NaN in Q reaches Y: the scan reports it
    qn = a["Q"].copy()
    qn[0, 0, 5, 3] = 0x7FC0  # bf16 NaN
    Qn = gh.to_dev(qn, "bf16")
    st = ets.attn_fwd(ets.ATTN_BF16, 2, 1, 1, n, n, d, d, Qn, K, V, {"causal": 1}, 0.125, 0, None, Y, LSE,
                      raise_on_error=False)
    assert st == ets.ATTN_ERR_NONFINITE
    monkeypatch.delenv("ATTN_DEBUG")
    st = ets.attn_fwd(ets.ATTN_BF16, 2, 1, 1, n, n, d, d, Qn, K, V, {"causal": 1}, 0.125, 0, None, Y, LSE,
                      raise_on_error=False)
    assert st == ets.ATTN_OK  # not checked on the normal path
