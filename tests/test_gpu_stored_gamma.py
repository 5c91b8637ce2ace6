"""The stored-gamma backward (bf16/fp16 with dropout, causal / window masks):
with a workspace of attn_bwd_workspace_size_fast bytes the dK/dV kernel also writes
every gamma_ij = p_ij (kappa_ij G_i . V_j - D_i) it forms, and the dQ product
dQ_i = c sum_j gamma_ij K_j reads them back (alphabetamath.cc, "Tiled
attention and its recomputed reverse pass are exact", paragraphs 4-6).

Each case runs the backward in both forms on the same forward output:
  * dQ, dK, dV of the stored form against the fp64 oracle (relative Frobenius
    <= 1e-2, the bf16/fp16 bar);
  * dK and dV bit-identical between the forms (the same dK/dV kernel, which
    only adds the stores);
  * dQ of the two forms within the same bar of each other.
Shapes cover ragged query and key tails (partly written tiles), a window
whose tiles start mid-way (the strided block layout), n_q != n_k without a
mask, grouped heads, dropout, and keys past the last 128-key block.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import dense
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

REL_TOL = 1e-2


def _inputs(B, H, H_kv, nq, nk, d, dtype, seed):
    w = workloads.DenseWorkload("t", B=B, H=H, H_kv=H_kv, n=max(nq, nk), d=d, dv=d, dtype=dtype, c=1.0, seed=seed)
    a = workloads.dense_arrays(w)
    out = {}
    for k, n in (("Q", nq), ("K", nk), ("V", nk), ("G", nq)):
        out[k] = np.ascontiguousarray(a[k][:, :, :n])
        out[k + "64"] = np.ascontiguousarray(a[k + "64"][:, :, :n])
    if H_kv != H:
        for k in ("K", "V"):
            out[k] = np.ascontiguousarray(out[k][:, :H_kv])
            out[k + "64"] = np.ascontiguousarray(out[k + "64"][:, :H_kv])
    return out


CASES = [
    # dtype, d, B, H, H_kv, nq, nk, causal, window, dropout (rate, seed)
    ("bf16", 128, 1, 2, 2, 200, 200, True, 0, (0.1, 3)),
    ("f16", 64, 2, 2, 2, 330, 330, True, 0, (0.25, 11)),
    ("bf16", 128, 1, 2, 2, 300, 300, True, 100, (0.1, 5)),
    ("bf16", 64, 1, 2, 2, 520, 520, True, 200, (0.3, 2**40 + 1)),
    ("f16", 128, 1, 2, 2, 260, 260, False, 90, (0.1, 8)),
    ("bf16", 64, 1, 2, 2, 150, 270, False, 0, (0.1, 9)),
    ("bf16", 128, 1, 4, 2, 530, 530, True, 0, (0.05, 10)),
    ("bf16", 128, 1, 2, 2, 400, 400, True, 0, (0.1, 12345)),
    ("f16", 64, 1, 2, 1, 700, 700, True, 0, (0.2, 7)),
]


@pytest.mark.parametrize("dtype,d,B,H,H_kv,nq,nk,causal,window,drop", CASES)
def test_stored_gamma_backward_matches_oracle_and_recompute(dtype, d, B, H, H_kv, nq, nk, causal, window, drop):
    import exact_tiled_softmax_amd as ets
    a = _inputs(B, H, H_kv, nq, nk, d, dtype, seed=nq + 31 * d)
    c = 1.0 / math.sqrt(d)
    mask = gh.mask_arg(causal=causal, window=window)
    dt = gh.DT[dtype]
    fast = ets.attn_bwd_workspace_size_fast(dt, B, H, H_kv, nq, nk, d, d, mask, drop)
    assert fast > ets.attn_bwd_workspace_size(dt, B, H, H_kv, nq, nk, d, d)
    rf = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], mask, c, dropout=drop, ws_form="fast")
    rm = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], mask, c, dropout=drop, ws_form="min")
    for k in ("dK", "dV"):
        assert np.array_equal(rf[k], rm[k]), k
    assert gh.rel_fro(rf["dQ"], rm["dQ"]) <= REL_TOL
    allowed = dense.Allowed(nq, nk, causal=causal, window=window)
    odrop = dense.Dropout(float(np.float32(drop[0])), seed=drop[1])
    dQ, dK, dV = dense.vjp(a["Q64"], a["K64"], a["V64"], allowed, c, a["G64"], dropout=odrop)
    for name, ref in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        err = gh.rel_fro(rf[name], ref)
        assert err <= REL_TOL, (name, err)


def test_fast_workspace_size_is_the_minimal_one_without_a_stored_form():
    # fp32, block masks and calls without dropout have no stored-gamma form
    import exact_tiled_softmax_amd as ets
    gh.torch_cuda()
    shape = (1, 2, 2, 128, 128, 64, 64)  # B, H, H_kv, n_q, n_k, d, dv
    drop = (0.1, 1)
    for dt, mask, dr in ((ets.ATTN_F32, {"causal": 1}, drop),
                         (ets.ATTN_BF16, {"causal": 1, "block_mask": gh.to_dev(np.ones((2, 2), np.uint8), "u8"),
                                          "block_q": 64, "block_k": 64}, drop),
                         (ets.ATTN_BF16, {"causal": 1}, None), (ets.ATTN_BF16, {"causal": 1}, (0.0, 1))):
        base = ets.attn_bwd_workspace_size(dt, *shape)
        assert ets.attn_bwd_workspace_size_fast(dt, *shape, mask, dr) == base
