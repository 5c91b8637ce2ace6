"""The dropout realisation xi, read back bit for bit from each kernel that
replays it (forward, dK/dV, dQ), against the oracle's Philox keep mask.

Inverted dropout multiplies each weight p_ij by xi_ij / (1 - rho), and the
reverse pass must use the same xi as the forward pass (alphabetamath.cc,
"A different dropout mask changes the reverse result").  The inputs below make
every output element a known function of a single xi_ij, so a wrong bit in any
kernel's replay shows up as a wrong element, not as a small change of a norm.

With Q = 0 every score is 0, so p_ij = 1 / |A_i| on the causal set A_i =
{0..i}.  Keys and rows are taken in blocks of d (block r: indices rd .. rd+d-1):

  forward / dV run:  V_j = e_{j-rd} for keys j of block r (0 elsewhere) and
                     G_i = e_{i-rd} for rows i of block r (0 elsewhere):
                       Y_i[c]  = p_i kappa xi_{i, rd+c}          (rd + c <= i)
                       dV_j[c] = p_i kappa xi_{i, j}, i = rd + c (j <= i)
  dQ run (twice: with the minimal workspace the dQ kernel replays xi itself;
  with the larger one it reads the gamma tiles the dK/dV kernel stored):
                     K_j = e_{j-rd} for keys of block r, V_j = G_i = e_0:
                       dQ_i[c] = scale p_i (kappa xi_{i, rd+c} - D_i),
                       D_i = G_i . Y_i = Y_i[0]
so xi is nonzero-ness of Y and dV, and the nearer of the two candidate values
for dQ (they differ by scale p_i kappa, far above the rounding error).
"""

import numpy as np
import pytest

import workloads
from oracle import philox
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _st(x, dtype):
    return workloads.round_to(x, dtype)[0]


def _decode(dtype, d, n, rate, seed, H=2):
    B = 1
    nb = (n + d - 1) // d
    tri = np.tril(np.ones((n, n), bool))
    xi_y = np.zeros((H, n, n), np.int8) - 1   # -1: not decoded
    xi_dv = np.zeros((H, n, n), np.int8) - 1
    xi_dq = np.zeros((H, n, n), np.int8) - 1
    xi_dqs = np.zeros((H, n, n), np.int8) - 1
    mask = gh.mask_arg(causal=True)
    zeros_qk = np.zeros((B, H, n, d))
    p = 1.0 / np.arange(1, n + 1)
    kappa = float(np.float32(1.0 / (1.0 - float(np.float32(rate)))))
    for r in range(nb):
        blk = np.arange(r * d, min(n, r * d + d))
        c = blk - r * d
        onehot = np.zeros((B, H, n, d))
        onehot[:, :, blk, c] = 1.0
        # forward / dV run
        res = gh.dense_run(dtype, _st(zeros_qk, dtype), _st(zeros_qk, dtype), _st(onehot, dtype),
                           _st(onehot, dtype), mask, 1.0, dropout=(rate, seed))
        for h in range(H):
            Y, dV = res["Y"][0, h], res["dV"][0, h]
            for cc, j in zip(c, blk):
                rows = np.arange(j, n)                     # rows that see key j
                xi_y[h, rows, j] = Y[rows, cc] != 0
                i = j                                      # dV column cc holds row i = rd + cc
                keys = np.arange(0, i + 1)
                xi_dv[h, i, keys] = dV[keys, cc] != 0
        # dQ run
        e0 = np.zeros((B, H, n, d))
        e0[..., 0] = 1.0
        for form, xi_out in (("min", xi_dq), ("fast", xi_dqs)):
            res = gh.dense_run(dtype, _st(zeros_qk, dtype), _st(onehot, dtype), _st(e0, dtype), _st(e0, dtype),
                               mask, 1.0, dropout=(rate, seed), ws_form=form)
            for h in range(H):
                Y, dQ = res["Y"][0, h], res["dQ"][0, h]
                D = Y[:, 0]
                for cc, j in zip(c, blk):
                    rows = np.arange(j, n)
                    kept = p[rows] * (kappa - D[rows])
                    dropped = -p[rows] * D[rows]
                    got = dQ[rows, cc]
                    xi_out[h, rows, j] = np.abs(got - kept) < np.abs(got - dropped)
    want = np.stack([philox.keep_mask(seed, float(np.float32(rate)), h, np.arange(n), np.arange(n))
                     for h in range(H)]).astype(np.int8)
    checks = [("forward", xi_y), ("dK/dV", xi_dv), ("dQ", xi_dq)]
    if dtype != "f32":  # the fp32 path has no stored-gamma form
        checks.append(("dQ from stored gamma", xi_dqs))
    for name, xi in checks:
        assert np.all(xi[:, tri] >= 0), f"{name}: pairs left undecoded"
        bad = np.argwhere((xi != want) & tri[None])
        assert bad.size == 0, f"{name}: {len(bad)} xi bits differ, first (head, row, key) {bad[:5].tolist()}"


@pytest.mark.parametrize("dtype,d,n", [("bf16", 128, 333), ("bf16", 64, 333), ("f16", 128, 300),
                                       ("f16", 64, 270), ("f32", 32, 100)])
def test_dropout_replay_is_bit_exact_in_every_kernel(dtype, d, n):
    _decode(dtype, d, n, rate=0.25, seed=2**33 + 4242)


def test_dropout_replay_at_the_workload_rate():
    # rho = 0.1 (threshold 6553 of 2^16), the dropout workload's rate and seed
    _decode("bf16", 128, 520, rate=0.1, seed=0)
