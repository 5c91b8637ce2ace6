"""Variable lengths and packed segments (the `lengths` and `starts` parts of
the allowed set) on the GPU, through the C ABI, against the fp64 oracle.

The course's attention intersects the causal range with each sequence's active
length and with packed-segment boundaries, reads a per-row lower key bound, and
keeps inactive padded rows at zero with no division (intale.github.io ch. 19,
"Change attention evaluation inside the existing model" and "Rescale earlier
mass before adding a new tile").  Tolerances as the other parity tests; rows
past a batch's length must be exactly zero (LSE -inf), as must the key and
value gradients of keys past it.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import dense
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

REL_TOL = 1e-2
LSE_TOL = 1e-3
F32_TOL = 1e-5


def _inputs(B, H, H_kv, n, d, dtype, seed):
    w = workloads.DenseWorkload("t", B=B, H=H, H_kv=H_kv, n=n, d=d, dv=d, dtype=dtype, c=1.0, seed=seed)
    return workloads.dense_arrays(w)


def _dev_i32(x):
    torch = gh.torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


def _run(dtype, a, c, causal=True, window=0, lengths=None, starts=None, block_mask=None, dense_mask=None,
         dropout=None):
    B, H, n, d = a["Q"].shape
    m = gh.mask_arg(causal=causal, window=window, block_mask=block_mask, dense_mask=dense_mask)
    if lengths is not None:
        m["lengths"] = _dev_i32(lengths)
    if starts is not None:
        m["starts"] = _dev_i32(starts)
    r = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], m, c, dropout=dropout)
    allowed = dense.Allowed(n, n, causal=causal, window=window, block_mask=block_mask, dense_mask=dense_mask,
                            lengths=lengths, starts=starts)
    drop = None if dropout is None else dense.Dropout(float(np.float32(dropout[0])), seed=dropout[1])
    Y, LSE = dense.forward(a["Q64"], a["K64"], a["V64"], allowed, c, dropout=drop)
    dQ, dK, dV = dense.vjp(a["Q64"], a["K64"], a["V64"], allowed, c, a["G64"], dropout=drop)
    ref = {"Y": Y, "LSE": LSE, "dQ": dQ, "dK": dK, "dV": dV}
    for k in ("Y", "dQ", "dK", "dV"):
        if dtype == "f32":
            err = float(np.max(np.abs(r[k] - ref[k])))
            assert err <= F32_TOL, f"{k} max abs {err}"
        else:
            err = gh.rel_fro(r[k], ref[k])
            assert err <= REL_TOL, f"{k} rel fro {err}"
    assert gh.lse_err(r["LSE"], LSE) <= (F32_TOL if dtype == "f32" else LSE_TOL)
    if lengths is not None:
        for b, L in enumerate(lengths):
            L = min(max(int(L), 0), n)
            assert np.all(r["Y"][b, :, L:] == 0) and np.all(np.isneginf(r["LSE"][b, :, L:]))
            assert np.all(r["dQ"][b, :, L:] == 0)
            assert np.all(r["dK"][b, :, L:] == 0) and np.all(r["dV"][b, :, L:] == 0)
    return r


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f16", 64)])
def test_lengths_causal(dtype, d):
    n = 333
    a = _inputs(3, 4, 2, n, d, dtype, 100 + d)
    _run(dtype, a, 1.0 / math.sqrt(d), lengths=[333, 130, 0])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_packed_segments_causal(dtype, d):
    n = 400
    a = _inputs(2, 2, 2, n, d, dtype, 110 + d)
    starts = np.stack([workloads.packed_starts([70, 1, 129, 64], n), workloads.packed_starts([400], n)])
    _run(dtype, a, 1.0 / math.sqrt(d), starts=starts)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_lengths_and_segments_with_window(dtype, d):
    n = 520
    a = _inputs(2, 4, 4, n, d, dtype, 120 + d)
    starts = np.stack([workloads.packed_starts([300, 100], n), workloads.packed_starts([17, 250], n)])
    _run(dtype, a, 1.0 / math.sqrt(d), window=150, lengths=[460, 267], starts=starts)


def test_long_sequences_reach_the_whole_tile_loops():
    # lengths long enough that every kernel runs stretches of whole tiles (and
    # dK/dV steps) before the ragged end of each batch
    n, d = 768, 128
    a = _inputs(2, 2, 2, n, d, "bf16", 130)
    _run("bf16", a, 1.0 / math.sqrt(d), lengths=[768, 700])


def test_arbitrary_lower_bounds_with_tile_mask_no_causal():
    # starts need not be segment starts: random per-row lower bounds (some above
    # the last key, giving empty rows), no causal mask, a tile mask
    n, d = 300, 64
    a = _inputs(2, 2, 1, n, d, "f16", 140)
    rng = np.random.default_rng(141)
    starts = rng.integers(-5, n + 10, (2, n)).astype(np.int32)
    nt = (n + 63) // 64
    bm = (rng.random((nt, nt)) < 0.6).astype(np.uint8)
    _run("f16", a, 0.125, causal=False, lengths=[300, 250], starts=starts, block_mask=bm)


def test_dense_mask_with_lengths_and_dropout():
    n, d = 200, 64
    a = _inputs(2, 2, 2, n, d, "bf16", 150)
    rng = np.random.default_rng(151)
    dm = rng.random((n, n)) < 0.5
    dm[np.arange(n), np.arange(n)] = True
    starts = np.stack([workloads.packed_starts([90], n), workloads.packed_starts([20, 20], n)])
    _run("bf16", a, 0.125, causal=False, lengths=[200, 150], starts=starts, dense_mask=dm, dropout=(0.2, 77))


def test_fp32_path_with_layout():
    n, d = 70, 24
    a = _inputs(2, 2, 1, n, d, "f32", 160)
    starts = np.stack([workloads.packed_starts([30, 5], n), workloads.packed_starts([1], n)])
    _run("f32", a, 0.3, lengths=[60, 70], starts=starts)


def test_lengths_out_of_range_are_clamped():
    # outside the debug checks, lengths below 0 or above n act as 0 and n
    n, d = 130, 64
    a = _inputs(2, 1, 1, n, d, "bf16", 170)
    _run("bf16", a, 0.125, lengths=[-7, 10 ** 6])
