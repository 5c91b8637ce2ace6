"""Parity of the HIP dense path with the fp64 oracle (GPU, through the C ABI).

Tolerances: fp32 max abs error <= 1e-5; bf16/fp16 relative Frobenius error
<= 1e-2 on Y, dQ, dK, dV and LSE max abs error <= 1e-3.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import dense
from tests import gpu_helpers as gh
from tests.conftest import golden

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
REL_TOL = 1e-2
LSE_TOL = 1e-3


def _inputs(B, H, H_kv, n, d, dv, dtype, seed):
    w = workloads.DenseWorkload("t", B=B, H=H, H_kv=H_kv, n=n, d=d, dv=dv, dtype=dtype, c=1.0, seed=seed)
    return workloads.dense_arrays(w)


def _oracle(a, allowed, c, drop=None):
    Y, LSE = dense.forward(a["Q64"], a["K64"], a["V64"], allowed, c, dropout=drop)
    dQ, dK, dV = dense.vjp(a["Q64"], a["K64"], a["V64"], allowed, c, a["G64"], dropout=drop)
    return {"Y": Y, "LSE": LSE, "dQ": dQ, "dK": dK, "dV": dV}


def _assert_close(got, ref, dtype, what=""):
    if dtype == "f32":
        for k in ("Y", "dQ", "dK", "dV"):
            if k in got:
                err = float(np.max(np.abs(got[k] - ref[k])))
                assert err <= F32_TOL, f"{what} {k} max abs {err}"
        assert gh.lse_err(got["LSE"], ref["LSE"]) <= F32_TOL, what
    else:
        for k in ("Y", "dQ", "dK", "dV"):
            if k in got:
                err = gh.rel_fro(got[k], ref[k])
                assert err <= REL_TOL, f"{what} {k} rel fro {err}"
        err = gh.lse_err(got["LSE"], ref["LSE"])
        assert err <= LSE_TOL, f"{what} LSE {err}"


# ------------------------------------------------------------ page examples


def _lane(x):
    return np.asarray(x, np.float32)[None, None]


@pytest.mark.parametrize("name", ["one_key.json", "empty_first_block.json", "merge_order.json"])
def test_page_examples_fp32(name):
    g = golden(name)
    i, e = g["inputs"], g["expected"]
    Q, K, V = _lane(i["Q"]), _lane(i["K"]), _lane(i["V"])
    n = Q.shape[2]
    G = _lane(i.get("G", np.zeros((n, V.shape[3]))))
    m = gh.mask_arg(dense_mask=np.asarray(i["allowed"], np.uint8))
    r = gh.dense_run("f32", Q, K, V, G, m, i["c"], block_b=i["b"])
    np.testing.assert_allclose(r["Y"][0, 0], e["Y"], atol=1e-6)
    np.testing.assert_allclose(r["LSE"][0, 0], g["derived"]["LSE"], atol=1e-6)
    if name == "one_key.json":
        np.testing.assert_allclose(r["dQ"][0, 0], e["dQ"], atol=1e-6)
        np.testing.assert_allclose(r["dK"][0, 0], e["dK"], atol=1e-6)
        np.testing.assert_allclose(r["dV"][0, 0], e["dV"], atol=1e-6)


def test_two_tile_example_fp32():
    g = golden("two_tile_online.json")
    i, e = g["inputs"], g["expected"]
    Q, K, V = _lane(i["Q"]), _lane(i["K"]), _lane(i["V"])
    G = np.zeros((1, 1, 4, 2), np.float32)
    r = gh.dense_run("f32", Q, K, V, G, gh.mask_arg(causal=True), i["c"], block_b=i["tiles"][1], backward=False)
    np.testing.assert_allclose(r["Y"][0, 0, 3], e["last_dense_output"], rtol=1e-6)
    Yo, _ = dense.forward(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64),
                          dense.Allowed(4, 4, causal=True), i["c"])
    assert float(np.abs(r["Y"] - Yo).max()) <= 1e-5


# ------------------------------------------------------------ fp32 path


@pytest.mark.parametrize("b", [16, 1, 7, 64, 100])
def test_fp32_config_single_head(b):
    # n = 64, d = v = 16, c = 1/4, causal, block size b (16 is the workload's)
    w = workloads.WORKLOADS["dense_causal_f32_n64_d16"]
    a = workloads.dense_arrays(w)
    r = gh.dense_run("f32", a["Q"], a["K"], a["V"], a["G"], gh.mask_arg(causal=True), w.c, block_b=b)
    ref = _oracle(a, dense.Allowed(w.n, w.n, causal=True), w.c)
    _assert_close(r, ref, "f32", f"b={b}")


def test_fp32_gqa_masks_ragged():
    a = _inputs(2, 4, 2, 45, 24, 40, "f32", 3)
    rng = np.random.default_rng(3)
    dm = rng.random((45, 45)) < 0.4
    dm[:, :9] = False
    dm[5] = False                          # an empty row
    m = gh.mask_arg(causal=True, window=20, dense_mask=dm)
    r = gh.dense_run("f32", a["Q"], a["K"], a["V"], a["G"], m, 0.3, block_b=8)
    ref = _oracle(a, dense.Allowed(45, 45, causal=True, window=20, dense_mask=dm), 0.3)
    _assert_close(r, ref, "f32")
    assert np.all(r["Y"][:, :, 5] == 0) and np.all(np.isneginf(r["LSE"][:, :, 5]))


# ------------------------------------------------------------ MFMA path


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f16", 64)])
def test_causal_ragged(dtype, d):
    n = 300  # several 64/128/256 tiles plus a ragged tail
    a = _inputs(1, 2, 2, n, d, d, dtype, 10 + d)
    c = 1.0 / math.sqrt(d)
    r = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], gh.mask_arg(causal=True), c)
    ref = _oracle(a, dense.Allowed(n, n, causal=True), c)
    _assert_close(r, ref, dtype, f"{dtype} d={d}")


@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 128)])
def test_window_and_block_mask(dtype, d):
    n = 333
    a = _inputs(1, 2, 2, n, d, d, dtype, 20 + d)
    rng = np.random.default_rng(21)
    nt = (n + 63) // 64
    bm = (rng.random((nt, nt)) < 0.5).astype(np.uint8)
    np.fill_diagonal(bm, 1)
    c = 1.0 / math.sqrt(d)
    m = gh.mask_arg(causal=True, window=100, block_mask=bm, block_q=64, block_k=64)
    r = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], m, c)
    ref = _oracle(a, dense.Allowed(n, n, causal=True, window=100, block_mask=bm), c)
    _assert_close(r, ref, dtype)


@pytest.mark.parametrize("causal,window,n,d", [(True, 300, 700, 128), (False, 200, 520, 64), (True, 64, 640, 128)])
def test_window_only_long_enough_for_whole_tiles(causal, window, n, d):
    # arithmetic masks long enough that every kernel has runs of tiles (and of
    # dK/dV steps) that every row of a workgroup sees whole, with ragged ends
    a = _inputs(1, 2, 2, n, d, d, "bf16", 80 + d)
    c = 1.0 / math.sqrt(d)
    r = gh.dense_run("bf16", a["Q"], a["K"], a["V"], a["G"], gh.mask_arg(causal=causal, window=window), c)
    ref = _oracle(a, dense.Allowed(n, n, causal=causal, window=window), c)
    _assert_close(r, ref, "bf16", f"causal={causal} window={window} n={n}")


def test_dense_mask_with_empty_leading_blocks_and_empty_rows():
    n, d = 130, 64
    a = _inputs(1, 2, 2, n, d, d, "bf16", 30)
    rng = np.random.default_rng(31)
    dm = rng.random((n, n)) < 0.3
    dm[:64, :70] = False                 # empty leading blocks for the first rows
    dm[np.arange(n), np.arange(n)] = True
    dm[[3, 77, 129]] = False             # rows with an empty allowed set
    m = gh.mask_arg(dense_mask=dm)
    r = gh.dense_run("bf16", a["Q"], a["K"], a["V"], a["G"], m, 0.125)
    ref = _oracle(a, dense.Allowed(n, n, dense_mask=dm), 0.125)
    _assert_close(r, ref, "bf16")
    assert np.all(r["Y"][:, :, [3, 77, 129]] == 0)
    assert np.all(np.isneginf(r["LSE"][:, :, [3, 77, 129]]))


@pytest.mark.parametrize("H,H_kv,n", [(4, 2, 200), (4, 1, 200), (4, 2, 530)])
def test_grouped_heads(H, H_kv, n):
    d = 128
    a = _inputs(2, H, H_kv, n, d, d, "bf16", 40 + H_kv)
    c = 1.0 / math.sqrt(d)
    r = gh.dense_run("bf16", a["Q"], a["K"], a["V"], a["G"], gh.mask_arg(causal=True), c)
    ref = _oracle(a, dense.Allowed(n, n, causal=True), c)
    _assert_close(r, ref, "bf16")


def test_no_mask_cross_lengths():
    # every key allowed, n_q != n_k
    a = _inputs(1, 2, 2, 96, 64, 64, "f16", 50)
    K, V = a["K"][:, :, :70], a["V"][:, :, :70]
    b2 = dict(a, K=K, V=V, K64=a["K64"][:, :, :70], V64=a["V64"][:, :, :70])
    r = gh.dense_run("f16", a["Q"], K, V, a["G"], None, 0.125)
    ref = _oracle(b2, dense.Allowed(96, 70), 0.125)
    _assert_close(r, ref, "f16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_causal_row_zero_is_exact(dtype):
    # p = e^0 = 1 and l = 1 on the first causal row: Y_0 = V_0 bit for bit
    a = _inputs(1, 2, 2, 128, 128, 128, dtype, 60)
    r = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], gh.mask_arg(causal=True), 0.1, backward=False)
    assert np.array_equal(r["Y"][:, :, 0], a["V64"][:, :, 0])


def test_zero_scale_gives_mean_of_allowed_values():
    n, d = 150, 64
    a = _inputs(1, 1, 1, n, d, d, "bf16", 70)
    r = gh.dense_run("bf16", a["Q"], a["K"], a["V"], a["G"], gh.mask_arg(causal=True), 0.0, backward=False)
    mean = np.cumsum(a["V64"][0, 0], axis=0) / np.arange(1, n + 1)[:, None]
    assert gh.rel_fro(r["Y"][0, 0], mean) <= REL_TOL
    np.testing.assert_allclose(r["LSE"][0, 0], np.log(np.arange(1, n + 1)), atol=LSE_TOL)


# ------------------------------------------------------------ dropout


def test_dropout_mask_is_bit_exact():
    import exact_tiled_softmax_amd as ets
    from oracle import philox
    torch = gh.torch_cuda()
    for rate, seed, (B, H, nq, nk) in [(0.1, 0, (2, 3, 37, 41)), (0.5, 2**40 + 12345, (1, 2, 64, 130)),
                                       (0.0, 7, (1, 1, 5, 9))]:
        xi = torch.full((B, H, nq, nk), 7, dtype=torch.uint8, device="cuda")
        ets.attn_dropout_mask(rate, seed, B, H, nq, nk, xi)
        got = xi.cpu().numpy()
        for b in range(B):
            for h in range(H):
                want = philox.keep_mask(seed, float(np.float32(rate)), b * H + h, np.arange(nq), np.arange(nk))
                assert np.array_equal(got[b, h], want.astype(np.uint8)), (rate, seed, b, h)


@pytest.mark.parametrize("dtype,d,n", [("bf16", 128, 256), ("f16", 64, 190), ("f32", 16, 64)])
def test_dropout_forward_backward(dtype, d, n):
    rate, seed = 0.1, 1234
    a = _inputs(1, 2, 2, n, d, d, dtype, 80 + d)
    c = 1.0 / math.sqrt(d)
    r = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], gh.mask_arg(causal=True), c, dropout=(rate, seed))
    drop = dense.Dropout(float(np.float32(rate)), seed=seed)
    ref = _oracle(a, dense.Allowed(n, n, causal=True), c, drop)
    _assert_close(r, ref, dtype)


# ------------------------------------------------------------ error paths


def test_invalid_arguments_touch_nothing():
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    a = _inputs(1, 2, 2, 64, 64, 64, "bf16", 90)
    Q, K, V = gh.to_dev(a["Q"], "bf16"), gh.to_dev(a["K"], "bf16"), gh.to_dev(a["V"], "bf16")
    Y = torch.full((1, 2, 64, 64), 123, dtype=torch.int16, device="cuda")
    LSE = torch.full((1, 2, 64), 5.0, device="cuda")
    bad = [
        dict(d=96, dv=96, code=ets.ATTN_ERR_UNSUPPORTED),         # no kernel for d = 96
        dict(scale=-1.0, code=ets.ATTN_ERR_INVALID_ARG),
        dict(scale=float("nan"), code=ets.ATTN_ERR_INVALID_ARG),
        dict(H_kv=3, code=ets.ATTN_ERR_INVALID_ARG),
        dict(block_b=32, code=ets.ATTN_ERR_UNSUPPORTED),
        dict(n_k=32, mask=gh.mask_arg(causal=True), code=ets.ATTN_ERR_INVALID_ARG),
        dict(dropout=(1.0, 0), code=ets.ATTN_ERR_INVALID_ARG),
    ]
    for case in bad:
        args = dict(d=64, dv=64, scale=0.125, H_kv=2, block_b=0, n_k=64, mask=None, dropout=None)
        args.update({k: v for k, v in case.items() if k != "code"})
        st = ets.attn_fwd(ets.ATTN_BF16, 1, 2, args["H_kv"], 64, args["n_k"], args["d"], args["dv"], Q, K, V,
                          args["mask"], args["scale"], args["block_b"], args["dropout"], Y, LSE,
                          raise_on_error=False)
        assert st == case["code"], case
    torch.cuda.synchronize()
    assert bool((Y == 123).all()) and bool((LSE == 5.0).all())


def test_mfma_probe_runs_and_counts():
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    n = ets.attn_mfma_probe(2, 8, sink, sink.numel())
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert n == cus * 8 * 8 * 8
    assert bool(torch.isfinite(sink[:cus]).all())


def test_issue_and_atomic_probes_run_and_count():
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    assert ets.attn_issue_probe(1, 4, 0, 8, sink, sink.numel()) == cus * 4 * 8 * 8
    assert ets.attn_issue_probe(2, 6, 1, 8, sink, sink.numel()) == cus * 8 * 8 * 8
    torch.cuda.synchronize()
    assert ets.attn_issue_probe(2, 7, 0, 8, sink, sink.numel(), raise_on_error=False) == 0  # 7: not built
    rows = 50
    table = torch.zeros(rows, 576, dtype=torch.float32, device="cuda")
    idx = torch.tensor([3, 49, 3, -1, 60, 0, 7, 3], dtype=torch.int32, device="cuda")
    n = ets.attn_atomic_probe(table, rows, idx, idx.numel(), 2, 1)
    torch.cuda.synchronize()
    assert n == 2 * 4 * 1 * 4 * 576
    counts = torch.zeros(rows)
    for k in range(32):  # 2 blocks x 4 waves x 1 group x 4 rows, indices taken cyclically
        r = int(idx[k % 8])
        if 0 <= r < rows:
            counts[r] += 1
    assert torch.equal(table.cpu(), counts[:, None].expand(rows, 576))


def test_lds_probe_reads_what_it_wrote():
    # the probe's LDS words are i * 2654435761 mod 2^32; workgroup w's first
    # lane XOR-folds the 16-byte reads at (1 KiB k + 64 it) mod 64 KiB
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    iters = 40
    n = ets.attn_lds_probe(8, iters, sink, sink.numel())
    torch.cuda.synchronize()
    assert n == cus * 8 * 64 * 16 * 16 * iters
    words = (np.arange(16384, dtype=np.uint64) * 2654435761) % (1 << 32)
    acc = 0
    for it in range(iters):
        for k in range(16):
            a = ((k * 1024 + it * 64) & 0xFFF0) // 4
            for w in range(4):
                acc ^= int(words[a + w])
    got = sink[:cus].cpu().numpy().view(np.uint32)
    assert np.all(got == acc)


@pytest.mark.parametrize("form", ["min", "fast"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_backward_phases_reproduce_attn_bwd(dtype, d, form):
    # attn_bwd_phase(1), (2), (4) in turn run the same kernels on the same
    # workspace as attn_bwd, so the gradients agree bit for bit (in the
    # stored-gamma form phase 4 reads the tiles phase 2 wrote)
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    n = 333
    a = _inputs(1, 4, 2, n, d, d, dtype, 77)
    c = 1.0 / math.sqrt(d)
    mask = gh.mask_arg(causal=True, window=200)
    drop = (0.15, 99) if form == "fast" else None  # the stored-gamma form needs dropout
    r = gh.dense_run(dtype, a["Q"], a["K"], a["V"], a["G"], mask, c, dropout=drop, ws_form=form)
    dev = r["_dev"]
    dt = gh.DT[dtype]
    shape = (dt, 1, 4, 2, n, n, d, d)
    q, k, v, g = (gh.to_dev(a[x], dtype) for x in ("Q", "K", "V", "G"))
    dQ, dK, dV = gh.empty(a["Q"].shape, dtype), gh.empty(a["K"].shape, dtype), gh.empty(a["V"].shape, dtype)
    nb = ets.attn_bwd_workspace_size(*shape) if form == "min" else ets.attn_bwd_workspace_size_fast(*shape, mask,
                                                                                                  drop)
    assert form == "min" or nb > ets.attn_bwd_workspace_size(*shape)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for ph in (1, 2, 4):
        ets.attn_bwd_phase(ph, *shape, q, k, v, dev["Y"], dev["LSE"], g, mask, c, 0, drop, dQ, dK, dV, ws, nb)
    torch.cuda.synchronize()
    for name, t in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        assert np.array_equal(gh.from_dev(t, dtype), r[name]), name

