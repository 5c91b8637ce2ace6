"""attn_bwd_noalloc (the backward for callers that cannot allocate: its
workspace is a fixed device array inside the library) against attn_bwd with a
caller workspace: same kernels, so the gradients agree bit for bit.  Two calls
in a row, the second on a smaller problem, so that the second call runs on the
array the first one left behind; then a call past the array's limit is refused
with nothing launched."""

import math

import numpy as np
import pytest

import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _grads(dtype, B, H, H_kv, n, d, mask, seed, noalloc):
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    w = workloads.DenseWorkload("t", B=B, H=H, H_kv=H_kv, n=n, d=d, dv=d, dtype=dtype, c=1.0, seed=seed)
    a = workloads.dense_arrays(w)
    dt = gh.DT[dtype]
    c = 1.0 / math.sqrt(d)
    q, k, v, g = (gh.to_dev(a[x], dtype) for x in ("Q", "K", "V", "G"))
    Y, LSE = gh.empty((B, H, n, d), dtype), torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    ets.attn_fwd(dt, B, H, H_kv, n, n, d, d, q, k, v, mask, c, 0, None, Y, LSE)
    dQ, dK, dV = gh.empty(a["Q"].shape, dtype), gh.empty(a["K"].shape, dtype), gh.empty(a["V"].shape, dtype)
    if noalloc:
        ets.attn_bwd_noalloc(dt, B, H, H_kv, n, n, d, d, q, k, v, Y, LSE, g, mask, c, 0, None, dQ, dK, dV)
    else:
        nb = ets.attn_bwd_workspace_size(dt, B, H, H_kv, n, n, d, d)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        ets.attn_bwd(dt, B, H, H_kv, n, n, d, d, q, k, v, Y, LSE, g, mask, c, 0, None, dQ, dK, dV, ws, nb)
    torch.cuda.synchronize()
    return [gh.from_dev(t, dtype) for t in (dQ, dK, dV)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_backward_matches_workspace_backward_twice(dtype):
    cases = [(2, 8, 4, 1000, 128, {"causal": 1}), (1, 2, 2, 333, 64, {"causal": 1, "window": 100})]
    for B, H, H_kv, n, d, mask in cases:  # the second call is smaller than the first
        ref = _grads(dtype, B, H, H_kv, n, d, mask, 7, noalloc=False)
        got = _grads(dtype, B, H, H_kv, n, d, mask, 7, noalloc=True)
        for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
            assert np.array_equal(x, y), (name, B, H, n, d)


def test_noalloc_refuses_problems_past_its_array():
    import exact_tiled_softmax_amd as ets
    torch = gh.torch_cuda()
    rows_max = (16 << 20) // 8 - 64           # 16 MiB holds two fp32 arrays of rows + 64 entries
    n = 4096
    H = rows_max // n + 1                      # one head too many
    sentinel = torch.full((8,), 99, dtype=torch.int16, device="cuda")
    P = sentinel.data_ptr()
    st = ets.attn_bwd_noalloc(ets.ATTN_BF16, 1, H, H, n, n, 64, 64, P, P, P, P, P, P, {"causal": 1}, 0.125, 0,
                              None, P, P, P, raise_on_error=False)
    assert st == ets.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((sentinel == 99).all())
