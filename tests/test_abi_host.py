"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host, before any launch (no GPU needed: every call below
fails validation, so nothing reaches the device)."""

import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:attn_status|size_t|const char\*)\s+(attn_\w+)\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_bwd", "attn_sparse_fwd", "attn_sparse_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import exact_tiled_softmax_amd as ets
    out = subprocess.run(["nm", "-D", "--defined-only", ets.library_path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(ets.lib, n)
        assert hasattr(ets, n), f"binding lacks {n}"


def test_status_strings():
    import exact_tiled_softmax_amd as ets
    assert ets.attn_status_string(ets.ATTN_OK) == "ok"
    assert "workspace" in ets.attn_status_string(ets.ATTN_ERR_WORKSPACE)
    assert ets.attn_status_string(99) == "unknown status"


def test_workspace_sizes():
    import exact_tiled_softmax_amd as ets
    assert ets.attn_bwd_workspace_size(ets.ATTN_BF16, 4, 16, 16, 2048, 2048, 128, 128) == 2 * (((4 * 16 * 2048 + 64) * 4 + 255) // 256 * 256)
    assert ets.attn_bwd_workspace_size(ets.ATTN_BF16, 0, 16, 16, 2048, 2048, 128, 128) == 0
    assert ets.attn_sparse_bwd_workspace_size(4096, 64, 16384, 576, 512, 2048) == 2 * 4096 * 64 * 4 + 16384 * 576 * 4
    assert ets.attn_sparse_bwd_det_workspace_size(4096, 64, 16384, 576, 512, 2048) == 2 * 4096 * 64 * 4 + 16384 * 576 * 8


def test_stored_gamma_workspace_sizes():
    # 16 KiB per (64-key, 128-query) tile a causal / window mask reaches, per
    # (batch, head), with dropout: n = 8192 causal has 64 query tiles, 64 * 65
    # tile slots; n = 2048, 16 * 17
    import exact_tiled_softmax_amd as ets
    drop = (0.1, 0)
    base = ets.attn_bwd_workspace_size(ets.ATTN_BF16, 1, 16, 16, 8192, 8192, 128, 128)
    fast = ets.attn_bwd_workspace_size_fast(ets.ATTN_BF16, 1, 16, 16, 8192, 8192, 128, 128, {"causal": 1}, drop)
    assert fast == base + 16 * 64 * 65 * 16384
    base = ets.attn_bwd_workspace_size(ets.ATTN_BF16, 4, 16, 16, 2048, 2048, 128, 128)
    fast = ets.attn_bwd_workspace_size_fast(ets.ATTN_BF16, 4, 16, 16, 2048, 2048, 128, 128, {"causal": 1}, drop)
    assert fast == base + 4 * 16 * 16 * 17 * 16384
    # causal + 256-key window: at most (256 + 126) // 64 + 2 = 7 key tiles per query tile
    fast = ets.attn_bwd_workspace_size_fast(ets.ATTN_F16, 2, 32, 32, 4096, 4096, 64, 64,
                                            {"causal": 1, "window": 256}, drop)
    assert fast == ets.attn_bwd_workspace_size(ets.ATTN_F16, 2, 32, 32, 4096, 4096, 64, 64) + 64 * 32 * 7 * 16384
    # no mask, n_q != n_k: every key tile of every query tile
    fast = ets.attn_bwd_workspace_size_fast(ets.ATTN_BF16, 1, 2, 2, 150, 270, 64, 64, None, drop)
    assert fast == ets.attn_bwd_workspace_size(ets.ATTN_BF16, 1, 2, 2, 150, 270, 64, 64) + 2 * 2 * 5 * 16384
    # no stored form: without dropout (or at rate 0), fp32, unsupported widths,
    # block masks, layouts; and a (batch, head) whose tiles pass 2 GiB
    for args, mask, dr in (((ets.ATTN_BF16, 1, 1, 1, 256, 256, 64, 64), {"causal": 1}, None),
                           ((ets.ATTN_BF16, 1, 1, 1, 256, 256, 64, 64), {"causal": 1}, (0.0, 3)),
                           ((ets.ATTN_F32, 1, 1, 1, 256, 256, 64, 64), {"causal": 1}, drop),
                           ((ets.ATTN_BF16, 1, 1, 1, 256, 256, 96, 96), {"causal": 1}, drop),
                           ((ets.ATTN_BF16, 1, 1, 1, 256, 256, 64, 64), {"causal": 1, "block_mask": P, "block_q": 64,
                                                                          "block_k": 64}, drop),
                           ((ets.ATTN_BF16, 1, 1, 1, 256, 256, 64, 64), {"causal": 1, "lengths": P}, drop),
                           ((ets.ATTN_BF16, 1, 1, 1, 1 << 16, 1 << 16, 64, 64), {"causal": 1}, drop)):
        assert ets.attn_bwd_workspace_size_fast(*args, mask, dr) == ets.attn_bwd_workspace_size(*args)


P = 0x10000  # a dummy aligned address: never dereferenced, every call fails validation


@pytest.mark.parametrize("case", [
    dict(B=0, code=1), dict(d=0, code=1), dict(H=3, H_kv=2, code=1), dict(scale=-0.5, code=1),
    dict(scale=float("inf"), code=1), dict(dt=7, code=1), dict(d=96, dv=96, code=2), dict(d=128, dv=64, code=2),
    dict(block_b=16, code=2), dict(dt=0, d=256, dv=16, code=2), dict(Q=None, code=1), dict(Q=P + 2, code=1),
    dict(dropout=(1.5, 0), code=1), dict(dropout=(float("nan"), 0), code=1),
    dict(mask={"causal": 1}, n_k=100, code=1), dict(mask={"window": -1}, code=1),
    dict(mask={"block_mask": P, "block_q": 0, "block_k": 64}, code=1),
])
def test_fwd_rejects_before_launch(case):
    import exact_tiled_softmax_amd as ets
    a = dict(dt=ets.ATTN_BF16, B=1, H=2, H_kv=2, n_q=64, n_k=64, d=64, dv=64, Q=P, scale=0.125, block_b=0,
             dropout=None, mask=None)
    a.update({k: v for k, v in case.items() if k != "code"})
    st = ets.attn_fwd(a["dt"], a["B"], a["H"], a["H_kv"], a["n_q"], a["n_k"], a["d"], a["dv"], a["Q"], P, P,
                      a["mask"], a["scale"], a["block_b"], a["dropout"], P, P, stream=0, raise_on_error=False)
    assert st == case["code"]


def test_bwd_rejects_small_workspace_before_launch():
    import exact_tiled_softmax_amd as ets
    need = ets.attn_bwd_workspace_size(ets.ATTN_BF16, 1, 2, 2, 64, 64, 64, 64)
    for ws, nbytes in ((None, need), (P, need - 1), (P + 8, need)):
        st = ets.attn_bwd(ets.ATTN_BF16, 1, 2, 2, 64, 64, 64, 64, P, P, P, P, P, P, None, 0.125, 0, None,
                          P, P, P, ws, nbytes, stream=0, raise_on_error=False)
        assert st == ets.ATTN_ERR_WORKSPACE
    with pytest.raises(ets.AttnError):
        ets.attn_bwd(ets.ATTN_BF16, 1, 2, 2, 64, 64, 64, 64, P, P, P, P, P, P, None, 0.125, 0, None,
                     P, P, P, None, 0, stream=0)


@pytest.mark.parametrize("case", [
    dict(dt=0, code=2), dict(H=32, code=2), dict(d_qk=512, code=2), dict(Tq=0, code=1),
    dict(d_v=600, code=1), dict(scale=-1.0, code=1), dict(idx=None, code=1), dict(KV=P + 4, code=1),
])
def test_sparse_fwd_rejects_before_launch(case):
    import exact_tiled_softmax_amd as ets
    a = dict(dt=ets.ATTN_BF16, Tq=8, H=64, Tkv=32, d_qk=576, d_v=512, topk=16, KV=P, idx=P, scale=0.04)
    a.update({k: v for k, v in case.items() if k != "code"})
    st = ets.attn_sparse_fwd(a["dt"], a["Tq"], a["H"], a["Tkv"], a["d_qk"], a["d_v"], a["topk"], P, a["KV"],
                             a["idx"], None, None, a["scale"], P, P, stream=0, raise_on_error=False)
    assert st == case["code"]


def test_sparse_bwd_needs_dsink_with_sink_and_a_workspace():
    import exact_tiled_softmax_amd as ets
    need = ets.attn_sparse_bwd_workspace_size(8, 64, 32, 576, 512, 16)
    st = ets.attn_sparse_bwd(ets.ATTN_BF16, 8, 64, 32, 576, 512, 16, P, P, P, None, P, 0.04, P, P, P, P, P,
                             None, P, need, stream=0, raise_on_error=False)
    assert st == ets.ATTN_ERR_INVALID_ARG
    st = ets.attn_sparse_bwd(ets.ATTN_BF16, 8, 64, 32, 576, 512, 16, P, P, P, None, None, 0.04, P, P, P, P, P,
                             None, P, need - 1, stream=0, raise_on_error=False)
    assert st == ets.ATTN_ERR_WORKSPACE


def test_sparse_lse_kind_is_checked_before_launch():
    import exact_tiled_softmax_amd as ets
    assert ets.attn_sparse_fwd_lse(2, ets.ATTN_BF16, 8, 64, 32, 576, 512, 16, P, P, P, None, None, 0.04, P, P,
                                   stream=0, raise_on_error=False) == ets.ATTN_ERR_INVALID_ARG
    need = ets.attn_sparse_bwd_workspace_size(8, 64, 32, 576, 512, 16)
    assert ets.attn_sparse_bwd_lse(-1, ets.ATTN_BF16, 8, 64, 32, 576, 512, 16, P, P, P, None, None, 0.04, P, P, P,
                                   P, P, None, P, need, stream=0, raise_on_error=False) == ets.ATTN_ERR_INVALID_ARG
    # a valid kind still goes through the same checks (missing workspace)
    assert ets.attn_sparse_bwd_lse(ets.ATTN_LSE_KV, ets.ATTN_BF16, 8, 64, 32, 576, 512, 16, P, P, P, None, None,
                                   0.04, P, P, P, P, P, None, None, need, stream=0,
                                   raise_on_error=False) == ets.ATTN_ERR_WORKSPACE


def test_sparse_deterministic_backward_needs_its_larger_workspace():
    import exact_tiled_softmax_amd as ets
    small = ets.attn_sparse_bwd_workspace_size(8, 64, 32, 576, 512, 16)
    need = ets.attn_sparse_bwd_det_workspace_size(8, 64, 32, 576, 512, 16)
    assert need > small
    st = ets.attn_sparse_bwd_det(ets.ATTN_LSE_TOTAL, ets.ATTN_BF16, 8, 64, 32, 576, 512, 16, P, P, P, None, None,
                                 0.04, P, P, P, P, P, None, P, need - 1, stream=0, raise_on_error=False)
    assert st == ets.ATTN_ERR_WORKSPACE
    st = ets.attn_sparse_bwd_det(5, ets.ATTN_BF16, 8, 64, 32, 576, 512, 16, P, P, P, None, None,
                                 0.04, P, P, P, P, P, None, P, need, stream=0, raise_on_error=False)
    assert st == ets.ATTN_ERR_INVALID_ARG


def test_dropout_mask_rejects_bad_rate():
    import exact_tiled_softmax_amd as ets
    assert ets.attn_dropout_mask(1.0, 0, 1, 1, 4, 4, P, stream=0, raise_on_error=False) == ets.ATTN_ERR_INVALID_ARG
    assert ets.attn_dropout_mask(0.1, 0, 1, 1, 4, 4, None, stream=0, raise_on_error=False) == ets.ATTN_ERR_INVALID_ARG


def test_mfma_probe_rejects_bad_arguments():
    import ctypes
    import exact_tiled_softmax_amd as ets
    for w, it, sink, n in ((3, 10, P, 256), (1, 0, P, 256), (1, 10, None, 256), (2, 10, P, 0)):
        cnt = ctypes.c_longlong(0)
        st = ets.lib.attn_mfma_probe(w, it, ets._ptr(sink), n, ctypes.byref(cnt), None)
        assert st == ets.ATTN_ERR_INVALID_ARG


def test_issue_atomic_and_lds_probes_reject_bad_arguments():
    import ctypes
    import exact_tiled_softmax_amd as ets
    cnt = ctypes.c_longlong(0)
    for w, k, tr, it, sink, n in ((3, 0, 0, 10, P, 256), (1, 5, 0, 10, P, 256), (1, 4, 0, 0, P, 256),
                                  (2, 4, 0, 10, None, 256), (1, 4, 2, 10, P, 256), (1, 4, -1, 10, P, 256)):
        st = ets.lib.attn_issue_probe(w, k, tr, it, ets._ptr(sink), n, ctypes.byref(cnt), None)
        assert st == ets.ATTN_ERR_INVALID_ARG
    for tab, rows, idx, n_idx, blocks, gpw in ((None, 8, P, 4, 1, 1), (P, 0, P, 4, 1, 1), (P, 8, None, 4, 1, 1),
                                               (P, 8, P, 0, 1, 1), (P, 8, P, 4, 0, 1), (P, 8, P, 4, 1, 0)):
        st = ets.lib.attn_atomic_probe(ets._ptr(tab), rows, ets._ptr(idx), n_idx, blocks, gpw, ctypes.byref(cnt), None)
        assert st == ets.ATTN_ERR_INVALID_ARG
    for w, it, sink, n in ((2, 10, P, 256), (32, 10, P, 256), (8, 0, P, 256), (8, 10, None, 256), (8, 10, P, 0)):
        assert ets.lib.attn_lds_probe(w, it, ets._ptr(sink), n, ctypes.byref(cnt), None) == ets.ATTN_ERR_INVALID_ARG


def test_one_hip_runtime_per_process():
    # the library binds to the HIP runtime PyTorch loads, whatever the import order
    code = ("import exact_tiled_softmax_amd, torch\n"
            "m = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(m))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT, check=True).stdout
    assert out.strip().splitlines()[-1] == "1"


@pytest.mark.parametrize("case", [
    # per-(batch, head) tensors must stay below 2^32 bytes (32-bit buffer extents)
    dict(n_q=1 << 24, n_k=1 << 24, d=128, dv=128, code=2),
    dict(n_k=1 << 24, d=128, dv=128, code=2),
    # at most 2^28 - 64 rows (32-bit workspace offsets)
    dict(B=2, H=1 << 8, H_kv=1 << 8, n_q=1 << 19, n_k=64, code=2),
    # fp32 path: B * H at most 65535
    dict(dt=0, B=256, H=256, H_kv=256, d=16, dv=16, code=2),
    # lengths need n_q == n_k and 4-byte aligned layout arrays
    dict(mask={"lengths": P}, n_k=100, code=1),
    dict(mask={"lengths": P + 2}, code=1),
    dict(mask={"starts": P + 1}, code=1),
])
def test_fwd_limits_and_layout_checks(case):
    import exact_tiled_softmax_amd as ets
    a = dict(dt=ets.ATTN_BF16, B=1, H=2, H_kv=2, n_q=64, n_k=64, d=64, dv=64, mask=None)
    a.update({k: v for k, v in case.items() if k != "code"})
    st = ets.attn_fwd(a["dt"], a["B"], a["H"], a["H_kv"], a["n_q"], a["n_k"], a["d"], a["dv"], P, P, P,
                      a["mask"], 0.125, 0, None, P, P, stream=0, raise_on_error=False)
    assert st == case["code"], case
    if case["code"] == 2:  # the backward applies the same limits
        st = ets.attn_bwd(a["dt"], a["B"], a["H"], a["H_kv"], a["n_q"], a["n_k"], a["d"], a["dv"], P, P, P, P, P, P,
                          a["mask"], 0.125, 0, None, P, P, P, P, 1 << 62, stream=0, raise_on_error=False)
        assert st == 2


def test_nonfinite_status_has_a_name():
    import exact_tiled_softmax_amd as ets
    assert ets.ATTN_ERR_NONFINITE == 5
    assert "non-finite" in ets.attn_status_string(ets.ATTN_ERR_NONFINITE)


def test_mask_struct_layout_matches_the_header():
    # attn_mask_t: int32 causal, int32 window, pointer, int32 block_q, int32
    # block_k, pointer, then the lengths and starts pointers
    import ctypes
    import exact_tiled_softmax_amd as ets
    names = [f[0] for f in ets.Mask._fields_]
    assert names == ["causal", "window", "block_mask", "block_q", "block_k", "dense_mask", "lengths", "starts"]
    assert ctypes.sizeof(ets.Mask) == 48
    text = open(HEADER).read()
    body = text[text.index("typedef struct {\n  int32_t causal;"):text.index("} attn_mask_t;")]
    assert body.index("lengths") < body.index("starts") and "const int32_t* lengths;" in body
