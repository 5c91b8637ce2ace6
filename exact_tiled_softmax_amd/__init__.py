"""Python binding of libattn.so (exact tiled masked softmax attention, gfx950).

Argument marshalling only: every function has the name, argument order and
meaning of the C entry point declared in include/attn.h and forwards to it
through ctypes.  Pointer arguments accept an integer device address, None, or
any object with ``data_ptr()`` (a torch tensor).  ``stream`` defaults to the
current torch stream when torch is importable, else the default stream.

The library must be built (``python exact_tiled_softmax_amd/build.py``);
importing this package raises if libattn.so is missing.  There is no fallback
implementation.
"""

import ctypes
import os

__all__ = [
    "ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_WORKSPACE", "ATTN_ERR_HIP",
    "ATTN_ERR_NONFINITE",
    "ATTN_F32", "ATTN_F16", "ATTN_BF16", "ATTN_LSE_TOTAL", "ATTN_LSE_KV", "AttnError", "Mask", "Dropout",
    "attn_fwd", "attn_bwd", "attn_bwd_phase", "attn_bwd_noalloc", "attn_bwd_workspace_size", "attn_bwd_workspace_size_fast", "attn_sparse_fwd", "attn_sparse_bwd",
    "attn_sparse_fwd_lse", "attn_sparse_bwd_lse", "attn_sparse_bwd_det", "attn_sparse_bwd_det_workspace_size",
    "attn_sparse_bwd_workspace_size", "attn_dropout_mask", "attn_mfma_probe", "attn_issue_probe", "attn_atomic_probe", "attn_lds_probe", "attn_status_string", "library_path", "lib",
]

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP, ATTN_ERR_NONFINITE = range(6)
ATTN_F32, ATTN_F16, ATTN_BF16 = range(3)
ATTN_LSE_TOTAL, ATTN_LSE_KV = range(2)

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libattn.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it with `python exact_tiled_softmax_amd/build.py` "
        "(there is no fallback implementation)")



def _share_torch_hip_runtime():
    """Make libattn.so bind to the HIP runtime PyTorch uses.

    The PyTorch wheel ships its own libamdhip64.so.  If libattn.so were loaded
    first it would pull in the system runtime, and a later `import torch` would
    add a second runtime to the process: device memory and streams from one,
    launches on the other.  Loading PyTorch's copy first (same SONAME) makes the
    dynamic linker resolve libattn.so against it.  Without PyTorch the system
    runtime is used."""
    import importlib.util
    import sys
    if "torch" in sys.modules:
        return
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        return
    path = os.path.join(os.path.dirname(spec.origin), "lib", "libamdhip64.so")
    if os.path.exists(path):
        ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)


_share_torch_hip_runtime()
lib = ctypes.CDLL(library_path)


class Mask(ctypes.Structure):
    """attn_mask_t: causal, window, block_mask (device ptr), block_q, block_k, dense_mask,
    lengths and starts (device ptrs)."""
    _fields_ = [("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("block_mask", ctypes.c_void_p), ("block_q", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("dense_mask", ctypes.c_void_p),
                ("lengths", ctypes.c_void_p), ("starts", ctypes.c_void_p)]


class Dropout(ctypes.Structure):
    """attn_dropout_t: rate (float), seed (uint64)."""
    _fields_ = [("rate", ctypes.c_float), ("seed", ctypes.c_uint64)]


_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_pm, _pd = ctypes.POINTER(Mask), ctypes.POINTER(Dropout)

lib.attn_status_string.restype = ctypes.c_char_p
lib.attn_status_string.argtypes = [_i]
lib.attn_fwd.restype = _i
lib.attn_fwd.argtypes = [_i] + [_i] * 7 + [_vp] * 3 + [_pm, _f, _i, _pd, _vp, _vp, _vp]
lib.attn_bwd_workspace_size.restype = _sz
lib.attn_bwd_workspace_size.argtypes = [_i] * 8
lib.attn_bwd_workspace_size_fast.restype = _sz
lib.attn_bwd_workspace_size_fast.argtypes = [_i] * 8 + [_pm, _pd]
lib.attn_bwd.restype = _i
lib.attn_bwd.argtypes = ([_i] + [_i] * 7 + [_vp] * 6 + [_pm, _f, _i, _pd] + [_vp] * 3 + [_vp, _sz, _vp])
lib.attn_bwd_noalloc.restype = _i
lib.attn_bwd_noalloc.argtypes = lib.attn_bwd.argtypes[:-3] + [_vp]
lib.attn_bwd_phase.restype = _i
lib.attn_bwd_phase.argtypes = [_i] + lib.attn_bwd.argtypes
lib.attn_sparse_fwd.restype = _i
lib.attn_sparse_fwd.argtypes = [_i] + [_i] * 6 + [_vp] * 5 + [_f, _vp, _vp, _vp]
lib.attn_sparse_bwd_workspace_size.restype = _sz
lib.attn_sparse_bwd_workspace_size.argtypes = [_i] * 6
lib.attn_sparse_bwd.restype = _i
lib.attn_sparse_bwd.argtypes = ([_i] + [_i] * 6 + [_vp] * 5 + [_f] + [_vp] * 3 + [_vp] * 3 + [_vp, _sz, _vp])
lib.attn_sparse_fwd_lse.restype = _i
lib.attn_sparse_fwd_lse.argtypes = [_i] + lib.attn_sparse_fwd.argtypes
lib.attn_sparse_bwd_lse.restype = _i
lib.attn_sparse_bwd_lse.argtypes = [_i] + lib.attn_sparse_bwd.argtypes
lib.attn_sparse_bwd_det.restype = _i
lib.attn_sparse_bwd_det.argtypes = [_i] + lib.attn_sparse_bwd.argtypes
lib.attn_sparse_bwd_det_workspace_size.restype = _sz
lib.attn_sparse_bwd_det_workspace_size.argtypes = [_i] * 6
lib.attn_dropout_mask.restype = _i
lib.attn_dropout_mask.argtypes = [_f, ctypes.c_uint64, _i, _i, _i, _i, _vp, _vp]
lib.attn_mfma_probe.restype = _i
lib.attn_mfma_probe.argtypes = [_i, _i, _vp, _i, ctypes.POINTER(ctypes.c_longlong), _vp]
lib.attn_issue_probe.restype = _i
lib.attn_issue_probe.argtypes = [_i, _i, _i, _i, _vp, _i, ctypes.POINTER(ctypes.c_longlong), _vp]
lib.attn_atomic_probe.restype = _i
lib.attn_atomic_probe.argtypes = [_vp, _i, _vp, _i, _i, _i, ctypes.POINTER(ctypes.c_longlong), _vp]
lib.attn_lds_probe.restype = _i
lib.attn_lds_probe.argtypes = [_i, _i, _vp, _i, ctypes.POINTER(ctypes.c_longlong), _vp]


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is not None:
        return s if isinstance(s, int) else getattr(s, "cuda_stream", s)
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
    except Exception:  # pragma: no cover - torch without a GPU
        pass
    return None


def _mask(m):
    if m is None:
        return None
    if isinstance(m, Mask):
        return ctypes.byref(m)
    d = dict(m)
    return ctypes.byref(Mask(int(d.get("causal", 0)), int(d.get("window", 0)), _ptr(d.get("block_mask")),
                             int(d.get("block_q", 0)), int(d.get("block_k", 0)), _ptr(d.get("dense_mask")),
                             _ptr(d.get("lengths")), _ptr(d.get("starts"))))


def _drop(d):
    if d is None:
        return None
    if isinstance(d, Dropout):
        return ctypes.byref(d)
    rate, seed = d
    return ctypes.byref(Dropout(float(rate), int(seed)))


def _check(status, where, raise_on_error):
    if raise_on_error and status != ATTN_OK:
        raise AttnError(status, where)
    return status


def attn_status_string(status):
    return lib.attn_status_string(int(status)).decode()


def attn_fwd(dt, B, H, H_kv, n_q, n_k, d, dv, Q, K, V, mask, scale, block_b, dropout, Y, LSE,
             stream=None, raise_on_error=True):
    st = lib.attn_fwd(dt, B, H, H_kv, n_q, n_k, d, dv, _ptr(Q), _ptr(K), _ptr(V), _mask(mask),
                      float(scale), int(block_b), _drop(dropout), _ptr(Y), _ptr(LSE), _stream(stream))
    return _check(st, "attn_fwd", raise_on_error)


def attn_bwd_workspace_size(dt, B, H, H_kv, n_q, n_k, d, dv):
    return lib.attn_bwd_workspace_size(dt, B, H, H_kv, n_q, n_k, d, dv)


def attn_bwd_workspace_size_fast(dt, B, H, H_kv, n_q, n_k, d, dv, mask, dropout):
    return lib.attn_bwd_workspace_size_fast(dt, B, H, H_kv, n_q, n_k, d, dv, _mask(mask), _drop(dropout))


def attn_bwd(dt, B, H, H_kv, n_q, n_k, d, dv, Q, K, V, Y, LSE, G, mask, scale, block_b, dropout,
             dQ, dK, dV, workspace, workspace_bytes, stream=None, raise_on_error=True):
    st = lib.attn_bwd(dt, B, H, H_kv, n_q, n_k, d, dv, _ptr(Q), _ptr(K), _ptr(V), _ptr(Y), _ptr(LSE),
                      _ptr(G), _mask(mask), float(scale), int(block_b), _drop(dropout), _ptr(dQ),
                      _ptr(dK), _ptr(dV), _ptr(workspace), int(workspace_bytes), _stream(stream))
    return _check(st, "attn_bwd", raise_on_error)


def attn_bwd_noalloc(dt, B, H, H_kv, n_q, n_k, d, dv, Q, K, V, Y, LSE, G, mask, scale, block_b, dropout,
                     dQ, dK, dV, stream=None, raise_on_error=True):
    st = lib.attn_bwd_noalloc(dt, B, H, H_kv, n_q, n_k, d, dv, _ptr(Q), _ptr(K), _ptr(V), _ptr(Y), _ptr(LSE),
                              _ptr(G), _mask(mask), float(scale), int(block_b), _drop(dropout), _ptr(dQ),
                              _ptr(dK), _ptr(dV), _stream(stream))
    return _check(st, "attn_bwd_noalloc", raise_on_error)


def attn_bwd_phase(phases, dt, B, H, H_kv, n_q, n_k, d, dv, Q, K, V, Y, LSE, G, mask, scale, block_b,
                   dropout, dQ, dK, dV, workspace, workspace_bytes, stream=None, raise_on_error=True):
    st = lib.attn_bwd_phase(int(phases), dt, B, H, H_kv, n_q, n_k, d, dv, _ptr(Q), _ptr(K), _ptr(V), _ptr(Y),
                            _ptr(LSE), _ptr(G), _mask(mask), float(scale), int(block_b), _drop(dropout),
                            _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(workspace), int(workspace_bytes),
                            _stream(stream))
    return _check(st, "attn_bwd_phase", raise_on_error)


def attn_sparse_fwd(dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length, attn_sink, scale,
                    O, LSE, stream=None, raise_on_error=True):
    st = lib.attn_sparse_fwd(dt, Tq, H, Tkv, d_qk, d_v, topk, _ptr(Q), _ptr(KV), _ptr(topk_idx),
                             _ptr(topk_length), _ptr(attn_sink), float(scale), _ptr(O), _ptr(LSE),
                             _stream(stream))
    return _check(st, "attn_sparse_fwd", raise_on_error)


def attn_sparse_fwd_lse(kind, dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length, attn_sink, scale,
                        O, LSE, stream=None, raise_on_error=True):
    st = lib.attn_sparse_fwd_lse(int(kind), dt, Tq, H, Tkv, d_qk, d_v, topk, _ptr(Q), _ptr(KV), _ptr(topk_idx),
                                 _ptr(topk_length), _ptr(attn_sink), float(scale), _ptr(O), _ptr(LSE),
                                 _stream(stream))
    return _check(st, "attn_sparse_fwd_lse", raise_on_error)


def attn_sparse_bwd_workspace_size(Tq, H, Tkv, d_qk, d_v, topk):
    return lib.attn_sparse_bwd_workspace_size(Tq, H, Tkv, d_qk, d_v, topk)


def attn_sparse_bwd(dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length, attn_sink, scale,
                    O, LSE, dO, dQ, dKV, dSink, workspace, workspace_bytes, stream=None,
                    raise_on_error=True):
    st = lib.attn_sparse_bwd(dt, Tq, H, Tkv, d_qk, d_v, topk, _ptr(Q), _ptr(KV), _ptr(topk_idx),
                             _ptr(topk_length), _ptr(attn_sink), float(scale), _ptr(O), _ptr(LSE),
                             _ptr(dO), _ptr(dQ), _ptr(dKV), _ptr(dSink), _ptr(workspace),
                             int(workspace_bytes), _stream(stream))
    return _check(st, "attn_sparse_bwd", raise_on_error)


def attn_sparse_bwd_lse(kind, dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length, attn_sink, scale,
                        O, LSE, dO, dQ, dKV, dSink, workspace, workspace_bytes, stream=None,
                        raise_on_error=True):
    st = lib.attn_sparse_bwd_lse(int(kind), dt, Tq, H, Tkv, d_qk, d_v, topk, _ptr(Q), _ptr(KV), _ptr(topk_idx),
                                 _ptr(topk_length), _ptr(attn_sink), float(scale), _ptr(O), _ptr(LSE),
                                 _ptr(dO), _ptr(dQ), _ptr(dKV), _ptr(dSink), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream))
    return _check(st, "attn_sparse_bwd_lse", raise_on_error)


def attn_sparse_bwd_det_workspace_size(Tq, H, Tkv, d_qk, d_v, topk):
    return lib.attn_sparse_bwd_det_workspace_size(Tq, H, Tkv, d_qk, d_v, topk)


def attn_sparse_bwd_det(kind, dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length, attn_sink, scale,
                        O, LSE, dO, dQ, dKV, dSink, workspace, workspace_bytes, stream=None,
                        raise_on_error=True):
    st = lib.attn_sparse_bwd_det(int(kind), dt, Tq, H, Tkv, d_qk, d_v, topk, _ptr(Q), _ptr(KV), _ptr(topk_idx),
                                 _ptr(topk_length), _ptr(attn_sink), float(scale), _ptr(O), _ptr(LSE),
                                 _ptr(dO), _ptr(dQ), _ptr(dKV), _ptr(dSink), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream))
    return _check(st, "attn_sparse_bwd_det", raise_on_error)


def attn_dropout_mask(rate, seed, B, H, n_q, n_k, xi, stream=None, raise_on_error=True):
    st = lib.attn_dropout_mask(float(rate), int(seed), B, H, n_q, n_k, _ptr(xi), _stream(stream))
    return _check(st, "attn_dropout_mask", raise_on_error)


def attn_mfma_probe(waves_per_simd, iters, sink, sink_len, stream=None, raise_on_error=True):
    """Launch the MFMA-rate probe; returns the number of MFMA instructions issued."""
    n = ctypes.c_longlong(0)
    st = lib.attn_mfma_probe(int(waves_per_simd), int(iters), _ptr(sink), int(sink_len), ctypes.byref(n),
                             _stream(stream))
    _check(st, "attn_mfma_probe", raise_on_error)
    return n.value


def attn_issue_probe(waves_per_simd, valu_per_mfma, trans, iters, sink, sink_len, stream=None, raise_on_error=True):
    """Launch the MFMA + VALU issue probe; returns the number of MFMA instructions issued."""
    n = ctypes.c_longlong(0)
    st = lib.attn_issue_probe(int(waves_per_simd), int(valu_per_mfma), int(trans), int(iters), _ptr(sink),
                              int(sink_len), ctypes.byref(n), _stream(stream))
    _check(st, "attn_issue_probe", raise_on_error)
    return n.value


def attn_atomic_probe(table, rows, idx, n_idx, blocks, groups_per_wave, stream=None, raise_on_error=True):
    """Launch the fp32 atomic-add rate probe; returns the number of adds issued."""
    n = ctypes.c_longlong(0)
    st = lib.attn_atomic_probe(_ptr(table), int(rows), _ptr(idx), int(n_idx), int(blocks), int(groups_per_wave),
                               ctypes.byref(n), _stream(stream))
    _check(st, "attn_atomic_probe", raise_on_error)
    return n.value


def attn_lds_probe(waves_per_cu, iters, sink, sink_len, stream=None, raise_on_error=True):
    """Launch the LDS read-bandwidth probe; returns the bytes read from LDS."""
    n = ctypes.c_longlong(0)
    st = lib.attn_lds_probe(int(waves_per_cu), int(iters), _ptr(sink), int(sink_len), ctypes.byref(n),
                            _stream(stream))
    _check(st, "attn_lds_probe", raise_on_error)
    return n.value
