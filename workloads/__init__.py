"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds only random draws, dtype rounding and index bookkeeping: none
of the attention arithmetic.  Both the fp64 oracle and the HIP library receive
their inputs from here, so a parity test compares the two on bit-identical
values.

Recipe (every workload):
  * one ``numpy.random.default_rng(seed)`` stream, seed 0 unless stated;
  * draws in float64 with ``standard_normal``, in the order Q, K, V, G
    (dense) or Q, KV, dO (sparse), then the structure of the workload
    (block mask; sink logits; top-k indices);
  * tensors are rounded to the storage dtype (float64 -> float32 -> bf16 or
    fp16, each step round-to-nearest-even) and the oracle receives the rounded
    values widened back to float64, so parity measures kernel error rather than
    input quantisation.
"""

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------- dtype helpers

DTYPES = ("f32", "f16", "bf16")


def f64_to_bf16_bits(x):
    """Round to bf16 through float32 (both steps round-to-nearest-even);
    returns uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_to(x, dtype):
    """(storage array, float64 widening of it) for dtype in f32/f16/bf16.

    Storage arrays: float32, float16, or uint16 bf16 bit patterns."""
    if dtype == "f32":
        s = np.asarray(x, dtype=np.float32)
        return s, s.astype(np.float64)
    if dtype == "f16":
        s = np.asarray(np.asarray(x, dtype=np.float32), dtype=np.float16)
        return s, s.astype(np.float64)
    if dtype == "bf16":
        s = f64_to_bf16_bits(x)
        return s, bf16_bits_to_f64(s)
    raise ValueError(dtype)


def widen(storage, dtype):
    """float64 values of a storage array."""
    if dtype == "bf16":
        return bf16_bits_to_f64(storage)
    return np.asarray(storage, dtype=np.float64)


# ------------------------------------------------------------------- workloads

@dataclass
class DenseWorkload:
    name: str
    B: int
    H: int
    H_kv: int
    n: int
    d: int
    dv: int
    dtype: str
    c: float
    causal: bool = True
    window: int = 0
    block_mask_p: float = 0.0       # >0: Bernoulli tile mask with this keep probability
    mask_tile: int = 64
    rho: float = 0.0                 # dropout rate
    drop_seed: int = 0
    block_b: int = 0                 # key-block size b (0 = library default)
    seed: int = 0


@dataclass
class SparseWorkload:
    name: str
    Tq: int
    H: int
    Tkv: int
    dqk: int
    dv: int
    topk: int
    dtype: str
    alpha: float
    sink: bool = True
    seed: int = 0


WORKLOADS = {
    # single head, n = 64, d = v = 16, fp32, c = 1/4, b = 16, causal
    "dense_causal_f32_n64_d16": DenseWorkload(
        "dense_causal_f32_n64_d16", B=1, H=1, H_kv=1, n=64, d=16, dv=16, dtype="f32",
        c=0.25, causal=True, block_b=16),
    # dense causal MHA, bf16: B=4, H=16, n=2048, d=v=128
    "dense_causal_bf16_b4h16_n2048_d128": DenseWorkload(
        "dense_causal_bf16_b4h16_n2048_d128", B=4, H=16, H_kv=16, n=2048, d=128, dv=128,
        dtype="bf16", c=1.0 / math.sqrt(128.0), causal=True),
    # sliding window 256 AND Bernoulli(0.5) 64x64 tile mask (diagonal kept), fp16
    "masked_window256_tiles64_f16_b2h32_n4096_d64": DenseWorkload(
        "masked_window256_tiles64_f16_b2h32_n4096_d64", B=2, H=32, H_kv=32, n=4096, d=64, dv=64,
        dtype="f16", c=1.0 / 8.0, causal=True, window=256, block_mask_p=0.5, mask_tile=64),
    # inverted dropout rho = 0.1, causal, bf16: B=1, H=16, n=8192, d=v=128
    "dropout_causal_bf16_b1h16_n8192_d128": DenseWorkload(
        "dropout_causal_bf16_b1h16_n8192_d128", B=1, H=16, H_kv=16, n=8192, d=128, dv=128,
        dtype="bf16", c=1.0 / math.sqrt(128.0), causal=True, rho=0.1, drop_seed=0),
    # shared-KV top-k sparse attention with sink, bf16
    "sparse_topk2048_sink_bf16_tq4096_h64_tkv16384_d576": SparseWorkload(
        "sparse_topk2048_sink_bf16_tq4096_h64_tkv16384_d576", Tq=4096, H=64, Tkv=16384,
        dqk=576, dv=512, topk=2048, dtype="bf16", alpha=1.0 / 24.0),
}


def dense_arrays(w, seed=None):
    """Q, K, V, G (storage and float64) plus the tile mask for a dense workload."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = {}
    shapes = {"Q": (w.B, w.H, w.n, w.d), "K": (w.B, w.H_kv, w.n, w.d),
              "V": (w.B, w.H_kv, w.n, w.dv), "G": (w.B, w.H, w.n, w.dv)}
    for name in ("Q", "K", "V", "G"):
        s, f = round_to(rng.standard_normal(shapes[name]), w.dtype)
        out[name] = s
        out[name + "64"] = f
    out["block_mask"] = None
    if w.block_mask_p > 0:
        nt = (w.n + w.mask_tile - 1) // w.mask_tile
        bm = (rng.random((nt, nt)) < w.block_mask_p).astype(np.uint8)
        np.fill_diagonal(bm, 1)
        out["block_mask"] = bm
    return out


def causal_prefix_end(t, Tq, Tkv):
    """KV position of query token t: the tokens are spread evenly over the KV
    pool, token t sitting at row (t+1)*Tkv/Tq - 1 (its prefix ends there)."""
    return (t + 1) * Tkv // Tq - 1


def sparse_arrays(w, seed=None):
    """Q, KV, dO (storage and float64), sink logits, top-k indices and lengths.

    Indices of token t are drawn uniformly without replacement from its causal
    prefix [0, causal_prefix_end(t)]; when the prefix is shorter than top-k the
    row is padded with -1 and topk_length[t] holds the valid count.  Valid
    indices keep their draw order."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = {}
    shapes = {"Q": (w.Tq, w.H, w.dqk), "KV": (w.Tkv, w.dqk), "dO": (w.Tq, w.H, w.dv)}
    for name in ("Q", "KV", "dO"):
        s, f = round_to(rng.standard_normal(shapes[name]), w.dtype)
        out[name] = s
        out[name + "64"] = f
    out["sink"] = rng.standard_normal(w.H).astype(np.float32) if w.sink else None
    idx = np.full((w.Tq, w.topk), -1, dtype=np.int32)
    length = np.zeros(w.Tq, dtype=np.int32)
    for t in range(w.Tq):
        end = causal_prefix_end(t, w.Tq, w.Tkv)
        L = min(w.topk, end + 1)
        idx[t, :L] = rng.choice(end + 1, size=L, replace=False)
        length[t] = L
    out["idx"] = idx
    out["length"] = length
    return out


def packed_starts(segments, n):
    """starts [n] for packed segments: row i's lower key bound is the first row
    of the segment holding it.  ``segments`` lists segment lengths that sum to
    at most n; rows past them form one last segment."""
    starts = np.zeros(n, dtype=np.int32)
    o = 0
    for s in list(segments) + [max(0, n - int(np.sum(segments)))]:
        starts[o:o + s] = o
        o += s
    return starts
