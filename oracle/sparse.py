"""Shared-KV top-k sparse attention with an attention sink, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows icavan.github.io, "DeepSeek Sparse Attention Forward and Backward":

  section 1   Q [Tq, H, Dqk], KV [Tkv, Dqk], topk_idxs [Tq, T],
              topk_length [Tq] (optional), attn_sink [H] (optional);
              K = KV[:, :Dqk], V = KV[:, :Dv] (the tied row).
  section 2   s_u = alpha k_u . q over the selected rows I;
              Z = e^z + sum_u e^{s_u};  p_u = e^{s_u} / Z;  p_sink = e^z / Z;
              o = sum_u p_u v_u;  the sink carries no value; z = -inf disables it.
  section 3   dP_u = g . v_u;  D = g . o;  dS_u = p_u (dP_u - D);
              dq = alpha sum_u dS_u k_u;  dK_sel[u] = alpha dS_u q;
              dV_sel[u] = p_u g;  tied merge: dKV[I_u, :Dv] += dK + dV,
              dKV[I_u, Dv:] += dK, reduced over every token and head;
              dz = -p_sink D summed over tokens per head.
  section 7.1 the saved LSE is the sink-inclusive ln Z (natural log).
  section 7.2 a KV-only LSE, ln sum_u e^{s_u}, leaves the sink out; a
              backward pass given it forms LSE_total = logaddexp(LSE_kv, z).

Slots u >= topk_length[t] are padding and are never read.  A token with no
valid slot and no sink has an empty row: O = 0 and LSE = -inf; with a sink it
has O = 0 and LSE = z.
"""

import numpy as np


def _token(Q, KV, idx, length, sink, alpha, dv, t):
    L = idx.shape[1] if length is None else int(length[t])
    I = np.asarray(idx[t, :L], dtype=np.int64)
    Ks = np.asarray(KV[I], dtype=np.float64)            # [L, Dqk]
    q = np.asarray(Q[t], dtype=np.float64)               # [H, Dqk]
    s = alpha * (q @ Ks.T)                                # [H, L]
    H = q.shape[0]
    z = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    top = np.max(s, axis=1) if L else np.full(H, -np.inf)
    M = np.maximum(top, z)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    Zs = np.exp(z - M_safe) + np.exp(s - M_safe[:, None]).sum(axis=1)
    lse = np.where(Zs > 0, M_safe + np.log(np.where(Zs > 0, Zs, 1.0)), -np.inf)
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)
    p = np.where(np.isfinite(lse)[:, None], np.exp(s - lse_safe[:, None]), 0.0)
    p_sink = np.where(np.isfinite(lse), np.exp(z - lse_safe), 0.0)
    return I, Ks, q, p, p_sink, lse


def forward(Q, KV, idx, length, sink, alpha, dv, tokens=None):
    """O [Tq, H, dv] and sink-inclusive LSE [Tq, H] (rows of ``tokens`` only
    when given; other rows are left zero)."""
    Tq, H, _ = Q.shape
    O = np.zeros((Tq, H, dv))
    LSE = np.zeros((Tq, H))
    for t in (range(Tq) if tokens is None else tokens):
        I, Ks, q, p, p_sink, lse = _token(Q, KV, idx, length, sink, alpha, dv, t)
        O[t] = p @ Ks[:, :dv]
        LSE[t] = lse
    return O, LSE


def lse_kv(Q, KV, idx, length, alpha, tokens=None):
    """KV-only LSE [Tq, H] (section 7.2): ln sum_u e^{s_u} over the selected
    rows, written out directly (-inf for a token with no selected row)."""
    Tq, H, _ = Q.shape
    out = np.zeros((Tq, H))
    for t in (range(Tq) if tokens is None else tokens):
        L = idx.shape[1] if length is None else int(length[t])
        if L == 0:
            out[t] = -np.inf
            continue
        Ks = np.asarray(KV[np.asarray(idx[t, :L], dtype=np.int64)], dtype=np.float64)
        s = alpha * (np.asarray(Q[t], dtype=np.float64) @ Ks.T)   # [H, L]
        top = s.max(axis=1)
        out[t] = top + np.log(np.exp(s - top[:, None]).sum(axis=1))
    return out


def lse_total_from_kv(lse_kv_, sink):
    """Section 7.2's normalisation: LSE_total = logaddexp(LSE_kv, z)."""
    if sink is None:
        return np.asarray(lse_kv_, dtype=np.float64)
    return np.logaddexp(lse_kv_, np.asarray(sink, dtype=np.float64)[None, :])


def vjp(Q, KV, idx, length, sink, alpha, dv, dO, tokens=None):
    """(dQ [Tq, H, Dqk], dKV [Tkv, Dqk], dSink [H]).

    With ``tokens`` given only those tokens contribute (to every output)."""
    Tq, H, Dqk = Q.shape
    dQ = np.zeros((Tq, H, Dqk))
    dKV = np.zeros(KV.shape)
    dSink = np.zeros(H)
    for t in (range(Tq) if tokens is None else tokens):
        I, Ks, q, p, p_sink, _ = _token(Q, KV, idx, length, sink, alpha, dv, t)
        g = np.asarray(dO[t], dtype=np.float64)          # [H, dv]
        Vs = Ks[:, :dv]
        o = p @ Vs
        D = (g * o).sum(axis=1)                          # [H]
        dP = g @ Vs.T                                    # [H, L]
        dS = p * (dP - D[:, None])
        dQ[t] = alpha * (dS @ Ks)
        dK_sel = alpha * (dS.T @ q)                      # [L, Dqk]
        dV_sel = p.T @ g                                 # [L, dv]
        dK_sel[:, :dv] += dV_sel
        np.add.at(dKV, I, dK_sel)
        dSink += -p_sink * D
    return dQ, dKV, dSink
