"""Dense masked softmax attention and its analytic VJP, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (per batch b, query head h, query row i; keys j):

  s_ij  = c * sum_r Q_ir K_jr
  A_i   = allowed key set of row i
  Y_i   = sum_{j in A_i} e^{s_ij} V_j / sum_{j in A_i} e^{s_ij}
  LSE_i = ln sum_{j in A_i} e^{s_ij}

This is the dense row that the tiled forward reaches exactly
(alphabetamath.cc, "Tiled attention and its recomputed reverse pass are
exact", proof paragraphs 1-2: disjoint key blocks preserve the summary and the
final division gives the dense masked row).  It is evaluated with the row
maximum m_i as a shift, which changes only rounding.

The reverse pass is the exact gradient of Phi = sum_i sum_a G_ia Y_ia (same
proof, paragraphs 4-6; intale.github.io ch. 19, "Reconstruct probabilities
when a gradient needs them"):

  p_ij   = e^{s_ij - m_i} / l_i            (zero outside A_i)
  D_i    = sum_a G_ia Y_ia
  dP_ij  = sum_a G_ia V_ja
  gamma  = p_ij (dP_ij - D_i)
  dQ_i   = c sum_j gamma_ij K_j,  dK_j = c sum_i gamma_ij Q_i,  dV_j = sum_i p_ij G_i

Inverted dropout (alphabetamath.cc, "A different dropout mask changes the
reverse result"): a fixed realisation xi multiplies each weight by
kappa_ij = xi_ij / (1 - rho).  The forward becomes Y_i = sum_j p_ij kappa_ij V_j;
l_i and the LSE keep the undropped p.  Differentiating that map at fixed xi
gives gamma_ij = p_ij (kappa_ij dP_ij - D_i) and dV_j = sum_i p_ij kappa_ij G_i,
with D_i = G_i . Y_i still (Y already carries kappa).  This dropout form of
gamma is derived here, not printed on the pages.

Rows with an empty allowed set (excluded by the theorem) follow the Rust
course's convention for rows without keys: Y_i = 0 with no division,
LSE_i = -inf, and the row contributes nothing to any gradient.

Grouped heads: query head h reads K/V head h // (H / H_kv), the adjacent group
map of the course's multi-head layer (intale.github.io ch. 19, "Change
attention evaluation inside the existing model"); the key and value gradients
of every query head in a group add into the shared head.

Variable lengths and packed segments (intale.github.io ch. 19: "Change
attention evaluation inside the existing model" intersects the causal range
with each sequence's active length and with packed-segment boundaries; the
update-rule listing under "Rescale earlier mass before adding a new tile"
reads a per-(batch, query row) lower key bound, its `starts`, and that
section's closing paragraph keeps inactive padded rows at zero with no
division).  Two more parts of the allowed set, per batch b:
  lengths[b]      rows i >= lengths[b] are inactive (empty allowed set) and
                  keys j >= lengths[b] are never allowed;
  starts[b, i]    keys j < starts[b, i] are not allowed for row i (for packed
                  segments: the first row of the segment holding row i).
"""

import numpy as np

from . import philox

_ROW_BUDGET = 1 << 22  # score entries per chunk


class Allowed:
    """The allowed-key sets A_i as the AND of the enabled parts.

    causal      j <= i
    window > 0  i - j < window            (a look-back window; with causal,
                                           the window keys include self)
    block_mask  block_mask[i // block_q, j // block_k] != 0
    dense_mask  dense_mask[i, j] != 0
    lengths     per batch b: i < lengths[b] and j < lengths[b]
    starts      per batch b: j >= starts[b, i]
    With no part enabled every key is allowed.  Only lengths and starts
    depend on the batch index.
    """

    def __init__(self, n_q, n_k, causal=False, window=0, block_mask=None,
                 block_q=64, block_k=64, dense_mask=None, lengths=None, starts=None):
        self.n_q, self.n_k = int(n_q), int(n_k)
        self.causal = bool(causal)
        self.window = int(window)
        self.block_mask = None if block_mask is None else np.asarray(block_mask) != 0
        self.block_q, self.block_k = int(block_q), int(block_k)
        self.dense_mask = None if dense_mask is None else np.asarray(dense_mask) != 0
        self.lengths = None if lengths is None else np.asarray(lengths, dtype=np.int64)
        self.starts = None if starts is None else np.asarray(starts, dtype=np.int64)

    def rows(self, rows, b=0):
        """bool [len(rows), n_k] for the given query row indices of batch b."""
        i = np.asarray(rows, dtype=np.int64)[:, None]
        j = np.arange(self.n_k, dtype=np.int64)[None, :]
        a = np.ones((i.shape[0], self.n_k), dtype=bool)
        if self.causal:
            a &= j <= i
        if self.window > 0:
            a &= (i - j) < self.window
        if self.block_mask is not None:
            a &= self.block_mask[i // self.block_q, j // self.block_k]
        if self.dense_mask is not None:
            a &= self.dense_mask[i[:, 0], :]
        if self.lengths is not None:
            n_active = int(self.lengths[b])
            a &= (i < n_active) & (j < n_active)
        if self.starts is not None:
            a &= j >= self.starts[b][i[:, 0]][:, None]
        return a

    def pair_count(self, b=0):
        """|A| = sum_i |A_i| (the number of allowed (i, j) pairs) of batch b."""
        total = 0
        step = max(1, _ROW_BUDGET // max(1, self.n_k))
        for i0 in range(0, self.n_q, step):
            total += int(self.rows(np.arange(i0, min(self.n_q, i0 + step)), b).sum())
        return total


class Dropout:
    """A dropout realisation: either an explicit xi array [B, H, n_q, n_k] or
    the Philox rule of ``philox.keep_mask`` (seed, rho)."""

    def __init__(self, rho, xi=None, seed=None):
        if not (0.0 <= rho < 1.0):
            raise ValueError("dropout rate must lie in [0, 1)")
        if (xi is None) == (seed is None):
            raise ValueError("give exactly one of xi or seed")
        self.rho = float(rho)
        self.xi = None if xi is None else np.asarray(xi) != 0
        self.seed = seed

    def kappa(self, b, h, H, rows, n_k):
        """xi / (1 - rho) for one lane, float64 [len(rows), n_k]."""
        if self.xi is not None:
            keep = self.xi[b, h][np.asarray(rows)]
        else:
            keep = philox.keep_mask(self.seed, self.rho, b * H + h, rows, np.arange(n_k))
        return keep.astype(np.float64) / (1.0 - self.rho)


def _kv_head(h, H, H_kv):
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    return h // (H // H_kv)


def _row_probabilities(q_rows, k, c, allowed_rows):
    """p (zero outside A), m and l for a block of query rows of one lane."""
    s = c * (q_rows @ k.T)
    masked = np.where(allowed_rows, s, -np.inf)
    m = masked.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(allowed_rows, np.exp(masked - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=l[:, None] > 0)
    return p, m, l


def forward_rows(Q, K, V, allowed, c, b, h, rows, dropout=None):
    """Y and LSE for selected query rows of lane (b, h).

    Returns (Y [len(rows), dv], LSE [len(rows)]), float64.
    """
    B, H, n_q, d = Q.shape
    g = _kv_head(h, H, K.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    k = np.asarray(K[b, g], dtype=np.float64)
    v = np.asarray(V[b, g], dtype=np.float64)
    Y = np.zeros((rows.size, v.shape[1]))
    LSE = np.full(rows.size, -np.inf)
    step = max(1, _ROW_BUDGET // max(1, k.shape[0]))
    for s0 in range(0, rows.size, step):
        r = rows[s0:s0 + step]
        p, m, l = _row_probabilities(np.asarray(Q[b, h, r], dtype=np.float64), k, c, allowed.rows(r, b))
        w = p if dropout is None else p * dropout.kappa(b, h, H, r, k.shape[0])
        Y[s0:s0 + step] = w @ v
        LSE[s0:s0 + step] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return Y, LSE


def forward(Q, K, V, allowed, c, dropout=None):
    """Y [B, H, n_q, dv] and LSE [B, H, n_q] for every lane and row."""
    B, H, n_q, _ = Q.shape
    Y = np.zeros((B, H, n_q, V.shape[3]))
    LSE = np.zeros((B, H, n_q))
    rows = np.arange(n_q)
    for b in range(B):
        for h in range(H):
            Y[b, h], LSE[b, h] = forward_rows(Q, K, V, allowed, c, b, h, rows, dropout)
    return Y, LSE


def vjp_lane(Q, K, V, allowed, c, G, b, h, dropout=None, rows=None):
    """Gradient pieces from query rows of lane (b, h).

    Returns (dQ_rows [len(rows), d], dK_part [n_k, d], dV_part [n_k, dv]):
    dQ for those rows and the contributions of those rows to the shared K/V
    head of this lane.
    """
    B, H, n_q, d = Q.shape
    g = _kv_head(h, H, K.shape[1])
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    k = np.asarray(K[b, g], dtype=np.float64)
    v = np.asarray(V[b, g], dtype=np.float64)
    dQ = np.zeros((rows.size, d))
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    step = max(1, _ROW_BUDGET // max(1, k.shape[0]))
    for s0 in range(0, rows.size, step):
        r = rows[s0:s0 + step]
        q = np.asarray(Q[b, h, r], dtype=np.float64)
        gr = np.asarray(G[b, h, r], dtype=np.float64)
        p, _, _ = _row_probabilities(q, k, c, allowed.rows(r, b))
        kap = None if dropout is None else dropout.kappa(b, h, H, r, k.shape[0])
        w = p if kap is None else p * kap
        y = w @ v
        D = (gr * y).sum(axis=1)
        dP = gr @ v.T
        gamma = p * ((dP if kap is None else kap * dP) - D[:, None])
        dQ[s0:s0 + step] = c * (gamma @ k)
        dK += c * (gamma.T @ q)
        dV += w.T @ gr
    return dQ, dK, dV


def vjp(Q, K, V, allowed, c, G, dropout=None):
    """(dQ, dK, dV) of Phi = sum G * Y over all lanes, float64."""
    B, H, n_q, d = Q.shape
    H_kv = K.shape[1]
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, H_kv)
            dq, dk, dv = vjp_lane(Q, K, V, allowed, c, G, b, h, dropout)
            dQ[b, h] = dq
            dK[b, g] += dk
            dV[b, g] += dv
    return dQ, dK, dV
