"""The block-summary recurrence for one query row, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows alphabetamath.cc, "Tiled attention and its recomputed reverse pass are
exact" (proof paragraph 1) and intale.github.io ch. 19, "Rescale earlier mass
before adding a new tile" (the update rule and the statement that a tile with
no eligible key leaves the state untouched):

  * the row starts in the empty state (no summary);
  * key blocks J_1, J_2, ... of b consecutive keys are visited in order;
  * a block whose allowed part J & A_i is empty leaves the state unchanged;
  * otherwise, with a = max of the block's allowed scores and
    m' = max(m, a):  alpha = e^{m - m'} (alpha = 0 when the state was empty),
    l' = alpha l + sum_j e^{s_j - m'},  z' = alpha z + sum_j e^{s_j - m'} V_j;
  * after the last block Y = z / l.

Used only to reproduce the intermediate summaries the pages print and to show
that the recurrence reaches the dense row (``dense.forward_rows``).
"""

import numpy as np


def summary_trace(scores, V, allowed, b, order=None):
    """Run the recurrence over one row.

    scores  [n_k] scaled scores s_j of the row
    V       [n_k, dv] value rows
    allowed [n_k] bool, the row's allowed set A_i
    b       key-block size
    order   optional sequence of block indices to visit (default: ascending)

    Returns (cards, Y): one card per visited block with keys
    ``interval`` (start, end), ``empty`` (bool: state after the block is
    still the empty state), ``m``, ``alpha``, ``l``, ``z``; and Y = z / l
    (None while the state is empty).
    """
    scores = np.asarray(scores, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    allowed = np.asarray(allowed, dtype=bool)
    n_k = scores.size
    n_blocks = (n_k + b - 1) // b
    blocks = range(n_blocks) if order is None else order
    m, l, z = None, None, None  # None == the empty state
    cards = []
    for blk in blocks:
        j0, j1 = blk * b, min(n_k, (blk + 1) * b)
        sel = np.nonzero(allowed[j0:j1])[0] + j0
        alpha = None
        if sel.size:
            a = scores[sel].max()
            if m is None:
                m_new, alpha = a, 0.0
                l_prev, z_prev = 0.0, np.zeros(V.shape[1])
            else:
                m_new = max(m, a)
                alpha = float(np.exp(m - m_new))
                l_prev, z_prev = l, z
            e = np.exp(scores[sel] - m_new)
            l = alpha * l_prev + e.sum()
            z = alpha * z_prev + e @ V[sel]
            m = m_new
        cards.append({
            "interval": (j0, j1),
            "empty": m is None,
            "m": m,
            "alpha": alpha,
            "l": l,
            "z": None if z is None else z.copy(),
        })
    Y = None if m is None else z / l
    return cards, Y
