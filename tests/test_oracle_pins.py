"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print for a worked example (fixtures under tests/golden/, each with its
citation), closed forms, invariants, special cases that reduce to a library
routine, finite differences, or an independent implementation.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import dense, fd, sparse, summary
from tests.conftest import golden


def _arr(x):
    return np.asarray(x, dtype=np.float64)


def _lane(x):
    """[n, f] -> [1, 1, n, f]"""
    return _arr(x)[None, None]


# ----------------------------------------------------------- page examples


def test_one_key_example():
    g = golden("one_key.json")
    i, e = g["inputs"], g["expected"]
    Q, K, V, G = (_lane(i[k]) for k in ("Q", "K", "V", "G"))
    A = dense.Allowed(1, 1, dense_mask=i["allowed"])
    Y, LSE = dense.forward(Q, K, V, A, i["c"])
    assert Y[0, 0].tolist() == e["Y"]
    assert LSE[0, 0].tolist() == g["derived"]["LSE"]
    cards, y = summary.summary_trace([e["score"]], i["V"], [True], i["b"])
    assert (cards[-1]["m"], cards[-1]["l"], cards[-1]["z"][0]) == tuple(e["summary"])
    dQ, dK, dV = dense.vjp(Q, K, V, A, i["c"], G)
    assert dQ[0, 0].tolist() == e["dQ"]
    assert dK[0, 0].tolist() == e["dK"]
    assert dV[0, 0].tolist() == e["dV"]


def test_empty_first_block_example():
    g = golden("empty_first_block.json")
    i, e = g["inputs"], g["expected"]
    Q, K, V = (_lane(i[k]) for k in ("Q", "K", "V"))
    A = dense.Allowed(2, 2, dense_mask=i["allowed"])
    Y, LSE = dense.forward(Q, K, V, A, i["c"])
    assert Y[0, 0].tolist() == e["Y"]
    np.testing.assert_allclose(LSE[0, 0], g["derived"]["LSE"], rtol=0, atol=1e-15)
    s = np.zeros(2)  # Q = K = 0
    for row, key in ((0, "row0_cards"), (1, "row1_cards")):
        cards, y = summary.summary_trace(s, i["V"], np.asarray(i["allowed"][row], bool), i["b"])
        for card, want in zip(cards, e[key]):
            if want is None:
                assert card["empty"]
            else:
                assert not card["empty"]
                assert (card["m"], card["l"], card["z"][0]) == tuple(want)
        assert y.tolist() == e["Y"][row]


def test_merge_order_example():
    g = golden("merge_order.json")
    i, e = g["inputs"], g["expected"]
    Q, K, V = (_lane(i[k]) for k in ("Q", "K", "V"))
    A = dense.Allowed(2, 2, dense_mask=i["allowed"])
    Y, LSE = dense.forward(Q, K, V, A, i["c"])
    np.testing.assert_allclose(Y[0, 0], e["Y"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(LSE[0, 0], g["derived"]["LSE"], rtol=0, atol=1e-15)
    s = np.array([0.0, math.log(2.0)])
    # each singleton block summary
    for blk, want in enumerate(e["block_summaries"]):
        cards, _ = summary.summary_trace(s, i["V"], [True, True], 1, order=[blk])
        np.testing.assert_allclose((cards[0]["m"], cards[0]["l"], cards[0]["z"][0]), want, atol=1e-15)
    # both merge orders give the same merged summary and output
    for order in ([0, 1], [1, 0]):
        cards, y = summary.summary_trace(s, i["V"], [True, True], 1, order=order)
        c = cards[-1]
        np.testing.assert_allclose((c["m"], c["l"], c["z"][0]), e["merged"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(y, [2.0], atol=1e-15)


def test_dropout_replay_example():
    g = golden("dropout_replay.json")
    i, e = g["inputs"], g["expected"]
    Q, K, V, G = (_lane(i[k]) for k in ("Q", "K", "V", "G"))
    A = dense.Allowed(2, 2, dense_mask=i["allowed"])
    xi = np.broadcast_to(np.asarray(i["xi"])[None, None, None, :], (1, 1, 2, 2))
    drop = dense.Dropout(i["rho"], xi=xi)
    Y, _ = dense.forward(Q, K, V, A, i["c"], dropout=drop)
    assert Y[0, 0, 0].tolist() == e["Y_row0"]
    _, _, dV = dense.vjp(Q, K, V, A, i["c"], G, dropout=drop)
    assert dV[0, 0].tolist() == e["dV"]
    xi2 = np.broadcast_to(np.asarray(i["xi_other"])[None, None, None, :], (1, 1, 2, 2))
    _, _, dV2 = dense.vjp(Q, K, V, A, i["c"], G, dropout=dense.Dropout(i["rho"], xi=xi2))
    assert dV2[0, 0].tolist() == e["dV_other"]
    # undropped weights of row 1 are (1/2, 1/2): kappa = 2 xi gives (1, 0)
    p, _, _ = dense._row_probabilities(np.zeros((1, 1)), np.zeros((2, 1)), 1.0, np.ones((1, 2), bool))
    assert p[0].tolist() == e["undropped_p_row0"]


def test_two_tile_online_example():
    g = golden("two_tile_online.json")
    i, e = g["inputs"], g["expected"]
    Q, K, V = (_lane(i[k]) for k in ("Q", "K", "V"))
    A = dense.Allowed(4, 4, causal=True)
    Y, _ = dense.forward(Q, K, V, A, i["c"])
    row = i["trace_row"]
    s = i["c"] * (_arr(i["Q"])[row] @ _arr(i["K"]).T)
    assert s.tolist() == e["last_scores"]
    cards, y = summary.summary_trace(s, i["V"], A.rows([row])[0], i["tiles"][1])
    for card, want in zip(cards, e["cards"]):
        assert card["interval"] == tuple(want["interval"])
        np.testing.assert_allclose(card["m"], want["m"], rtol=1e-15)
        np.testing.assert_allclose(card["alpha"], want["alpha"], rtol=1e-15, atol=0)
        np.testing.assert_allclose(card["l"], want["l"], rtol=1e-15)
        np.testing.assert_allclose(card["z"], want["u"], rtol=1e-15)
    np.testing.assert_allclose(y, e["last_tiled_output"], rtol=1e-15)
    np.testing.assert_allclose(Y[0, 0, row], e["last_dense_output"], rtol=1e-15)
    # every row: tiled recurrence vs dense within the page's tolerance
    worst = 0.0
    for r in range(4):
        sr = i["c"] * (_arr(i["Q"])[r] @ _arr(i["K"]).T)
        _, yr = summary.summary_trace(sr, i["V"], A.rows([r])[0], i["tiles"][1])
        worst = max(worst, float(np.abs(yr - Y[0, 0, r]).max()))
    assert worst <= e["absolute_tolerance"]
    # the other rows have closed forms: row 0 sees key 0 only, rows 1, 2 are
    # softmax-weighted means of V over their prefixes
    assert Y[0, 0, 0].tolist() == [1.0, 10.0]
    for r in (1, 2):
        w = np.exp(np.arange(r + 1.0))
        np.testing.assert_allclose(Y[0, 0, r], (w / w.sum()) @ _arr(i["V"])[: r + 1], rtol=1e-15)


def test_sparse_tiny_example():
    g = golden("dsa_tiny.json")
    r, pr, dv_ = g["realisation"], g["printed"], g["derived"]
    Q, KV, dO = _arr(r["Q"]), _arr(r["KV"]), _arr(r["dO"])
    idx = np.asarray(r["idx"], dtype=np.int32)
    sink = _arr(r["sink"])
    O, LSE = sparse.forward(Q, KV, idx, None, sink, r["alpha"], r["dv"])
    np.testing.assert_allclose(O[0, 0, 0], pr["o"], atol=1e-15)
    np.testing.assert_allclose(LSE, dv_["LSE"], atol=1e-15)
    dQ, dKV, dSink = sparse.vjp(Q, KV, idx, None, sink, r["alpha"], r["dv"], dO)
    np.testing.assert_allclose(dSink, [pr["dz"]], atol=1e-15)
    # dKV rows are (p_u g, dS_u) for this realisation
    np.testing.assert_allclose(dKV[:, 0], np.asarray(pr["p"]) * pr["g"], atol=1e-15)
    np.testing.assert_allclose(dKV[:, 1], pr["dS"], atol=1e-15)
    np.testing.assert_allclose(dKV, dv_["dKV"], atol=1e-15)
    np.testing.assert_allclose(dQ, dv_["dQ"], atol=1e-15)
    # logit gradients sum to zero (softmax shift invariance)
    assert abs(sum(pr["dS"]) + dSink[0]) < 1e-15


# ------------------------------------------------------ closed forms, invariants


def _rand(shape, rng):
    return rng.standard_normal(shape)


def test_zero_scale_gives_mean_over_allowed_set():
    rng = np.random.default_rng(1)
    Q, K, V = _rand((1, 1, 9, 3), rng), _rand((1, 1, 9, 3), rng), _rand((1, 1, 9, 2), rng)
    mask = rng.random((9, 9)) < 0.5
    mask[np.arange(9), rng.integers(0, 9, 9)] = True
    A = dense.Allowed(9, 9, dense_mask=mask)
    Y, LSE = dense.forward(Q, K, V, A, 0.0)
    for i in range(9):
        np.testing.assert_allclose(Y[0, 0, i], V[0, 0][mask[i]].mean(axis=0), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(LSE[0, 0, i], math.log(mask[i].sum()), rtol=1e-14)


def test_single_allowed_key_copies_value_and_causal_row_zero():
    rng = np.random.default_rng(2)
    Q, K, V = _rand((1, 1, 6, 4), rng), _rand((1, 1, 6, 4), rng), _rand((1, 1, 6, 3), rng)
    pick = rng.integers(0, 6, 6)
    mask = np.zeros((6, 6), bool)
    mask[np.arange(6), pick] = True
    Y, LSE = dense.forward(Q, K, V, dense.Allowed(6, 6, dense_mask=mask), 0.7)
    assert np.array_equal(Y[0, 0], V[0, 0][pick])
    np.testing.assert_allclose(LSE[0, 0], 0.7 * np.einsum("id,id->i", Q[0, 0], K[0, 0][pick]), rtol=1e-14)
    Yc, LSEc = dense.forward(Q, K, V, dense.Allowed(6, 6, causal=True), 0.7)
    assert np.array_equal(Yc[0, 0, 0], V[0, 0, 0])


def test_hard_attention_selects_the_right_key_and_value():
    # one dominant score per row: Y_i equals V at the chosen key (pins the
    # orientation of Q K^T and the V index)
    n, d = 7, 8
    rng = np.random.default_rng(3)
    perm = rng.permutation(n)
    Q = np.zeros((1, 1, n, d))
    K = np.zeros((1, 1, n, d))
    Q[0, 0, np.arange(n), np.arange(n) % d] = 1.0
    K[0, 0, perm, np.arange(n) % d] = 1.0
    K[0, 0] += 1e-3 * rng.standard_normal((n, d))
    V = rng.standard_normal((1, 1, n, 3))
    Y, _ = dense.forward(Q, K, V, dense.Allowed(n, n), 2000.0)
    np.testing.assert_allclose(Y[0, 0], V[0, 0, perm], rtol=0, atol=1e-12)


def test_row_shift_invariance_via_extra_feature():
    # appending feature 1 to Q and t to K adds c*t to every score of every row:
    # Y is unchanged and the LSE shifts by c*t
    rng = np.random.default_rng(4)
    n, d = 10, 5
    Q, K, V = _rand((1, 2, n, d), rng), _rand((1, 2, n, d), rng), _rand((1, 2, n, 4), rng)
    A = dense.Allowed(n, n, causal=True, window=4)
    c, t = 0.3, 2.5
    Y, LSE = dense.forward(Q, K, V, A, c)
    Q2 = np.concatenate([Q, np.ones((1, 2, n, 1))], axis=3)
    K2 = np.concatenate([K, np.full((1, 2, n, 1), t)], axis=3)
    Y2, LSE2 = dense.forward(Q2, K2, V, A, c)
    np.testing.assert_allclose(Y2, Y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(LSE2, LSE + c * t, rtol=1e-13)


def test_unmasked_matches_library_softmax():
    rng = np.random.default_rng(5)
    n, d = 12, 6
    Q, K, V = _rand((2, 3, n, d), rng), _rand((2, 3, n, d), rng), _rand((2, 3, n, 5), rng)
    Y, LSE = dense.forward(Q, K, V, dense.Allowed(n, n), 0.4)
    S = 0.4 * np.matmul(Q, np.swapaxes(K, -1, -2))
    np.testing.assert_allclose(Y, np.matmul(scipy.special.softmax(S, axis=-1), V), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(LSE, scipy.special.logsumexp(S, axis=-1), rtol=1e-13)


def test_empty_row_is_zero_with_minus_inf_lse():
    rng = np.random.default_rng(6)
    Q, K, V, G = (_rand((1, 1, 4, 3), rng) for _ in range(4))
    mask = np.ones((4, 4), bool)
    mask[2] = False
    A = dense.Allowed(4, 4, dense_mask=mask)
    Y, LSE = dense.forward(Q, K, V, A, 1.0)
    assert np.all(Y[0, 0, 2] == 0) and LSE[0, 0, 2] == -np.inf
    dQ, dK, dV = dense.vjp(Q, K, V, A, 1.0, G)
    assert np.all(dQ[0, 0, 2] == 0)
    # row 2 contributes nothing: changing G_2 changes no gradient
    G2 = G.copy()
    G2[0, 0, 2] = 100.0
    for a, b in zip((dQ, dK, dV), dense.vjp(Q, K, V, A, 1.0, G2)):
        np.testing.assert_array_equal(a, b)


def test_gradient_sum_invariants():
    # sum_j gamma_ij = 0 per row  =>  sum_j dK_j = 0 ;  sum_j dV_j = sum_i G_i
    rng = np.random.default_rng(7)
    n, d = 16, 4
    Q, K, V, G = _rand((2, 2, n, d), rng), _rand((2, 2, n, d), rng), _rand((2, 2, n, 3), rng), _rand((2, 2, n, 3), rng)
    A = dense.Allowed(n, n, causal=True, window=5)
    _, dK, dV = dense.vjp(Q, K, V, A, 0.5, G)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-13)
    np.testing.assert_allclose(dV.sum(axis=2), G.sum(axis=2), rtol=1e-13, atol=1e-13)


def test_summary_recurrence_reaches_the_dense_row():
    # the theorem of the first page: for any block size b and any allowed set
    # (including empty leading blocks) the recurrence equals the dense row
    rng = np.random.default_rng(8)
    n, d = 23, 3
    Q, K, V = _rand((1, 1, n, d), rng), _rand((1, 1, n, d), rng), _rand((1, 1, n, 2), rng)
    mask = rng.random((n, n)) < 0.3
    mask[:, :6] = False
    mask[np.arange(n), np.arange(n)] = True
    A = dense.Allowed(n, n, dense_mask=mask)
    Y, _ = dense.forward(Q, K, V, A, 0.8)
    for b in (1, 2, 5, 8, 23, 40):
        for i in range(n):
            s = 0.8 * (Q[0, 0, i] @ K[0, 0].T)
            cards, y = summary.summary_trace(s, V[0, 0], mask[i], b)
            np.testing.assert_allclose(y, Y[0, 0, i], rtol=1e-13, atol=1e-14)
            # the empty leading block leaves the state empty
            assert cards[0]["empty"] == (not mask[i, :b].any())


# ------------------------------------------------------------ finite differences


def _phi_dense(A, c, drop):
    def fn(arrs):
        Q, K, V, G = arrs
        Y, _ = dense.forward(Q, K, V, A, c, dropout=drop)
        return float((G * Y).sum())
    return fn


@pytest.mark.parametrize("case", ["mha_random_mask", "gqa_window", "dropout_xi"])
def test_dense_vjp_matches_finite_differences(case):
    rng = np.random.default_rng({"mha_random_mask": 10, "gqa_window": 11, "dropout_xi": 12}[case])
    n, d, dv = 6, 3, 2
    H, H_kv = (2, 1) if case == "gqa_window" else (1, 1)
    Q, K = rng.standard_normal((1, H, n, d)), rng.standard_normal((1, H_kv, n, d))
    V, G = rng.standard_normal((1, H_kv, n, dv)), rng.standard_normal((1, H, n, dv))
    drop = None
    if case == "mha_random_mask":
        mask = rng.random((n, n)) < 0.5
        mask[:, :2] = False                  # empty leading block for b = 2
        mask[np.arange(n), np.arange(n)] = True
        A = dense.Allowed(n, n, dense_mask=mask)
    elif case == "gqa_window":
        A = dense.Allowed(n, n, causal=True, window=3)
    else:
        A = dense.Allowed(n, n, causal=True)
        drop = dense.Dropout(0.3, xi=rng.random((1, H, n, n)) < 0.7)
    c = 0.9
    dQ, dK, dV = dense.vjp(Q, K, V, A, c, G, dropout=drop)
    Q0, K0, V0 = Q.copy(), K.copy(), V.copy()
    num = fd.gradient(_phi_dense(A, c, drop), [Q, K, V, G])
    assert np.array_equal(Q, Q0) and np.array_equal(K, K0) and np.array_equal(V, V0)
    for a, b in zip((dQ, dK, dV), num[:3]):
        np.testing.assert_allclose(a, b, rtol=0, atol=4e-6)


@pytest.mark.parametrize("with_sink", [True, False])
def test_sparse_vjp_matches_finite_differences(with_sink):
    rng = np.random.default_rng(20 + with_sink)
    Tq, H, Tkv, dqk, dv, T = 3, 2, 7, 4, 3, 4
    Q, KV, dO = rng.standard_normal((Tq, H, dqk)), rng.standard_normal((Tkv, dqk)), rng.standard_normal((Tq, H, dv))
    idx = np.array([[5, 1, -1, -1], [0, 6, 2, 3], [4, 4, 1, 0]], dtype=np.int32)  # padded row; repeated index
    length = np.array([2, 4, 4], dtype=np.int32)
    sink = rng.standard_normal(H) if with_sink else None
    alpha = 0.6
    dQ, dKV, dSink = sparse.vjp(Q, KV, idx, length, sink, alpha, dv, dO)

    def fn(arrs):
        q, kv, s = arrs
        O, _ = sparse.forward(q, kv, idx, length, s if with_sink else None, alpha, dv)
        return float((dO * O).sum())

    s_arr = sink.copy() if with_sink else np.zeros(H)
    num = fd.gradient(fn, [Q, KV, s_arr])
    np.testing.assert_allclose(dQ, num[0], atol=4e-6)
    np.testing.assert_allclose(dKV, num[1], atol=4e-6)
    if with_sink:
        np.testing.assert_allclose(dSink, num[2], atol=4e-6)
    # rows never selected get exactly zero
    unused = sorted(set(range(Tkv)) - set(idx[0, :2]) - set(idx[1]) - set(idx[2]))
    assert np.all(dKV[unused] == 0)


def test_sparse_without_sink_reduces_to_dense_on_gathered_rows():
    rng = np.random.default_rng(30)
    Tq, H, Tkv, dqk, dv, T = 4, 3, 20, 6, 4, 5
    Q, KV, dO = rng.standard_normal((Tq, H, dqk)), rng.standard_normal((Tkv, dqk)), rng.standard_normal((Tq, H, dv))
    idx = np.stack([rng.choice(Tkv, T, replace=False) for _ in range(Tq)]).astype(np.int32)
    alpha = 0.35
    O, LSE = sparse.forward(Q, KV, idx, None, None, alpha, dv)
    dQ, dKV, _ = sparse.vjp(Q, KV, idx, None, None, alpha, dv, dO)
    dKV_ref = np.zeros_like(KV)
    for t in range(Tq):
        Kt = KV[idx[t]][None, None]               # [1, 1, T, dqk]
        Vt = KV[idx[t], :dv][None, None]
        q = Q[t][None, :, None, :]                # [1, H, 1, dqk] per head as one row
        for h in range(H):
            A = dense.Allowed(1, T)
            Y, L = dense.forward(q[:, h:h + 1], Kt, Vt, A, alpha)
            np.testing.assert_allclose(O[t, h], Y[0, 0, 0], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(LSE[t, h], L[0, 0, 0], rtol=1e-13)
            g = dO[t, h][None, None, None, :]
            dq, dk, dvv = dense.vjp(q[:, h:h + 1], Kt, Vt, A, alpha, g)
            np.testing.assert_allclose(dQ[t, h], dq[0, 0, 0], rtol=1e-12, atol=1e-13)
            np.add.at(dKV_ref, idx[t], dk[0, 0])
            np.add.at(dKV_ref[:, :dv], idx[t], dvv[0, 0])
    np.testing.assert_allclose(dKV, dKV_ref, rtol=1e-12, atol=1e-13)


def test_sparse_sink_probability_and_empty_rows():
    rng = np.random.default_rng(31)
    Q, KV = rng.standard_normal((2, 2, 3)), rng.standard_normal((5, 3))
    idx = np.array([[1, 3], [-1, -1]], dtype=np.int32)
    length = np.array([2, 0], dtype=np.int32)
    sink = np.array([0.3, -1.0])
    O, LSE = sparse.forward(Q, KV, idx, length, sink, 0.5, 2)
    # token with no valid slot: O = 0 and LSE = z
    assert np.all(O[1] == 0)
    np.testing.assert_array_equal(LSE[1], sink)
    # token 0: LSE = ln(e^z + sum e^s)
    s = 0.5 * Q[0] @ KV[[1, 3]].T
    np.testing.assert_allclose(LSE[0], scipy.special.logsumexp(np.c_[s, sink], axis=1), rtol=1e-14)
    O2, LSE2 = sparse.forward(Q, KV, idx, length, None, 0.5, 2)
    assert np.all(O2[1] == 0) and np.all(LSE2[1] == -np.inf)


def test_sparse_kv_only_lse_closed_form():
    # icavan.github.io, DSA page, section 7.2: scores (0, ln 3) give LSE_kv = ln 4;
    # a sink logit z = ln 4 makes LSE_total = logaddexp(ln 4, ln 4) = ln 8
    Q = np.ones((1, 1, 1))
    KV = np.array([[0.0], [np.log(3.0)]])
    idx = np.array([[0, 1]], dtype=np.int32)
    kv = sparse.lse_kv(Q, KV, idx, None, 1.0)
    np.testing.assert_allclose(kv, [[np.log(4.0)]], rtol=1e-15)
    tot = sparse.lse_total_from_kv(kv, np.array([np.log(4.0)]))
    np.testing.assert_allclose(tot, [[np.log(8.0)]], rtol=1e-15)
    _, LSE = sparse.forward(Q, KV, idx, None, np.array([np.log(4.0)]), 1.0, 1)
    np.testing.assert_allclose(LSE, tot, rtol=1e-15)


def test_sparse_kv_only_lse_normalises_to_the_sink_inclusive_lse():
    # the two conventions computed on separate paths: the forward sums e^z into
    # Z directly, lse_kv leaves it out and logaddexp adds it back
    rng = np.random.default_rng(32)
    Q, KV = rng.standard_normal((5, 3, 4)), rng.standard_normal((9, 4))
    idx = rng.integers(0, 9, (5, 6)).astype(np.int32)
    length = np.array([6, 0, 3, 1, 6], dtype=np.int32)
    sink = rng.standard_normal(3)
    kv = sparse.lse_kv(Q, KV, idx, length, 0.7)
    assert np.all(kv[1] == -np.inf)
    _, LSE = sparse.forward(Q, KV, idx, length, sink, 0.7, 2)
    np.testing.assert_allclose(sparse.lse_total_from_kv(kv, sink), LSE, rtol=1e-13)
    _, LSE0 = sparse.forward(Q, KV, idx, length, None, 0.7, 2)  # no sink: the two agree
    np.testing.assert_array_equal(sparse.lse_total_from_kv(kv, None), kv)
    np.testing.assert_allclose(kv[[0, 2, 3, 4]], LSE0[[0, 2, 3, 4]], rtol=1e-13)
    assert np.all(LSE0[1] == -np.inf)


# ------------------------------------------------------------- input rounding


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    import workloads
    x = np.random.default_rng(40).standard_normal(100000) * np.float64(3.0) ** np.random.default_rng(41).integers(-20, 20, 100000)
    bits = workloads.f64_to_bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    np.testing.assert_array_equal(workloads.bf16_bits_to_f64(bits),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# ------------------------------------------------------------ allowed sets
# The parts of A_i other than causal are pinned here against hand-enumerated
# sets and closed-form counts, so that a slip in a comparison (< vs <=), a
# swapped block_q / block_k or a per-batch index mistake fails.


def test_window_and_tile_mask_sets_hand_enumerated():
    # n = 6, causal, look-back window 3 (i - j < 3), tile mask on 2-row x 3-key
    # tiles [[1, 0], [0, 1], [1, 1]]: rows {0,1} keep keys {0,1,2}, rows {2,3}
    # keep keys {3,4,5}, rows {4,5} keep every key
    bm = np.array([[1, 0], [0, 1], [1, 1]], np.uint8)
    A = dense.Allowed(6, 6, causal=True, window=3, block_mask=bm, block_q=2, block_k=3)
    want = [[0], [0, 1], [], [3], [2, 3, 4], [3, 4, 5]]
    got = A.rows(np.arange(6))
    for i in range(6):
        assert np.flatnonzero(got[i]).tolist() == want[i], i
    # the window alone (no causal): keys j with i - j < 3, including every later key
    Aw = dense.Allowed(4, 4, window=3)
    assert [np.flatnonzero(r).tolist() for r in Aw.rows(np.arange(4))] == [[0, 1, 2, 3], [0, 1, 2, 3],
                                                                          [0, 1, 2, 3], [1, 2, 3]]


@pytest.mark.parametrize("n,W", [(1, 1), (7, 3), (64, 64), (200, 37), (333, 256), (4096, 256)])
def test_causal_window_pair_count_closed_form(n, W):
    # sum_i min(i + 1, W) = W (W + 1) / 2 + (n - W) W for n >= W, else n (n + 1) / 2
    want = W * (W + 1) // 2 + (n - W) * W if n >= W else n * (n + 1) // 2
    assert dense.Allowed(n, n, causal=True, window=W).pair_count() == want


def test_causal_tile_mask_pair_count_closed_form():
    # with T x T tiles a kept diagonal tile holds T (T + 1) / 2 causal pairs and
    # a kept tile below the diagonal T^2; tiles above the diagonal hold none
    rng = np.random.default_rng(30)
    T, nt = 5, 7
    bm = (rng.random((nt, nt)) < 0.5).astype(np.uint8)
    want = sum(int(bm[r, c]) * (T * T if r > c else (T * (T + 1) // 2 if r == c else 0))
               for r in range(nt) for c in range(nt))
    assert dense.Allowed(T * nt, T * nt, causal=True, block_mask=bm, block_q=T, block_k=T).pair_count() == want
    # rectangular tiles: only the row index is divided by block_q
    bq, bk = 2, 4
    bm2 = np.zeros((4, 2), np.uint8)
    bm2[1, 0] = 1   # rows 2, 3 x keys 0..3
    bm2[3, 1] = 1   # rows 6, 7 x keys 4..7
    A2 = dense.Allowed(8, 8, block_mask=bm2, block_q=bq, block_k=bk)
    assert A2.pair_count() == 16
    assert np.flatnonzero(A2.rows([6])[0]).tolist() == [4, 5, 6, 7]
    assert not A2.rows([4])[0].any()


def test_bench_pair_count_agrees_with_closed_forms():
    import bench
    import workloads
    for name, w in workloads.WORKLOADS.items():
        if not isinstance(w, workloads.DenseWorkload) or w.n > 4096:
            continue
        bm = workloads.dense_arrays(w)["block_mask"]
        A = dense.Allowed(w.n, w.n, causal=w.causal, window=w.window, block_mask=bm,
                          block_q=w.mask_tile, block_k=w.mask_tile)
        assert bench.dense_pairs(w, bm) == A.pair_count(), name
    w = workloads.WORKLOADS["dense_causal_bf16_b4h16_n2048_d128"]
    assert bench.dense_pairs(w, None) == 2048 * 2049 // 2


def test_lengths_and_starts_sets_hand_enumerated():
    # batch 0: active length 4 of n = 5, no starts effect; batch 1: two packed
    # segments [0, 2) and [2, 5) (starts = segment starts), causal
    starts = np.array([[0, 0, 0, 0, 0], [0, 0, 2, 2, 2]])
    A = dense.Allowed(5, 5, causal=True, lengths=[4, 5], starts=starts)
    got0 = [np.flatnonzero(r).tolist() for r in A.rows(np.arange(5), b=0)]
    got1 = [np.flatnonzero(r).tolist() for r in A.rows(np.arange(5), b=1)]
    assert got0 == [[0], [0, 1], [0, 1, 2], [0, 1, 2, 3], []]
    assert got1 == [[0], [0, 1], [2], [2, 3], [2, 3, 4]]
    # a lower bound above the row itself empties a causal row; without causal
    # the keys past the active length stay excluded
    A2 = dense.Allowed(4, 4, lengths=[3], starts=[[1, 3, 0, 0]])
    assert [np.flatnonzero(r).tolist() for r in A2.rows(np.arange(4))] == [[1, 2], [], [0, 1, 2], []]
    assert A.pair_count(0) == 10 and A.pair_count(1) == 1 + 2 + 1 + 2 + 3


def test_inactive_rows_reduce_to_the_unpadded_sequence():
    # lengths[b] = L: the first L rows equal attention over the L-token
    # sequence alone; inactive rows are zero with LSE -inf and add nothing to
    # any gradient (the course's inactive padded rows)
    rng = np.random.default_rng(31)
    n, d, dv, L = 9, 3, 2, 6
    Q, K, V, G = _rand((2, 1, n, d), rng), _rand((2, 1, n, d), rng), _rand((2, 1, n, dv), rng), _rand((2, 1, n, dv), rng)
    A = dense.Allowed(n, n, causal=True, lengths=[L, n])
    Y, LSE = dense.forward(Q, K, V, A, 0.7)
    dQ, dK, dV = dense.vjp(Q, K, V, A, 0.7, G)
    sl = slice(0, L)
    Ys, LSEs = dense.forward(Q[:1, :, sl], K[:1, :, sl], V[:1, :, sl], dense.Allowed(L, L, causal=True), 0.7)
    dQs, dKs, dVs = dense.vjp(Q[:1, :, sl], K[:1, :, sl], V[:1, :, sl], dense.Allowed(L, L, causal=True), 0.7,
                              G[:1, :, sl])
    np.testing.assert_allclose(Y[0, 0, sl], Ys[0, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(LSE[0, 0, sl], LSEs[0, 0], rtol=1e-13)
    assert np.all(Y[0, 0, L:] == 0) and np.all(np.isneginf(LSE[0, 0, L:]))
    for full, short in ((dQ, dQs), (dK, dKs), (dV, dVs)):
        np.testing.assert_allclose(full[0, 0, sl], short[0, 0], rtol=1e-12, atol=1e-13)
        assert np.all(full[0, 0, L:] == 0)
    # batch 1 is untouched by batch 0's length
    Yf, _ = dense.forward(Q[1:], K[1:], V[1:], dense.Allowed(n, n, causal=True), 0.7)
    np.testing.assert_allclose(Y[1], Yf[0], rtol=1e-13, atol=1e-14)


def test_packed_segments_reduce_to_separate_sequences():
    # causal attention over packed segments (starts = first row of each row's
    # segment) equals causal attention over each segment on its own
    rng = np.random.default_rng(32)
    segs = [4, 1, 6, 3]
    n, d, dv = sum(segs), 4, 3
    Q, K, V, G = _rand((1, 2, n, d), rng), _rand((1, 1, n, d), rng), _rand((1, 1, n, dv), rng), _rand((1, 2, n, dv), rng)
    starts = np.concatenate([np.full(s, o) for s, o in zip(segs, np.cumsum([0] + segs[:-1]))])[None]
    A = dense.Allowed(n, n, causal=True, starts=starts)
    Y, LSE = dense.forward(Q, K, V, A, 0.6)
    dQ, dK, dV = dense.vjp(Q, K, V, A, 0.6, G)
    o = 0
    for s in segs:
        sl = slice(o, o + s)
        As = dense.Allowed(s, s, causal=True)
        Ys, LSEs = dense.forward(Q[:, :, sl], K[:, :, sl], V[:, :, sl], As, 0.6)
        dQs, dKs, dVs = dense.vjp(Q[:, :, sl], K[:, :, sl], V[:, :, sl], As, 0.6, G[:, :, sl])
        np.testing.assert_allclose(Y[:, :, sl], Ys, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(LSE[:, :, sl], LSEs, rtol=1e-13)
        for full, short in ((dQ, dQs), (dK, dKs), (dV, dVs)):
            np.testing.assert_allclose(full[:, :, sl], short, rtol=1e-12, atol=1e-13)
        o += s


def test_layout_vjp_matches_finite_differences():
    rng = np.random.default_rng(33)
    n, d, dv = 6, 3, 2
    Q, K, V, G = _rand((2, 1, n, d), rng), _rand((2, 1, n, d), rng), _rand((2, 1, n, dv), rng), _rand((2, 1, n, dv), rng)
    starts = np.array([[0, 0, 1, 1, 3, 3], [0, 1, 1, 2, 2, 5]])
    A = dense.Allowed(n, n, causal=True, lengths=[5, 6], starts=starts)
    dQ, dK, dV = dense.vjp(Q, K, V, A, 0.8, G)
    num = fd.gradient(_phi_dense(A, 0.8, None), [Q, K, V, G])
    for a, b in zip((dQ, dK, dV), num[:3]):
        np.testing.assert_allclose(a, b, rtol=0, atol=4e-6)
