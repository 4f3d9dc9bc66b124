"""Pins of the float64 oracle to what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: values printed on the
handbook page "7. Gated DeltaNet: the token-by-token recurrence" (fixtures under
tests/golden/, each with its citation), closed forms, invariants stated on that
page and on the learn-llm page 13_linear_attention_viz, and brute force.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gdn_testutil import read_golden_kv, read_golden_rows


def _one_head(tokens, S0=None, *, scale=1.0, delta=True, normalize=True):
    """Run the oracle on a single (sequence, head) given a list of (q, k, v, g, beta)."""
    q = np.array([t[0] for t in tokens], dtype=np.float64)[:, None, :]
    k = np.array([t[1] for t in tokens], dtype=np.float64)[:, None, :]
    v = np.array([t[2] for t in tokens], dtype=np.float64)[:, None, :]
    g = np.array([[t[3]] for t in tokens], dtype=np.float64)
    b = np.array([[t[4]] for t in tokens], dtype=np.float64)
    s0 = None if S0 is None else np.asarray(S0, dtype=np.float64)[None, None]
    o, S = oracle.run(q, k, v, g, b, [0, len(tokens)], s0, scale=scale, delta=delta,
                      normalize=normalize)
    return o[:, 0, :], S[0, 0]


K1, K2 = [1.0, 0.0], [0.0, 1.0]


def _read(q):
    # a pure read: beta = 0 writes nothing and g = 0 keeps the table
    return (q, K1, [0.0, 0.0], 0.0, 0.0)


def test_two_dim_table_write_then_read():
    """Handbook, "The memory table": write k1->(3,1), k2->(-1,2), read three queries."""
    gold = read_golden_kv("two_dim_table.txt")
    toks = [(K1, K1, [3.0, 1.0], 0.0, 1.0), (K2, K2, [-1.0, 2.0], 0.0, 1.0),
            _read([1.0, 0.0]), _read([0.0, 1.0]), _read([0.6, 0.8])]
    o, S = _one_head(toks)
    np.testing.assert_allclose(S[0], gold["table_row_k1"], atol=1e-14)
    np.testing.assert_allclose(S[1], gold["table_row_k2"], atol=1e-14)
    np.testing.assert_allclose(o[2], gold["read_q_1_0"], atol=1e-14)
    np.testing.assert_allclose(o[3], gold["read_q_0_1"], atol=1e-14)
    np.testing.assert_allclose(o[4], gold["read_q_0.6_0.8"], atol=1e-14)


@pytest.mark.parametrize("variant", ["linear", "deltanet", "gated"])
def test_rewrite_key(variant):
    """Handbook, "Step by step" figure and list: rewrite k1 -> (5, 0) three ways."""
    gold = read_golden_kv("two_dim_table.txt")
    table = np.array([gold["table_row_k1"], gold["table_row_k2"]])
    g = math.log(gold["gated_alpha"][0]) if variant == "gated" else 0.0
    toks = [(K1, K1, [5.0, 0.0], g, 1.0), _read(K1), _read(K2)]
    o, _ = _one_head(toks, S0=table, delta=(variant != "linear"))
    np.testing.assert_allclose(o[1], gold[f"{variant}_read_k1"], atol=1e-14)
    np.testing.assert_allclose(o[2], gold[f"{variant}_read_k2"], atol=1e-14)


@pytest.mark.parametrize("row", read_golden_rows("decay_residue.txt"))
def test_decay_residue(row):
    """Handbook toy script part 3: a row never written again keeps alpha^n of itself.

    k1 is rewritten every step (beta = 1) while k2's row only decays.
    """
    alpha = float(row[0])
    for n, printed, fmt in ((10, row[1], "{:.3f}"), (50, row[2], "{:.3g}")):
        table = np.array([[3.0, 1.0], [-1.0, 2.0]])
        toks = [(K1, K1, [5.0, 0.0], math.log(alpha), 1.0)] * n
        _, S = _one_head(toks, S0=table)
        residue = S[1] / table[1]
        np.testing.assert_allclose(residue, alpha ** n, rtol=1e-12)
        assert fmt.format(residue[0]) == printed
        np.testing.assert_allclose(S[0], [5.0, 0.0], atol=1e-12)


def _fill(K, V, delta):
    """Write every (k, v) with beta = 1, alpha = 1 into an empty 128x128 table; read each k back."""
    n, d = K.shape
    o, S = oracle.run(K[:, None, :], K[:, None, :], V[:, None, :], np.zeros((n, 1)),
                      np.ones((n, 1)), [0, n], None, delta=delta)
    Khat = K / np.linalg.norm(K, axis=1, keepdims=True)
    read = Khat @ S[0, 0]
    return np.linalg.norm(read - V, axis=1) / np.linalg.norm(V, axis=1)


def _capacity_inputs():
    torch.manual_seed(0)
    Q, _ = torch.linalg.qr(torch.randn(128, 128))
    V0 = torch.randn(128, 128)
    sets = [(Q.double().numpy(), V0.double().numpy())]
    for n in (256, 1024):
        K = torch.nn.functional.normalize(torch.randn(n, 128), dim=-1)
        V = torch.randn(n, 128)
        sets.append((K.double().numpy(), V.double().numpy()))
    return sets


def test_capacity_orthogonal_and_random_keys():
    """Handbook toy script part 4: 128 orthonormal keys read back exactly; random keys blur.

    The inputs are redrawn with the same seeded generator and draw order as the
    page's experiment, so the printed percentages are matched exactly.
    """
    rows = read_golden_rows("capacity.txt")
    sets = _capacity_inputs()
    for (K, V), row in zip(sets, rows):
        plain = _fill(K, V, delta=False)
        dlt = _fill(K, V, delta=True)
        if row[0] == "128":
            # the page's keys are float32-orthonormal: 0% at the printed precision ...
            assert round(100 * plain.mean()) == 0 and round(100 * dlt.mean()) == 0
            # ... and exactly orthonormal keys (float64 QR) read back exactly
            Q64, _ = np.linalg.qr(K)
            assert _fill(Q64, V, delta=False).max() < 1e-12
            assert _fill(Q64, V, delta=True).max() < 1e-12
            continue
        got = [plain.mean(), dlt.mean(), dlt[-16:].mean(), dlt[:16].mean()]
        want = [float(x) for x in row[1:]]
        assert [round(100 * x) for x in got] == want, (got, want)
        # closed form for the plain table: crosstalk ~ sqrt((n-1)/d)
        assert abs(plain.mean() - math.sqrt((len(K) - 1) / 128)) < 0.05


def test_repeated_write_halves_the_error():
    """Handbook "Run it": one unit (k, v) written 6 times, beta = 0.5, g = 0, q = k.

    Reproduces the printed distances (delta rule halves each time; plain linear
    attention overshoots as |t/2 - 1| |v|) with the page's seeded draws and the
    page's 1/sqrt(dk) query scale.
    """
    rows = read_golden_rows("repeated_write.txt")
    torch.manual_seed(0)
    k = torch.nn.functional.normalize(torch.randn(128), dim=-1).double().numpy()
    v = torch.randn(128).double().numpy()
    toks = [(k, k, v, 0.0, 0.5)] * 6
    o_d, _ = _one_head(toks, scale=128 ** -0.5)
    o_p, _ = _one_head(toks, scale=128 ** -0.5, delta=False)
    vn = np.linalg.norm(v)
    for t, row in enumerate(rows):
        dd = np.linalg.norm(o_d[t] * math.sqrt(128) - v)
        dp = np.linalg.norm(o_p[t] * math.sqrt(128) - v)
        assert f"{dd:.3f}" == row[1] and f"{dp:.3f}" == row[2]
        np.testing.assert_allclose(dd, vn * 0.5 ** (t + 1), rtol=1e-12)
        np.testing.assert_allclose(dp, vn * abs((t + 1) / 2 - 1), rtol=1e-12, atol=1e-12)


def test_projection_at_beta_one():
    """Handbook "Common questions" (beta = 1, unit k reads back exactly v) and the
    learn-llm note that I - k k^T is a projection: holds for any alpha and table."""
    rng = np.random.default_rng(11)
    for _ in range(5):
        d = 16
        S0 = rng.standard_normal((d, d))
        k = rng.standard_normal(d)
        v = rng.standard_normal(d)
        g = -rng.uniform(0, 3)
        o, S = _one_head([(k, k, v, g, 1.0)], S0=S0)
        kh = k / np.linalg.norm(k)
        np.testing.assert_allclose(S.T @ kh, v, atol=1e-12)
        np.testing.assert_allclose(o[0], v, atol=1e-12)


def test_unnormalised_key_error_factor():
    """learn-llm note on |k|: S'k = Sk + beta (v - Sk)|k|^2, so with |k|^2 = 4 and
    beta = 1 each rewrite multiplies the error by |1 - beta |k|^2| = 3."""
    rng = np.random.default_rng(12)
    d = 8
    u = rng.standard_normal(d)
    k = 2.0 * u / np.linalg.norm(u)
    v = rng.standard_normal(d)
    S = rng.standard_normal((d, d))
    err = np.linalg.norm(S.T @ k - v)
    for _ in range(4):
        _, S = _one_head([(k, k, v, 0.0, 1.0)], S0=S, normalize=False)
        new = np.linalg.norm(S.T @ k - v)
        np.testing.assert_allclose(new / err, 3.0, rtol=1e-10)
        err = new


def test_delta_step_is_one_sgd_step():
    """Handbook "Step by step" (DeltaNet) and learn-llm: with alpha = 1 the write is one
    gradient step of 1/2 |S^T k - v|^2 with learning rate beta.  The gradient here is
    taken by central differences, independent of the update formula."""
    rng = np.random.default_rng(13)
    d = 6
    S0 = rng.standard_normal((d, d))
    k = rng.standard_normal(d)
    kh = k / np.linalg.norm(k)
    v = rng.standard_normal(d)
    beta = 0.37
    _, S1 = _one_head([(k, k, v, 0.0, beta)], S0=S0)

    def loss(S):
        r = S.T @ kh - v
        return 0.5 * float(r @ r)

    grad = np.zeros_like(S0)
    h = 1e-3
    for i in range(d):
        for j in range(d):
            E = np.zeros_like(S0)
            E[i, j] = h
            grad[i, j] = (loss(S0 + E) - loss(S0 - E)) / (2 * h)
    np.testing.assert_allclose(S1, S0 - beta * grad, atol=1e-9)


def _rand_seq(rng, T, d, dv):
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, dv))
    g = -rng.uniform(0, 1, T)
    b = rng.uniform(0, 1, T)
    return q, k, v, g, b


def test_plain_linear_attention_is_the_causal_sum():
    """Handbook "The memory table": sum_j (q.k_j) v_j = (sum_j k_j v_j^T)^T q.
    Without the subtraction and with alpha = 1 the oracle must give the brute-force
    causal sum o_t = sum_{j<=t} (q_t . k_j) beta_j v_j."""
    rng = np.random.default_rng(14)
    T, d, dv = 23, 8, 5
    q, k, v, _, b = _rand_seq(rng, T, d, dv)
    toks = [(q[t], k[t], v[t], 0.0, b[t]) for t in range(T)]
    o, _ = _one_head(toks, delta=False)
    qh = q / np.linalg.norm(q, axis=1, keepdims=True)
    kh = k / np.linalg.norm(k, axis=1, keepdims=True)
    for t in range(T):
        want = sum((qh[t] @ kh[j]) * b[j] * v[j] for j in range(t + 1))
        np.testing.assert_allclose(o[t], want, atol=1e-12)


def test_mamba2_row_is_the_decayed_causal_sum():
    """learn-llm update-rule table, Mamba2 row S_t = a_t S_{t-1} + v_t k_t^T (here with
    beta): o_t = (prod_{s<=t} a_s) S0^T q_t + sum_{j<=t} (prod_{j<s<=t} a_s)(q_t.k_j) beta_j v_j."""
    rng = np.random.default_rng(15)
    T, d, dv = 19, 7, 4
    q, k, v, g, b = _rand_seq(rng, T, d, dv)
    S0 = rng.standard_normal((d, dv))
    toks = [(q[t], k[t], v[t], g[t], b[t]) for t in range(T)]
    o, _ = _one_head(toks, S0=S0, delta=False)
    qh = q / np.linalg.norm(q, axis=1, keepdims=True)
    kh = k / np.linalg.norm(k, axis=1, keepdims=True)
    a = np.exp(g)
    for t in range(T):
        want = np.prod(a[: t + 1]) * (S0.T @ qh[t])
        for j in range(t + 1):
            want = want + np.prod(a[j + 1: t + 1]) * (qh[t] @ kh[j]) * b[j] * v[j]
        np.testing.assert_allclose(o[t], want, atol=1e-12)


def test_alpha_to_zero_sees_only_the_current_token():
    """Handbook "Questions" 3: alpha -> 0 empties the table each step, so the read is
    only the current token's own write: o_t = beta_t (q_t . k_t) v_t."""
    rng = np.random.default_rng(16)
    T, d, dv = 9, 8, 8
    q, k, v, _, b = _rand_seq(rng, T, d, dv)
    S0 = rng.standard_normal((d, dv))
    toks = [(q[t], k[t], v[t], -1e4, b[t]) for t in range(T)]
    o, S = _one_head(toks, S0=S0)
    qh = q / np.linalg.norm(q, axis=1, keepdims=True)
    kh = k / np.linalg.norm(k, axis=1, keepdims=True)
    for t in range(T):
        np.testing.assert_allclose(o[t], b[t] * (qh[t] @ kh[t]) * v[t], atol=1e-13)
    np.testing.assert_allclose(S, np.outer(kh[-1], b[-1] * v[-1]), atol=1e-13)


def test_zero_key_writes_nothing():
    """Normalising a zero vector gives zero (the x / max(|x|, eps) form), so a zero key
    neither reads nor writes and only the decay acts."""
    rng = np.random.default_rng(17)
    d = 4
    S0 = rng.standard_normal((d, d))
    _, S = _one_head([(np.ones(d), np.zeros(d), np.ones(d), math.log(0.5), 1.0)], S0=S0)
    np.testing.assert_allclose(S, 0.5 * S0, atol=1e-15)


def test_scale_is_linear_in_the_read_only():
    """The query scale multiplies the read and never touches the table."""
    rng = np.random.default_rng(18)
    T, d = 12, 8
    q, k, v, g, b = _rand_seq(rng, T, d, d)
    toks = [(q[t], k[t], v[t], g[t], b[t]) for t in range(T)]
    o1, S1 = _one_head(toks)
    o2, S2 = _one_head(toks, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(o2, o1 / math.sqrt(d), atol=1e-14)
    np.testing.assert_allclose(S2, S1, atol=0)
