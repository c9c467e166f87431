"""Pins for the RoPE / append oracle (oracle/rope.py), from the defining
properties of a rotary embedding rather than its formula:

* position 0 is the identity, and each channel pair keeps its length;
* scores depend only on the offset: <R(m)q, R(n)k> = <R(m+t)q, R(n+t)k>;
* rotations compose: R(a) R(b) = R(a + b);
* with pair j read as the complex number x_j + i x_{j+d/2}, a rotation is
  the product with exp(i p theta_j), theta_j = base**(-2j/d) (numpy complex
  arithmetic, a second statement of the same map);
* tree positions: a child of the root sits at P, a node at depth k at
  P - 1 + k, so siblings share a position and a chain is consecutive.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("d", [2, 64, 128])
def test_identity_and_pair_lengths(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d))
    np.testing.assert_allclose(oracle.rope(x, 0), x, rtol=0, atol=0)
    for p in (1, 17, 4096, 32783):
        y = oracle.rope(x, p)
        h = d // 2
        np.testing.assert_allclose(y[:, :h] ** 2 + y[:, h:] ** 2, x[:, :h] ** 2 + x[:, h:] ** 2,
                                   rtol=1e-12)


def test_scores_depend_on_offset_only():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n, t in ((5, 2, 100), (4096, 10, 7), (0, 33, 3000)):
        a = oracle.rope(q, m) @ oracle.rope(k, n)
        b = oracle.rope(q, m + t) @ oracle.rope(k, n + t)
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def test_composition_and_complex_form():
    rng = np.random.default_rng(2)
    d, base = 64, 10000.0
    x = rng.standard_normal(d)
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, 37), 1000), oracle.rope(x, 1037),
                               rtol=1e-9, atol=1e-12)
    h = d // 2
    z = x[:h] + 1j * x[h:]
    for p in (3, 2048):
        w = z * np.exp(1j * p * base ** (-2.0 * np.arange(h) / d))
        np.testing.assert_allclose(oracle.rope(x, p), np.concatenate([w.real, w.imag]),
                                   rtol=1e-9, atol=1e-12)


def test_tree_positions():
    par = np.array([-1, -1, 0, 2, 1, -1], dtype=np.int32)
    assert oracle.tree_positions(par, 6, 100).tolist() == [100, 100, 101, 102, 101, 100]
    chain = np.arange(-1, 7, dtype=np.int32)
    assert oracle.tree_positions(chain, 8, 10).tolist() == list(range(10, 18))


def test_append_rows_and_slots():
    rng = np.random.default_rng(3)
    B, n_max, Hq, Hkv, d = 2, 5, 4, 2, 8
    q = rng.standard_normal((B, n_max, Hq, d))
    k = rng.standard_normal((B, n_max, Hkv, d))
    v = rng.standard_normal((B, n_max, Hkv, d))
    par = np.array([[-1, 0, 1, 0, -1], [-1, 0, 0, 0, 0]], dtype=np.int32)
    P, n = np.array([7, 3]), np.array([5, 2])
    qo, rows = oracle.rope_append(q, k, v, P, par, n, n_max, False)
    assert sorted(rows[0]) == [7, 8, 9, 10, 11] and sorted(rows[1]) == [3, 4]
    assert np.isnan(qo[1, 2:]).all()
    np.testing.assert_allclose(qo[0, 2], oracle.rope(q[0, 2], 9))   # depth 3: 7 - 1 + 3
    np.testing.assert_array_equal(rows[0][9][1], v[0, 2])
    # expand: slot s is node n - n_q + s
    qe, rows_e = oracle.rope_append(q[:, :2], k[:, :2], v[:, :2], P, par, n, 2, True)
    np.testing.assert_allclose(qe[0, 0], oracle.rope(q[0, 0], 8))  # node 3, depth 2
    np.testing.assert_allclose(qe[0, 1], oracle.rope(q[0, 1], 7))  # node 4, depth 1
    assert sorted(rows_e[0]) == [10, 11] and sorted(rows_e[1]) == [3, 4]
