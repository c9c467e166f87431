"""The structured inputs of the full-size parity tests (gen.structured) and
the closed form the counting test expects, checked on the CPU against the
oracle at small sizes: so that the expected values of the GPU tests are
themselves right."""
import numpy as np
import pytest

from helpers import counting_expected

import oracle
from gen import random_case
from gen.structured import TILE, counting_inputs, needle_inputs


def _small(seed, paged, chain):
    return random_case(seed, B=3, Hq=8, Hkv=2, d=64, P_range=(0, 400), n_max=20, dtype="bf16",
                       paged=paged, chain=chain)


@pytest.mark.parametrize("seed,paged,chain", [(1, False, False), (2, True, False),
                                              (3, False, True), (4, True, True)])
def test_counting_closed_form_equals_oracle(seed, paged, chain):
    c = counting_inputs(_small(seed, paged, chain))
    O, L = oracle.verify(c)
    Ox, Lx = counting_expected(c, c.n_max, lambda n: list(range(c.n_max)))
    rows = ~np.isnan(Ox[..., 0, 0])
    assert np.array_equal(rows, ~np.isnan(O[..., 0, 0]))
    np.testing.assert_allclose(O[rows], Ox[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(L[~np.isnan(Lx)], Lx[~np.isnan(Lx)], rtol=1e-13)
    # expand rows: the w newest nodes
    w = 3
    Oe, Le = oracle.expand(c, c.q[:, :w], w)
    Oxe, Lxe = counting_expected(c, w, lambda n: [n - w + r for r in range(w)])
    r = ~np.isnan(Oxe[..., 0, 0])
    np.testing.assert_allclose(Oe[r], Oxe[r], rtol=1e-12, atol=1e-15)


def test_counting_codes_see_a_dropped_tile():
    """Mutation check on the oracle side: hiding one prefix tile from the
    mask changes its code channel by a whole tile's count and the LSE by
    ln(l / (l - 32)), far outside the bars the GPU test uses."""
    c = counting_inputs(_small(5, False, True))
    b = int(np.argmax(c.prefix_len))
    assert c.prefix_len[b] >= 2 * TILE
    O, L = oracle.verify(c, batches=[b])
    c2 = counting_inputs(_small(5, False, True))
    c2.v = c2.v.copy()
    c2.v[b, TILE: 2 * TILE] = c2.v[b, 0: TILE]   # tile 1 now carries tile 0's codes
    O2, _ = oracle.verify(c2, batches=[b])
    diff = np.abs(O2[b, :, :, :2] - O[b, :, :, :2])
    assert np.nanmin(diff) > 0.01 * np.nanmax(np.abs(O[b, :, :, :2]))


@pytest.mark.parametrize("paged", [False, True])
def test_needle_inputs_are_exact_and_spread(paged):
    c = needle_inputs(_small(6, paged, False), seed=9)
    O, L = oracle.verify(c)
    ok = ~np.isnan(O[..., 0, 0])
    # every row's identity channel reads back its (sequence, KV head) code exactly
    from gen.structured import id_code
    for b in range(c.B):
        for h in range(c.Hq):
            r = ok[b]
            np.testing.assert_allclose(O[b, r, h, -1], id_code(b, h // c.G, c.Hkv), rtol=1e-12)
    # each needle carries a share of the mass no smaller than 1/(4 x needles seen)
    for b in range(c.B):
        P = int(c.prefix_len[b])
        if P == 0:
            continue
        ntile = (P + TILE - 1) // TILE
        lse = L[b][:, ok[b]]
        # every needle scores at least (12/16)(38/64) d scale, the other positions 0
        s_min = 0.75 * (38 / 64) * c.d * c.scale
        assert np.all(lse >= np.log(ntile * np.exp(s_min)) - 1e-12)


def test_counting_closed_form_on_a_batch_slice():
    """The second batch of an alternating pair is a slice of the resident
    requests: its expected identity codes are the slice's, not its indices'."""
    import copy
    c = counting_inputs(random_case(8, B=6, Hq=8, Hkv=2, d=64, P_range=(10, 300), n_max=8,
                                    paged=True))
    sl = slice(3, 6)
    s = copy.copy(c)
    s.q, s.prefix_len, s.parent, s.n_nodes = c.q[sl], c.prefix_len[sl], c.parent[sl], c.n_nodes[sl]
    s.block_table, s.B = c.block_table[sl], 3
    s.planted = dict(c.planted, id_codes=c.planted["id_codes"][sl])
    O, L = oracle.verify(s)
    Ox, Lx = counting_expected(s, s.n_max, lambda n: list(range(s.n_max)))
    r = ~np.isnan(Ox[..., 0, 0])
    np.testing.assert_allclose(O[r], Ox[r], rtol=1e-12, atol=1e-15)
