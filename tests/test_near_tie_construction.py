"""The near-tie router inputs (tests/ties.py) do what the routing tests
need, checked on the CPU: the pair's logits are equal in exact arithmetic,
differ between fp32 summation orders, and sit at the intended ranks, where
the oracle sees a near tie (gap far below the tolerated 1e-5)."""
import numpy as np
import pytest

import oracle
from ties import association_dependent, exact_dot, near_tie_case, seq_dot32

SHAPES = [(256, 16, 2), (256, 16, 4), (4096, 64, 4)]


@pytest.mark.parametrize("D,E,K", SHAPES)
@pytest.mark.parametrize("where", ["boundary", "inside"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_near_tie_case(D, E, K, where, seed):
    Wr, x, e1, e2 = near_tie_case(D, E, K, seed, where)
    assert Wr.dtype == np.float32 and x.dtype == np.float32
    # equal in exact arithmetic (the same multiset of exact products)
    p1 = sorted((Wr[e1].astype(np.float64) * x.astype(np.float64)).tolist())
    p2 = sorted((Wr[e2].astype(np.float64) * x.astype(np.float64)).tolist())
    assert p1 == p2
    assert exact_dot(Wr[e1], x) == exact_dot(Wr[e2], x)
    # but not under one fp32 association
    assert association_dependent(Wr[e1], Wr[e2], x)
    assert seq_dot32(Wr[e1], x) != seq_dot32(Wr[e2], x)
    # the oracle (fp64, summed in index order): a near tie far below the
    # tolerated gap, the pair where intended
    lo = oracle.router(Wr, x.astype(np.float64))
    assert abs(lo[e1] - lo[e2]) <= 1e-12 * abs(lo[e1])
    order = sorted(range(E), key=lambda e: (-lo[e], e))
    ranks = sorted((order.index(e1), order.index(e2)))
    assert ranks == ([K - 1, K] if where == "boundary" else [0, 1])
    sel, gap = oracle.topk(lo, K)
    if where == "boundary":
        assert gap < 1e-5 and len({e1, e2} & set(int(e) for e in sel)) == 1
    else:
        assert set(int(e) for e in sel[:2]) == {e1, e2}
        # every other gap is wide: only the pair's order is decided by rounding
        assert gap > 1e-3 * lo[e1]
