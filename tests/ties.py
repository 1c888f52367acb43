"""Router inputs whose logits tie in exact arithmetic but not in fp32.

Two experts e1 < e2 get logits that are equal as real numbers: the input x
has two equal halves and router row e2 is row e1 with its halves swapped, so
both dot products add up the same products, only in another order.  An fp32
sum of those products depends on the order it takes, so the two logits
differ by a few units in the last place, one way or the other depending on
how the sum is associated.  Which of the two experts a top-K takes is then
decided by rounding: the routing of any two code paths that sum the logits
differently can disagree here, which is what these inputs are for.
"""
import math

import numpy as np


def near_tie_case(D, E, K, seed, where="boundary", sigma=0.05):
    """Router weights Wr [E][D] (fp32) and input x [D] (fp32) with the tied
    pair (e1, e2) placed at ranks K-1 and K of the exact ordering
    (where="boundary": which one is selected is decided by rounding) or at
    ranks 0 and 1 (where="inside": both selected, their order decided by
    rounding).  The other ranked rows are the pair's row times powers of two
    (exact multiples); every remaining row is scaled down by powers of two
    until its logit is below half the pair's.  Returns (Wr, x, e1, e2)."""
    assert D % 2 == 0 and E >= K + 2
    if where == "boundary":
        assert K >= 1
    rng = np.random.default_rng(seed)
    for _ in range(64):
        h = rng.standard_normal(D // 2).astype(np.float32)
        x = np.concatenate([h, h])
        Wr = (rng.standard_normal((E, D)) * sigma).astype(np.float32)
        e1, e2 = sorted(int(e) for e in rng.choice(E, size=2, replace=False))
        row = Wr[e1].copy()
        if exact_dot(row, x) < 0:
            row = -row
        Wr[e1] = row
        Wr[e2] = np.concatenate([row[D // 2:], row[:D // 2]])
        lt = exact_dot(row, x)
        if lt <= 0:
            continue
        others = [e for e in range(E) if e not in (e1, e2)]
        # ranked rows above the pair (boundary: K-1 of them) or below it (inside: K-2)
        n_above = K - 1 if where == "boundary" else 0
        n_below = 0 if where == "boundary" else max(0, K - 2)
        picks = [int(e) for e in rng.choice(others, size=n_above + n_below, replace=False)]
        for j, e in enumerate(picks[:n_above]):
            Wr[e] = row * np.float32(2.0 ** (j + 1))          # logits 2, 4, 8, ... times the pair's
        for j, e in enumerate(picks[n_above:]):
            Wr[e] = row * np.float32(2.0 ** -(j + 1))         # logits 1/2, 1/4, ... times the pair's
        thr = 0.25 if where == "boundary" else 2.0 ** -(n_below + 2)
        for e in others:
            if e in picks:
                continue
            while exact_dot(Wr[e], x) >= thr * lt:
                Wr[e] = Wr[e] * np.float32(0.25)
        if not association_dependent(Wr[e1], Wr[e2], x):
            continue
        return Wr, x, e1, e2
    raise RuntimeError("no near tie found")


def exact_dot(w, x):
    """The dot product of two fp32 vectors, correctly rounded to fp64 (each
    product is exact in fp64, and fsum adds them exactly)."""
    return math.fsum((np.asarray(w, np.float64) * np.asarray(x, np.float64)).tolist())


def seq_dot32(w, x):
    """The dot product summed left to right in fp32."""
    acc = np.float32(0.0)
    for p in (np.asarray(w, np.float32) * np.asarray(x, np.float32)):
        acc = np.float32(acc + p)
    return acc


def association_dependent(w1, w2, x):
    """True when the two rows' fp32 dot products, each summed left to right,
    differ (though their exact values are equal)."""
    return seq_dot32(w1, x) != seq_dot32(w2, x)
