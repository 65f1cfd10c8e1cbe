"""The GPU tests' acceptance rules, checked on the CPU: check_selection and
check_forward must accept the oracle's own results and reject planted
mistakes of the kinds a wrong kernel would make."""
import numpy as np
import pytest

import oracle
from helpers import NEAR_TIE_REL, check_forward, check_selection, csr_rows

# two disjoint groups clear of the text columns, as in the long-context workload
NB, TB = 40, 2
GROUPS = ((2, 30, 6), (30, 40, 3))


def _scores(seed=0, n=6):
    S = np.random.default_rng(seed).standard_normal((n, NB))
    return S


def _oracle_rows(S, qb):
    rp, ci = oracle.select_rows(S, qb, TB, GROUPS)
    return csr_rows(rp, ci)


def test_accepts_the_oracle_selection():
    S = _scores()
    qb = [0, 1, 5, 17, 38, 39]          # two text rows, four others
    rows = _oracle_rows(S, qb)
    assert check_selection(rows, rows, S, qb, TB, GROUPS, nB=NB) == 0


def _one_row_case():
    S = _scores(1, 1)
    qb = [7]
    rows = _oracle_rows(S, qb)
    return S, qb, rows


def _near_tie_shift(S, rows, src, dst):
    """Make the best dropped column of group dst a near-tie of that group's k-th
    score and the worst kept column of group src a near-tie of its own, and
    return a row that keeps one more of dst and one fewer of src."""
    S = S.copy()
    row = set(rows[0])
    (c0, c1, k0), (d0, d1, k1) = GROUPS[src], GROUPS[dst]
    s = S[0]
    tol = NEAR_TIE_REL * np.abs(s).max()
    kept_src = sorted((c for c in row if c0 <= c < c1), key=lambda c: s[c])
    drop = kept_src[0]                   # the src group's k-th (lowest kept)
    out_dst = sorted((c for c in range(d0, d1) if c not in row), key=lambda c: -s[c])
    add = out_dst[0]
    kth_dst = min(s[c] for c in row if d0 <= c < d1)
    S[0, add] = kth_dst - 0.1 * tol      # within the band of the dst group's k-th score
    bad = sorted((row - {drop}) | {add})
    return S, bad


def test_rejects_a_count_shift_between_groups_even_at_near_ties():
    S, qb, rows = _one_row_case()
    S2, bad = _near_tie_shift(S, rows, 0, 1)
    good = _oracle_rows(S2, qb)
    with pytest.raises(AssertionError, match="columns of group"):
        check_selection([bad], good, S2, qb, TB, GROUPS, nB=NB)


def test_accepts_a_near_tie_swap_inside_a_group():
    S, qb, rows = _one_row_case()
    s = S[0].copy()
    c0, c1, k = GROUPS[0]
    kept = sorted((c for c in rows[0] if c0 <= c < c1), key=lambda c: s[c])
    dropped = sorted((c for c in range(c0, c1) if c not in rows[0]), key=lambda c: -s[c])
    tol = NEAR_TIE_REL * np.abs(s).max()
    s[dropped[0]] = s[kept[0]] - 0.1 * tol   # the best dropped column now ties the k-th
    S2 = s[None, :]
    good = _oracle_rows(S2, qb)
    swapped = sorted((set(good[0]) - {kept[0]}) | {dropped[0]})
    if swapped == good[0]:
        swapped = sorted((set(good[0]) - {dropped[0]}) | {kept[0]})
    assert check_selection([swapped], good, S2, qb, TB, GROUPS, nB=NB) == 1


def test_rejects_a_swap_that_is_not_a_near_tie():
    S, qb, rows = _one_row_case()
    c0, c1, _ = GROUPS[0]
    kept = [c for c in rows[0] if c0 <= c < c1]
    far = [c for c in range(c0, c1) if c not in rows[0]]
    s = S[0]
    worst = min(far, key=lambda c: s[c])
    bad = sorted((set(rows[0]) - {kept[0]}) | {worst})
    with pytest.raises(AssertionError, match="not a near-tie"):
        check_selection([bad], rows, S, qb, TB, GROUPS, nB=NB)


@pytest.mark.parametrize("mutate,msg", [
    (lambda r: r[::-1], "ascending"),
    (lambda r: sorted(r + [r[-1]]), "ascending"),
    (lambda r: r[1:], "text column"),
    (lambda r: r[:-1] + [NB], "outside"),
])
def test_rejects_malformed_rows(mutate, msg):
    S, qb, rows = _one_row_case()
    with pytest.raises(AssertionError, match=msg):
        check_selection([mutate(list(rows[0]))], rows, S, qb, TB, GROUPS, nB=NB)


def test_rejects_a_text_row_that_is_not_dense():
    S = _scores(2, 1)
    qb = [1]
    rows = _oracle_rows(S, qb)
    assert rows[0] == list(range(NB))
    with pytest.raises(AssertionError, match="text row"):
        check_selection([rows[0][:-1]], rows, S, qb, TB, GROUPS, nB=NB)


def test_forward_tolerance_scales_with_v():
    rng = np.random.default_rng(3)
    O = rng.standard_normal((64, 16))
    L = rng.standard_normal(64)
    err = np.zeros_like(O)
    err[0, 0] = 5e-2                      # beyond 2e-2 for unit V, within 3 x 2e-2
    check_forward(O + err, L, O, L, "scaled", v_scale=3.0)
    with pytest.raises(AssertionError, match="max"):
        check_forward(O + err, L, O, L, "unit")
    with pytest.raises(AssertionError, match="LSE"):
        check_forward(O, L + 2e-3, O, L, "lse", v_scale=3.0)
