"""Shared helpers for the GPU parity tests: tensor marshalling and the
acceptance rules (tolerances, near-tie selection)."""
import math

import numpy as np
import torch

# Tolerances of the forward against the fp64 oracle (bf16 inputs and output,
# fp32 accumulation): max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <= 1e-3.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
# Selection: indices must match exactly except where the oracle's score of a
# differing column lies within this relative band (of the row's largest
# |score|) of the group's k-th score.
NEAR_TIE_REL = 1e-4


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_forward(O_gpu: np.ndarray, L_gpu: np.ndarray, O_or: np.ndarray, L_or: np.ndarray,
                  what: str = "", v_scale: float = 1.0):
    """Compare GPU O/LSE (already gathered to the oracle's rows) with the oracle.

    The O bounds are stated for unit-scale V; O is a convex combination of
    V rows and every rounding error in it (bf16 P, bf16 O) scales with V, so
    for V of standard deviation v_scale both bounds are scaled by it (a
    relative tolerance).  The LSE bound does not depend on V."""
    assert O_gpu.shape == O_or.shape, (O_gpu.shape, O_or.shape)
    d = np.abs(O_gpu - O_or)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    assert mx <= O_MAX_ABS * v_scale, f"{what}: max |dO| = {mx:.3e}"
    assert mean <= O_MEAN_ABS * v_scale, f"{what}: mean |dO| = {mean:.3e}"
    fin = np.isfinite(L_or)
    np.testing.assert_array_equal(np.isfinite(L_gpu), fin, err_msg=f"{what}: LSE finiteness")
    assert np.all(L_gpu[~fin] == L_or[~fin]), f"{what}: -inf LSE rows"
    if fin.any():
        dl = float(np.abs(L_gpu[fin] - L_or[fin]).max())
        assert dl <= LSE_MAX_ABS, f"{what}: max |dLSE| = {dl:.3e}"
    return mx, mean


def csr_rows(row_ptr: np.ndarray, col_idx: np.ndarray):
    return [col_idx[row_ptr[x]:row_ptr[x + 1]].tolist() for x in range(len(row_ptr) - 1)]


def check_csr_valid(row_ptr: np.ndarray, col_idx: np.ndarray, nB: int):
    assert row_ptr[0] == 0
    assert np.all(np.diff(row_ptr) >= 0)
    for x in range(len(row_ptr) - 1):
        c = col_idx[row_ptr[x]:row_ptr[x + 1]]
        assert np.all(np.diff(c) > 0), f"row {x} not strictly ascending"
        assert c.size == 0 or (c[0] >= 0 and c[-1] < nB)


def _groups_disjoint_clear(groups, text_blocks):
    """True when the groups with k > 0 are pairwise disjoint and leave the
    text columns alone: then every non-text row holds exactly k_g columns of
    each group [c_g, e_g) besides the text columns, and nothing else."""
    live = sorted((c0, c1) for (c0, c1, kk) in groups if kk > 0)
    for (a0, a1), (b0, _) in zip(live, live[1:]):
        if b0 < a1:
            return False
    return all(c0 >= text_blocks for (c0, _) in live)


def check_selection(gpu_rows, or_rows, S_or: np.ndarray, qblock, text_blocks, groups, nB=None):
    """Acceptance of a GPU selection against the oracle's, row by row.

    Every GPU row must be strictly ascending, unique and inside [0, nB); a
    text row must keep every column; another row must keep the text columns
    and, when the groups are disjoint and clear of the text columns, exactly
    k_g columns of each group and nothing outside the groups.  A row may
    differ from the oracle's only by near-ties: each differing column's oracle
    score lies within NEAR_TIE_REL * max|S_row| of its group's k-th largest
    oracle score.  Returns the number of rows that differ."""
    differ = 0
    exact_counts = _groups_disjoint_clear(groups, text_blocks)
    for x, (g, o) in enumerate(zip(gpu_rows, or_rows)):
        s = S_or[x]
        n_cols = len(s) if nB is None else nB
        ga = np.asarray(g, dtype=np.int64)
        assert np.all(np.diff(ga) > 0), f"row {x}: columns not strictly ascending: {g}"
        assert ga.size == 0 or (ga[0] >= 0 and ga[-1] < n_cols), f"row {x}: column outside [0, {n_cols})"
        i = int(qblock[x])
        tb = min(text_blocks, n_cols)
        if i < text_blocks:
            assert g == list(range(n_cols)), f"row {x}: text row not dense"
        else:
            assert set(range(tb)) <= set(g), f"row {x}: text column missing"
            if exact_counts:
                inside = set(range(tb))
                for (c0, c1, kk) in groups:
                    if kk <= 0:
                        continue
                    cnt = int(np.count_nonzero((ga >= c0) & (ga < c1)))
                    assert cnt == kk, f"row {x}: {cnt} columns of group [{c0}, {c1}) kept, {kk} asked"
                    inside.update(range(c0, c1))
                assert set(g) <= inside, f"row {x}: a kept column lies outside the text columns and groups"
        if g == o:
            continue
        differ += 1
        assert i >= text_blocks, f"row {x}: text row differs"
        tol = NEAR_TIE_REL * float(np.abs(s).max())
        gs, os_ = set(g), set(o)
        for col in gs ^ os_:
            ok = False
            for (c0, c1, kk) in groups:
                if c0 <= col < c1 and kk > 0:
                    kth = np.sort(s[c0:c1])[::-1][kk - 1]
                    ok = ok or abs(s[col] - kth) <= tol
            assert ok, (f"row {x}: column {col} differs (score {s[col]:.6e}) and is not a near-tie; "
                        f"gpu={sorted(gs)} oracle={sorted(os_)}")
        assert len(gs) == len(os_), f"row {x}: {len(gs)} vs {len(os_)} kept blocks"
    return differ


def sample_rows(B, H, N, n, seed, must=()):
    """Flat token rows (b*H + h)*N + t: a seeded random sample plus `must`."""
    r = np.random.default_rng(seed)
    rows = set(int(x) for x in r.choice(B * H * N, size=min(n, B * H * N), replace=False))
    rows.update(int(x) for x in must)
    return np.array(sorted(rows), dtype=np.int64)
