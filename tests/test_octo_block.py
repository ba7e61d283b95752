"""The triplet encoder scans 4 of the 9 cells of the joint-rounding window.

The oracle's joint rounding (OCTOPUS summary, Method steps 5-6, read as the
3x3 window around the point's (xi, eta) cell) keeps the candidate of least
error, which for positive norm codes is the candidate of largest projection
t . n_hat.  The GPU encoder scans only the 2x2 block of the window on the side
of the point's quadrant of its cell.  That is exact if the largest projection
over the other five cells never exceeds the block's.  This test checks that
property in float64 on the stored (fp32) direction tables at every bit width:
random points over the whole square, thin strips along the outer edges (where
the map folds the square's border onto itself and mirror cells tie) and along
the interior folds (xi = 0, eta = 0, |xi| + |eta| = 1).  The block is formed
as in the kernel: the two grid columns (rows) whose centres bracket xi (eta),
and next to an outer column that column and its neighbour.
"""

import numpy as np
import pytest

from oracle import tq_oracle as O


def _block_lo(v, nd):
    """Lower column of the block, as the kernel forms it: the lower of the two
    column centres around v, floor((v + 1) nd / 2 - 1/2), clamped to
    [0, nd - 2] (next to an outer column: that column and its neighbour)."""
    return np.clip(np.floor((v + 1.0) * (nd / 2) - 0.5).astype(np.int64), 0, nd - 2)


def _block_margin(xi, eta, dirs, nd):
    """(best projection in the quadrant block) - (best over the other cells
    of the 3x3 window), for the unit directions at (xi, eta)."""
    n = O.oct_unmap(xi, eta)
    jx = np.clip(np.floor((xi + 1.0) * (nd / 2)).astype(np.int64), 0, nd - 1)
    je = np.clip(np.floor((eta + 1.0) * (nd / 2)).astype(np.int64), 0, nd - 1)
    a0, c0 = _block_lo(xi, nd), _block_lo(eta, nd)
    # the block lies inside the window of the point's cell
    assert np.all((a0 >= jx - 1) & (a0 + 1 <= jx + 1) & (c0 >= je - 1) & (c0 + 1 <= je + 1))
    best_in = np.full(xi.shape, -np.inf)
    best_out = np.full(xi.shape, -np.inf)
    for da in (-1, 0, 1):
        for dc in (-1, 0, 1):
            a, c = jx + da, je + dc
            ok = (a >= 0) & (a < nd) & (c >= 0) & (c < nd)
            p = np.sum(n * dirs[np.clip(a, 0, nd - 1), np.clip(c, 0, nd - 1)], axis=-1)
            p = np.where(ok, p, -np.inf)
            inside = ((a == a0) | (a == a0 + 1)) & ((c == c0) | (c == c0 + 1))
            best_in = np.where(inside, np.maximum(best_in, p), best_in)
            best_out = np.where(~inside, np.maximum(best_out, p), best_out)
    return best_in - best_out


@pytest.mark.parametrize("b", [2, 3, 4])
def test_best_window_cell_lies_in_the_quadrant_block(b):
    dirs, _ = O.octo_codebooks(128, b)
    nd = 1 << O.octo_bits(b)[0]
    rng = np.random.default_rng(2024 + b)
    points = [(rng.uniform(-1, 1, 400_000), rng.uniform(-1, 1, 400_000))]
    s = np.linspace(-1.0, 1.0, 40_001)
    for eps in (1e-9, 1e-6, 1e-3):
        z = np.zeros_like(s)
        points += [(-1 + eps + z, s), (1 - eps + z, s), (s, -1 + eps + z), (s, 1 - eps + z)]
        for sg in (-1.0, 1.0):
            points += [(sg * eps + z, s), (s, sg * eps + z)]
            diag = 1.0 - np.abs(s) + sg * eps
            ok = np.abs(diag) <= 1.0
            points += [(s[ok], diag[ok]), (s[ok], -diag[ok])]
    worst = min(float(np.min(_block_margin(x, e, dirs, nd))) for x, e in points)
    assert worst >= 0.0, f"a cell outside the quadrant block wins by {-worst:.3e}"


def test_block_scan_matches_the_full_window_on_the_oracles_codes():
    """Codes from the 2x2 scan equal the oracle's 3x3 joint rounding on
    random triplets (ties aside, which have measure zero)."""
    for b in (2, 3, 4):
        dirs, crho = O.octo_codebooks(128, b)
        nd = 1 << O.octo_bits(b)[0]
        rng = np.random.default_rng(77 + b)
        t = rng.standard_normal((200_000, 3)) * rng.uniform(0.01, 0.4, (200_000, 1))
        ref = O.octo_encode_triplets(t, b, dirs, crho)
        rho = np.sqrt(np.sum(t * t, axis=-1))
        xi, eta = O.oct_map(t / rho[:, None])
        a0, c0 = _block_lo(xi, nd), _block_lo(eta, nd)
        best = np.full(rho.shape, -np.inf)
        A = np.zeros(rho.shape, np.int64)
        C = np.zeros(rho.shape, np.int64)
        for da in (0, 1):
            for dc in (0, 1):
                a, c = a0 + da, c0 + dc
                p = np.sum(t * dirs[a, c], axis=-1)
                take = p > best
                best, A, C = np.where(take, p, best), np.where(take, a, A), np.where(take, c, C)
        assert np.array_equal(A, ref["a"]) and np.array_equal(C, ref["c"]), b


@pytest.mark.parametrize("b", [2, 3, 4])
def test_map_error_leaves_the_block_choice(b):
    """The GPU map is approximate (a polynomial arctangent within 1.6e-7 rad,
    fp32 arithmetic), so its xi and eta differ slightly from the oracle's.
    Shifted by 2e-5 in any direction (about 100 times that), the block still
    holds the window's best cell."""
    dirs, _ = O.octo_codebooks(128, b)
    nd = 1 << O.octo_bits(b)[0]
    rng = np.random.default_rng(31 + b)
    xi, eta = rng.uniform(-1, 1, 400_000), rng.uniform(-1, 1, 400_000)
    n = O.oct_unmap(xi, eta)
    jx = np.clip(np.floor((xi + 1.0) * (nd / 2)).astype(np.int64), 0, nd - 1)
    je = np.clip(np.floor((eta + 1.0) * (nd / 2)).astype(np.int64), 0, nd - 1)
    best = np.full(xi.shape, -np.inf)
    A = np.zeros(xi.shape, np.int64)
    C = np.zeros(xi.shape, np.int64)
    for da in (-1, 0, 1):
        for dc in (-1, 0, 1):
            a, c = jx + da, je + dc
            ok = (a >= 0) & (a < nd) & (c >= 0) & (c < nd)
            p = np.where(ok, np.sum(n * dirs[np.clip(a, 0, nd - 1), np.clip(c, 0, nd - 1)], axis=-1), -np.inf)
            take = p > best
            best, A, C = np.where(take, p, best), np.where(take, a, A), np.where(take, c, C)
    for sx in (-1.0, 1.0):
        for sy in (-1.0, 1.0):
            a0 = _block_lo(np.clip(xi + sx * 2e-5, -1, 1), nd)
            c0 = _block_lo(np.clip(eta + sy * 2e-5, -1, 1), nd)
            inside = ((A == a0) | (A == a0 + 1)) & ((C == c0) | (C == c0 + 1))
            assert np.all(inside), int(np.sum(~inside))
