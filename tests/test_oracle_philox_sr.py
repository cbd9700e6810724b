"""Pins of the oracle's Philox generator and stochastic rounding."""
import numpy as np

import oracle as O
from golden_data import golden


def test_philox_known_answers():
    for v in golden("philox4x32_10_kat")["vectors"]:
        ctr = [int(h, 16) for h in v["ctr"]]
        key = [int(h, 16) for h in v["key"]]
        out = [int(h, 16) for h in v["out"]]
        assert list(O.philox4x32_10(ctr, key)) == out


def test_uniform_lanes_follow_philox_words():
    # Element idx reads 16-bit lane idx % 8 of the block n = idx / 8.
    seed, stream = 0x0123456789ABCDEF, 7
    for n in [0, 1, 12345, (1 << 33) + 5]:
        w = O.philox4x32_10([n & 0xFFFFFFFF, n >> 32, stream, 0],
                            [seed & 0xFFFFFFFF, seed >> 32])
        halves = []
        for word in w:
            halves += [int(word) & 0xFFFF, int(word) >> 16]
        u = O.sr_uniform(seed, stream, [8 * n + j for j in range(8)])
        assert np.array_equal(u, (np.array(halves, np.float32) + 0.5) / 65536)


def test_uniform_is_uniform():
    u = O.sr_uniform(42, 0, np.arange(1 << 20))
    assert u.min() > 0 and u.max() < 1
    hist = np.bincount((u * 64).astype(np.int64), minlength=64)
    expect = (1 << 20) / 64
    chi2 = ((hist - expect) ** 2 / expect).sum()
    assert chi2 < 120          # 63 dof; p ~ 1e-5 cut
    assert abs(u.mean() - 0.5) < 5 * (1 / np.sqrt(12)) / np.sqrt(1 << 20)
    # different streams and seeds give different draws
    assert not np.array_equal(u[:64], O.sr_uniform(42, 1, np.arange(64)))
    assert not np.array_equal(u[:64], O.sr_uniform(43, 0, np.arange(64)))


def test_sr_worked_example_monte_carlo():
    g = golden("requant_chain")
    # forward: 5.4 in a block of scale 9 -> 0.6 -> RTN 0.5 -> 4.5
    fwd = np.float32(g["value"]) / np.float32(g["fwd_scale"])
    assert abs(fwd - g["fwd_scaled"]) < 1e-6
    assert O.round_to(fwd, O.E2M1)[()] == g["fwd_code_value"]
    assert g["fwd_code_value"] * g["fwd_scale"] == g["fwd_value"]
    # backward: 4.5 in a block of scale 2 -> 2.25 -> SR between 2 and 3
    v = np.float32(g["fwd_value"]) / np.float32(g["bwd_scale"])
    assert v == g["bwd_scaled"]
    n = 1_000_000
    u = O.sr_uniform(0xC0FFEE, 3, np.arange(n))
    q = O.round_to(np.full(n, v, np.float32), O.E2M1, O.SR, u)
    assert set(np.unique(q)) == {2.0, 3.0}
    p_up = (q == 3.0).mean()
    sigma = np.sqrt(g["p_up"] * g["p_down"] / n)
    assert abs(p_up - g["p_up"]) < 5 * sigma
    mean = float(q.astype(np.float64).mean()) * g["bwd_scale"]
    assert abs(mean - g["mean"]) < 5 * sigma * g["bwd_scale"]


def _grid(fmt):
    if fmt == O.E2M1:
        return np.array([O.e2m1_value(c) for c in range(8)])
    return np.array([O.e4m3_value(b) for b in range(0x7F)])


def test_sr_exact_expectation_sweep():
    """E[q(x)] over all 2^16 uniforms equals x up to the 2^-17 lattice bias."""
    h = np.arange(1 << 16, dtype=np.float32)
    u_all = (h + np.float32(0.5)) / np.float32(65536.0)
    rng = np.random.default_rng(1)
    for fmt in (O.E2M1, O.E4M3):
        grid = _grid(fmt)
        vmax = grid[-1]
        # across every interval of the grid: interior points, near both ends
        lo, hi = grid[:-1], grid[1:]
        fr = np.concatenate([rng.uniform(0, 1, 3), [1e-3, 0.5, 1 - 1e-3]])
        xs = (lo[:, None] + (hi - lo)[:, None] * fr[None, :]).reshape(-1).astype(np.float32)
        xs = np.concatenate([xs, -xs[:20]])
        for x in xs:
            q = O.round_to(np.full(u_all.size, x, np.float32), fmt, O.SR, u_all).astype(
                np.float64)
            a = abs(float(x))
            k = np.searchsorted(grid, a, side="right") - 1
            a_lo, a_hi = grid[k], grid[min(k + 1, grid.size - 1)]
            # only the two neighbours are ever returned
            assert set(np.abs(np.unique(q))) <= {a_lo, a_hi}
            step = a_hi - a_lo
            bias = abs(q.mean() - float(x))
            assert bias <= step * 2.0 ** -16 + 1e-7 * a, (fmt, x, bias, step)
        # saturating end: x beyond the last grid point stays at vmax
        q = O.round_to(np.full(16, vmax, np.float32), fmt, O.SR, u_all[:16])
        assert np.all(q == vmax)


def test_sr_on_grid_is_deterministic():
    for fmt in (O.E2M1, O.E4M3):
        grid = _grid(fmt).astype(np.float32)
        u = O.sr_uniform(9, 9, np.arange(grid.size))
        assert np.array_equal(O.round_to(grid, fmt, O.SR, u), grid)
        assert np.array_equal(O.round_to(-grid, fmt, O.SR, u), -grid)


def test_sr_decision_is_exact():
    """floor(t + u) is decided on the exact sum (the pages define SR by its
    probability of rounding up; no intermediate rounding may move t + u
    across a grid point).  t + u = 1 - 2^-25 must round down although the
    nearest FP32 number to it is 1.0; t + u = 1 exactly rounds up."""
    u = np.float32([1.0 - 2.0 ** -17])               # the largest uniform, h = 65535
    # E2M1 bottom binade: step 1/2, t = 2|x|
    below = np.float32([2.0 ** -18 - 2.0 ** -26])     # t = 2^-17 - 2^-25
    at = np.float32([2.0 ** -18])                     # t = 2^-17
    assert O.round_to(below, O.E2M1, O.SR, u)[0] == 0.0
    assert O.round_to(at, O.E2M1, O.SR, u)[0] == 0.5
    assert O.round_to(-below, O.E2M1, O.SR, u)[0] == 0.0
    # E4M3 subnormal binade: step 2^-9, t = |x| * 2^9
    below8 = np.float32([(2.0 ** -17 - 2.0 ** -25) * 2.0 ** -9])
    at8 = np.float32([2.0 ** -26])
    assert O.round_to(below8, O.E4M3, O.SR, u)[0] == 0.0
    assert O.round_to(at8, O.E4M3, O.SR, u)[0] == 2.0 ** -9
