"""Host model of the error GEMM's work-item orders (csrc/lds_dma.h ``tile_of``, csrc/err_gemm.hip
``tri_tile`` and ``quad_tile``) and of the quadratic form's block decomposition.

The GPU kernels walk their tiles in a persistent loop: work item G runs on compute unit G % grid as
that unit's (G / grid)-th tile. This model repeats the index arithmetic and checks that
* every order is a bijection onto its tiles (every tile computed once, no tile twice);
* the quadratic form's pairs of row tiles give every compute unit the same number of K steps
  on the large layers' shapes;
* the decomposition the kQuad kernel computes - row tile I over K from its diagonal block to d_in,
  the diagonal block's G entries halved, the tile's sum doubled, K walked down in the first tile of a
  pair and up in the second - adds up to sum_o delta[o] G delta[o]^T exactly (float64, random
  symmetric G), for ragged d_in (last block 128 wide), ragged d_out, odd and even row-tile counts
  and compute-unit counts below and above the number of pairs.
The GPU parity tests (tests/test_parity_gpu_gram.py, tests/test_parity_gpu_full.py) check the
kernels themselves against the oracle; this model pins the orders' arithmetic on the CPU.
"""
import numpy as np
import pytest

SUPER = 16
XCDS = 8


def tile_of(G, tiles_m, n_cols):
    """Token tile and column of item G in the 16 x 16 super-block order (XCD-aware)."""
    n_sbm, n_sbn = -(-tiles_m // SUPER), -(-n_cols // SUPER)
    r = min(G // (SUPER * n_cols), n_sbm - 1)
    G1 = G - SUPER * r * n_cols
    h = min(SUPER, tiles_m - SUPER * r)
    c = min(G1 // (h * SUPER), n_sbn - 1)
    G2 = G1 - c * h * SUPER
    w = min(SUPER, n_cols - SUPER * c)
    if h == SUPER and w == SUPER:
        x, q = G2 % XCDS, G2 // XCDS
        return SUPER * r + (x // 4) * 8 + q % 8, SUPER * c + (x % 4) * 4 + q // 8
    if w == SUPER:
        x, q = G2 % XCDS, G2 // XCDS
        assert q < 2 * h
        return SUPER * r + q % h, SUPER * c + 2 * x + q // h
    return SUPER * r + G2 % h, SUPER * c + G2 // h


def tri_of(G, tiles):
    r, rem = 0, G
    while rem >= tiles - r:
        rem -= tiles - r
        r += 1
    return r, r + rem


def tri_tile(G, tiles):
    """Upper-triangle tile of item G in super-block rows (kStore: G = X^T X)."""
    r0, rem = 0, G
    while True:
        h = min(SUPER, tiles - r0)
        n_diag, n_right = h * (h + 1) // 2, h * (tiles - r0 - h)
        if rem < n_diag:
            a, b = tri_of(rem, h)
            return a + r0, b + r0
        rem -= n_diag
        if rem < n_right:
            a, b = tile_of(rem, h, tiles - r0 - h)
            return a + r0, b + r0 + h
        rem -= n_right
        r0 += SUPER


def quad_tile(G, R, n_cols, grid):
    """Row tile, column and K direction (True: downwards) of kQuad item G."""
    n_pairs = (R // 2) * n_cols
    if G < 2 * n_pairs:
        full, rem = n_pairs // grid, n_pairs % grid
        if G < 2 * full * grid:
            c = G // grid
            p, second = (c >> 1) * grid + (G - c * grid), c & 1
        else:
            g = G - 2 * full * grid
            second = int(g >= rem)
            p = full * grid + (g - rem if second else g)
        tm, col = tile_of(p, R // 2, n_cols)
        if second:
            tm = R - 1 - tm
        return tm, col, not second
    return R // 2, G - 2 * n_pairs, False


@pytest.mark.parametrize("tiles_m", [1, 2, 7, 15, 16, 17, 31, 33, 55, 112])
@pytest.mark.parametrize("n_cols", [1, 3, 16, 40, 97])
def test_tile_of_is_a_bijection(tiles_m, n_cols):
    seen = {tile_of(G, tiles_m, n_cols) for G in range(tiles_m * n_cols)}
    assert seen == {(m, c) for m in range(tiles_m) for c in range(n_cols)}


def test_partial_rows_give_each_xcd_two_columns():
    # 15 rows high: item G of a full-width super-block goes to XCD G % 8, which takes columns 2x, 2x+1
    for G in range(15 * 16):
        _, col = tile_of(G, 15, 64)
        assert col // 2 == G % XCDS


@pytest.mark.parametrize("tiles", [1, 2, 15, 16, 17, 33, 43, 112])
def test_tri_tile_is_a_bijection_onto_the_upper_triangle(tiles):
    seen = [tri_tile(G, tiles) for G in range(tiles * (tiles + 1) // 2)]
    assert all(a <= b < tiles for a, b in seen)
    assert len(set(seen)) == len(seen) == tiles * (tiles + 1) // 2


def _panels_per_xcd(order, tiles):
    """Mean over rounds of 256 items of the most distinct X panels one XCD's tiles need."""
    n = tiles * (tiles + 1) // 2
    worst = []
    for r0 in range(0, n, 256):
        panels = {}
        for G in range(r0, min(r0 + 256, n)):
            a, b = order(G, tiles)
            panels.setdefault(G % XCDS, set()).update((a, b))
        worst.append(max(len(v) for v in panels.values()))
    return float(np.mean(worst))


def test_tri_tile_shares_panels_inside_each_xcd():
    # stress layer's G (112 tile rows): the tiles an XCD runs together need far fewer distinct X
    # panels than in row order (13 inside a super-block row, more where a round spans two)
    blocked, rows = _panels_per_xcd(tri_tile, 112), _panels_per_xcd(tri_of, 112)
    assert blocked < 17 and rows > 30


@pytest.mark.parametrize("R,n_cols,grid", [(1, 5, 5), (2, 3, 6), (3, 4, 12), (4, 200, 256), (34, 2, 68),
                                           (43, 320, 256), (112, 1280, 256), (16, 960, 256), (5, 7, 3)])
def test_quad_tile_is_a_bijection(R, n_cols, grid):
    seen = set()
    for G in range(R * n_cols):
        tm, col, _ = quad_tile(G, R, n_cols, grid)
        assert 0 <= tm < R and 0 <= col < n_cols
        seen.add((tm, col))
    assert len(seen) == R * n_cols


@pytest.mark.parametrize("d_in,d_out,n_cand", [(28672, 8192, 40), (8192, 57344, 20), (4096, 12288, 20)])
def test_quad_pairs_balance_the_compute_units(d_in, d_out, n_cand):
    T, n_cols = -(-d_in // 256), -(-d_out // 256) * n_cand
    grid = min(T * n_cols, 256)
    steps = np.zeros(grid)
    for G in range(T * n_cols):
        tm, _, _ = quad_tile(G, T, n_cols, grid)
        steps[G % grid] += (d_in - 256 * tm) // 64
    assert steps.max() == steps.min()


def _quad_form_by_tiles(Gm, D, grid_cap):
    """The kQuad kernel's arithmetic in float64: per item, K steps of 64 in walk order, A = G's rows of
    the row tile (halved in the diagonal block), B = delta's rows of the column tile, the epilogue's
    sum of acc * delta[o, j], doubled."""
    n_cand, d_out, d_in = D.shape
    T, tn = -(-d_in // 256), -(-d_out // 256)
    n_cols = tn * n_cand
    grid = min(T * n_cols, grid_cap)
    sums = np.zeros((n_cand, T * tn))
    for G in range(T * n_cols):
        tm, col, down = quad_tile(G, T, n_cols, grid)
        k0 = 256 * tm
        k_steps, nd = (d_in - k0) // 64, min(256, d_in - k0) // 64
        d0, d1 = (k_steps - nd, k_steps) if down else (0, nd)
        cand, t = divmod(col, tn)
        rows, outs = slice(k0, min(k0 + 256, d_in)), slice(256 * t, min(256 * t + 256, d_out))
        acc = np.zeros((outs.stop - outs.start, rows.stop - rows.start))
        for kt in range(k_steps):
            pos = k_steps - 1 - kt if down else kt
            ks = slice(k0 + 64 * pos, k0 + 64 * pos + 64)
            half = d0 <= kt < d1
            assert half == (ks.start < k0 + 256)  # the halved steps are exactly the diagonal block's
            acc += D[cand][outs][:, ks] @ ((0.5 if half else 1.0) * Gm[rows, ks]).T
        sums[cand, tm * tn + t] = 2.0 * np.sum(acc * D[cand][outs][:, rows])
    return sums.sum(axis=1)


@pytest.mark.parametrize("d_in,d_out,n_cand,grid_cap", [(128, 100, 1, 256), (384, 300, 3, 256), (640, 513, 2, 5),
                                                       (1152, 256, 1, 7), (1024, 2560 // 8, 20, 40),
                                                       (2304, 700, 2, 3)])
def test_quad_decomposition_is_the_quadratic_form(d_in, d_out, n_cand, grid_cap):
    rng = np.random.default_rng(d_in + d_out)
    X = rng.standard_normal((d_in + 5, d_in))
    Gm = X.T @ X
    D = rng.standard_normal((n_cand, d_out, d_in))
    want = np.einsum("koi,ij,koj->k", D, Gm, D)
    got = _quad_form_by_tiles(Gm, D, grid_cap)
    np.testing.assert_allclose(got, want, rtol=1e-10)


def test_a_dropped_doubling_is_caught():
    # the model's check has teeth: counting the blocks right of the diagonal once gives another value
    rng = np.random.default_rng(1)
    X = rng.standard_normal((400, 384))
    Gm = X.T @ X
    D = rng.standard_normal((1, 130, 384))
    want = np.einsum("koi,ij,koj->k", D, Gm, D)
    once = sum(D[0][:, 256 * i:256 * i + 256] @ Gm[256 * i:256 * i + 256, 256 * j:256 * j + 256]
               @ D[0][:, 256 * j:256 * j + 256].T for i in range(2) for j in range(i, 2)).trace()
    assert abs(once - want[0]) > 1e-6 * abs(want[0])
