"""Pins of the seeded input generator (CPU only): the Lloyd fit against the exact
half-normal Lloyd-Max solution, the RTN encoder against a brute-force nearest-level search,
the crest factor the model card quotes for Gaussian weights, and the quality direction
(Lloyd grid beats E2M1 on Gaussian weights)."""
import numpy as np
import pytest
from scipy.stats import norm

import oracle
import synth


def _density_lloyd(n=8, iters=2000):
    """Lloyd-Max levels of the half-normal density |N(0,1)| by fixed-point iteration:
    cut points at midpoints, each level at the conditional mean of its cell,
    E[r | a < r < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a))."""
    lv = norm.ppf(0.5 + 0.5 * (np.arange(n) + 0.5) / n)
    for _ in range(iters):
        cuts = np.concatenate([[0.0], 0.5 * (lv[1:] + lv[:-1]), [np.inf]])
        a, b = cuts[:-1], cuts[1:]
        lv = (norm.pdf(a) - norm.pdf(b)) / (norm.cdf(b) - norm.cdf(a))
    return lv


def test_lloyd_grid_close_to_density_solution():
    exact = _density_lloyd()
    grid = synth.lloyd_grid(1, 0)
    assert grid.dtype == np.float32 and grid.shape == (8,)
    assert np.all(np.diff(grid) > 0) and grid[0] > 0
    np.testing.assert_allclose(grid, exact, atol=0.03)
    # the largest level sits in the tail: about 2.73 for 16-level Gaussian Lloyd-Max
    assert 2.6 < exact[-1] < 2.8


def test_lloyd_grid_seeded_per_layer():
    a, b, c = synth.lloyd_grid(3, 0), synth.lloyd_grid(3, 0), synth.lloyd_grid(3, 1)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)


def test_crest_factor_matches_model_card():
    # GLM-5.2-NF4-Lloyd-Experts-GPTQ, "What this is": Gaussian weights have crest factor
    # ~2.365 (ratio of block-32 max |w| to the block RMS, averaged)
    w = synth.normal_matrix(synth.key(99, 0), 6250, 1024)       # 200k blocks of 32
    blk = w.reshape(-1, 32).astype(np.float64)
    cf = np.mean(np.abs(blk).max(1) / np.sqrt((blk ** 2).mean(1)))
    assert abs(cf - 2.365) < 0.01
    assert abs(w.std() - synth.WEIGHT_SIGMA) < 2e-4


def _brute_rtn(w, grid):
    """Nearest-level search written out: for each block the smallest e with gmax 2^e >= amax,
    then argmin_i | |w|/2^e - grid_i | with ties to the lower index."""
    N, K = w.shape
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, K // 32), np.uint8)
    g = grid.astype(np.float64)
    for n in range(N):
        for b in range(K // 32):
            blk = w[n, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            e = -200
            while g[-1] * 2.0 ** e < amax:
                e += 1
            scales[n, b] = e + 127
            r = np.abs(blk) / 2.0 ** e
            d = np.abs(r[:, None] - g[None, :])
            idx = np.argmin(d, axis=1)                  # first minimum: lower index on ties
            codes[n, 32 * b:32 * b + 32] = idx | np.where(blk < 0, 8, 0)
    return codes, scales


@pytest.mark.parametrize("which", ["lloyd", "e2m1"])
def test_rtn_encoder_matches_bruteforce(which):
    grid = synth.lloyd_grid(1, 0) if which == "lloyd" else synth.E2M1_GRID
    w = synth.normal_matrix(synth.key(7, 1), 24, 256)
    # exact ties and zero blocks
    w[0, :32] = 0.0
    w[1, :32] *= 0.1
    w[1, 0] = np.float32(grid[7] * 2.0 ** -6)          # amax exactly gmax * 2^-6
    w[1, 1] = np.float32(0.5 * (grid[2] + grid[3]) * 2.0 ** -6)   # a midpoint (if exact)
    codes, scales = synth.rtn_encode(w, grid)
    bc, bs = _brute_rtn(w, grid)
    np.testing.assert_array_equal(scales, bs)
    np.testing.assert_array_equal(oracle.unpack_codes(codes), bc)
    assert scales[0, 0] == 0 and (codes[0, :16] == 0).all()
    assert scales[1, 0] == 127 - 6


def test_rtn_error_bound_and_quality_direction():
    w = synth.normal_matrix(synth.key(8, 2), 256, 1024)
    lloyd = synth.lloyd_grid(1, 0)
    errs = {}
    for name, grid in (("lloyd", lloyd), ("e2m1", synth.E2M1_GRID)):
        codes, scales = synth.rtn_encode(w, grid)
        v = oracle.dequant_f64_exact(codes, scales, grid)
        step = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=1)
        gaps = np.diff(np.concatenate([[0.0], grid.astype(np.float64)]))
        bound = max(grid[0], 0.5 * gaps.max()) * step
        assert np.all(np.abs(v - w) <= bound + 1e-30)
        errs[name] = np.sqrt(((v - w) ** 2).sum() / (w.astype(np.float64) ** 2).sum())
    # GLM-5.2-NF4-Lloyd-Experts-GPTQ: the fitted grid gives lower weight error than E2M1
    assert errs["lloyd"] < errs["e2m1"]
    assert 0.08 < errs["lloyd"] < 0.14


def test_generator_permutation_consistency():
    """Stored gate row n / down column n hold logical channel perms[e, n]."""
    E, H, I = 2, 64, 64
    a = synth.make_layer(11, E, H, I)
    b = synth.make_layer(11, E, H, I, permute="random")
    for e in range(E):
        p = b.perms[e]
        np.testing.assert_array_equal(b.gate_codes[e], a.gate_codes[e][p])
        np.testing.assert_array_equal(b.up_scales[e], a.up_scales[e][p])
    # down columns: the draws move with the permutation (the bytes differ because the
    # 32-blocks are re-formed). The gathered branch and the contiguous branch of the
    # generator evaluate the same Box-Muller draw with differently vectorised libm calls,
    # so values agree to the last fp32 ulp, not bit for bit.
    k = synth.key(11, synth.S_WEIGHTS, 0, 0, 2)
    d0 = synth.normal_matrix(k, H, I)
    d1 = synth.normal_matrix(k, H, I, col_src=b.perms[0])
    np.testing.assert_allclose(d1, d0[:, b.perms[0]], rtol=1e-6, atol=1e-9)


def test_logits_zipf_skew():
    T, E = 2048, 256
    lg = synth.make_logits(3, T, E, zipf_s=1.0)
    ids, _ = oracle.route_topk(lg, 8)
    counts = np.bincount(ids.ravel(), minlength=E)
    top8 = np.sort(counts)[::-1][:8].sum() / counts.sum()
    assert top8 > 0.4                     # a few experts carry most of the routed mass
    flat = synth.make_logits(2, T, E)
    ids2, _ = oracle.route_topk(flat, 8)
    c2 = np.bincount(ids2.ravel(), minlength=E)
    assert np.sort(c2)[::-1][:8].sum() / c2.sum() < 0.1
    for t in range(0, T, 97):
        assert len(np.unique(lg[t])) == E


def test_router_weights_seeded_and_scaled():
    H, E = 6144, 256
    a = synth.make_router(4, E, H)
    np.testing.assert_array_equal(a, synth.make_router(4, E, H))
    assert not np.array_equal(a, synth.make_router(4, E, H, layer=1))
    assert a.dtype == np.uint16 and a.shape == (E, H)
    lg = oracle.router_logits(synth.make_x(4, 64, H), a)
    assert 0.9 < lg.std() < 1.1          # logits about N(0, 1) with x ~ N(0, 1)
