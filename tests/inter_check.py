"""Element-wise check of the intermediate I = bf16(silu(g) * u) of the GPU against the oracle.

The GPU accumulates g and u in fp32 and the oracle in fp64; both round I once to bf16. An
element may therefore land one bf16 ulp away where the two sums straddle a rounding boundary,
and further only where g or u nearly cancel, so that the fp32 accumulation error is large
relative to the value. The check:
  * every element equal, or within 1 ulp of the oracle's, or (beyond 1 ulp) within the fp32
    accumulation bound of that element: |dI| <= ulp + K 2^-24 (|silu'(g) u| S_g +
    |silu(g)| S_u) + 2^-22 |silu(g) u|, with S_g = sum_h |x_h Wg[n, h]| (likewise S_u) and
    K the contraction length (every rounding of any summation order is covered);
  * the fraction of elements that are not bit-equal (signed zeros equal) at most
    FLIP_FRACTION_MAX: a systematic error of a fraction of an ulp (for instance 1e-3 relative)
    moves far more elements than that.
"""
import numpy as np

import oracle

FLIP_FRACTION_MAX = 0.01


def bf16_ulp(v):
    """Spacing of bf16 numbers at the fp64 values v (bf16 values): 2^(e - 7)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    e = np.floor(np.log2(a)).astype(np.int64)
    return np.ldexp(1.0, e - 7)


def _element_bound(lw, x, t, e, n, ulp):
    tab = lw.tables[int(lw.table_id[e])]
    wg = oracle.bf16_to_f64(oracle.dequant_bf16(lw.gate_codes[e, n:n + 1],
                                                lw.gate_scales[e, n:n + 1], tab))[0]
    wu = oracle.bf16_to_f64(oracle.dequant_bf16(lw.up_codes[e, n:n + 1],
                                                lw.up_scales[e, n:n + 1], tab))[0]
    xt = x[t]
    g, u = float(xt @ wg), float(xt @ wu)
    sg, su = float(np.abs(xt) @ np.abs(wg)), float(np.abs(xt) @ np.abs(wu))
    sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))
    gamma = x.shape[1] * 2.0 ** -24
    return ulp + gamma * (abs(dsilu * u) * sg + abs(silu) * su) + 2.0 ** -22 * abs(silu * u)


def check_inter(gpu_bits, ref_bits, token_of_row, expert_of_row, x_bits, lw, label=""):
    """gpu_bits, ref_bits: bf16 bits [R, I] in natural channel order; row r is the pair of
    token token_of_row[r] on expert expert_of_row[r]. Returns (not bit-equal, beyond 1 ulp)."""
    g = oracle.bf16_to_f64(gpu_bits)
    r = oracle.bf16_to_f64(ref_bits)
    assert g.shape == r.shape
    same = (g == r) | (np.isnan(g) & np.isnan(r))
    flips = int((~same).sum())
    diff = np.abs(g - r)
    ulp = bf16_ulp(r)
    over = ~same & ~(diff <= ulp)
    bad = []
    if over.any():
        x = oracle.bf16_to_f64(x_bits)
        for ri, n in zip(*np.nonzero(over)):
            b = _element_bound(lw, x, int(token_of_row[ri]), int(expert_of_row[ri]), int(n),
                               float(ulp[ri, n]))
            if not diff[ri, n] <= b:
                bad.append((int(ri), int(n), float(g[ri, n]), float(r[ri, n]), b))
    frac = flips / max(g.size, 1)
    print(f"inter {label}: {g.size} elements, {flips} not bit-equal ({frac:.2e}), "
          f"{int(over.sum())} beyond 1 ulp", flush=True)
    assert not bad, f"elements beyond their fp32 accumulation bound (row, n, gpu, ref, bound): {bad[:8]}"
    assert frac <= FLIP_FRACTION_MAX, f"{flips} of {g.size} elements not bit-equal"
    return flips, int(over.sum())
