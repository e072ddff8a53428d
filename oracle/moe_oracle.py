"""Plain, slow, fp64 CPU oracle of the routed-expert MoE forward over 4-bit codebook experts.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or call this module. It shares no code with the GPU library
(``codebook_quantized_moe_amd``) and imports nothing from it.

Sources (the pages' titles; the section named on each function):

* [card]  GLM-5.2-NF4-Lloyd-Experts-GPTQ model card (aidendle94): the storage format --
  "Contents" (4-bit codes + E8M0 block scales, block 32 along K, low nibble = even K) and
  "Codes are indices into the per-layer grid" (the low 3 bits of a code pick one of the 8
  grid magnitudes, bit 3 is the sign, and the block's scale byte s multiplies by
  2^(s - 127); the grid holds absolute magnitudes, with no per-block normalisation) and
  "What this is" (the E2M1 table {0, .5, 1, 1.5, 2, 3, 4, 6}).
* [brief] "Round 7 -- Rewrite the GLM-5.2 routed-expert encoder" (CODEX_ROUND7.md of
  GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78): model geometry (256 routed experts, top-8, hidden 6144,
  moe_intermediate 2048); decision 4 (I_e = silu(X Wg^T) * (X Wu^T)); decision 6 (down is
  the [K=2048, N=6144] contraction of I_e); decision 7 (a consistent intermediate-channel
  permutation of gate-N, up-N and down-K is exact because SwiGLU is elementwise).
* [readme] README of GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "What had to be fixed" / "Shared
  residual rotations": expert outputs are router-weighted and summed back per token.
* [dense6] GLM-5.2-EXL3-DENSE6-MTP78 model card, "Quant recipe": the router (mlp.gate) is held
  in BF16; [brief] "Target pipeline": a layer's routing is the router applied to its
  activations.
* [readme] "Checkpoint layout update (2026-08-10): BF16 shared experts, merged online K6" and
  "What changed and why": every routed layer also carries one shared-expert MLP (gate, up,
  down projections; 5.74 GB of BF16 over the 76 layers, i.e. 3 * 6144 * 2048 weights per
  layer) whose gate and up run as one merged launch.

Readings where the pages are silent (each is listed with its reason in the design notes):

* gating: softmax over the k selected logits (textbook top-k gating), or the logistic
  sigmoid of each selected logit renormalised over the k (the other textbook form); either
  way the k experts are the k largest logits (the sigmoid is increasing);
* router logits: the plain product of the bf16 activations and the bf16 router rows;
* top-k order: IEEE-754 totalOrder on the fp32 logit bits, descending, ties (identical
  bits) to the lower expert id;
* permutation: pairs p = t*k + j sorted by (expert, p), i.e. a stable sort; pairs whose id
  is outside [0, E) are placed after all valid pairs, in p order;
* dequant rounding: the exact product, rounded once to bf16 (round-to-nearest-even);
  code 8 of a table whose entry 0 is 0 gives -0; scale byte 255 gives NaN (OCP MX E8M0);
* the intermediate I is rounded to bf16 (the one stored activation inside the layer);
  everything else accumulates in fp64;
* shared expert: a SwiGLU MLP of the routed experts' shape and storage format, run on every
  token with weight 1 and added to the routed sum before the residual (the usual
  shared-expert MoE; the pages give its tensors and size, not the sum);
* encoding: nearest magnitude with ties to the lower index, the sign bit for negative
  weights only, exponents clamped to [-127, 127], all-zero blocks at byte 0, blocks with a
  non-finite weight at byte 255 with zero codes; the grid fit takes its ratios (the data)
  with the block exponents of the starting table and moves the levels by weighted Lloyd
  rounds on them (an empty cell keeps its magnitude); the arm choice keeps the fitted grid
  on a tie.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64", "rne_bf16", "total_order_key", "router_logits", "route_topk",
    "permute_by_expert",
    "unpack_codes", "dequant_bf16", "layer_forward", "expert_inter", "shared_expert_forward",
    "stack_forward",
    "block_scale_bytes", "rtn_encode", "reconstruction_sq_error", "lloyd_stats",
    "lloyd_update", "fit_grid", "select_arms", "E2M1_TABLE",
]

# [card] "What this is": the MXFP4 (E2M1) magnitudes, one per 3-bit magnitude index.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


# ----------------------------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def rne_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Written from the bf16 format itself (1 sign bit, 8 exponent bits with bias 127,
    7 stored significand bits; gradual underflow below 2^-126 in steps of 2^-133), one
    rounding straight from fp64 (no detour through fp32, which would round twice for values
    in bf16's subnormal range). NaN -> 0x7FC0 with the input's sign; overflow -> +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint32) << np.uint32(15)
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.uint32)

    nan = np.isnan(a)
    inf = np.isinf(a)
    fin = ~(nan | inf)

    # normal range of the result: |x| >= 2^-126. |x| = m * 2^ex with m in [0.5, 1).
    m, ex = np.frexp(np.where(fin, a, 1.0))
    q = ex.astype(np.int64) - 1                      # |x| = (2m) * 2^q, 2m in [1, 2)
    normal = fin & (a >= 2.0 ** -126)
    # significand in units of the quantum 2^(q-7): in [128, 256); exact power-of-two scaling
    sig = np.ldexp(np.where(normal, a, 0.0), np.where(normal, 7 - q, 0))
    r = np.rint(sig)                                  # numpy rint: round half to even
    carry = r >= 256.0
    r = np.where(carry, 128.0, r)
    q = np.where(carry, q + 1, q)
    over = normal & (q > 127)
    nbits = (((q + 127).astype(np.uint32) & np.uint32(0xFF)) << np.uint32(7)) | \
        ((r.astype(np.int64) - 128).astype(np.uint32) & np.uint32(0x7F))
    out = np.where(normal & ~over, nbits, out)
    out = np.where(over | inf, np.uint32(0x7F80), out)

    # subnormal range: multiples of 2^-133; a result of 128 units is the smallest normal.
    sub = fin & (a < 2.0 ** -126)
    units = np.rint(np.ldexp(np.where(sub, a, 0.0), 133))
    out = np.where(sub, units.astype(np.uint32), out)

    out = np.where(nan, np.uint32(0x7FC0), out)
    return (out | sign).astype(np.uint16)


# ----------------------------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------------------------

def total_order_key(logits) -> np.ndarray:
    """uint32 keys whose unsigned order is IEEE-754 totalOrder of the fp32 values."""
    b = np.ascontiguousarray(logits, dtype=np.float32).view(np.uint32)
    neg = (b >> np.uint32(31)).astype(bool)
    return np.where(neg, ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def router_logits(x_bits, router_bits) -> np.ndarray:
    """Router logits l[t, e] = sum_h x[t, h] * Wr[e, h] over the bf16 values, in fp64.

    [dense6] "Quant recipe": the router weight is kept in BF16; [brief] "Target pipeline":
    routing_L = router(acts_L). x_bits uint16 [T, H], router_bits uint16 [E, H].
    Returns float64 [T, E].
    """
    x = bf16_to_f64(x_bits)
    wr = bf16_to_f64(router_bits)
    return x @ wr.T


def route_topk(logits, k: int, gating: str = "softmax"):
    """Top-k experts per token and their gate values.

    [brief] model geometry: each token selects 8 of 256 routed experts. Order of the k ids:
    logit descending (totalOrder), ties to the lower expert id. Gate values, in fp64, over
    the k selected logits: "softmax", w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0); or
    "sigmoid", s_j = 1 / (1 + exp(-l_j)) and w_j = s_j / sum_i s_i.
    Returns ids int32 [T, k], w float64 [T, k].
    """
    if gating not in ("softmax", "sigmoid"):
        raise ValueError(gating)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    assert 1 <= k <= E
    key = total_order_key(logits).astype(np.int64)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -key[t]))  # primary: key descending; secondary: id ascending
        sel = order[:k]
        ids[t] = sel
        lv = logits[t, sel].astype(np.float64)
        if gating == "softmax":
            ex = np.exp(lv - lv[0])
            w[t] = ex / ex.sum()
        else:
            sg = 1.0 / (1.0 + np.exp(-lv))
            w[t] = sg / sg.sum()
    return ids, w


def permute_by_expert(ids, E: int):
    """Group the T*k (token, slot) pairs by expert.

    Pair p = t*k + j. Pairs are ordered by (expert id, p) ascending (a stable counting sort);
    pairs whose id is outside [0, E) come last, in p order.
    Returns offsets int32 [E+1] (offsets[e] = number of valid pairs with id < e; offsets[E]
    = number of valid pairs), sorted_pair int32 [T*k] (sorted position -> p) and pair_pos
    int32 [T*k] (p -> sorted position).
    """
    e = np.asarray(ids, dtype=np.int64).ravel()
    P = e.size
    p = np.arange(P)
    valid = (e >= 0) & (e < E)
    bucket = np.where(valid, e, E)
    counts = np.bincount(bucket, minlength=E + 1)[:E]
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_pair = np.lexsort((p, bucket))
    pair_pos = np.empty(P, np.int64)
    pair_pos[sorted_pair] = p
    return offsets.astype(np.int32), sorted_pair.astype(np.int32), pair_pos.astype(np.int32)


# ----------------------------------------------------------------------------------------------
# dequantisation
# ----------------------------------------------------------------------------------------------

def unpack_codes(codes) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes; [card] "Contents": low nibble = even K."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = c & 0x0F
    out[..., 1::2] = c >> 4
    return out


def dequant_f64_exact(codes, scales, table) -> np.ndarray:
    """The exact (unrounded) weight values of one matrix, in fp64.

    [card] "Codes are indices into the per-layer grid": mag = code & 7 indexes the 8-entry
    table, sign = -1 when bit 3 is set, w = sign * table[mag] * 2^(scale_byte - 127), one
    scale byte per 32 consecutive K of a row. Scale byte 255 -> NaN (reading).
    The product of an fp32 table entry and 2^(s - 127), s in [0, 254], is exact in fp64.
    """
    c = unpack_codes(codes)
    s = np.repeat(np.asarray(scales, dtype=np.int64), 32, axis=-1)
    assert s.shape == c.shape
    tab = np.asarray(table, dtype=np.float32).astype(np.float64)
    mag = tab[c & 7]
    neg = (c & 8) != 0
    v = np.ldexp(mag, s - 127)
    v = np.where(neg, -v, v)                       # -0.0 for a zero magnitude
    v = np.where(s == 255, np.where(neg, -np.nan, np.nan), v)
    return v


def dequant_bf16(codes, scales, table) -> np.ndarray:
    """Dequantised weights as bf16 bit patterns (uint16): one RNE rounding of the exact value."""
    return rne_bf16(dequant_f64_exact(codes, scales, table))


def _expert_dense(codes, scales, table):
    return bf16_to_f64(dequant_bf16(codes, scales, table))


# ----------------------------------------------------------------------------------------------
# encoding (the quantizer) and the grid fit
# ----------------------------------------------------------------------------------------------

def block_scale_bytes(w_bits, gmax: float) -> np.ndarray:
    """Scale byte of every block of 32 along K of bf16 weights [..., K].

    [card] "Codes are indices into the per-layer grid": a block's exponent e is the least
    integer for which the grid's top magnitude times 2^e reaches the block's largest
    magnitude, stored as the byte e + 127. Readings: e is clamped to [-127, 127]; an
    all-zero block gets byte 0; a block holding an Inf or NaN gets byte 255 (it decodes to
    NaN).
    """
    w = bf16_to_f64(w_bits)
    blocks = w.reshape(w.shape[:-1] + (w.shape[-1] // 32, 32))
    out = np.empty(blocks.shape[:-1], np.uint8)
    g = float(np.float32(gmax))
    for idx in np.ndindex(out.shape):
        b = blocks[idx]
        if not np.all(np.isfinite(b)):
            out[idx] = 255
            continue
        amax = float(np.max(np.abs(b)))
        if amax == 0.0:
            out[idx] = 0
            continue
        e = math.frexp(amax / g)[1]
        while math.ldexp(g, e) < amax:
            e += 1
        while math.ldexp(g, e - 1) >= amax:
            e -= 1
        out[idx] = min(max(e, -127), 127) + 127
    return out


def rtn_encode(w_bits, table):
    """Round-to-nearest encoding of bf16 weights [N, K] against 8 ascending magnitudes.

    [card] "Codes are indices into the per-layer grid" (bits 0..2 index the grid, bit 3 is the
    sign, w = sign * grid[mag] * 2^(s - 127)) and "Contents" (block 32 along K, two codes per
    byte, the even K in the low nibble). Each weight takes the magnitude nearest to
    |w| / 2^e, ties to the lower index (reading); bit 3 is set for negative weights (reading:
    -0 keeps a clear sign bit). Returns codes uint8 [N, K/2], scales uint8 [N, K/32].
    """
    tab = np.asarray(table, dtype=np.float32).astype(np.float64)
    w = bf16_to_f64(w_bits)
    N, K = w.shape
    scales = block_scale_bytes(w_bits, tab[7])
    e = np.repeat(scales.astype(np.int64), 32, axis=1) - 127
    r = np.abs(w) * np.ldexp(1.0, -e)                 # exact: a power-of-two rescale
    mid = 0.5 * (tab[:-1] + tab[1:])                  # exact in fp64
    mag = np.zeros((N, K), np.int64)
    for i in range(7):
        mag += r > mid[i]
    codes4 = (mag | np.where(w < 0, 8, 0)).astype(np.uint8)
    bad = np.repeat(scales == 255, 32, axis=1)
    codes4[bad] = 0
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def reconstruction_sq_error(w_bits, codes, scales, table) -> np.ndarray:
    """Per row: sum over K of (w - w_hat)^2 in fp64, w_hat the bf16 dequantisation."""
    w = bf16_to_f64(w_bits)
    wh = bf16_to_f64(dequant_bf16(codes, scales, table))
    return np.sum((w - wh) ** 2, axis=1)


def lloyd_stats(w_bits, table, gmax=None):
    """One weighted Lloyd-Max step's sums over bf16 weights [N, K] for 8 ascending magnitudes.

    [card] "What this is": the layer's 8 magnitudes come from a Lloyd-Max fit to the
    block-normalised magnitudes r = |W| / 2^e of every expert's three matrices taken together,
    where a ratio counts with weight (2^e)^2, the factor by which its squared error scales back
    to weight space. e is each block's exponent for the
    top magnitude gmax (block_scale_bytes; default table[7]) and each ratio goes to its
    nearest magnitude of `table` (the rtn_encode rule). Returns float64 [3, 8]: per magnitude
    m, sum (2^e)^2 r, sum (2^e)^2 and sum (2^e)^2 (r - table[m])^2 over the ratios it holds.
    Blocks with a non-finite weight are skipped.
    """
    tab = np.asarray(table, dtype=np.float32).astype(np.float64)
    w = bf16_to_f64(w_bits)
    scales = block_scale_bytes(w_bits, tab[7] if gmax is None else gmax)
    keep = np.repeat(scales != 255, 32, axis=1)
    e = np.repeat(scales.astype(np.int64), 32, axis=1) - 127
    r = np.abs(w) * np.ldexp(1.0, -e)
    mid = 0.5 * (tab[:-1] + tab[1:])
    mag = np.zeros(w.shape, np.int64)
    for i in range(7):
        mag += r > mid[i]
    wt = np.ldexp(1.0, 2 * e)
    out = np.zeros((3, 8), np.float64)
    for m in range(8):
        sel = keep & (mag == m)
        out[0, m] = np.sum(wt[sel] * r[sel])
        out[1, m] = np.sum(wt[sel])
        out[2, m] = np.sum(wt[sel] * (r[sel] - tab[m]) ** 2)
    return out


def lloyd_update(table, stats) -> np.ndarray:
    """The next table: each magnitude moves to the weighted mean of its ratios (a magnitude
    that holds no ratio stays), rounded to fp32."""
    tab = np.asarray(table, dtype=np.float32).astype(np.float64)
    s1, s0 = stats[0], stats[1]
    new = np.where(s0 > 0, s1 / np.where(s0 > 0, s0, 1.0), tab)
    return new.astype(np.float32)


def fit_grid(mats, table0, iters: int):
    """Weighted Lloyd-Max over the pooled ratios of several bf16 matrices: the ratios and their
    weights are fixed by table0's top magnitude (the data of the fit), then iters rounds of
    assignment and update (lloyd_stats summed over the matrices, lloyd_update) move the
    levels; the weighted squared error of the ratios never goes up. Returns the fp32 table
    (the matrices are then encoded against it, with its own top magnitude)."""
    tab = np.asarray(table0, dtype=np.float32)
    g0 = float(tab[7])
    for _ in range(iters):
        st = sum(lloyd_stats(m, tab, gmax=g0) for m in mats)
        tab = lloyd_update(tab, st)
    return tab


def select_arms(err_a, err_b) -> np.ndarray:
    """Per expert, arm 0 (the fitted grid) unless arm 1 (E2M1) has the strictly smaller
    reconstruction error ([card] "Provenance": the winner is chosen per expert against an
    E2M1 control arm). err_*: float64 [E]. Returns table ids uint8 [E]."""
    return (np.asarray(err_b) < np.asarray(err_a)).astype(np.uint8)


# ----------------------------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------------------------

def _silu(g):
    return g / (1.0 + np.exp(-g))


def _swiglu_rows(xs, lw, e):
    """silu(Wg_e x) * (Wu_e x) in fp64 for the activation rows xs [R, H] (fp64 values of bf16
    activations), [brief] decision 4."""
    tab = lw.tables[int(lw.table_id[e])]
    wg = _expert_dense(lw.gate_codes[e], lw.gate_scales[e], tab)
    g = xs @ wg.T
    del wg
    wu = _expert_dense(lw.up_codes[e], lw.up_scales[e], tab)
    u = xs @ wu.T
    return _silu(g) * u


def expert_inter(x_bits, lw, e, tokens) -> np.ndarray:
    """The intermediate rows of expert e for the given tokens, as layer_forward forms them:
    bf16 bits [len(tokens), I] of silu(Wg_e x_t) * (Wu_e x_t), one RNE rounding of the fp64
    value. Checks every row of one (hot) expert without the other experts' work."""
    return rne_bf16(_swiglu_rows(bf16_to_f64(np.asarray(x_bits)[np.asarray(tokens)]), lw, e))


def shared_expert_forward(x_bits, sw, round_inter=True):
    """The shared expert on every token, in fp64 ([readme] "Checkpoint layout update ...: BF16
    shared experts, merged online K6": one gate/up/down MLP per layer beside the routed ones).

    sw: weights of one expert in the routed layout (gate_codes [1, I, H/2], ..., tables,
    table_id [1]). Per token t: I_t = bf16(silu(Wg x_t) * (Wu x_t)) (round_inter),
    z_t = Wd I_t. Returns dict(inter=bf16 bits [T, I], z=fp64 [T, H]).
    """
    x = bf16_to_f64(x_bits)
    tab = sw.tables[int(sw.table_id[0])]
    wg = _expert_dense(sw.gate_codes[0], sw.gate_scales[0], tab)
    wu = _expert_dense(sw.up_codes[0], sw.up_scales[0], tab)
    a = _silu(x @ wg.T) * (x @ wu.T)
    del wg, wu
    inter = rne_bf16(a)
    if round_inter:
        a = bf16_to_f64(inter)
    wd = _expert_dense(sw.down_codes[0], sw.down_scales[0], tab)
    return dict(inter=inter, z=a @ wd.T)


def layer_forward(x_bits, logits, k, lw, residual_bits=None, tokens=None, round_inter=True,
                  routing=None, shared=None):
    """One routed-MoE layer forward in fp64.

    x_bits: bf16 bits [T, H]; logits fp32 [T, E]; lw: an object with gate_codes,
    gate_scales, up_codes, up_scales ([E, I, H/2], [E, I, H/32]), down_codes, down_scales
    ([E, H, I/2], [E, H, I/32]), tables [n_tables, 8] fp32 and table_id [E].

    Per pair p = (t, j) routed to expert e ([brief] decisions 4 and 6; [readme]):
        g = Wg_e x_t,  u = Wu_e x_t                       (fp64 over bf16 values)
        I_p = bf16(silu(g) * u)                           (round_inter)
        z_p = Wd_e I_p                                    (fp64)
        y_t = sum_j w[t, j] * z_(t, j)  (+ residual_t)
    tokens: optional subset of token ids for which y is computed (routing is always done
    for all tokens). routing: optional precomputed (ids, w) to use instead of route_topk.
    shared: optional shared-expert weights (see shared_expert_forward); its z_t is added to
    y_t (for the tokens computed), and the output dict gains shared_inter and shared_z.
    Returns a dict with ids, w, offsets, sorted_pair, pair_pos, inter (bf16 bits
    [T*k, I] by sorted position; rows of tokens outside ``tokens`` are zero) and y
    (fp64 [T, H]; rows outside ``tokens`` are zero) and, with a residual, x_next bits.
    """
    x = bf16_to_f64(x_bits)
    T, H = x.shape
    E = lw.table_id.shape[0]
    I = lw.gate_codes.shape[1]
    if routing is None:
        ids, w = route_topk(logits, k)
    else:
        ids, w = routing
    offsets, sorted_pair, pair_pos = permute_by_expert(ids, E)
    want = np.ones(T, bool) if tokens is None else np.isin(np.arange(T), tokens)
    inter = np.zeros((T * k, I), np.uint16)
    y = np.zeros((T, H), np.float64)
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size == 0:
            continue
        pairs = sorted_pair[rows]
        tok = pairs // k
        slot = pairs % k
        keep = want[tok]
        if not keep.any():
            continue
        rows, pairs, tok, slot = rows[keep], pairs[keep], tok[keep], slot[keep]
        tab = lw.tables[int(lw.table_id[e])]
        a = _swiglu_rows(x[tok], lw, e)
        if round_inter:
            ib = rne_bf16(a)
            inter[rows] = ib
            a = bf16_to_f64(ib)
        wd = _expert_dense(lw.down_codes[e], lw.down_scales[e], tab)
        z = a @ wd.T
        del wd
        np.add.at(y, tok, w[tok, slot][:, None] * z)
    out = dict(ids=ids, w=w, offsets=offsets, sorted_pair=sorted_pair, pair_pos=pair_pos,
               inter=inter, y=y)
    if shared is not None:
        rows = np.flatnonzero(want)
        sh = shared_expert_forward(np.asarray(x_bits)[rows], shared, round_inter=round_inter)
        y[rows] += sh["z"]
        out["shared_inter"] = np.zeros((T, sh["inter"].shape[1]), np.uint16)
        out["shared_inter"][rows] = sh["inter"]
        out["shared_z"] = np.zeros((T, H), np.float64)
        out["shared_z"][rows] = sh["z"]
    if residual_bits is not None:
        out["x_next"] = rne_bf16(bf16_to_f64(residual_bits) + y)
    return out


def stack_forward(x_bits, layers, k):
    """Free-running stack: X_{l+1} = bf16(X_l + y_l) (fp64 sum, one rounding).

    layers: iterable of (logits, lw) per layer. Returns the final bf16 bits.
    """
    xb = np.asarray(x_bits, dtype=np.uint16)
    for logits, lw in layers:
        xb = layer_forward(xb, logits, k, lw, residual_bits=xb)["x_next"]
    return xb
