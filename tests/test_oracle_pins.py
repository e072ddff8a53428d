"""Pins of the CPU oracle against facts fixed outside it: the pages' hand-worked decode
values, closed forms of the bf16 format, library routines (torch's fp32->bf16 conversion,
torch.topk, Python's sort, transformers' Mixtral experts and router) and algebraic
invariants (consistent intermediate-channel permutation). CPU only."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_bits_to_bf16(v):
    """bf16 bits of a value that is exactly representable in bf16 (the top half of fp32)."""
    b = np.array(v, dtype=np.float32).view(np.uint32)
    assert (b & 0xFFFF) == 0
    return int(b >> 16)


# ----------------------------------------------------------------------------------------------
# bf16 rounding
# ----------------------------------------------------------------------------------------------

def test_rne_matches_torch_on_fp32_values():
    g = np.random.default_rng(1)
    # wide exponent range, both signs, fp32 subnormals, and values near the overflow edge
    x = (g.standard_normal(200_000) * np.exp2(g.integers(-140, 127, 200_000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3961e38,
                                     1.1754942e-38, 1e-45, -1e-45], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.rne_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_rne_single_rounding_closed_forms():
    # 1 + 2^-8 is exactly halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert oracle.rne_bf16(np.array([1 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1 + 2^-6
    assert oracle.rne_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # just above the midpoint (not representable in fp32): rounds up; a detour through
    # fp32 would land on the tie and round down to 1.0
    assert oracle.rne_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    # bf16 subnormals are multiples of 2^-133
    assert oracle.rne_bf16(np.array([2.0 ** -133]))[0] == 0x0001
    assert oracle.rne_bf16(np.array([0.5 * 2.0 ** -133]))[0] == 0x0000      # tie -> even (0)
    assert oracle.rne_bf16(np.array([1.5 * 2.0 ** -133]))[0] == 0x0002      # tie -> even (2)
    assert oracle.rne_bf16(np.array([-127.5 * 2.0 ** -133]))[0] == 0x8080   # -> min normal
    # largest finite bf16 is (2 - 2^-7) * 2^127; the midpoint to 2^128 rounds to inf
    assert oracle.rne_bf16(np.array([(2 - 2.0 ** -7) * 2.0 ** 127]))[0] == 0x7F7F
    assert oracle.rne_bf16(np.array([(2 - 2.0 ** -8) * 2.0 ** 127]))[0] == 0x7F80
    assert oracle.rne_bf16(np.array([-0.0]))[0] == 0x8000
    assert oracle.rne_bf16(np.array([np.nan]))[0] == 0x7FC0


# ----------------------------------------------------------------------------------------------
# decode: the pages' formula on hand-built bytes
# ----------------------------------------------------------------------------------------------

def _tables():
    lloyd = np.array([0.2108, 0.4, 0.7, 0.95, 1.25, 1.6, 2.1, 2.75], np.float32)
    return {"e2m1": oracle.E2M1_TABLE, "lloyd_m0": lloyd}


def _read_golden():
    rows = []
    with open(os.path.join(GOLDEN, "decode_examples.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            tab, s, byte, ev, od = line.split()
            rows.append((tab, int(s), int(byte, 16), ev, od))
    return rows


def _golden_bits(tok):
    v = float(tok)
    if tok.startswith("-") and v == 0.0:
        return 0x8000
    return _f32_bits_to_bf16(v)


@pytest.mark.parametrize("row", _read_golden(), ids=lambda r: f"{r[0]}-s{r[1]}-{r[2]:#04x}")
def test_decode_golden_bytes(row):
    tab, s, byte, ev, od = row
    table = _tables()[tab]
    # one row of 32 codes (16 bytes), the example byte first, one scale byte
    codes = np.zeros((1, 16), np.uint8)
    codes[0, 0] = byte
    scales = np.array([[s]], np.uint8)
    bits = oracle.dequant_bf16(codes, scales, table)
    assert bits.shape == (1, 32)
    assert int(bits[0, 0]) == _golden_bits(ev), "even K (low nibble)"
    assert int(bits[0, 1]) == _golden_bits(od), "odd K (high nibble)"


def test_nibble_order_distinct_codes():
    # byte j holds codes for K = 2j (low nibble) and 2j+1 (high nibble)
    codes = np.array([[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] + [0] * 8], np.uint8)
    c = oracle.unpack_codes(codes)[0]
    np.testing.assert_array_equal(c[:16], np.arange(16))
    v = oracle.bf16_to_f64(oracle.dequant_bf16(codes, np.array([[127]], np.uint8),
                                               oracle.E2M1_TABLE))[0, :16]
    expect = np.array([0, .5, 1, 1.5, 2, 3, 4, 6]) * 1.0
    np.testing.assert_array_equal(v[:8], expect)
    np.testing.assert_array_equal(v[8:], -expect)
    assert np.signbit(v[8])


def test_e2m1_zero_codes_every_scale():
    s = np.arange(255, dtype=np.uint8)[:, None]                 # every scale byte but 255
    codes = np.tile(np.array([[0x80] + [0] * 15], np.uint8), (255, 1))
    bits = oracle.dequant_bf16(codes, s, oracle.E2M1_TABLE)
    assert (bits[:, 0] == 0x0000).all()          # code 0 -> +0
    assert (bits[:, 1] == 0x8000).all()          # code 8 -> -0
    assert (bits[:, 2:] == 0x0000).all()


def test_scale_byte_edges_closed_form():
    t = oracle.E2M1_TABLE
    def dq(byte, s):
        codes = np.zeros((1, 16), np.uint8)
        codes[0, 0] = byte
        return oracle.dequant_bf16(codes, np.array([[s]], np.uint8), t)[0, :2]
    # s = 0: 0.5 * 2^-127 = 2^-128 = 32 * 2^-133 -> subnormal bits 0x0020; 1.5*2^-127 -> 96
    assert list(dq(0x31, 0)) == [0x0020, 0x0060]
    # s = 254: low nibble 7: 6 * 2^127 overflows -> +inf; high nibble 1: 0.5 * 2^127 = 2^126
    assert list(dq(0x17, 254)) == [0x7F80, 0x7E80]
    # s = 255 -> NaN carrying the code's sign
    assert list(dq(0x81, 255)) == [0x7FC0, 0xFFC0]
    # a Lloyd magnitude with bits below bf16 precision, scaled into the subnormal range:
    # (1 + 2^-8 + 2^-20) * 2^-127 = 64.25.. * 2^-133 -> 64 units
    tab = np.array([1 + 2.0 ** -8 + 2.0 ** -20] * 8, np.float32)
    codes = np.zeros((1, 16), np.uint8)
    b = oracle.dequant_bf16(codes, np.array([[0]], np.uint8), tab)
    assert b[0, 0] == 0x0040


# ----------------------------------------------------------------------------------------------
# routing and permutation
# ----------------------------------------------------------------------------------------------

def test_topk_matches_sort_and_torch_topk():
    g = np.random.default_rng(2)
    for (T, E, k) in [(16, 4, 2), (8, 256, 8), (33, 64, 64), (5, 17, 1)]:
        logits = g.standard_normal((T, E)).astype(np.float32)
        ids, w = oracle.route_topk(logits, k)
        for t in range(T):
            brute = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(ids[t]) == brute
        tv, ti = torch.topk(torch.from_numpy(logits), k, dim=1, sorted=True)
        np.testing.assert_array_equal(ids, ti.numpy())


def test_topk_gate_weights_match_mixtral_router():
    from transformers import MixtralConfig
    from transformers.models.mixtral.modeling_mixtral import MixtralTopKRouter
    g = np.random.default_rng(3)
    T, E, k = 12, 256, 8
    logits = g.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route_topk(logits, k)
    cfg = MixtralConfig(hidden_size=E, num_local_experts=E, num_experts_per_tok=k)
    r = MixtralTopKRouter(cfg).double()
    with torch.no_grad():
        r.weight.copy_(torch.eye(E, dtype=torch.float64))   # router logits = the given logits
        # the router's softmax runs in fp32 (.float()); feed fp64 logits and compare at fp32
        _, scores, idx = r(torch.from_numpy(logits.astype(np.float64)))
    np.testing.assert_array_equal(ids, idx.numpy())
    np.testing.assert_allclose(w, scores.double().numpy(), rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)


def test_sigmoid_gate_closed_forms():
    """Sigmoid gating: the k largest logits, s_j = 1/(1 + exp(-l_j)), renormalised."""
    # selected logits (x, -x): s = (sigmoid(x), 1 - sigmoid(x)) already sums to 1
    x = 0.7
    ids, w = oracle.route_topk(np.array([[x, -3.0, -x, -5.0]], np.float32), 2, gating="sigmoid")
    assert ids.tolist() == [[0, 2]]
    xf = float(np.float32(x))
    np.testing.assert_allclose(w[0], [1 / (1 + np.exp(-xf)), 1 / (1 + np.exp(xf))], rtol=1e-15)
    # logits (ln 3, 0): s = (3/4, 1/2) -> w = (0.6, 0.4)
    l3 = np.float32(np.log(3.0))
    _, w = oracle.route_topk(np.array([[0.0, l3, -1.0]], np.float32), 2, gating="sigmoid")
    s3 = 1 / (1 + np.exp(-float(l3)))
    np.testing.assert_allclose(w[0], [s3 / (s3 + 0.5), 0.5 / (s3 + 0.5)], rtol=1e-15)
    np.testing.assert_allclose(w[0], [0.6, 0.4], rtol=1e-7)
    # equal logits: uniform weights; the same experts as softmax gating
    _, w = oracle.route_topk(np.full((1, 8), 0.25, np.float32), 4, gating="sigmoid")
    np.testing.assert_allclose(w, 0.25, rtol=1e-15)
    g = np.random.default_rng(4)
    logits = g.standard_normal((6, 64)).astype(np.float32)
    i1, _ = oracle.route_topk(logits, 8)
    i2, w2 = oracle.route_topk(logits, 8, gating="sigmoid")
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(w2.sum(1), 1.0, rtol=1e-14)


def test_router_logits_closed_forms():
    """Router logits are the plain product of bf16 activations and bf16 router rows."""
    T, H, E = 3, 64, 5
    one = oracle.rne_bf16(np.ones((T, H)))
    rows = oracle.rne_bf16(np.arange(E, dtype=np.float64)[:, None] * np.ones((1, H)))
    np.testing.assert_array_equal(oracle.router_logits(one, rows), np.arange(E)[None, :] * H * np.ones((T, 1)))
    # a one-hot activation row picks one column of the router
    g = np.random.default_rng(8)
    wr = oracle.rne_bf16(g.standard_normal((E, H)))
    x = np.zeros((1, H))
    x[0, 17] = 1.0
    np.testing.assert_array_equal(oracle.router_logits(oracle.rne_bf16(x), wr)[0],
                                  oracle.bf16_to_f64(wr)[:, 17])


def test_router_and_sigmoid_gate_match_glm4_moe_router():
    """Against transformers' GLM-4.5 MoE router with one group, no score bias, renormalised
    top-k and scaling 1: logits (fp32 there), expert sets and gate weights."""
    from transformers import Glm4MoeConfig
    from transformers.models.glm4_moe.modeling_glm4_moe import Glm4MoeTopkRouter
    g = np.random.default_rng(5)
    T, H, E, k = 12, 128, 256, 8
    x = oracle.rne_bf16(g.standard_normal((T, H)))
    wr = oracle.rne_bf16(0.1 * g.standard_normal((E, H)))
    logits = oracle.router_logits(x, wr)
    ids, w = oracle.route_topk(logits.astype(np.float32), k, gating="sigmoid")
    cfg = Glm4MoeConfig(hidden_size=H, n_routed_experts=E, num_experts_per_tok=k, n_group=1,
                        topk_group=1, norm_topk_prob=True, routed_scaling_factor=1.0)
    r = Glm4MoeTopkRouter(cfg)
    with torch.no_grad():
        r.weight.copy_(torch.from_numpy(oracle.bf16_to_f64(wr)).float())
        rl, tw, ti = r(torch.from_numpy(oracle.bf16_to_f64(x)).float())
    np.testing.assert_allclose(logits, rl.double().numpy(), rtol=1e-5, atol=1e-5)
    for t in range(T):
        ref = dict(zip(ti[t].tolist(), tw[t].double().tolist()))
        assert sorted(ref) == sorted(ids[t].tolist())
        np.testing.assert_allclose(w[t], [ref[e] for e in ids[t]], rtol=2e-6, atol=1e-7)


def test_topk_ties_and_signed_zero():
    logits = np.array([[1.0, 3.0, 3.0, -0.0, 0.0, 3.0]], np.float32)
    ids, w = oracle.route_topk(logits, 5)
    # equal values: lower id first; +0 ranks above -0 (IEEE totalOrder)
    assert list(ids[0]) == [1, 2, 5, 0, 4]
    np.testing.assert_allclose(w[0, :3], w[0, 0])


def test_permute_is_stable_counting_sort():
    g = np.random.default_rng(4)
    for (T, k, E) in [(16, 2, 4), (8, 8, 256), (300, 8, 64), (1, 1, 1)]:
        ids = g.integers(0, E, (T, k)).astype(np.int32)
        off, sp, pp = oracle.permute_by_expert(ids, E)
        flat = ids.ravel()
        brute = sorted(range(T * k), key=lambda p: (flat[p], p))
        assert list(sp) == brute
        assert off[0] == 0 and off[E] == T * k
        for e in range(E):
            assert off[e + 1] - off[e] == (flat == e).sum()
        np.testing.assert_array_equal(sp[pp], np.arange(T * k))


def test_permute_invalid_ids_go_last():
    ids = np.array([[3, -1], [0, 7], [2, 0]], np.int32)
    off, sp, pp = oracle.permute_by_expert(ids, 4)
    assert off[4] == 4                      # 4 valid pairs
    assert list(sp) == [2, 5, 4, 0, 1, 3]   # e0: p2, p5; e2: p4; e3: p0; invalid: p1, p3


# ----------------------------------------------------------------------------------------------
# the layer: against transformers' Mixtral experts (an independent SwiGLU MoE implementation)
# ----------------------------------------------------------------------------------------------

def _mixtral_forward(x, ids, w, gate, up, down):
    from transformers import MixtralConfig
    from transformers.models.mixtral.modeling_mixtral import MixtralExperts
    E, I, H = gate.shape
    cfg = MixtralConfig(hidden_size=H, intermediate_size=I, num_local_experts=E,
                        num_experts_per_tok=ids.shape[1], hidden_act="silu")
    m = MixtralExperts(cfg).double()
    with torch.no_grad():
        m.gate_up_proj.copy_(torch.from_numpy(np.concatenate([gate, up], axis=1)))
        m.down_proj.copy_(torch.from_numpy(down))
        y = m(torch.from_numpy(x), torch.from_numpy(ids.astype(np.int64)), torch.from_numpy(w))
    return y.numpy()


def _dense(lw, perm_back=False):
    E = lw.table_id.shape[0]
    g, u, d = [], [], []
    for e in range(E):
        tab = lw.tables[lw.table_id[e]]
        ge = oracle.bf16_to_f64(oracle.dequant_bf16(lw.gate_codes[e], lw.gate_scales[e], tab))
        ue = oracle.bf16_to_f64(oracle.dequant_bf16(lw.up_codes[e], lw.up_scales[e], tab))
        de = oracle.bf16_to_f64(oracle.dequant_bf16(lw.down_codes[e], lw.down_scales[e], tab))
        if perm_back:   # stored channel n holds logical channel perms[e, n]
            inv = np.argsort(lw.perms[e])
            ge, ue, de = ge[inv], ue[inv], de[:, inv]
        g.append(ge), u.append(ue), d.append(de)
    return np.stack(g), np.stack(u), np.stack(d)


@pytest.fixture(scope="module")
def tiny():
    c = synth.WORKLOADS["tiny"]
    lw = synth.make_layer(1, c.E, c.H, c.I)
    x = synth.make_x(1, c.T, c.H)
    logits = synth.make_logits(1, c.T, c.E)
    return c, lw, x, logits


def test_layer_matches_mixtral_experts(tiny):
    c, lw, x, logits = tiny
    out = oracle.layer_forward(x, logits, c.k, lw, round_inter=False)
    g, u, d = _dense(lw)
    ref = _mixtral_forward(oracle.bf16_to_f64(x), out["ids"], out["w"], g, u, d)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)


def test_layer_all_experts_selected_matches_mixtral(tiny):
    c, lw, x, logits = tiny
    out = oracle.layer_forward(x, logits, c.E, lw, round_inter=False)     # k = E
    g, u, d = _dense(lw)
    ref = _mixtral_forward(oracle.bf16_to_f64(x), out["ids"], out["w"], g, u, d)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)


def test_layer_dense_bruteforce_scatter(tiny):
    """Every expert on every token, gate values scattered into a zero [T, E] matrix."""
    c, lw, x, logits = tiny
    out = oracle.layer_forward(x, logits, c.k, lw, round_inter=False)
    g, u, d = _dense(lw)
    xf = torch.from_numpy(oracle.bf16_to_f64(x))
    G = np.zeros((c.T, c.E))
    for t in range(c.T):
        G[t, out["ids"][t]] = out["w"][t]
    y = torch.zeros(c.T, c.H, dtype=torch.float64)
    for e in range(c.E):
        h = torch.nn.functional.silu(xf @ torch.from_numpy(g[e]).T) * (xf @ torch.from_numpy(u[e]).T)
        y += torch.from_numpy(G[:, e:e + 1]) * (h @ torch.from_numpy(d[e]).T)
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-14)


def test_layer_intermediate_is_bf16_of_swiglu(tiny):
    c, lw, x, logits = tiny
    a = oracle.layer_forward(x, logits, c.k, lw, round_inter=True)
    b = oracle.layer_forward(x, logits, c.k, lw, round_inter=False)
    rel = np.linalg.norm(a["y"] - b["y"], axis=1) / np.linalg.norm(b["y"], axis=1)
    assert rel.max() < 4e-3                     # bf16 rounding of I only
    assert (a["inter"] != 0).any()


def test_layer_tokens_subset_equals_full(tiny):
    c, lw, x, logits = tiny
    full = oracle.layer_forward(x, logits, c.k, lw)
    sub = oracle.layer_forward(x, logits, c.k, lw, tokens=[3, 7])
    np.testing.assert_array_equal(sub["y"][[3, 7]], full["y"][[3, 7]])


# ----------------------------------------------------------------------------------------------
# consistent intermediate-channel permutation ("Round 7" brief, decision 7)
# ----------------------------------------------------------------------------------------------

def _relayout_block_perm(lw, perms):
    """Bytes of the same experts with intermediate channels permuted: stored channel n takes
    logical channel perms[e, n]. perms must move whole 32-blocks / permute within blocks so the
    down K-blocks (scales) stay whole. Works on unpacked codes (low nibble = even K)."""
    import copy
    q = copy.deepcopy(lw)
    E = lw.table_id.shape[0]
    for e in range(E):
        p = perms[e]
        q.gate_codes[e] = lw.gate_codes[e][p]
        q.gate_scales[e] = lw.gate_scales[e][p]
        q.up_codes[e] = lw.up_codes[e][p]
        q.up_scales[e] = lw.up_scales[e][p]
        c = oracle.unpack_codes(lw.down_codes[e])[:, p]
        q.down_codes[e] = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        q.down_scales[e] = lw.down_scales[e][:, p[::32] // 32]
    return q


def test_block_permutation_relayout_invariance(tiny):
    c, lw, x, logits = tiny
    g = np.random.default_rng(5)
    perms = np.stack([np.concatenate([b * 32 + g.permutation(32) for b in g.permutation(c.I // 32)])
                      for _ in range(c.E)])
    q = _relayout_block_perm(lw, perms)
    a = oracle.layer_forward(x, logits, c.k, lw)
    b = oracle.layer_forward(x, logits, c.k, q)
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-13, atol=1e-15)
    # I is permuted per row: same multiset of values
    np.testing.assert_array_equal(np.sort(a["inter"], 1), np.sort(b["inter"], 1))


def test_random_permutation_baked_in_equals_unpermuted_dense():
    """Weights drawn, permuted (stored channel n = logical perms[e, n]) and then encoded:
    the routed forward on the stored bytes equals the dense forward on the un-permuted
    dequantised weights (exact up to fp64 re-association)."""
    E, H, I, k, T = 4, 256, 128, 2, 16
    lw = synth.make_layer(1, E, H, I, permute="random", e2m1_experts=(2,))
    x = synth.make_x(1, T, H)
    logits = synth.make_logits(1, T, E)
    out = oracle.layer_forward(x, logits, k, lw, round_inter=False)
    g, u, d = _dense(lw, perm_back=True)
    ref = _mixtral_forward(oracle.bf16_to_f64(x), out["ids"], out["w"], g, u, d)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)
    assert (lw.perms[0] != np.arange(I)).any()


def test_stack_residual_rounding(tiny):
    c, lw, x, logits = tiny
    one = oracle.layer_forward(x, logits, c.k, lw, residual_bits=x)
    ref = oracle.rne_bf16(oracle.bf16_to_f64(x) + one["y"])
    np.testing.assert_array_equal(one["x_next"], ref)
    two = oracle.stack_forward(x, [(logits, lw), (logits, lw)], c.k)
    step = oracle.layer_forward(one["x_next"], logits, c.k, lw, residual_bits=one["x_next"])
    np.testing.assert_array_equal(two, step["x_next"])


def _plain_bf16(v):
    """fp64 values -> the nearest bf16 values, ties to even (normal range): 8 significant bits,
    written from the format (frexp gives v = m 2^e with 1/2 <= |m| < 1)."""
    m, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def _plain_decode(codes, scales, table):
    """[card] "Contents" / "Codes are indices into the per-layer grid", element by element:
    code c of byte k // 2 (low nibble for even k), w = (-1)^(bit 3) table[c & 7] 2^(s - 127)
    with s the scale byte of k // 32, rounded once to bf16."""
    N, half = codes.shape
    out = np.empty((N, 2 * half))
    for kk in range(2 * half):
        b = codes[:, kk // 2].astype(np.int64)
        c = (b >> 4) if kk % 2 else (b & 15)
        mag = np.asarray(table, np.float32).astype(np.float64)[c & 7]
        out[:, kk] = np.where(c & 8, -1.0, 1.0) * mag * 2.0 ** (scales[:, kk // 32].astype(np.int64) - 127)
    return _plain_bf16(out)


def test_stack_two_distinct_layers_against_a_plain_loop():
    """Two layers with their own grid, weights, logits and E2M1 expert, X carried in bf16:
    the oracle's free-running stack against a loop written from the definitions (full sort
    for the top-k, softmax over the k, element-wise decode, SwiGLU, gate-weighted sum,
    X + y rounded to bf16 once). Weights N(0, 0.2), so that y is comparable to X and
    swapping the two layers changes most of the result."""
    T, H, I, E, k = 6, 128, 64, 5, 2
    layers = [(synth.make_logits(71, T, E, layer=l),
               synth.make_layer(71, E, H, I, layer=l, e2m1_experts=(l,), sigma=0.2))
              for l in range(2)]
    assert not np.array_equal(layers[0][1].tables[0], layers[1][1].tables[0])
    x0 = synth.make_x(71, T, H)
    got = oracle.bf16_to_f64(oracle.stack_forward(x0, layers, k))
    X = (x0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for logits, lw in layers:
        Y = np.zeros((T, H))
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            lg = np.array([float(logits[t, e]) for e in order])
            p = np.exp(lg - lg.max())
            p /= p.sum()
            for j, e in enumerate(order):
                tab = lw.tables[int(lw.table_id[e])]
                wg = _plain_decode(lw.gate_codes[e], lw.gate_scales[e], tab)
                wu = _plain_decode(lw.up_codes[e], lw.up_scales[e], tab)
                wd = _plain_decode(lw.down_codes[e], lw.down_scales[e], tab)
                g, u = wg @ X[t], wu @ X[t]
                a = _plain_bf16(g / (1.0 + np.exp(-g)) * u)
                Y[t] += p[j] * (wd @ a)
        X = _plain_bf16(X + Y)
    ulp = np.ldexp(1.0, np.frexp(np.abs(X))[1] - 8)
    assert np.all(np.abs(got - X) <= ulp)
    assert np.mean(got == X) >= 0.99
    swapped = oracle.bf16_to_f64(oracle.stack_forward(x0, layers[::-1], k))
    assert np.mean(swapped == got) < 0.5


# ----------------------------------------------------------------------------------------------
# shared expert
# ----------------------------------------------------------------------------------------------

def _with_shared_as_expert(lw, sw):
    """The routed layer with the shared expert appended as expert E (same table set)."""
    assert np.array_equal(lw.tables, sw.tables)
    cat = lambda a, b: np.concatenate([a, b], axis=0)
    return synth.LayerWeights(cat(lw.gate_codes, sw.gate_codes), cat(lw.gate_scales, sw.gate_scales),
                              cat(lw.up_codes, sw.up_codes), cat(lw.up_scales, sw.up_scales),
                              cat(lw.down_codes, sw.down_codes), cat(lw.down_scales, sw.down_scales),
                              lw.tables, cat(lw.table_id, sw.table_id))


def test_shared_expert_is_a_routed_expert_with_weight_one(tiny):
    """Adding the shared expert equals routing every token to one more expert, the shared one,
    with gate weight 1 (through the routed path pinned above)."""
    c, lw, x, logits = tiny
    sw = synth.make_shared(1, c.H, c.I)
    out = oracle.layer_forward(x, logits, c.k, lw, shared=sw, residual_bits=x)
    ids = np.concatenate([out["ids"], np.full((c.T, 1), c.E, np.int32)], axis=1)
    w = np.concatenate([out["w"], np.ones((c.T, 1))], axis=1)
    aug = oracle.layer_forward(x, None, c.k + 1, _with_shared_as_expert(lw, sw), routing=(ids, w),
                               residual_bits=x)
    np.testing.assert_allclose(out["y"], aug["y"], rtol=1e-12, atol=1e-14)
    shared_rows = aug["pair_pos"].reshape(c.T, c.k + 1)[:, c.k]
    np.testing.assert_array_equal(out["shared_inter"], aug["inter"][shared_rows])
    assert not np.array_equal(out["y"], oracle.layer_forward(x, logits, c.k, lw)["y"])


def test_shared_expert_matches_glm4_moe_mlp(tiny):
    """Against transformers' GLM-4.5 MoE dense MLP (its shared-expert module) on the dequantized
    weights, in fp64 without the bf16 rounding of the intermediate."""
    import torch
    from transformers import Glm4MoeConfig
    from transformers.models.glm4_moe.modeling_glm4_moe import Glm4MoeMLP
    c, _, x, _ = tiny
    sw = synth.make_shared(1, c.H, c.I)
    g, u, d = _dense(sw)
    cfg = Glm4MoeConfig(hidden_size=c.H, intermediate_size=c.I, hidden_act="silu")
    mlp = Glm4MoeMLP(cfg, intermediate_size=c.I).double()
    with torch.no_grad():
        mlp.gate_proj.weight.copy_(torch.from_numpy(g[0]))
        mlp.up_proj.weight.copy_(torch.from_numpy(u[0]))
        mlp.down_proj.weight.copy_(torch.from_numpy(d[0]))
        ref = mlp(torch.from_numpy(oracle.bf16_to_f64(x))).numpy()
    z = oracle.shared_expert_forward(x, sw, round_inter=False)["z"]
    np.testing.assert_allclose(z, ref, rtol=1e-12, atol=1e-14)
    # with the intermediate rounded, the stored inter is bf16 of SwiGLU
    sh = oracle.shared_expert_forward(x, sw)
    a = oracle.bf16_to_f64(x) @ g[0].T
    np.testing.assert_array_equal(sh["inter"], oracle.rne_bf16(a / (1 + np.exp(-a)) *
                                                             (oracle.bf16_to_f64(x) @ u[0].T)))


def test_shared_expert_token_subset(tiny):
    c, lw, x, logits = tiny
    sw = synth.make_shared(1, c.H, c.I)
    full = oracle.layer_forward(x, logits, c.k, lw, shared=sw)
    part = oracle.layer_forward(x, logits, c.k, lw, shared=sw, tokens=[3, 11])
    np.testing.assert_array_equal(part["y"][[3, 11]], full["y"][[3, 11]])
    np.testing.assert_array_equal(part["shared_z"][[3, 11]], full["shared_z"][[3, 11]])
    assert not part["y"][0].any()


# ----------------------------------------------------------------------------------------------
# encoding (quantizer) and the weighted grid fit
# ----------------------------------------------------------------------------------------------

def _bits(a):
    return synth.bf16_bits_from_f32(np.asarray(a, np.float32))


def test_block_scale_closed_forms():
    g = synth.lloyd_grid(1, 0)
    gmax = float(g[7])
    row = np.zeros((6, 32), np.float32)
    row[0, 5] = 6.0                       # E2M1: amax = gmax * 2^0 exactly
    row[1, 5] = np.float32(6.0 * 2 ** -9)                  # amax = gmax * 2^-9
    row[2, 7] = np.nextafter(np.float32(6.0 * 2 ** -9), np.float32(1))  # just above (bf16 below)
    row[3, 0] = np.inf
    row[4, 3] = np.nan
    bits = _bits(row)
    bits[2, 7] = _bits([6.0 * 2 ** -9])[0] + 1             # the next bf16 above 6 * 2^-9
    s = oracle.block_scale_bytes(bits, 6.0)[:, 0]
    assert s.tolist() == [127, 118, 119, 255, 255, 0]
    # the smallest e with gmax * 2^e >= amax, on the Lloyd grid's gmax
    w = oracle.bf16_to_f64(_bits(np.random.default_rng(2).standard_normal((50, 32)) * 0.02))
    sb = oracle.block_scale_bytes(_bits(w), gmax)[:, 0].astype(int) - 127
    amax = np.abs(w).max(1)
    assert np.all(gmax * 2.0 ** sb >= amax) and np.all(gmax * 2.0 ** (sb - 1) < amax)
    # clamps: far below 2^-127 * gmax gets byte 0
    tiny = np.zeros((1, 32), np.uint16)
    tiny[0, 0] = 1                                          # the smallest bf16 subnormal
    assert oracle.block_scale_bytes(tiny, gmax)[0, 0] == 0


def _brute_codes(w_bits, scales, table):
    """Nearest of the 16 codes, each decoded by the pinned decoder at the block's scale; ties
    to the lower magnitude, then to the sign of w (negative only for w < 0)."""
    w = oracle.bf16_to_f64(w_bits)
    N, K = w.shape
    values = {}
    out = np.empty((N, K), np.uint8)
    for n in range(N):
        for k in range(K):
            s = int(scales[n, k // 32])
            if s not in values:
                values[s] = [oracle.dequant_f64_exact(np.full((1, 16), c | (c << 4), np.uint8),
                                                      np.array([[s]], np.uint8), table)[0, 0]
                             for c in range(16)]
            vals = values[s]
            neg = bool(w[n, k] < 0)
            out[n, k] = min(range(16), key=lambda c: (abs(w[n, k] - vals[c]), c & 7,
                                                      bool(c & 8) != neg))
    return out


@pytest.mark.parametrize("which", ["lloyd", "e2m1"])
def test_rtn_encode_matches_bruteforce_and_decoder(which):
    table = synth.lloyd_grid(1, 0) if which == "lloyd" else oracle.E2M1_TABLE
    g = np.random.default_rng(3)
    w = (g.standard_normal((6, 128)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                                         # all-zero block
    w[1, 32:64] = (np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4) *
                   np.tile([1, -1], 16))                    # E2M1 midpoints: exact ties
    w[2, 0] = -0.0
    bits = _bits(w)
    codes, scales = oracle.rtn_encode(bits, table)
    c4 = oracle.unpack_codes(codes)
    dec = oracle.dequant_f64_exact
    assert np.array_equal(scales, oracle.block_scale_bytes(bits, table[7]))
    want = _brute_codes(bits, scales, table)
    np.testing.assert_array_equal(c4, want)
    # round trip: each weight within half the largest gap (or the top overshoot) of the grid
    wh = dec(codes, scales, table)
    tab = np.asarray(table, np.float64)
    half = max(np.max(np.diff(tab)) / 2, tab[0])
    e = np.repeat(scales.astype(int) - 127, 32, axis=1)
    assert np.all(np.abs(oracle.bf16_to_f64(bits) - wh) <= half * 2.0 ** e + 1e-300)
    if which == "e2m1":
        # midpoints tie to the lower magnitude
        np.testing.assert_array_equal(c4[1, 32:40] & 7, [0, 1, 2, 3, 4, 5, 6, 7])


@pytest.mark.parametrize("which", ["lloyd", "e2m1"])
def test_rtn_encode_matches_generator_encoder(which):
    """The input generator's C encoder (written separately, on fp32 input) agrees on weights
    that are bf16 values."""
    table = synth.lloyd_grid(2, 1) if which == "lloyd" else synth.E2M1_GRID
    w = oracle.bf16_to_f64(_bits(synth.normal_matrix(synth.key(9, 2), 16, 512))).astype(np.float32)
    c1, s1 = synth.rtn_encode(w, table)
    c2, s2 = oracle.rtn_encode(_bits(w), table)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_reconstruction_error_and_arm_selection():
    g = np.random.default_rng(6)
    lloyd = synth.lloyd_grid(1, 0)
    gauss = _bits(g.standard_normal((32, 256)) * 0.02)
    # weights exactly on the E2M1 grid (block maxima 6 * 2^e): E2M1 reconstructs them exactly
    on = (oracle.E2M1_TABLE[g.integers(0, 8, (32, 256))] * np.where(g.random((32, 256)) < .5, -1, 1)
          * 2.0 ** -8).astype(np.float32)
    on[:, ::32] = 6 * 2.0 ** -8
    on = _bits(on)
    errs = {}
    for name, w in (("gauss", gauss), ("on", on)):
        for arm, tab in ((0, lloyd), (1, oracle.E2M1_TABLE)):
            c, s = oracle.rtn_encode(w, tab)
            e = oracle.reconstruction_sq_error(w, c, s, tab)
            wh = oracle.bf16_to_f64(oracle.dequant_bf16(c, s, tab))
            np.testing.assert_allclose(e, ((oracle.bf16_to_f64(w) - wh) ** 2).sum(1), rtol=1e-15)
            errs[name, arm] = e.sum()
    assert errs["on", 1] == 0.0 and errs["on", 0] > 0
    assert errs["gauss", 0] < errs["gauss", 1]             # the fitted grid wins on Gaussians
    ids = oracle.select_arms([errs["gauss", 0], errs["on", 0], 1.0],
                             [errs["gauss", 1], errs["on", 1], 1.0])
    assert ids.tolist() == [0, 1, 0]                       # a tie keeps the fitted grid


def test_lloyd_stats_closed_form():
    tab = oracle.E2M1_TABLE
    w = np.zeros((1, 64), np.float32)
    w[0, :4] = [6.0, 1.0, -1.0, 0.6]                    # e = 0: ratios 6, 1, 1, 0.6 (-> 0.5)
    w[0, 32:35] = [24.0, -4.0, 1.0]                     # e = 2: ratios 6, 1, 0.25 (tie -> 0)
    st = oracle.lloyd_stats(_bits(w), tab)
    r06 = float(oracle.bf16_to_f64(_bits([0.6]))[0])
    # level 0 holds 28 zeros at weight 1, 29 zeros and 0.25 at weight 16
    np.testing.assert_allclose(st[:, 0], [16 * 0.25, 28 + 30 * 16, 16 * 0.25 ** 2], rtol=1e-15)
    np.testing.assert_allclose(st[:, 1], [r06, 1, (r06 - 0.5) ** 2], rtol=1e-15)
    np.testing.assert_allclose(st[:, 2], [2 + 16, 2 + 16, 0], rtol=1e-15)
    np.testing.assert_allclose(st[:, 7], [6 + 16 * 6, 1 + 16, 0], rtol=1e-15)


def test_weighted_lloyd_step_matches_sklearn_kmeans():
    """One update equals one iteration of scikit-learn's weighted k-means (Lloyd) on the
    ratios, started from the table, with the (2^e)^2 weights as sample weights."""
    from sklearn.cluster import KMeans
    g = np.random.default_rng(7)
    w = g.standard_normal((24, 256)) * 0.02 * np.exp(g.standard_normal((24, 1)))
    bits = _bits(w)
    tab = synth.lloyd_grid(1, 0)
    st = oracle.lloyd_stats(bits, tab)
    assert np.all(st[1] > 0)                              # no empty cell (sklearn would move it)
    new = oracle.lloyd_update(tab, st)
    e = np.repeat(oracle.block_scale_bytes(bits, tab[7]).astype(int) - 127, 32, axis=1)
    r = (np.abs(oracle.bf16_to_f64(bits)) * 2.0 ** -e).reshape(-1, 1)
    km = KMeans(n_clusters=8, init=np.asarray(tab, np.float64).reshape(-1, 1), n_init=1,
                max_iter=1, algorithm="lloyd", tol=0.0)
    km.fit(r, sample_weight=(2.0 ** (2 * e)).ravel())
    np.testing.assert_allclose(new, np.sort(km.cluster_centers_.ravel()).astype(np.float32),
                               rtol=1e-6)
    # on its fixed ratios (exponents of the starting table) the weighted distortion of the
    # fit never goes up, round by round
    d = [st[2].sum()]
    for it in range(1, 5):
        fitted = oracle.fit_grid([bits], tab, it)
        d.append(oracle.lloyd_stats(bits, fitted, gmax=tab[7])[2].sum())
    assert all(b <= a * (1 + 1e-12) for a, b in zip(d, d[1:])) and d[-1] < d[0]
