"""GPU parity of libmoeq against the fp64 CPU oracle, through the C ABI.

Bars: routing ids, the permutation and every dequantised weight bit-exact; gate values to
fp32 rounding; the intermediate to bf16 rounding; layer outputs within 5e-3 row-relative
(||y_gpu - y_ref|| / ||y_ref|| per token row, y_ref in fp64 over the same bf16 weights and
activations)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from inter_check import check_inter

pytestmark = pytest.mark.gpu

ROW_REL_TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import codebook_quantized_moe_amd  # noqa: F401  (fails loudly when not built)


@pytest.fixture(params=["decode", "prefill"])
def path(request, monkeypatch):
    """Run the projections through the decode kernels or the prefill kernels."""
    monkeypatch.setenv("MOEQ_FORCE_PATH", request.param)
    return request.param


def _mq():
    import codebook_quantized_moe_amd as mq
    return mq


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def u16(t):
    return host(t).view(np.uint16)


def row_rel(y_gpu_bits, y_ref):
    g = oracle.bf16_to_f64(y_gpu_bits)
    num = np.linalg.norm(g - y_ref, axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    return num / np.maximum(den, 1e-300)


def run_layer(lw, x_bits, logits, k, residual=False):
    mq = _mq()
    T, H = x_bits.shape
    E, I = lw.table_id.shape[0], lw.gate_codes.shape[1]
    w = mq.DeviceWeights.from_host(lw)
    L = mq.MoeLayer(T, H, I, E, k)
    x = dev(x_bits.view(np.int16))
    y = L.forward(x, dev(logits), w, residual=x if residual else None)
    torch.cuda.synchronize()
    return dict(ids=host(L.topk_ids).reshape(T, k), w=host(L.topk_w).reshape(T, k),
                offsets=host(L.offsets), sorted_pair=host(L.sorted_pair),
                pair_pos=host(L.pair_pos), inter=u16(L.inter), y=u16(y))


def unslot(inter, I):
    return inter[:, _mq().inter_slot(np.arange(I))]


def check_layer(out, ref, k, lw, x, tokens=None, inter_rows=True):
    """Routing and permutation bit-exact, gate values to fp32 rounding, the intermediate
    element-wise (inter_check), y within the row-relative bar; rows of `tokens` (default all)."""
    np.testing.assert_array_equal(out["ids"], ref["ids"])
    np.testing.assert_allclose(out["w"], ref["w"], rtol=2e-6, atol=1e-7)
    np.testing.assert_array_equal(out["offsets"], ref["offsets"])
    np.testing.assert_array_equal(out["sorted_pair"], ref["sorted_pair"])
    np.testing.assert_array_equal(out["pair_pos"], ref["pair_pos"])
    T = out["y"].shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    if inter_rows:
        I = ref["inter"].shape[1]
        rows = ref["pair_pos"].reshape(T, k)[toks].ravel()
        pairs = ref["sorted_pair"][rows]
        check_inter(unslot(out["inter"], I)[rows], ref["inter"][rows], pairs // k,
                    ref["ids"].ravel()[pairs], x, lw, label=f"{T} tokens")
    rel = row_rel(out["y"][toks], ref["y"][toks])
    assert np.all(np.isfinite(rel)) and rel.max() <= ROW_REL_TOL, rel.max()
    return rel.max()


# ----------------------------------------------------------------------------------------------
# dequant: bit-exact for every scale byte and every code, several tables
# ----------------------------------------------------------------------------------------------

def test_debug_dequant_bitexact_all_bytes_and_scales():
    mq = _mq()
    E, N, K = 3, 256, 128
    g = np.random.default_rng(11)
    codes = g.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    codes[:, :, :16] = np.arange(256, dtype=np.uint8).reshape(16, 16)[np.arange(N) % 16]
    scales = np.empty((E, N, K // 32), np.uint8)
    scales[:] = (np.arange(N)[:, None] + np.arange(K // 32)[None, :] * 64) % 256
    odd = np.array([0.0, 1e-40, 2.0 ** -126, 1 + 2.0 ** -8 + 2.0 ** -20, 1 + 3 * 2.0 ** -8,
                    3.0e38, 1.99609375, 0.2108], np.float32)
    tables = np.stack([synth.lloyd_grid(1, 0), synth.E2M1_GRID, odd]).astype(np.float32)
    table_id = np.array([0, 1, 2], np.uint8)
    out = torch.empty((E, N, K), dtype=torch.int16, device="cuda")
    mq.moeq_debug_dequant(dev(codes), dev(scales), E, N, K, tables, dev(table_id), out)
    got = u16(out)
    for e in range(E):
        ref = oracle.dequant_bf16(codes[e], scales[e], tables[table_id[e]])
        mism = np.argwhere(got[e] != ref)
        assert mism.size == 0, (e, mism[:5], got[e][tuple(mism[0])], ref[tuple(mism[0])])


def test_debug_dequant_invalid_table_id_is_nan():
    mq = _mq()
    E, N, K = 2, 16, 64
    codes = np.full((E, N, K // 2), 0x31, np.uint8)
    scales = np.full((E, N, K // 32), 127, np.uint8)
    tables = np.stack([synth.E2M1_GRID]).astype(np.float32)
    out = torch.empty((E, N, K), dtype=torch.int16, device="cuda")
    mq.moeq_debug_dequant(dev(codes), dev(scales), E, N, K, tables,
                          dev(np.array([0, 1], np.uint8)), out)
    v = oracle.bf16_to_f64(u16(out))
    assert np.all(v[0, :, 0::2] == 0.5) and np.all(v[0, :, 1::2] == 1.5)
    assert np.all(np.isnan(v[1]))


# ----------------------------------------------------------------------------------------------
# routing and permutation: bit-exact
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,zipf", [(16, 4, 2, None), (8, 256, 8, None), (2048, 256, 8, 1.0),
                                        (33, 64, 64, None), (1, 17, 1, None), (5, 256, 256, None)])
def test_route_topk_bitexact(T, E, k, zipf):
    mq = _mq()
    logits = synth.make_logits(7, T, E, zipf_s=zipf)
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    mq.moeq_route_topk(dev(logits), T, E, k, ids, w)
    rid, rw = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(host(ids).reshape(T, k), rid)
    np.testing.assert_allclose(host(w).reshape(T, k), rw, rtol=2e-6, atol=1e-7)


def test_route_ties_and_signed_zero():
    mq = _mq()
    logits = np.array([[1.0, 3.0, 3.0, -0.0, 0.0, 3.0] + [-5.0] * 58,
                       [np.float32(-np.inf)] * 60 + [2.0, 2.0, -1.0, 2.0]], np.float32)
    T, E, k = 2, 64, 5
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    mq.moeq_route_topk(dev(logits), T, E, k, ids, w)
    rid, _ = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(host(ids).reshape(T, k), rid)


@pytest.mark.parametrize("T,E,k,zipf", [(16, 4, 2, None), (8, 256, 8, None), (2048, 256, 8, 1.0),
                                        (33, 64, 64, None), (1, 17, 1, None), (5, 256, 256, None)])
def test_route_sigmoid_gating(T, E, k, zipf):
    mq = _mq()
    logits = synth.make_logits(8, T, E, zipf_s=zipf)
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    mq.moeq_route_topk(dev(logits), T, E, k, ids, w, gating=mq.MOEQ_GATING_SIGMOID_TOPK)
    rid, rw = oracle.route_topk(logits, k, "sigmoid")
    np.testing.assert_array_equal(host(ids).reshape(T, k), rid)
    np.testing.assert_allclose(host(w).reshape(T, k), rw, rtol=2e-6, atol=1e-7)


def test_route_sigmoid_gating_extreme_logits():
    """Selected logits far below zero (sigmoid underflows fp32 below about -104), straddling
    the sign, and far above zero (sigmoid rounds to one): weights stay finite and exact."""
    mq = _mq()
    E, k = 64, 8
    g = np.random.default_rng(5)
    rows = [g.uniform(-300, -250, E), g.uniform(-110, -80, E), g.uniform(-4, 4, E),
            g.uniform(60, 90, E), np.concatenate([g.uniform(-95, -90, E - 1), [0.5]]),
            np.concatenate([g.uniform(-300, -200, E - 2), [-1e-30, 1e-30]])]
    logits = np.array(rows, np.float32)
    T = logits.shape[0]
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    mq.moeq_route_topk(dev(logits), T, E, k, ids, w, gating=mq.MOEQ_GATING_SIGMOID_TOPK)
    rid, rw = oracle.route_topk(logits, k, "sigmoid")
    gw = host(w).reshape(T, k)
    np.testing.assert_array_equal(host(ids).reshape(T, k), rid)
    assert np.all(np.isfinite(gw))
    np.testing.assert_allclose(gw, rw, rtol=2e-6, atol=1e-7)


def _router_case(seed, T, H, E):
    x = synth.make_x(seed, T, H)
    wr = synth.make_router(seed, E, H)
    return x, wr


def _router_bound(x, wr):
    """Rounding bound of an fp32 sum of exact bf16 products in which a term meets at most
    n = H/16 + 8 roundings (one per 16-wide MFMA step of the longest chain, plus the adds
    inside an MFMA and between wavefronts): n * 2^-24 * sum_h |x_h w_h| (|.| by clearing the
    sign bits)."""
    n = x.shape[1] // 16 + 8
    ax = (x & np.uint16(0x7FFF)).astype(np.uint16)
    aw = (wr & np.uint16(0x7FFF)).astype(np.uint16)
    return n * 2.0 ** -24 * oracle.router_logits(ax, aw)


@pytest.mark.parametrize("T,H,E", [(8, 6144, 256),      # decode batch: few-tokens kernel, K / 16
                                   (37, 576, 17),       # ragged tokens and experts, K / 2
                                   (1, 64, 1),          # one token, one expert, one K step
                                   (64, 640, 256),      # last few-tokens size, K / 4
                                   (65, 1024, 48),      # first many-tokens size
                                   (100, 1088, 200),    # K groups with a ragged last group
                                   (2048, 6144, 256)])  # prefill batch
def test_router_logits(T, H, E):
    mq = _mq()
    x, wr = _router_case(31, T, H, E)
    logits = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    mq.moeq_router_logits(dev(x.view(np.int16)), T, H, dev(wr.view(np.int16)), E, logits)
    got = host(logits)
    rows = np.arange(T) if T <= 256 else np.unique(np.r_[0, T - 1, np.arange(0, T, 61)])
    ref = oracle.router_logits(x[rows], wr)
    bound = _router_bound(x[rows], wr)
    assert np.all(np.isfinite(got))
    err = np.abs(got[rows].astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / bound).max())
    again = torch.empty_like(logits)
    mq.moeq_router_logits(dev(x.view(np.int16)), T, H, dev(wr.view(np.int16)), E, again)
    np.testing.assert_array_equal(host(again).view(np.uint32), got.view(np.uint32))


def test_layer_routed_sigmoid(path):
    """Router -> sigmoid top-k -> the expert path, all on the GPU; the selection and gates are
    checked by applying the oracle's routing to the GPU's fp32 logits."""
    mq = _mq()
    T, E, H, I, k = 37, 8, 576, 320, 4
    lw, x, _ = _case(27, T, E, H, I, k, e2m1_experts=(1,), permute="random")
    wr = synth.make_router(27, E, H)
    w = mq.DeviceWeights.from_host(lw)
    L = mq.MoeLayer(T, H, I, E, k, gating=mq.MOEQ_GATING_SIGMOID_TOPK)
    y = L.forward_routed(dev(x.view(np.int16)), dev(wr.view(np.int16)), w)
    out = dict(ids=host(L.topk_ids).reshape(T, k), w=host(L.topk_w).reshape(T, k),
               offsets=host(L.offsets), sorted_pair=host(L.sorted_pair),
               pair_pos=host(L.pair_pos), inter=u16(L.inter), y=u16(y))
    gl = host(L.logits)
    assert np.all(np.abs(gl - oracle.router_logits(x, wr)) <= _router_bound(x, wr))
    routing = oracle.route_topk(gl, k, "sigmoid")
    ref = oracle.layer_forward(x, gl, k, lw, routing=routing)
    check_layer(out, ref, k, lw, x)


@pytest.mark.parametrize("T,k,E", [(16, 2, 4), (8, 8, 256), (2048, 8, 256), (8192, 8, 256),
                                   (1, 1, 1), (129, 3, 7), (21, 3, 5), (13, 5, 256)])
def test_permute_bitexact(T, k, E):
    """Up to 64 pairs one wavefront (1, 32, 63, 64 pairs here), then one workgroup (65, 387),
    then three launches."""
    mq = _mq()
    ids = np.random.default_rng(T * 31 + E).integers(0, E, T * k).astype(np.int32)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    mq.moeq_permute_by_expert(dev(ids), T, k, E, off, sp, pp)
    ro, rs, rp = oracle.permute_by_expert(ids.reshape(T, k), E)
    np.testing.assert_array_equal(host(off), ro)
    np.testing.assert_array_equal(host(sp), rs)
    np.testing.assert_array_equal(host(pp), rp)


def test_permute_invalid_ids_are_placed_last():
    mq = _mq()
    ids = np.array([3, -1, 0, 7, 2, 0, 4, 1000], np.int32)
    E = 4
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(8, dtype=torch.int32, device="cuda")
    pp = torch.empty(8, dtype=torch.int32, device="cuda")
    mq.moeq_permute_by_expert(dev(ids), 4, 2, E, off, sp, pp)
    ro, rs, rp = oracle.permute_by_expert(ids.reshape(4, 2), E)
    np.testing.assert_array_equal(host(off), ro)
    np.testing.assert_array_equal(host(sp), rs)
    np.testing.assert_array_equal(host(pp), rp)
    assert host(off)[E] == 4


@pytest.mark.parametrize("P,E", [(64, 256), (64, 3), (65, 256)])
def test_permute_invalid_ids_small(P, E):
    """Invalid ids (negative and >= E) mixed with repeated valid ones, at the largest size of the
    one-wavefront form and one pair beyond it."""
    mq = _mq()
    g = np.random.default_rng(P * 7 + E)
    ids = g.integers(-2, E + 2, P).astype(np.int32)
    ids[::9] = E + 1000
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(P, dtype=torch.int32, device="cuda")
    pp = torch.empty(P, dtype=torch.int32, device="cuda")
    mq.moeq_permute_by_expert(dev(ids), P, 1, E, off, sp, pp)
    ro, rs, rp = oracle.permute_by_expert(ids.reshape(P, 1), E)
    np.testing.assert_array_equal(host(off), ro)
    np.testing.assert_array_equal(host(sp), rs)
    np.testing.assert_array_equal(host(pp), rp)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("P,E", [(4096, 256), (4097, 17), (40000, 256), (65536 + 1000, 64)])
def test_permute_many_pairs_with_invalid_ids(P, E):
    """The three-launch form (blocks of 1024 pairs, the last one larger), skewed ids and
    invalid ids scattered through several blocks."""
    mq = _mq()
    g = np.random.default_rng(P)
    ids = np.minimum(g.zipf(1.3, P) - 1, E - 1).astype(np.int32)
    bad = g.choice(P, 37, replace=False)
    ids[bad] = g.choice([-1, E, E + 5, 1 << 30, -(1 << 30)], 37)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(P, dtype=torch.int32, device="cuda")
    pp = torch.empty(P, dtype=torch.int32, device="cuda")
    mq.moeq_permute_by_expert(dev(ids), P, 1, E, off, sp, pp)
    ro, rs, rp = oracle.permute_by_expert(ids.reshape(P, 1), E)
    np.testing.assert_array_equal(host(off), ro)
    np.testing.assert_array_equal(host(sp), rs)
    np.testing.assert_array_equal(host(pp), rp)
    assert host(off)[E] == P - 37


# ----------------------------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------------------------

def _case(cfg_id, T, E, H, I, k, **kw):
    lw = synth.make_layer(cfg_id, E, H, I, **kw)
    x = synth.make_x(cfg_id, T, H)
    logits = synth.make_logits(cfg_id, T, E)
    return lw, x, logits


def test_layer_tiny_config(path):
    c = synth.WORKLOADS["tiny"]
    lw, x, logits = _case(1, c.T, c.E, c.H, c.I, c.k)
    out = run_layer(lw, x, logits, c.k)
    ref = oracle.layer_forward(x, logits, c.k, lw)
    check_layer(out, ref, c.k, lw, x)


def test_layer_empty_batch(path):
    """No tokens: the routing front end still writes expert_offsets (all zero), every other
    call is a no-op on empty (NULL-address) tensors, and the output is empty."""
    mq = _mq()
    c = synth.WORKLOADS["tiny"]
    lw, _, _ = _case(1, c.T, c.E, c.H, c.I, c.k)
    w = mq.DeviceWeights.from_host(lw)
    L = mq.MoeLayer(0, c.H, c.I, c.E, c.k)
    L.offsets.fill_(-7)
    x = torch.empty((0, c.H), dtype=torch.int16, device="cuda")
    lg = torch.empty((0, c.E), dtype=torch.float32, device="cuda")
    y = L.forward(x, lg, w, residual=x, out=x)
    assert tuple(y.shape) == (0, c.H)
    np.testing.assert_array_equal(host(L.offsets), np.zeros(c.E + 1, np.int32))
    L.offsets.fill_(-7)
    L.permute()
    np.testing.assert_array_equal(host(L.offsets), np.zeros(c.E + 1, np.int32))
    assert tuple(L.forward_fused(x, lg, w).shape) == (0, c.H)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,E,H,I,k", [(37, 8, 576, 320, 4),     # >16 rows per expert, K tails
                                       (37, 16, 1024, 512, 4),    # 16-byte aligned scale rows
                                       # down over whole 2048-wide K chunks (no K bound checks)
                                       # with a last 128-row block half past H; gate|up K tail
                                       (37, 8, 2112, 2048, 4),
                                       (5, 4, 4096, 2048, 2),     # whole chunks in both
                                       (1, 16, 256, 128, 16),     # k = E, one token
                                       (64, 4, 256, 192, 4)])     # k = E, 64 rows per expert
def test_layer_ragged_shapes(T, E, H, I, k, path):
    lw, x, logits = _case(21, T, E, H, I, k, e2m1_experts=(1,), permute="random")
    out = run_layer(lw, x, logits, k)
    ref = oracle.layer_forward(x, logits, k, lw)
    check_layer(out, ref, k, lw, x)


@pytest.mark.parametrize("groups", [1, 3])
@pytest.mark.parametrize("T,E,H,I,k", [(64, 4, 256, 192, 4), (1, 16, 256, 128, 16),
                                       (37, 8, 576, 320, 4)])
def test_layer_prefill_few_workgroups(T, E, H, I, k, groups, monkeypatch):
    """The many-rows kernels with every item on one (or three) workgroups: consecutive items
    and drained work queues on one workgroup (a claim race here once mixed up items)."""
    monkeypatch.setenv("MOEQ_FORCE_PATH", "prefill")
    monkeypatch.setenv("MOEQ_PREFILL_WORKGROUPS", str(groups))
    lw, x, logits = _case(24, T, E, H, I, k, e2m1_experts=(1,), permute="random")
    out = run_layer(lw, x, logits, k)
    ref = oracle.layer_forward(x, logits, k, lw)
    check_layer(out, ref, k, lw, x)


def test_layer_residual_in_place(path):
    mq = _mq()
    T, E, H, I, k = 16, 4, 256, 128, 2
    lw, x, logits = _case(22, T, E, H, I, k)
    w = mq.DeviceWeights.from_host(lw)
    L = mq.MoeLayer(T, H, I, E, k)
    xb = dev(x.view(np.int16))
    L.forward(xb, dev(logits), w, residual=xb, out=xb)        # y written over the residual
    ref = oracle.layer_forward(x, logits, k, lw, residual_bits=x)
    got = oracle.bf16_to_f64(u16(xb))
    expect = oracle.bf16_to_f64(ref["x_next"])
    rel = np.linalg.norm(got - expect, axis=1) / np.linalg.norm(expect, axis=1)
    assert rel.max() < 5e-3


def test_layer_invalid_expert_id_gives_nan_row(path):
    mq = _mq()
    T, E, H, I, k = 4, 4, 256, 128, 2
    lw, x, logits = _case(23, T, E, H, I, k)
    w = mq.DeviceWeights.from_host(lw)
    L = mq.MoeLayer(T, H, I, E, k)
    ids = np.array([[0, 1], [2, 9], [3, 0], [1, 2]], np.int32)
    wts = np.full((T, k), 0.5, np.float32)
    L.topk_ids.copy_(dev(ids.ravel()))
    L.topk_w.copy_(dev(wts.ravel()))
    L.permute()
    L.gateup(dev(x.view(np.int16)), w)
    L.down(w)
    y = oracle.bf16_to_f64(u16(L.combine()))
    assert host(L.offsets)[E] == 7
    assert np.all(np.isnan(y[1])) and np.all(np.isfinite(y[[0, 2, 3]]))
    ref = oracle.layer_forward(x, None, k, lw, routing=(ids.clip(0, E - 1),
                                                        wts.astype(np.float64)))
    rel = row_rel(u16(L.y)[[0, 2, 3]], ref["y"][[0, 2, 3]])
    assert rel.max() < ROW_REL_TOL


def test_layer_invalid_table_id_gives_nan_rows(path):
    T, E, H, I, k = 16, 4, 256, 128, 2
    lw, x, logits = _case(24, T, E, H, I, k)
    lw.table_id[2] = 7                       # only 2 tables exist
    out = run_layer(lw, x, logits, k)
    ids = out["ids"]
    y = oracle.bf16_to_f64(out["y"])
    uses2 = (ids == 2).any(1)
    assert uses2.any() and np.all(np.isnan(y[uses2])) and np.all(np.isfinite(y[~uses2]))


def test_layer_deterministic(path):
    T, E, H, I, k = 37, 8, 576, 320, 4
    lw, x, logits = _case(25, T, E, H, I, k)
    a = run_layer(lw, x, logits, k)
    b = run_layer(lw, x, logits, k)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


# ----------------------------------------------------------------------------------------------
# full GLM sizes
# ----------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def glm_layer():
    c = synth.WORKLOADS["glm_decode_t8"]
    return synth.make_layer(2, c.E, c.H, c.I)


@pytest.mark.timeout(600)
def test_glm_decode_t8_full(glm_layer):
    c = synth.WORKLOADS["glm_decode_t8"]
    x = synth.make_x(2, c.T, c.H)
    logits = synth.make_logits(2, c.T, c.E)
    out = run_layer(glm_layer, x, logits, c.k)
    ref = oracle.layer_forward(x, logits, c.k, glm_layer)
    check_layer(out, ref, c.k, glm_layer, x)


def _tile_class_tokens(out, k, seed, n_random=1):
    """Tokens whose pairs sit at every tile class of the most-loaded expert under the 128-row
    tiles of the many-rows kernels (the first row of its first tile, the last row of its
    first full tile, the first and the last row of its last tile, partial when its row count
    is not a multiple of 128), a token on the least-loaded expert (at most 32 rows: a tile
    whose 32-row MFMA tiles are mostly skipped), and random tokens. Returns (tokens, hot)."""
    off, sp = out["offsets"], out["sorted_pair"]
    counts = np.diff(off)
    hot = int(np.argmax(counts))
    b, n = int(off[hot]), int(counts[hot])
    rows = {b, b + min(127, n - 1), b + (n - 1) // 128 * 128, b + n - 1}
    toks = {int(sp[r]) // k for r in rows}
    live = np.flatnonzero(counts > 0)
    small = int(live[np.argmin(counts[live])])
    assert counts[small] <= 32
    toks.add(int(sp[off[small]]) // k)
    g = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(out["y"].shape[0]), sorted(toks))
    toks |= {int(t) for t in g.choice(rest, size=n_random, replace=False)}
    return sorted(toks), hot


def _check_expert_rows(out, x, lw, k, e, label):
    """The intermediate of every row of expert e, element-wise against the oracle."""
    off, sp = out["offsets"], out["sorted_pair"]
    rows = np.arange(off[e], off[e + 1])
    assert rows.size > 0
    toks = sp[rows] // k
    I = lw.gate_codes.shape[1]
    ref = oracle.expert_inter(x, lw, e, toks)
    check_inter(unslot(out["inter"], I)[rows], ref, toks, np.full(rows.size, e), x, lw,
                label=f"{label}: expert {e}, {rows.size} rows")


@pytest.mark.timeout(600)
def test_glm_prefill_t2048_zipf_sampled():
    """2048 tokens under Zipf routing: every row of the hottest expert (16 tiles of the
    many-rows kernels) element-wise, y of tokens at each of its tile classes and on the
    least-loaded expert; then the rank-1 Zipf expert re-packed on the E2M1 grid (its table
    id set to E2M1), which must route identically and give its rows from the E2M1 table."""
    c = synth.WORKLOADS["glm_prefill_t2048_zipf"]
    lw = synth.make_layer(3, c.E, c.H, c.I)
    x = synth.make_x(3, c.T, c.H)
    logits = synth.make_logits(3, c.T, c.E, zipf_s=c.zipf_s)
    out = run_layer(lw, x, logits, c.k)
    toks, hot = _tile_class_tokens(out, c.k, 3)
    _check_expert_rows(out, x, lw, c.k, hot, "hottest")
    ref = oracle.layer_forward(x, logits, c.k, lw, tokens=toks)
    check_layer(out, ref, c.k, lw, x, tokens=toks)

    e1 = int(np.argmax(synth.zipf_bias(3, c.E, c.zipf_s)))        # rank 1 of the Zipf bias
    sub = synth.make_layer(3, c.E, c.H, c.I, e2m1_experts=(e1,), experts=[e1])
    for name in ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes",
                 "down_scales"):
        getattr(lw, name)[e1] = getattr(sub, name)[e1]
    lw.table_id[e1] = 1
    out2 = run_layer(lw, x, logits, c.k)
    np.testing.assert_array_equal(out2["sorted_pair"], out["sorted_pair"])
    assert np.diff(out2["offsets"])[e1] > 128
    _check_expert_rows(out2, x, lw, c.k, e1, "rank-1 on E2M1")
    t1 = [int(out2["sorted_pair"][out2["offsets"][e1 + 1] - 1]) // c.k]
    ref2 = oracle.layer_forward(x, logits, c.k, lw, tokens=t1)
    check_layer(out2, ref2, c.k, lw, x, tokens=t1)


@pytest.mark.timeout(600)
def test_glm_prefill_t8192_e2m1_permuted_sampled():
    """8192 tokens, Zipf routing, the E2M1 experts of the model card's defect table and a
    random intermediate-channel permutation baked into gate-N, up-N and down-K: every row of
    the hottest expert and of every E2M1 expert that has rows, element-wise; y of tokens at
    each tile class of the hottest expert, on the least-loaded expert and on an E2M1 expert."""
    c = synth.WORKLOADS["glm_prefill_t8192_zipf_e2m1_perm"]
    lw = synth.make_layer(5, c.E, c.H, c.I, e2m1_experts=c.e2m1, permute=c.permute)
    x = synth.make_x(5, c.T, c.H)
    logits = synth.make_logits(5, c.T, c.E, zipf_s=c.zipf_s)
    out = run_layer(lw, x, logits, c.k)
    toks, hot = _tile_class_tokens(out, c.k, 5)
    _check_expert_rows(out, x, lw, c.k, hot, "hottest")
    counts = np.diff(out["offsets"])
    on = [e for e in c.e2m1 if counts[e] > 0]
    assert on
    for e in on:
        _check_expert_rows(out, x, lw, c.k, e, "E2M1")
    toks = sorted(set(toks) | {int(out["sorted_pair"][out["offsets"][on[0]]]) // c.k})
    ref = oracle.layer_forward(x, logits, c.k, lw, tokens=toks)
    check_layer(out, ref, c.k, lw, x, tokens=toks)


def test_block_permutation_relayout_gpu(path):
    """A permutation that moves whole 32-channel blocks and channels within blocks can be
    applied to the stored bytes exactly; outputs agree up to fp32 re-association. A changed
    summation order can move an intermediate value across a bf16 rounding boundary: one such
    flip changes y by about 2^-8 of that channel's share, hence a bound well above fp32
    re-association (~1e-6) yet far below the parity bar."""
    import copy
    T, E, H, I, k = 64, 8, 512, 256, 4
    lw, x, logits = _case(26, T, E, H, I, k)
    g = np.random.default_rng(7)
    perms = np.stack([np.concatenate([b * 32 + g.permutation(32) for b in g.permutation(I // 32)])
                      for _ in range(E)])
    q = copy.deepcopy(lw)
    for e in range(E):
        p = perms[e]
        q.gate_codes[e], q.gate_scales[e] = lw.gate_codes[e][p], lw.gate_scales[e][p]
        q.up_codes[e], q.up_scales[e] = lw.up_codes[e][p], lw.up_scales[e][p]
        cd = oracle.unpack_codes(lw.down_codes[e])[:, p]
        q.down_codes[e] = (cd[:, 0::2] | (cd[:, 1::2] << 4)).astype(np.uint8)
        q.down_scales[e] = lw.down_scales[e][:, p[::32] // 32]
    a = oracle.bf16_to_f64(run_layer(lw, x, logits, k)["y"])
    b = oracle.bf16_to_f64(run_layer(q, x, logits, k)["y"])
    rel = np.linalg.norm(a - b, axis=1) / np.linalg.norm(a, axis=1)
    assert rel.max() < 1e-3
    assert np.median(rel) < 1e-6


# ----------------------------------------------------------------------------------------------
# shared expert beside the routed ones
# ----------------------------------------------------------------------------------------------

def _run_shared(sw, x):
    mq = _mq()
    T, H = x.shape
    I = sw.gate_codes.shape[1]
    w = mq.DeviceWeights.from_host(sw)
    inter = torch.empty((T, I), dtype=torch.int16, device="cuda")
    z = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    nws = mq.moeq_shared_workspace_bytes(T, H, I)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    mq.moeq_shared_expert(dev(x.view(np.int16)), T, H, I, w.gate_codes, w.gate_scales,
                          w.up_codes, w.up_scales, w.down_codes, w.down_scales, w.tables,
                          w.table_id, inter, z, ws, nws)
    return u16(inter), host(z)


@pytest.mark.parametrize("T,H,I", [(16, 256, 128),       # tiny geometry
                                   (37, 576, 320),       # K tails, ragged rows
                                   (1, 256, 128),        # one token
                                   (8, 6144, 2048),      # GLM decode batch
                                   (200, 1024, 512)])    # many rows (prefill kernels)
def test_shared_expert(T, H, I, path):
    sw = synth.make_shared(41, H, I)
    x = synth.make_x(41, T, H)
    inter, z = _run_shared(sw, x)
    ref = oracle.shared_expert_forward(x, sw)
    check_inter(unslot(inter, I), ref["inter"], np.arange(T), np.zeros(T, np.int64), x, sw,
                label="shared expert")
    rel = np.linalg.norm(z - ref["z"], axis=1) / np.linalg.norm(ref["z"], axis=1)
    assert np.all(np.isfinite(z)) and rel.max() <= ROW_REL_TOL, rel.max()


def test_shared_expert_invalid_table_id_gives_nan():
    sw = synth.make_shared(42, 256, 128)
    sw.table_id[0] = 5
    _, z = _run_shared(sw, synth.make_x(42, 4, 256))
    assert np.isnan(z).all()


@pytest.mark.parametrize("T,E,H,I,k", [(16, 4, 256, 128, 2), (37, 8, 576, 320, 4)])
def test_layer_with_shared_expert(T, E, H, I, k, path):
    """Routed path on the main stream, the shared expert on a side stream, summed in the
    combine with the residual; y in place over X."""
    mq = _mq()
    lw, x, logits = _case(43, T, E, H, I, k, e2m1_experts=(1,), permute="random")
    sw = synth.make_shared(43, H, I)
    L = mq.MoeLayer(T, H, I, E, k, shared_I=I)
    xb = dev(x.view(np.int16))
    L.forward(xb, dev(logits), mq.DeviceWeights.from_host(lw), residual=xb, out=xb,
              shared=mq.DeviceWeights.from_host(sw))
    ref = oracle.layer_forward(x, logits, k, lw, residual_bits=x, shared=sw)
    got = oracle.bf16_to_f64(u16(xb))
    expect = oracle.bf16_to_f64(ref["x_next"])
    rel = np.linalg.norm(got - expect, axis=1) / np.linalg.norm(expect, axis=1)
    assert rel.max() < ROW_REL_TOL, rel.max()
    # the shared term is really there: without it the result is far off
    plain = oracle.bf16_to_f64(oracle.layer_forward(x, logits, k, lw, residual_bits=x)["x_next"])
    assert (np.linalg.norm(got - plain, axis=1) / np.linalg.norm(plain, axis=1)).max() > 1e-2


@pytest.mark.timeout(600)
def test_glm_decode_t8_with_shared_expert(glm_layer):
    mq = _mq()
    c = synth.WORKLOADS["glm_decode_t8"]
    x = synth.make_x(2, c.T, c.H)
    logits = synth.make_logits(2, c.T, c.E)
    sw = synth.make_shared(2, c.H, c.I)
    L = mq.MoeLayer(c.T, c.H, c.I, c.E, c.k, shared_I=c.I)
    y = L.forward(dev(x.view(np.int16)), dev(logits), mq.DeviceWeights.from_host(glm_layer),
                  shared=mq.DeviceWeights.from_host(sw))
    ref = oracle.layer_forward(x, logits, c.k, glm_layer, shared=sw)
    rel = row_rel(u16(y), ref["y"])
    assert np.all(np.isfinite(rel)) and rel.max() <= ROW_REL_TOL, rel.max()


# ----------------------------------------------------------------------------------------------
# encoding (quantizer), grid fit and arm choice
# ----------------------------------------------------------------------------------------------

def _special_weights(seed, E, N, K):
    """bf16 bits [E, N, K]: N(0, 0.02) with scale spread per row, plus blocks that exercise
    the rules: all zero, exact E2M1 midpoint ties, -0, subnormals, huge values, Inf/NaN."""
    g = np.random.default_rng(seed)
    w = (g.standard_normal((E, N, K)) * 0.02 * np.exp(g.standard_normal((E, N, 1)))).astype(np.float32)
    w[0, 0, :32] = 0.0
    w[0, 1, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4) * np.tile([1, -1], 16)
    w[0, 2, 5] = -0.0
    w[0, 3, 32:64] = np.float32(1e-39) * g.standard_normal(32).astype(np.float32)   # subnormal
    w[0, 4, :32] *= 1e30
    bits = synth.bf16_bits_from_f32(w)
    bits[0, 5, 40] = 0x7F80                      # +Inf
    bits[0, 6, 70] = 0xFFC1                      # NaN
    return bits


def test_quantize_bitexact():
    mq = _mq()
    E, N, K = 3, 40, 256
    bits = _special_weights(51, E, N, K)
    tables = np.stack([synth.lloyd_grid(1, 0), oracle.E2M1_TABLE]).astype(np.float32)
    tid = np.array([0, 1, 0], np.uint8)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda")
    err = torch.empty(E * N, dtype=torch.float64, device="cuda")
    mq.moeq_quantize(dev(bits.view(np.int16)), E, N, K, tables, dev(tid), codes, scales, err)
    gc, gs, ge = host(codes), host(scales), host(err).reshape(E, N)
    for e in range(E):
        tab = tables[tid[e]]
        rc, rs = oracle.rtn_encode(bits[e], tab)
        np.testing.assert_array_equal(gs[e], rs)
        np.testing.assert_array_equal(gc[e], rc)
        re = oracle.reconstruction_sq_error(bits[e], rc, rs, tab)
        np.testing.assert_array_equal(np.isnan(ge[e]), np.isnan(re))
        ok = ~np.isnan(re)
        np.testing.assert_allclose(ge[e][ok], re[ok], rtol=1e-12, atol=1e-300)
    assert gs[0, 5, 1] == 255 and gs[0, 6, 2] == 255 and gs[0, 0, 0] == 0
    # a second call gives the same bytes; codes-only and error-only calls agree with the full one
    err2 = torch.empty_like(err)
    mq.moeq_quantize(dev(bits.view(np.int16)), E, N, K, tables, dev(tid), None, None, err2)
    np.testing.assert_array_equal(host(err2).view(np.uint64), host(err).view(np.uint64))


# tables of the boundary test: a Lloyd grid, E2M1, E2M1 scaled far down and up (so that block
# exponents clamp at +-127 and thresholds reach the ends of the bf16 range), repeated
# magnitudes, and a table whose first midpoint is 0
BOUNDARY_TABLES = np.stack([synth.lloyd_grid(1, 0), oracle.E2M1_TABLE,
                            oracle.E2M1_TABLE * np.float32(2.0 ** -20),
                            oracle.E2M1_TABLE * np.float32(2.0 ** 20),
                            np.array([0.1, 0.1, 0.5, 0.5, 0.5, 1, 2, 2], np.float32),
                            np.array([0, 0, 0, 0, 0, 0, 0, 1], np.float32)]).astype(np.float32)


def _boundary_weights(seed, N, K):
    """bf16 bits [E, N, K], expert t for table t: every block draws its exponent across the
    whole bf16 range (block maxima from subnormal to near the largest finite value), spreads
    its other magnitudes over 12 binades below the maximum, and places weights exactly on
    midpoints times 2^e (ties) and one bf16 step either side of them."""
    g = np.random.default_rng(seed)
    E = len(BOUNDARY_TABLES)
    out = np.zeros((E, N, K), np.uint16)
    for t, tab in enumerate(BOUNDARY_TABLES):
        gmax = float(tab[7])
        mid = 0.5 * (tab[:-1].astype(np.float64) + tab[1:].astype(np.float64))
        # the exponent at which 2^e times the smallest nonzero midpoint, rounded down to bf16,
        # becomes a normal number; the first blocks straddle it, then two blocks whose e clamps
        lo = mid[mid > 0].min()
        e_edge = -126 - int(np.floor(np.log2(lo)))
        fixed = [gmax * 2.0 ** (e_edge + d) * 0.75 for d in range(-2, 3)] + \
                [3.0e38 * 0.9, gmax * 2.0 ** -140]
        nblk = 0
        for n in range(N):
            for b in range(K // 32):
                ex = int(g.integers(-150, 130))
                amax = min(gmax * 2.0 ** ex * g.uniform(0.5, 1.0), 3.0e38)
                if nblk < len(fixed):
                    amax = fixed[nblk]
                elif g.random() < 0.05:
                    amax = 3.0e38 * g.uniform(0.3, 1.0)
                nblk += 1
                v = amax * 2.0 ** (-g.uniform(0, 12, 32)) * np.where(g.random(32) < .5, -1, 1)
                v[0] = amax
                v[g.random(32) < 0.05] = 0.0
                bits = synth.bf16_bits_from_f32(v.astype(np.float32))
                e = int(oracle.block_scale_bytes(bits[None], gmax)[0, 0]) - 127
                for j in range(2, 32, 3):
                    with np.errstate(over="ignore"):        # beyond fp32: skipped below
                        tie = int(synth.bf16_bits_from_f32(
                            np.array([mid[g.integers(0, 7)] * 2.0 ** e], np.float32))[0])
                    step = int(g.integers(-1, 2))
                    cand = tie + step if 0 < (tie & 0x7FFF) < 0x7F7F else tie
                    if (cand & 0x7FFF) <= (int(bits[0]) & 0x7FFF):
                        bits[j] = (cand & 0x7FFF) | (0x8000 if g.random() < .5 else 0)
                out[t, n, b * 32:(b + 1) * 32] = bits
    return out


def test_quantize_exponent_and_threshold_boundaries():
    """The scale byte and the nearest magnitude against the oracle, bit for bit, across block
    exponents on both sides of every range limit the kernel's integer decision has (thresholds
    leaving the normal range, exponents clamped at +-127) and on exact ties."""
    mq = _mq()
    N, K = 24, 256
    bits = _boundary_weights(57, N, K)
    for group in ((0, 1, 2, 3), (4, 5)):               # at most 4 tables per call
        tabs = BOUNDARY_TABLES[list(group)]
        gb = np.ascontiguousarray(bits[list(group)])
        E = len(group)
        tid = np.arange(E, dtype=np.uint8)
        codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda")
        err = torch.empty(E * N, dtype=torch.float64, device="cuda")
        mq.moeq_quantize(dev(gb.view(np.int16)), E, N, K, tabs, dev(tid), codes, scales, err)
        gc, gs, ge = host(codes), host(scales), host(err).reshape(E, N)
        err2 = torch.empty_like(err)
        mq.moeq_quantize(dev(gb.view(np.int16)), E, N, K, tabs, dev(tid), None, None, err2)
        np.testing.assert_array_equal(host(err2).view(np.uint64), host(err).view(np.uint64))
        for i, t in enumerate(group):
            tab = BOUNDARY_TABLES[t]
            rc, rs = oracle.rtn_encode(gb[i], tab)
            np.testing.assert_array_equal(gs[i], rs, err_msg=f"table {t}")
            np.testing.assert_array_equal(gc[i], rc, err_msg=f"table {t}")
            re = oracle.reconstruction_sq_error(gb[i], rc, rs, tab)
            np.testing.assert_allclose(ge[i], re, rtol=1e-12, atol=1e-300, err_msg=f"table {t}")


def test_quantize_invalid_table_id_gives_nan_blocks():
    mq = _mq()
    E, N, K = 2, 8, 96
    bits = _special_weights(52, E, N, K)
    codes = torch.full((E, N, K // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda")
    err = torch.empty(E * N, dtype=torch.float64, device="cuda")
    mq.moeq_quantize(dev(bits.view(np.int16)), E, N, K, oracle.E2M1_TABLE[None],
                     dev(np.array([0, 3], np.uint8)), codes, scales, err)
    assert (host(scales)[1] == 255).all() and (host(codes)[1] == 0).all()
    assert np.isnan(host(err)[N:]).all()


def test_lloyd_stats_and_pooling():
    mq = _mq()
    tab = synth.lloyd_grid(1, 0)
    mats = [_special_weights(53, 2, 24, 192), _special_weights(54, 3, 16, 256)]
    stats = torch.empty(24, dtype=torch.float64, device="cuda")
    ref = np.zeros((3, 8))
    for i, m in enumerate(mats):
        E, N, K = m.shape
        need = mq.moeq_lloyd_workspace_bytes(E, N)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        mq.moeq_lloyd_stats(dev(m.view(np.int16)), E, N, K, tab, 2.5, i > 0, stats, ws, need)
        ref += sum(oracle.lloyd_stats(m[e], tab, gmax=2.5) for e in range(E))
    np.testing.assert_allclose(host(stats).reshape(3, 8), ref, rtol=1e-12)


@pytest.mark.timeout(600)
def test_grid_fit_and_layer_encode_end_to_end(path):
    """Fit the grid (weighted Lloyd), choose arms and encode a layer on the GPU; then run the
    encoded layer forward on the GPU: all against the oracle."""
    from codebook_quantized_moe_amd import encode
    mq = _mq()
    T, E, H, I, k = 24, 6, 256, 128, 2
    g = np.random.default_rng(55)
    def draw(shape):
        return synth.bf16_bits_from_f32(g.standard_normal(shape) * 0.02)
    gate, up, down = draw((E, I, H)), draw((E, I, H)), draw((E, H, I))
    # expert 4: weights exactly on the E2M1 grid, so E2M1 reconstructs it exactly
    for m in (gate, up, down):
        vals = oracle.E2M1_TABLE[g.integers(0, 8, m.shape[1:])] * np.where(
            g.random(m.shape[1:]) < .5, -1, 1) * 2.0 ** -8
        vals[:, ::32] = 6 * 2.0 ** -8
        m[4] = synth.bf16_bits_from_f32(vals)
    mats = [dev(m.view(np.int16)) for m in (gate, up, down)]
    g0 = synth.lloyd_grid(1, 0)
    grid, dist = encode.fit_grid(mats, g0, 3)
    ref_grid = oracle.fit_grid([m[e] for m in (gate, up, down) for e in range(E)], g0, 3)
    np.testing.assert_allclose(grid, ref_grid, rtol=1e-6)
    assert all(b <= a * (1 + 1e-12) for a, b in zip(dist, dist[1:]))
    enc = encode.encode_layer(*mats, grid)
    # arms and bytes, decided by the oracle on the GPU's own grid
    errs = np.zeros((E, 2))
    for m in (gate, up, down):
        for e in range(E):
            for t, tb in enumerate((grid, oracle.E2M1_TABLE)):
                c, s = oracle.rtn_encode(m[e], tb)
                errs[e, t] += oracle.reconstruction_sq_error(m[e], c, s, tb).sum()
    np.testing.assert_allclose(host(enc["expert_err"]), errs, rtol=1e-12)
    tid = oracle.select_arms(errs[:, 0], errs[:, 1])
    np.testing.assert_array_equal(host(enc["table_id"]), tid)
    assert tid[4] == 1 and tid.sum() == 1
    lw = synth.LayerWeights(*(np.empty(0),) * 6, tables=enc["tables"], table_id=tid)
    for name, m in (("gate", gate), ("up", up), ("down", down)):
        cs = [oracle.rtn_encode(m[e], enc["tables"][tid[e]]) for e in range(E)]
        np.testing.assert_array_equal(host(enc[name + "_codes"]), np.stack([c for c, _ in cs]))
        np.testing.assert_array_equal(host(enc[name + "_scales"]), np.stack([s for _, s in cs]))
        setattr(lw, name + "_codes", np.stack([c for c, _ in cs]))
        setattr(lw, name + "_scales", np.stack([s for _, s in cs]))
    # the encoded layer through the forward path
    x = synth.make_x(55, T, H)
    logits = synth.make_logits(55, T, E)
    w = mq.DeviceWeights(enc["gate_codes"], enc["gate_scales"], enc["up_codes"],
                         enc["up_scales"], enc["down_codes"], enc["down_scales"],
                         enc["tables"], enc["table_id"])
    L = mq.MoeLayer(T, H, I, E, k)
    y = L.forward(dev(x.view(np.int16)), dev(logits), w)
    ref = oracle.layer_forward(x, logits, k, lw)
    rel = row_rel(u16(y), ref["y"])
    assert rel.max() <= ROW_REL_TOL, rel.max()


@pytest.mark.timeout(600)
def test_quantize_glm_expert_sampled_rows():
    """A GLM-size expert matrix (2048 x 6144) in the launch the layer encoder uses; sampled
    rows against the oracle."""
    mq = _mq()
    N, K = 2048, 6144
    bits = synth.bf16_bits_from_f32(synth.normal_matrix(synth.key(56, 1), N, K))
    tables = np.stack([synth.lloyd_grid(2, 0), oracle.E2M1_TABLE]).astype(np.float32)
    codes = torch.empty((1, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, N, K // 32), dtype=torch.uint8, device="cuda")
    err = torch.empty(N, dtype=torch.float64, device="cuda")
    mq.moeq_quantize(dev(bits.view(np.int16)), 1, N, K, tables, dev(np.zeros(1, np.uint8)),
                     codes, scales, err)
    rows = [0, 1, 777, 2047]
    rc, rs = oracle.rtn_encode(bits[rows], tables[0])
    np.testing.assert_array_equal(host(codes)[0, rows], rc)
    np.testing.assert_array_equal(host(scales)[0, rows], rs)
    np.testing.assert_allclose(host(err)[rows], oracle.reconstruction_sq_error(bits[rows], rc, rs, tables[0]),
                               rtol=1e-12)


# ----------------------------------------------------------------------------------------------
# the decode layer as one cooperative launch
# ----------------------------------------------------------------------------------------------

@pytest.mark.timeout(600)
@pytest.mark.parametrize("T,E,H,I,k,gating", [(16, 4, 256, 128, 2, 0), (37, 8, 576, 320, 4, 1),
                                              (1, 16, 256, 128, 16, 0), (8, 256, 6144, 2048, 8, 0),
                                              (64, 256, 6144, 2048, 8, 1)])
def test_moe_decode_single_launch(T, E, H, I, k, gating, monkeypatch):
    """Bit-identical to the per-step calls on the few-rows kernels (the same kernels' phases,
    the same summation orders) and within the bar of the oracle; residual updated in place;
    a second call with other inputs (the barrier word is reset per call)."""
    monkeypatch.setenv("MOEQ_FORCE_PATH", "decode")
    mq = _mq()
    if H == 6144:
        lw = synth.make_layer(2, E, H, I) if T == 8 else synth.make_layer(61, E, H, I)
    else:
        lw = synth.make_layer(61, E, H, I, e2m1_experts=(1,), permute="random")
    w = mq.DeviceWeights.from_host(lw)
    L = mq.MoeLayer(T, H, I, E, k, gating=gating)
    for call in range(2):
        x = synth.make_x(61, T, H, batch=call)
        logits = synth.make_logits(61, T, E, batch=call)
        xb, lg = dev(x.view(np.int16)), dev(logits)
        ref_bits = u16(L.forward(xb, lg, w, residual=xb, out=torch.empty_like(xb)))
        y = L.forward_fused(xb, lg, w, residual=xb, out=xb)            # in place over x
        mq.moeq_moe_decode_check(L.f_ws)
        np.testing.assert_array_equal(u16(y), ref_bits)
        # the oracle on the small shapes and on the first call of the GLM layers (all 8
        # tokens; the first and last of 64); the bit-identity above ties the rest to the
        # per-step calls, which their own tests hold to the oracle
        if H != 6144 or call == 0:
            routing = oracle.route_topk(logits, k, "sigmoid" if gating else "softmax")
            if T <= 16:
                tokens = None
            else:
                tokens = [0, T - 1] if H == 6144 else list(range(0, T, 9))
            ref = oracle.layer_forward(x, logits, k, lw, residual_bits=x, routing=routing,
                                       tokens=tokens)
            toks = np.arange(T) if tokens is None else np.asarray(tokens)
            got = oracle.bf16_to_f64(u16(y))[toks]
            expect = oracle.bf16_to_f64(ref["x_next"])[toks]
            rel = np.linalg.norm(got - expect, axis=1) / np.linalg.norm(expect, axis=1)
            assert rel.max() < ROW_REL_TOL, rel.max()


@pytest.mark.parametrize("T,E,k,gating", [(1, 17, 1, 0), (8, 256, 8, 0), (7, 40, 9, 1),
                                          (64, 256, 8, 1), (65, 64, 4, 0), (2048, 256, 8, 1)])
def test_route_permute_equals_the_two_calls(T, E, k, gating):
    """One launch up to 64 tokens, two beyond: the same five arrays, bit for bit, as
    moeq_route_topk then moeq_permute_by_expert, and the oracle's routing."""
    mq = _mq()
    logits = dev(synth.make_logits(71, T, E, zipf_s=1.0 if T > 64 else None))
    def bufs():
        i32 = dict(dtype=torch.int32, device="cuda")
        return (torch.empty(T * k, **i32), torch.empty(T * k, dtype=torch.float32, device="cuda"),
                torch.empty(E + 1, **i32), torch.empty(T * k, **i32), torch.empty(T * k, **i32))
    a, b = bufs(), bufs()
    mq.moeq_route_permute(logits, T, E, k, *a, gating=gating)
    mq.moeq_route_topk(logits, T, E, k, b[0], b[1], gating=gating)
    mq.moeq_permute_by_expert(b[0], T, k, E, b[2], b[3], b[4])
    for x, y in zip(a, b):
        np.testing.assert_array_equal(host(x).view(np.uint32), host(y).view(np.uint32))
    rid, rw = oracle.route_topk(host(logits), k, "sigmoid" if gating else "softmax")
    np.testing.assert_array_equal(host(a[0]).reshape(T, k), rid)
    ro, rs, rp = oracle.permute_by_expert(rid, E)
    np.testing.assert_array_equal(host(a[2]), ro)
    np.testing.assert_array_equal(host(a[3]), rs)
