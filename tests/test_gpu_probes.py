"""Probes of the weights the two projection kernels decode, through the C ABI.

moeq_down with one-hot intermediate rows and gate weight 1: row r of expert e carries 1.0 at
channel c_r and zeros elsewhere, so yp[r, h] = 1.0 * Wd_e[h, c_r] exactly (every other product
is a zero, the sum of zeros and one product is exact in fp32, and the gate weight 1 changes
nothing). One row per channel reads back the whole down matrix as the kernel decoded it, which
must equal the oracle's dequantisation bit for bit (signed zeros compare equal: a sum that
holds a -0 product and +0 products is +0).

moeq_gateup_swiglu with one-hot activation rows: row r of expert e is 1.0 at column h_r, so
g = Wg_e[n, h_r] and u = Wu_e[n, h_r] exactly, and I[r, n] = bf16(silu(g) * u) can differ
from the oracle's only by the rounding of silu in fp32 (at most one bf16 ulp, rarely).

Both kernel families (MOEQ_FORCE_PATH), the GLM shape (K/32 a multiple of 16: scale rows on
16-byte boundaries, the aligned staging forms) and ragged shapes (K/32 = 18 and 20: the
unaligned staging forms; K % 128 = 64 and 0: the two prefill super-stage forms), each with an
expert on the E2M1 table beside experts on the layer's Lloyd grid.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from inter_check import bf16_ulp

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

ONE_BF16 = 0x3F80


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import codebook_quantized_moe_amd  # noqa: F401  (fails loudly when not built)


@pytest.fixture(params=["decode", "prefill"])
def path(request, monkeypatch):
    monkeypatch.setenv("MOEQ_FORCE_PATH", request.param)
    return request.param


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# (H, I, E): GLM geometry with two experts (4096 probe rows, the few-rows kernels' maximum);
# down K = I = 576 (K/32 = 18, K % 128 = 64) and 640 (K/32 = 20, K % 128 = 0); gate|up
# K = H = 576 and 640 likewise
SHAPES = [(6144, 2048, 2), (576, 576, 3), (640, 640, 3)]


def _layer(H, I, E):
    """Expert 1 on the E2M1 table, the others on the layer's Lloyd grid."""
    return synth.make_layer(61, E, H, I, e2m1_experts=(1,))


@pytest.mark.parametrize("H,I,E", SHAPES)
def test_down_decodes_every_weight_bitexact(H, I, E, path):
    import codebook_quantized_moe_amd as mq
    lw = _layer(H, I, E)
    w = mq.DeviceWeights.from_host(lw)
    R = E * I                                       # one row per (expert, channel)
    offsets = (np.arange(E + 1) * I).astype(np.int32)
    sorted_pair = np.arange(R, dtype=np.int32)
    inter = np.zeros((R, I), np.uint16)
    inter[np.arange(R), np.tile(mq.inter_slot(np.arange(I)), E)] = ONE_BF16
    yp = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    nws = mq.moeq_workspace_bytes(R, 1, E, H, I)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    mq.moeq_down(dev(inter.view(np.int16)), R, H, I, E, 1, dev(offsets), dev(sorted_pair),
                 dev(np.ones(R, np.float32)), w.down_codes, w.down_scales, w.tables, w.table_id,
                 yp, ws, nws)
    got = host(yp)
    for e in range(E):
        want = oracle.dequant_bf16(lw.down_codes[e], lw.down_scales[e],
                                   lw.tables[int(lw.table_id[e])])          # [H, I] bf16 bits
        want = (want.astype(np.uint32) << 16).view(np.float32).T             # [I, H]
        g = got[e * I:(e + 1) * I]
        same = g == want
        assert same.all(), (f"expert {e} (table {int(lw.table_id[e])}): "
                            f"{int((~same).sum())} of {same.size} weights differ, first at "
                            f"{np.argwhere(~same)[:4].tolist()}")


@pytest.mark.parametrize("H,I,E", SHAPES)
def test_gateup_decodes_every_column(H, I, E, path):
    import codebook_quantized_moe_amd as mq
    lw = _layer(H, I, E)
    w = mq.DeviceWeights.from_host(lw)
    # rows per expert: every column of K when it fits the few-rows kernels' 4096 rows,
    # else 2048 columns h_r = 97 r mod H (97 is prime to H = 6144 = 3 * 2^11 and 1 mod 32,
    # so the columns are distinct and take every position inside a 32-block)
    Rpe = H if E * H <= 4096 else 4096 // E
    cols = (np.arange(Rpe) * 97) % H
    R = E * Rpe
    x = np.zeros((R, H), np.uint16)
    x[np.arange(R), np.tile(cols, E)] = ONE_BF16
    offsets = (np.arange(E + 1) * Rpe).astype(np.int32)
    sorted_pair = np.arange(R, dtype=np.int32)
    inter = torch.empty((R, I), dtype=torch.int16, device="cuda")
    nws = mq.moeq_workspace_bytes(R, 1, E, H, I)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    mq.moeq_gateup_swiglu(dev(x.view(np.int16)), R, H, I, E, 1, dev(offsets), dev(sorted_pair),
                          w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, w.tables,
                          w.table_id, inter, ws, nws)
    got = host(inter).view(np.uint16)[:, mq.inter_slot(np.arange(I))]
    flips = 0
    for e in range(E):
        want = oracle.expert_inter(x[e * Rpe:(e + 1) * Rpe], lw, e, np.arange(Rpe))
        gv = oracle.bf16_to_f64(got[e * Rpe:(e + 1) * Rpe])
        wv = oracle.bf16_to_f64(want)
        diff = np.abs(gv - wv)
        assert np.all(diff <= bf16_ulp(wv)), (
            f"expert {e}: {int((diff > bf16_ulp(wv)).sum())} elements beyond one bf16 ulp, "
            f"first at {np.argwhere(diff > bf16_ulp(wv))[:4].tolist()}")
        flips += int((gv != wv).sum())
    print(f"gate|up probe: {R * I} elements, {flips} one ulp apart", flush=True)
    assert flips <= 0.002 * R * I
