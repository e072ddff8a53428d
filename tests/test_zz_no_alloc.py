"""The allocation-free gate|up entry point (moeq_gateup_swiglu_static) against
moeq_gateup_swiglu with a caller workspace, through the C ABI: two calls in a row, the second
with a smaller input (first the many-rows kernels, then the few-rows kernels), with the same
results bit for bit; a call that needs more than the static scratch is refused and launches
nothing."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import codebook_quantized_moe_amd  # noqa: F401  (fails loudly when not built)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_static_scratch_matches_the_workspace_call():
    import codebook_quantized_moe_amd as mq
    E, H, I, k = 8, 1024, 512, 4
    lw = synth.make_layer(81, E, H, I, e2m1_experts=(3,))
    w = mq.DeviceWeights.from_host(lw)
    # 300 tokens: 1200 rows, the many-rows kernels; then 5 tokens: 20 rows, the few-rows ones
    for T in (300, 5):
        x = dev(synth.make_x(81, T, H, batch=T).view(np.int16))
        logits = dev(synth.make_logits(81, T, E, batch=T))
        L = mq.MoeLayer(T, H, I, E, k)
        L.route_permute(logits)
        L.gateup(x, w)                                   # caller workspace
        want = host(L.inter)
        got = torch.full_like(L.inter, -1)
        mq.moeq_gateup_swiglu_static(x, T, H, I, E, k, L.offsets, L.sorted_pair, w.gate_codes,
                                     w.gate_scales, w.up_codes, w.up_scales, w.tables,
                                     w.table_id, got)
        rows = int(host(L.offsets)[E])
        assert rows == T * k
        np.testing.assert_array_equal(host(got)[:rows], want[:rows])


def test_static_scratch_refuses_a_call_beyond_its_size():
    import codebook_quantized_moe_amd as mq
    E, H, I, k = 4, 6144, 128, 1
    T = (mq.MOEQ_STATIC_SCRATCH_BYTES - 256) // (2 * H) + 1    # one token more than fits
    assert mq.moeq_workspace_bytes(T, k, E, H, I) > mq.MOEQ_STATIC_SCRATCH_BYTES
    # real buffers of the full sizes (all routed to nothing), so that even a launch would stay
    # in bounds
    x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    sorted_pair = torch.zeros(T * k, dtype=torch.int32, device="cuda")
    codes = torch.zeros((E, I, H // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((E, I, H // 32), dtype=torch.uint8, device="cuda")
    table_id = torch.zeros(E, dtype=torch.uint8, device="cuda")
    inter = torch.zeros((T * k, I), dtype=torch.int16, device="cuda")
    tables = np.array([[0.1, 0.3, 0.6, 0.9, 1.2, 1.6, 2.0, 2.7]], np.float32)
    with pytest.raises(mq.MoeqError) as ei:
        mq.moeq_gateup_swiglu_static(x, T, H, I, E, k, offsets, sorted_pair, codes, scales,
                                     codes, scales, tables, table_id, inter)
    assert ei.value.status == mq.MOEQ_EWORKSPACE
    assert "static" in mq.moeq_last_error()
    torch.cuda.synchronize()
    assert int(inter.abs().sum()) == 0
