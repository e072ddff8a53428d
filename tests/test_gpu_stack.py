"""Decode through a stack of MoE layers with a residual carried in bf16, on the GPU.

The 32-layer GLM-shaped stack (64 tokens, 32 distinct layers with their own grids and
weights, ~5.1 GB each) runs on the device layer by layer with the residual added in place,
X_{l+1} = bf16(X_l + y_l). The oracle checks it teacher-forced: at sampled layers the GPU's
own X_l is fed to both sides with no residual, routing is compared for all tokens and y_l
for sampled tokens (a full-size fp64 free-running stack is beyond a test's time: every token
touches 256 expert dequantizations). The free-running composition is checked against the
oracle's stack on a small shape instead, with the same calls.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

ROW_REL_TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import codebook_quantized_moe_amd  # noqa: F401  (fails loudly when not built)


def _rows_rel(gpu_bits, ref):
    g = oracle.bf16_to_f64(gpu_bits)
    return np.linalg.norm(g - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)


@pytest.mark.timeout(300)
def test_stack_free_running_small():
    """16 layers of a small shape (H 256, I 128, E 16, top-2, 24 tokens), residual in place,
    against the oracle's free-running stack."""
    import codebook_quantized_moe_amd as mq
    T, H, I, E, k, L = 24, 256, 128, 16, 2, 16
    x0 = synth.make_x(91, T, H)
    layers = []
    for l in range(L):
        lw = synth.make_layer(91, E, H, I, layer=l)
        logits = synth.make_logits(91, T, E, layer=l)
        layers.append((logits, lw))
    ref = oracle.stack_forward(x0, layers, k)
    ml = mq.MoeLayer(T, H, I, E, k)
    X = torch.from_numpy(x0.view(np.int16)).cuda()
    for logits, lw in layers:
        w = mq.DeviceWeights.from_host(lw)
        ml.forward(X, torch.from_numpy(logits).cuda(), w, residual=X, out=X)
    torch.cuda.synchronize()
    got = X.cpu().numpy().view(np.uint16)
    rel = _rows_rel(got, oracle.bf16_to_f64(ref))
    assert np.all(np.isfinite(rel)) and rel.max() <= ROW_REL_TOL, rel.max()


class _Stack:
    """The 32-layer stack's device state, advanced a few layers per test (each test stays
    well under a few minutes: every GLM layer is generated on the host first)."""

    def __init__(self):
        import codebook_quantized_moe_amd as mq
        self.mq = mq
        self.c = c = synth.WORKLOADS["glm_stack32_decode_t64"]
        self.ml = mq.MoeLayer(c.T, c.H, c.I, c.E, c.k)
        self.X = torch.from_numpy(synth.make_x(4, c.T, c.H).view(np.int16)).cuda()
        self.layer = 0

    def advance(self, upto, checked):
        """Layers [self.layer, upto): X_{l+1} = bf16(X_l + y_l) in place; at the layers in
        `checked` (layer -> sampled token), y_l is compared teacher-forced with the oracle."""
        c, ml, X = self.c, self.ml, self.X
        for l in range(self.layer, upto):
            lw = synth.make_layer(4, c.E, c.H, c.I, layer=l, sigma=c.sigma)
            w = self.mq.DeviceWeights.from_host(lw)
            logits = synth.make_logits(4, c.T, c.E, layer=l)
            lg = torch.from_numpy(logits).cuda()
            if l in checked:
                torch.cuda.synchronize()
                x_bits = X.cpu().numpy().view(np.uint16).copy()
                y = ml.forward(X, lg, w)                   # teacher-forced: no residual
                torch.cuda.synchronize()
                ids = ml.topk_ids.cpu().numpy().reshape(c.T, c.k)
                tok = checked[l]
                ref = oracle.layer_forward(x_bits, logits, c.k, lw, tokens=[tok])
                np.testing.assert_array_equal(ids, ref["ids"])
                rel = _rows_rel(y.cpu().numpy().view(np.uint16)[[tok]], ref["y"][[tok]])
                assert np.isfinite(rel[0]) and rel[0] <= ROW_REL_TOL, (l, rel[0])
            ml.forward(X, lg, w, residual=X, out=X)        # X_{l+1} = bf16(X_l + y_l)
            del w
            print(f"stack layer {l} done", flush=True)
        self.layer = upto
        torch.cuda.synchronize()
        xf = oracle.bf16_to_f64(X.cpu().numpy().view(np.uint16))
        assert np.all(np.isfinite(xf)) and np.abs(xf).max() < 64.0


@pytest.fixture(scope="module")
def stack32():
    return _Stack()


@pytest.mark.timeout(600)
def test_glm_stack32_layers_0_7(stack32):
    stack32.advance(8, {0: 5})


@pytest.mark.timeout(600)
def test_glm_stack32_layers_8_15(stack32):
    assert stack32.layer == 8
    stack32.advance(16, {13: 40})


@pytest.mark.timeout(600)
def test_glm_stack32_layers_16_23(stack32):
    assert stack32.layer == 16
    stack32.advance(24, {})


@pytest.mark.timeout(600)
def test_glm_stack32_layers_24_31(stack32):
    assert stack32.layer == 24
    stack32.advance(32, {31: 63})
