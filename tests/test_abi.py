"""The C-ABI calls reject bad arguments before launching anything.

These pass a fake device address (FAKE) to calls that must fail in their host-side checks, so
they run only where no GPU is visible: on a machine with a GPU a regression in those checks
would launch kernels on that address.
"""
import numpy as np
import pytest
import torch

import codebook_quantized_moe_amd as mq

pytestmark = pytest.mark.skipif(
    torch.cuda.is_available(),
    reason="fake device addresses: host-side validation is tested only where no GPU is visible")

GOOD_TABLES = np.array([[0.13, 0.39, 0.66, 0.94, 1.26, 1.62, 2.07, 2.73],
                        [0, .5, 1, 1.5, 2, 3, 4, 6]], np.float32)
FAKE = 4096   # a non-null, 16-byte aligned address; never dereferenced by a failing call


def _status(fn, *args, **kw):
    with pytest.raises(mq.MoeqError) as ei:
        fn(*args, **kw)
    return ei.value.status


def test_route_validation():
    assert _status(mq.moeq_route_topk, FAKE, 4, 256, 0, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_route_topk, FAKE, 4, 8, 9, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_route_topk, FAKE, 4, 300, 8, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_route_topk, None, 4, 256, 8, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_route_topk, FAKE, 4, 256, 8, FAKE, FAKE, gating=3,
                   stream=0) == mq.MOEQ_EINVAL
    assert "gating" in mq.moeq_last_error()
    mq.moeq_route_topk(None, 0, 256, 8, None, None, stream=0)       # T = 0: no-op, OK


def test_router_validation():
    f = mq.moeq_router_logits
    assert _status(f, FAKE, 4, 0, FAKE, 256, FAKE, stream=0) == mq.MOEQ_EINVAL      # H <= 0
    assert _status(f, FAKE, -1, 64, FAKE, 256, FAKE, stream=0) == mq.MOEQ_EINVAL    # T < 0
    assert _status(f, FAKE, 4, 64, FAKE, 0, FAKE, stream=0) == mq.MOEQ_EINVAL       # E < 1
    assert _status(f, FAKE, 4, 64, FAKE, 257, FAKE, stream=0) == mq.MOEQ_EINVAL     # E > 256
    assert _status(f, FAKE, 4, 96, FAKE, 256, FAKE, stream=0) == mq.MOEQ_EUNSUPPORTED
    assert "multiple of 64" in mq.moeq_last_error()
    assert _status(f, FAKE, 1 << 20, 1024, FAKE, 256, FAKE, stream=0) == mq.MOEQ_EUNSUPPORTED
    assert _status(f, None, 4, 64, FAKE, 256, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(f, FAKE, 4, 64, FAKE, 256, None, stream=0) == mq.MOEQ_EINVAL
    assert _status(f, FAKE + 8, 4, 64, FAKE, 256, FAKE, stream=0) == mq.MOEQ_EUNSUPPORTED
    assert _status(f, FAKE, 4, 64, FAKE, 256, FAKE + 2, stream=0) == mq.MOEQ_EUNSUPPORTED
    f(None, 0, 64, None, 256, None, stream=0)                       # T = 0: no-op, OK
    # the sigmoid gating is a known mode: a bad size still fails on the size, not the mode
    assert _status(mq.moeq_route_topk, FAKE, 4, 8, 9, FAKE, FAKE,
                   gating=mq.MOEQ_GATING_SIGMOID_TOPK, stream=0) == mq.MOEQ_EINVAL
    assert "gating" not in mq.moeq_last_error()
    mq.moeq_route_topk(None, 0, 256, 8, None, None, gating=mq.MOEQ_GATING_SIGMOID_TOPK, stream=0)


def test_permute_validation():
    assert _status(mq.moeq_permute_by_expert, FAKE, 4, 8, 0, FAKE, FAKE, FAKE,
                   stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_permute_by_expert, None, 4, 8, 256, FAKE, FAKE, FAKE,
                   stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_permute_by_expert, FAKE, 4, 8, 256, None, FAKE, FAKE,
                   stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_permute_by_expert, FAKE, 1 << 29, 8, 256, FAKE, FAKE, FAKE,
                   stream=0) == mq.MOEQ_EINVAL


def _gateup(**over):
    a = dict(x=FAKE, T=8, H=6144, I=2048, E=256, k=8, expert_offsets=FAKE, sorted_pair=FAKE,
             gate_codes=FAKE, gate_scales=FAKE, up_codes=FAKE, up_scales=FAKE,
             tables=GOOD_TABLES, table_id=FAKE, inter=FAKE, ws=None, ws_bytes=0, stream=0)
    a.update(over)
    return a


def test_gateup_validation():
    bad = [
        (dict(H=6000), mq.MOEQ_EUNSUPPORTED),
        (dict(I=100), mq.MOEQ_EUNSUPPORTED),
        (dict(k=0), mq.MOEQ_EINVAL),
        (dict(E=257), mq.MOEQ_EINVAL),
        (dict(x=None), mq.MOEQ_EINVAL),
        (dict(table_id=None), mq.MOEQ_EINVAL),
        (dict(gate_codes=FAKE + 8), mq.MOEQ_EUNSUPPORTED),
        (dict(gate_scales=FAKE + 2), mq.MOEQ_EUNSUPPORTED),
        (dict(tables=np.zeros((5, 8), np.float32)), mq.MOEQ_EINVAL),
        (dict(tables=np.array([[np.nan] * 8], np.float32)), mq.MOEQ_EINVAL),
        (dict(tables=np.array([[np.inf] + [1] * 7], np.float32)), mq.MOEQ_EINVAL),
        (dict(tables=np.array([[-0.0] + [1] * 7], np.float32)), mq.MOEQ_EINVAL),
        (dict(tables=np.array([[1.0] * 7 + [-2.0]], np.float32)), mq.MOEQ_EINVAL),
    ]
    for over, code in bad:
        assert _status(mq.moeq_gateup_swiglu, **_gateup(**over)) == code, over


def test_projections_accept_no_tokens():
    """T = 0 is a no-op with NULL per-token arrays (an empty tensor's address is NULL), as for
    routing, permutation and combine; sizes and tables are still checked first."""
    none = dict(x=None, T=0, expert_offsets=None, sorted_pair=None, inter=None)
    mq.moeq_gateup_swiglu(**_gateup(**none))
    assert mq.moeq_last_error() == ""
    mq.moeq_down(None, 0, 6144, 2048, 256, 8, None, None, None, FAKE, FAKE, GOOD_TABLES, FAKE,
                 None, stream=0)
    assert mq.moeq_last_error() == ""
    assert _status(mq.moeq_gateup_swiglu, **_gateup(H=6000, **none)) == mq.MOEQ_EUNSUPPORTED
    assert _status(mq.moeq_gateup_swiglu,
                   **_gateup(tables=np.array([[np.nan] * 8], np.float32), **none)) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_down, None, -1, 6144, 2048, 256, 8, None, None, None, FAKE, FAKE,
                   GOOD_TABLES, FAKE, None, stream=0) == mq.MOEQ_EINVAL


def test_down_and_combine_validation():
    assert _status(mq.moeq_down, FAKE, 8, 6144, 2048, 256, 8, FAKE, FAKE, None, FAKE, FAKE,
                   GOOD_TABLES, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL       # topk_w NULL
    assert _status(mq.moeq_down, FAKE, 8, 6144, 2048, 256, 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                   GOOD_TABLES, FAKE, FAKE + 4, stream=0) == mq.MOEQ_EUNSUPPORTED
    assert _status(mq.moeq_unpermute_combine, FAKE, FAKE, FAKE, 8, 8, 256, 6146, None, FAKE,
                   stream=0) == mq.MOEQ_EUNSUPPORTED
    assert _status(mq.moeq_unpermute_combine, None, FAKE, FAKE, 8, 8, 256, 6144, None, FAKE,
                   stream=0) == mq.MOEQ_EINVAL
    assert _status(mq.moeq_unpermute_combine, FAKE, FAKE, FAKE, 8, 8, 256, 6144, FAKE + 2, FAKE,
                   stream=0) == mq.MOEQ_EUNSUPPORTED


def test_debug_dequant_validation():
    assert _status(mq.moeq_debug_dequant, FAKE, FAKE, 1, 1, 96, GOOD_TABLES, FAKE, FAKE,
                   stream=0) == mq.MOEQ_EUNSUPPORTED
    assert _status(mq.moeq_debug_dequant, FAKE, FAKE, 0, 1, 64, GOOD_TABLES, FAKE, FAKE,
                   stream=0) == mq.MOEQ_EINVAL


def test_last_error_is_cleared_on_success():
    _status(mq.moeq_route_topk, None, 4, 256, 8, FAKE, FAKE, stream=0)
    assert mq.moeq_last_error() != ""
    mq.moeq_route_topk(None, 0, 256, 8, None, None, stream=0)
    assert mq.moeq_last_error() == ""


def test_workspace_contract():
    # 256 bytes of work-queue counters + T * H bf16 values (the pair-split copy of x),
    # rounded up to 256 bytes; 0 for T = 0
    assert mq.moeq_workspace_bytes(8, 8, 256, 6144, 2048) == 256 + 8 * 6144 * 2
    assert mq.moeq_workspace_bytes(3, 8, 256, 64, 64) == 256 + 512
    assert mq.moeq_workspace_bytes(0, 8, 256, 6144, 2048) == 0
    need = mq.moeq_workspace_bytes(8, 8, 256, 6144, 2048)
    assert _status(mq.moeq_gateup_swiglu, **_gateup()) == mq.MOEQ_EWORKSPACE
    assert _status(mq.moeq_gateup_swiglu, **_gateup(ws=FAKE, ws_bytes=need - 1)) == \
        mq.MOEQ_EWORKSPACE
    assert _status(mq.moeq_gateup_swiglu, **_gateup(ws=FAKE + 8, ws_bytes=need)) == \
        mq.MOEQ_EUNSUPPORTED
    assert str(need) in mq.moeq_last_error() or "aligned" in mq.moeq_last_error()


def _shared(**over):
    ws_need = mq.moeq_shared_workspace_bytes(8, 6144, 2048)
    a = dict(x=FAKE, T=8, H=6144, I=2048, gate_codes=FAKE, gate_scales=FAKE, up_codes=FAKE,
             up_scales=FAKE, down_codes=FAKE, down_scales=FAKE, tables=GOOD_TABLES,
             table_id=FAKE, inter=FAKE, z=FAKE, ws=FAKE, ws_bytes=ws_need, stream=0)
    a.update(over)
    return a


def test_shared_expert_contract():
    # identity routing (256 + 2 * 256-rounded T ints) + the projections' workspace for T rows
    assert mq.moeq_shared_workspace_bytes(8, 6144, 2048) == \
        256 + 2 * 256 + mq.moeq_workspace_bytes(8, 1, 1, 6144, 2048)
    assert mq.moeq_shared_workspace_bytes(100, 64, 64) == \
        256 + 2 * 512 + mq.moeq_workspace_bytes(100, 1, 1, 64, 64)
    assert mq.moeq_shared_workspace_bytes(0, 6144, 2048) == 0
    need = mq.moeq_shared_workspace_bytes(8, 6144, 2048)
    bad = [
        (dict(ws=None), mq.MOEQ_EWORKSPACE),
        (dict(ws_bytes=need - 1), mq.MOEQ_EWORKSPACE),
        (dict(ws=FAKE + 16), mq.MOEQ_EUNSUPPORTED),         # 256-byte alignment
        (dict(H=6000, ws_bytes=1 << 30), mq.MOEQ_EUNSUPPORTED),
        (dict(I=100), mq.MOEQ_EUNSUPPORTED),
        (dict(T=-1), mq.MOEQ_EINVAL),
        (dict(x=None), mq.MOEQ_EINVAL),
        (dict(down_codes=None), mq.MOEQ_EINVAL),           # the down projection is checked too
        (dict(down_scales=FAKE + 2), mq.MOEQ_EUNSUPPORTED),
        (dict(z=FAKE + 4), mq.MOEQ_EUNSUPPORTED),
        (dict(table_id=None), mq.MOEQ_EINVAL),
        (dict(tables=np.array([[np.nan] * 8], np.float32)), mq.MOEQ_EINVAL),
    ]
    for over, code in bad:
        assert _status(mq.moeq_shared_expert, **_shared(**over)) == code, over
        assert "moeq_shared_expert" in mq.moeq_last_error()
    mq.moeq_shared_expert(**_shared(T=0, x=None, ws=None, ws_bytes=0))   # T = 0: no-op, OK
    f = mq.moeq_unpermute_combine_shared
    assert _status(f, FAKE, FAKE, FAKE, 8, 8, 256, 6144, FAKE + 4, None, FAKE,
                   stream=0) == mq.MOEQ_EUNSUPPORTED
    assert _status(f, FAKE, FAKE, FAKE, 8, 8, 256, 6146, FAKE, None, FAKE,
                   stream=0) == mq.MOEQ_EUNSUPPORTED
    assert _status(f, None, FAKE, FAKE, 8, 8, 256, 6144, FAKE, None, FAKE,
                   stream=0) == mq.MOEQ_EINVAL
    f(None, None, None, 0, 8, 256, 6144, None, None, None, stream=0)   # T = 0: no-op, OK


def test_quantizer_validation():
    q = mq.moeq_quantize
    ok = dict(w=FAKE, E=2, N=4, K=64, tables=GOOD_TABLES, table_id=FAKE, codes=FAKE, scales=FAKE,
              row_err=FAKE, stream=0)
    bad = [
        (dict(K=48), mq.MOEQ_EUNSUPPORTED),
        (dict(K=16), mq.MOEQ_EINVAL),
        (dict(E=0), mq.MOEQ_EINVAL),
        (dict(w=None), mq.MOEQ_EINVAL),
        (dict(table_id=None), mq.MOEQ_EINVAL),
        (dict(codes=FAKE + 8), mq.MOEQ_EUNSUPPORTED),
        (dict(row_err=FAKE + 4), mq.MOEQ_EUNSUPPORTED),
        (dict(tables=np.array([[0, .5, 1, 1.5, 2, 3, 6, 4]], np.float32)), mq.MOEQ_EINVAL),
        (dict(tables=np.zeros((1, 8), np.float32)), mq.MOEQ_EINVAL),
    ]
    for over, code in bad:
        a = dict(ok)
        a.update(over)
        assert _status(q, **a) == code, over
    assert "non-decreasing" in mq.moeq_last_error() or "positive" in mq.moeq_last_error()
    ls = mq.moeq_lloyd_stats
    need = mq.moeq_lloyd_workspace_bytes(2, 4)
    assert need == 2 * 24 * 8                  # 8 rows: 2 workgroups of 24 fp64 sums
    assert _status(ls, FAKE, 2, 4, 64, GOOD_TABLES[0], 0.0, 0, FAKE, FAKE, need,
                   stream=0) == mq.MOEQ_EINVAL                        # gmax must be > 0
    assert _status(ls, FAKE, 2, 4, 64, GOOD_TABLES[0], 2.73, 0, FAKE, FAKE, need - 1,
                   stream=0) == mq.MOEQ_EWORKSPACE
    assert _status(ls, FAKE, 2, 4, 64, GOOD_TABLES[0], 2.73, 0, None, FAKE, need,
                   stream=0) == mq.MOEQ_EINVAL
    sa = mq.moeq_select_arms
    assert _status(sa, FAKE, FAKE, 0, 4, 0, FAKE, None, stream=0) == mq.MOEQ_EINVAL
    assert _status(sa, FAKE, FAKE, 2, 4, 1, FAKE, None, stream=0) == mq.MOEQ_EINVAL  # accumulate


def test_moe_decode_validation():
    f = mq.moeq_moe_decode
    need = mq.moeq_moe_decode_workspace_bytes(8, 8, 256, 6144, 2048)
    assert need > 8 * 8 * 6144 * 4                       # holds the expert outputs
    ok = dict(x=FAKE, logits=FAKE, T=8, H=6144, I=2048, E=256, k=8, gate_codes=FAKE,
              gate_scales=FAKE, up_codes=FAKE, up_scales=FAKE, down_codes=FAKE, down_scales=FAKE,
              tables=GOOD_TABLES, table_id=FAKE, residual=None, y=FAKE, ws=FAKE, ws_bytes=need,
              stream=0)
    bad = [
        (dict(T=1024, ws_bytes=1 << 40), mq.MOEQ_EUNSUPPORTED),      # T * k above 4096 rows
        (dict(ws_bytes=need - 1), mq.MOEQ_EWORKSPACE),
        (dict(ws=FAKE + 16), mq.MOEQ_EUNSUPPORTED),
        (dict(logits=None), mq.MOEQ_EINVAL),
        (dict(gating=7), mq.MOEQ_EINVAL),
        (dict(H=6000), mq.MOEQ_EUNSUPPORTED),
        (dict(down_codes=None), mq.MOEQ_EINVAL),
        (dict(E=300), mq.MOEQ_EINVAL),
    ]
    for over, code in bad:
        a = dict(ok)
        a.update(over)
        assert _status(f, **a) == code, over
    a = dict(ok)
    a.update(T=0, x=None, ws=None, ws_bytes=0)
    f(**a)                                                 # T = 0: no-op, OK
    assert _status(mq.moeq_moe_decode_check, None, stream=0) == mq.MOEQ_EINVAL


def test_route_permute_validation():
    f = mq.moeq_route_permute
    assert _status(f, FAKE, 4, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(f, FAKE, 4, 256, 8, FAKE, FAKE, None, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(f, None, 4, 256, 8, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0) == mq.MOEQ_EINVAL
    assert _status(f, FAKE, 4, 256, 8, FAKE, FAKE, FAKE, FAKE, FAKE, gating=5,
                   stream=0) == mq.MOEQ_EINVAL
