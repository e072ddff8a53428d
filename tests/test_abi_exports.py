"""The C-ABI library loads and exports every symbol include/moeq.h declares (no compute
call: these run with or without a GPU)."""
import ctypes
import os
import re

import numpy as np

import codebook_quantized_moe_amd as mq

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moeq.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(moeq_[a-z_]+)\s*\(", src))
    names.discard("moeq_inter_slot")           # static inline helper in the header
    return sorted(names)


def test_header_symbols_exported():
    names = _declared()
    assert set(names) == set(mq.EXPORTED)
    lib = ctypes.CDLL(mq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_inter_slot_matches_header_rule():
    c = np.arange(64)
    s = mq.inter_slot(c)
    assert sorted(s) == list(range(64))
    np.testing.assert_array_equal(s[:8], [0, 4, 1, 5, 2, 6, 3, 7])


def test_lloyd_update_on_the_host_equals_the_oracle():
    """moeq_lloyd_update runs on the host (no device work): the next table from the sums of a
    grid-fit round, an empty cell keeping its magnitude, against the oracle's update."""
    import oracle
    g = np.random.default_rng(5)
    table = np.sort(g.uniform(0.05, 3.0, 8)).astype(np.float32)
    stats = np.abs(g.standard_normal((3, 8))) * 10.0
    stats[0] = stats[1] * (table + g.uniform(-0.05, 0.05, 8))     # weighted means near the levels
    stats[:, 3] = 0.0                                              # an empty cell
    nxt, err = mq.moeq_lloyd_update(stats.ravel(), table)
    np.testing.assert_array_equal(nxt, oracle.lloyd_update(table, stats))
    assert nxt[3] == table[3]
    assert err == sum(float(v) for v in stats[2])
    lib = ctypes.CDLL(mq.LIB_PATH)
    lib.moeq_lloyd_update.argtypes = [ctypes.c_void_p] * 4
    assert lib.moeq_lloyd_update(None, table.ctypes.data, nxt.ctypes.data, None) == mq.MOEQ_EINVAL
