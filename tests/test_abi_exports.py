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
