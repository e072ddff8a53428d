"""Encoding a layer's bf16 experts into the 4-bit format on the GPU, over libmoeq's calls.

Plumbing only: torch holds the device buffers; every pass over the weights is a libmoeq
kernel (moeq_lloyd_stats, moeq_quantize, moeq_select_arms). The host reads back the 24 sums
of each grid-fit round and moeq_lloyd_update forms the next 8 magnitudes from them (the
tables travel to the kernels as host arrays).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (moeq_lloyd_stats, moeq_lloyd_update, moeq_lloyd_workspace_bytes, moeq_quantize,
               moeq_select_arms)

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)


def fit_grid(mats, table0, iters: int, stream=None):
    """Weighted Lloyd-Max over the pooled ratios of the bf16 matrices `mats` (device int16
    tensors [E, N, K]): block exponents from table0's top magnitude, then `iters` rounds of
    assignment and update. Returns (fp32 table, per-round sum of weighted squared error)."""
    dev = mats[0].device
    tab = np.asarray(table0, np.float32).copy()
    g0 = float(tab[7])
    stats = torch.zeros(24, dtype=torch.float64, device=dev)
    need = max(moeq_lloyd_workspace_bytes(m.shape[0], m.shape[1]) for m in mats)
    ws = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    dist = []
    for _ in range(iters):
        for i, m in enumerate(mats):
            E, N, K = m.shape
            moeq_lloyd_stats(m, E, N, K, tab, g0, i > 0, stats, ws, need, stream=stream)
        tab, err = moeq_lloyd_update(stats.cpu().numpy(), tab)
        dist.append(err)
    return tab, dist


def encode_layer(gate, up, down, grid, stream=None):
    """Encode one layer's experts (device int16 bf16 bits: gate, up [E, I, H], down [E, H, I])
    against the fitted grid and E2M1, each expert keeping the table with the smaller total
    reconstruction error over its three matrices (ties keep the grid). Returns a dict of
    device tensors: {gate,up,down}_{codes,scales}, table_id [E] u8, expert_err [E, 2] fp64,
    and the host tables [2, 8]."""
    dev = gate.device
    E = gate.shape[0]
    tables = np.stack([np.asarray(grid, np.float32), E2M1])
    ids = [torch.full((E,), t, dtype=torch.uint8, device=dev) for t in (0, 1)]
    table_id = torch.empty(E, dtype=torch.uint8, device=dev)
    expert_err = torch.zeros(2 * E, dtype=torch.float64, device=dev)
    for i, m in enumerate((gate, up, down)):
        _, N, K = m.shape
        errs = [torch.empty(E * N, dtype=torch.float64, device=dev) for _ in range(2)]
        for t in (0, 1):
            moeq_quantize(m, E, N, K, tables, ids[t], None, None, errs[t], stream=stream)
        moeq_select_arms(errs[0], errs[1], E, N, i > 0, table_id, expert_err, stream=stream)
    out = dict(table_id=table_id, expert_err=expert_err.view(E, 2), tables=tables)
    for name, m in (("gate", gate), ("up", up), ("down", down)):
        _, N, K = m.shape
        codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
        moeq_quantize(m, E, N, K, tables, table_id, codes, scales, None, stream=stream)
        out[name + "_codes"], out[name + "_scales"] = codes, scales
    return out
