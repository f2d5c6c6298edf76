"""Test helpers: decode the published v_f8 layout and compare the HIP path
with the oracle.  (Test code: may import the oracle.)"""
from __future__ import annotations

import numpy as np
import torch

from oracle import fp8_e4m3 as F8
from oracle import sage_oracle as O

KV_TILE = 128


def v_layout_index(d: int):
    """For one 128-key tile: (key, chan) of every byte offset, from sage.h's formula."""
    off = np.arange(KV_TILE * d)
    i = off % 16
    L = (off // 16) % 64
    p = (off // 1024) % 2
    cb = (off // 2048) % (d // 32)
    kb = off // (2048 * (d // 32))
    chan = cb * 32 + (L % 32)
    s = p * 16 + i
    g = L // 32
    key = kb * 64 + (s // 16) * 32 + ((s % 16) // 4) * 8 + g * 4 + (s % 4)
    return key, chan


def v_natural(v_f8: np.ndarray, N: int, d: int) -> np.ndarray:
    """uint8 [B, H_kv, ntile*128*d] in the sage.h layout -> uint8 [B, H_kv, N, d]."""
    B, Hk, tot = v_f8.shape
    nt = tot // (KV_TILE * d)
    key, chan = v_layout_index(d)
    out = np.zeros((B, Hk, nt * KV_TILE, d), dtype=np.uint8)
    raw = v_f8.reshape(B, Hk, nt, KV_TILE * d)
    for t in range(nt):
        out[:, :, t * KV_TILE + key, chan] = raw[:, :, t, :]
    return out[:, :, :N], out[:, :, N:]


def to_np(t):
    return t.detach().cpu().numpy()


def compare_output(o_gpu: torch.Tensor, o_ref: np.ndarray, max_abs=2e-2, cos_min=0.9995):
    a = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    m = O.metrics(a, o_ref)
    assert np.isfinite(a).all(), "non-finite output"
    assert m["max_abs"] <= max_abs and m["cos"] >= cos_min, m
    return m
