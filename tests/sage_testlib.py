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


def _dtype_name(t) -> str:
    return {torch.float16: "fp16", torch.bfloat16: "bf16"}[t.dtype]


def compare_output(o_gpu: torch.Tensor, o_ref: np.ndarray, max_abs=2e-2, cos_min=0.9995):
    """The HIP output against the oracle's float64 result rounded once to the
    output dtype (as the kernel rounds its own): max-abs <= 2e-2 and cosine >= 0.9995."""
    a = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    ref = O.round_output(np.asarray(o_ref, dtype=np.float64), _dtype_name(o_gpu))
    m = O.metrics(a, ref)
    assert np.isfinite(a).all(), "non-finite output"
    assert m["max_abs"] <= max_abs and m["cos"] >= cos_min, m
    return m


def v4_natural(v_f4: np.ndarray, v_e8: np.ndarray, N: int, d: int):
    """The sage.h MXFP4 V layout -> (E2M1 codes uint8 [B, H_kv, Np, d], exponents
    int64 [B, H_kv, Np/32, d]), Np = N rounded up to 128."""
    B, Hk, tot = v_f4.shape
    nt = tot // (64 * d)
    ncb = d // 32
    raw = v_f4.reshape(B, Hk, nt, 2, ncb, 64, 16)
    lo, hi = raw & 0xF, raw >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(B, Hk, nt, 2, ncb, 64, 32)     # nibble p
    codes = np.zeros((B, Hk, nt * 128, d), dtype=np.uint8)
    p = np.arange(32)
    kin = 8 * ((p % 16) // 4) + 4 * (p // 16) + (p % 4)                       # key in block
    for h in range(2):
        for cb in range(ncb):
            for lane in range(64):
                chan = cb * 32 + lane % 32
                key0 = h * 64 + (lane // 32) * 32
                for t in range(nt):
                    codes[:, :, t * 128 + key0 + kin, chan] = nib[:, :, t, h, cb, lane, :]
    sc = v_e8.reshape(B, Hk, nt, 2, 64, 4)[..., :ncb].astype(np.int64) - 127     # [.., h, lane, cb]
    e = np.zeros((B, Hk, nt * 4, d), dtype=np.int64)
    for h in range(2):
        for lane in range(64):
            g = lane // 32
            for cb in range(ncb):
                chan = cb * 32 + lane % 32
                e[:, :, np.arange(nt) * 4 + 2 * h + g, chan] = sc[:, :, :, h, lane, cb]
    return codes, e


def compare_output_mx(o_gpu, o_ref, max_abs=2e-2, cos_min=0.9995):
    """MXFP4 P V: the kernel and the oracle decide the E2M1 codes and block exponents on
    the same float32 P~ values, so the bar is the FP8 one."""
    return compare_output(o_gpu, o_ref, max_abs=max_abs, cos_min=cos_min)


def lse_tol(N, lse_ref, corr=0.0):
    """Bound on |lse_gpu - lse_oracle|.  Both sides take ln 2 (m + log2 l) from the same
    float32 running max m and the same float32 P~ (up to one ulp of an exponential); l
    is a float32 sum of at most N positive terms on the GPU (relative error <= N 2^-24)
    and float64 in the oracle; log2, the add and the multiply by ln 2 each round once at
    the magnitude of the result (|lse| + 20 bounds |m| + |log2 l| here).  The correction
    is an fp32 dot product, within ~1e-6 of its magnitude."""
    return N * 2.0 ** -23 + (np.abs(lse_ref) + 20.0) * 2.0 ** -21 + 1e-6 * np.abs(corr) + 1e-6
