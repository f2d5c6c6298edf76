"""MI355X (gfx950) quantized attention forward pass: Python binding.

A thin ctypes layer over ``libsage_amd.so`` (the C ABI in ``include/sage.h``).
It only marshals arguments: every step of the method runs in the HIP
kernels; PyTorch provides device memory and the current stream.  There is no
CPU fallback -- if the library is not built or no GPU is visible, calls fail.

The method (SageAttention2 detail page, Algorithm 1, with INT8 Q/K):
smooth K by its token mean, quantize Q (per 128, 32 or 1 tokens) and K (per 64
tokens) to INT8 with FP32 scales, quantize V per channel to FP8 E4M3, then run a tiled
online-softmax attention with INT8 QK^T and FP8 PV (P scaled by 448).

Entry points (same names as the C ABI):
    sage_buffer_sizes(B, H, H_kv, N, d, q_group=128) -> dict of byte sizes
    sage_quant_qk(q, k, smooth_k=True, q_group=128, smooth_q=False)
        -> dict(q_i8, q_scale, k_i8, k_scale, k_mean[, q_mean])
    sage_delta_s(k, qk, sm_scale, i0=0, nrows=None) -> fp32 [B, H, nrows, N] (smooth Q rows)
    sage_quant_v(v) -> dict(v_f8, v_scale)
    sage_quant_qkv(q, k, v, smooth_k=True, q_group=128, smooth_q=False) -> (qk, vq): both in one call
    sage_quant_v_mxfp4(v) -> dict(v_f4, v_e8) (MXFP4 V)
    sage_attn_fwd(qk, vq, causal=..., sm_scale=..., out_dtype=...) -> o
    sage_attn_fwd_lse(qk, vq, causal=..., sm_scale=..., lse_corr=None) -> (o, lse)
    sage_attn_fwd_smooth_q(qk, vq, k, causal=..., sm_scale=..., return_lse=False,
        lse_corr=None, workspace=None) -> o or (o, lse) (smoothed Q, Delta S in chunks)
    sage_attn_fwd_mxfp4(qk, vq4, causal=..., sm_scale=..., return_lse=False) -> o or (o, lse)
    sage_lse_correction(q, k_mean, sm_scale) -> fp32 [B, H, N]
    sage_qk_int32(q_i8, k_i8, b, h) -> int32 [N, N] (diagnostic)
    sage_quant_qk_noalloc(q, k, smooth_k=True, q_group=128, smooth_q=False, out=...)
        -> as sage_quant_qk, with the library's fixed scratch array (allocates nothing)
    sage_mfma_peak(kind=0, iters=48000, nwg=256) -> (ops, clocks, sink, wall_khz)
        (roofline diagnostic: a dense MFMA loop and the clock it runs at)
and the composition ``sageattn(q, k, v, is_causal=False, sm_scale=None,
smooth_k=True, return_lse=False, q_group=128, smooth_q=False)``.  ``q_group`` is the number of
consecutive Q tokens per scale: 128 (per block), 32 (per wave, the per-warp
granularity) or 1 (per query, the per-thread granularity); the attention
entry points read it from the length of ``q_scale``.  ``smooth_q`` subtracts each
128-token Q block's mean before quantizing and adds the Delta S term back to
the scores (Algorithm 1's GEMV compensation), computed a chunk of heads and Q blocks at a
time into a bounded workspace.  ``pv="mxfp4"`` runs P V in MXFP4
(E2M1 with E8M0 scales per 32 keys, the OCP format the pages name for MI350-class
GPUs) on the FP4 matrix cores.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["SageError", "library_path", "load_library", "sage_buffer_sizes", "sage_quant_qk",
           "sage_quant_v", "sage_quant_v_mxfp4", "sage_delta_s", "sage_attn_fwd",
           "sage_attn_fwd_lse", "sage_attn_fwd_smooth_q", "sage_attn_fwd_mxfp4",
           "sage_lse_correction",
           "sage_qk_int32", "sage_quant_qk_noalloc", "sage_quant_qkv", "sage_mfma_peak",
           "sageattn", "SagePlan",
           "smooth_q_workspace", "BLKQ", "BLKK",
           "KV_TILE", "Q_GROUPS", "SCRATCH_BYTES"]

BLKQ, BLKK, KV_TILE = 128, 64, 128
Q_GROUPS = (128, 32, 1)   # Q tokens per scale: per block, per wave, per query
_FP16, _BF16 = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))


class SageError(RuntimeError):
    def __init__(self, status: int, msg: str, where: str):
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


class _Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_f8", "v_scale", "o",
        "ws_quant_qk", "ws_quant_v", "q_mean", "ws_smooth_q", "v_f4", "v_e8", "ws_quant_qkv")]


_lib = None


def library_path() -> str:
    return os.path.join(_HERE, "libsage_amd.so")


def load_library():
    """Load libsage_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m quantized_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sage_abi_version.restype = i
    lib.sage_status_str.argtypes = [i]
    lib.sage_status_str.restype = ctypes.c_char_p
    lib.sage_buffer_sizes.argtypes = [i, i, i, i, i, i, ctypes.POINTER(_Sizes)]
    lib.sage_quant_qk.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp,
                                  sz, vp]
    lib.sage_delta_s.argtypes = [vp, i, vp, vp, i, i, i, i, i, ctypes.c_float, i, i, vp, vp]
    lib.sage_quant_v.argtypes = [vp, i, i, i, i, i, vp, vp, vp, sz, vp]
    lib.sage_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                  ctypes.c_float, vp]
    lib.sage_attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, i,
                                      i, i, ctypes.c_float, vp]
    lib.sage_attn_fwd_smooth_q.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, vp, i, vp, vp,
                                           i, i, i, i, i, i, i, ctypes.c_float, vp, sz, vp]
    lib.sage_lse_correction.argtypes = [vp, i, vp, i, i, i, i, i, ctypes.c_float, vp, vp]
    lib.sage_quant_v_mxfp4.argtypes = [vp, i, i, i, i, i, vp, vp, vp]
    lib.sage_attn_fwd_mxfp4.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, i,
                                        i, ctypes.c_float, vp]
    lib.sage_qk_int32.argtypes = [vp, vp, i, i, i, i, i, i, i, vp, vp]
    lib.sage_quant_qk_noalloc.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, vp, vp, vp, vp, vp,
                                          vp, vp]
    lib.sage_quant_qkv.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp,
                                   vp, vp, vp, sz, vp]
    lib.sage_mfma_peak.argtypes = [i, i, i, vp, vp, ctypes.POINTER(i), vp]
    for f in ("sage_buffer_sizes", "sage_quant_qk", "sage_delta_s", "sage_quant_v", "sage_attn_fwd",
              "sage_attn_fwd_lse", "sage_lse_correction", "sage_qk_int32", "sage_quant_v_mxfp4",
              "sage_attn_fwd_mxfp4", "sage_quant_qk_noalloc", "sage_quant_qkv",
              "sage_attn_fwd_smooth_q", "sage_mfma_peak"):
        getattr(lib, f).restype = i
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        msg = load_library().sage_status_str(status).decode()
        raise SageError(status, msg, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dt(dtype) -> int:
    if dtype == torch.float16:
        return _FP16
    if dtype == torch.bfloat16:
        return _BF16
    raise TypeError(f"q/k/v must be float16 or bfloat16, got {dtype}")


def _need_gpu(*ts):
    for t in ts:
        if not (isinstance(t, torch.Tensor) and t.is_cuda):
            raise ValueError("all tensors must be CUDA (HIP) device tensors")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_sizes(where: str, sizes: dict, **bufs):
    """Each given buffer must hold at least the bytes sage_buffer_sizes names for
    the shapes (a shorter one would be read or written past its end)."""
    for name, t in bufs.items():
        if t is not None and _nbytes(t) < sizes[name]:
            raise ValueError(f"{where}: {name} holds {_nbytes(t)} bytes; the shapes need "
                             f"{sizes[name]}")


def _check_tensor(where: str, name: str, t, shape, dtype):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{where}: {name} must be {dtype} {list(shape)}, got {t.dtype} "
                         f"{list(t.shape)}")


def sage_buffer_sizes(B: int, H: int, H_kv: int, N: int, d: int, q_group: int = BLKQ) -> dict:
    s = _Sizes()
    _check(load_library().sage_buffer_sizes(B, H, H_kv, N, d, q_group, ctypes.byref(s)),
           "sage_buffer_sizes")
    return {n: getattr(s, n) for n, _ in _Sizes._fields_}


def _q_group_of(q_scale: torch.Tensor, N: int) -> int:
    """The Q granularity a q_scale tensor was written for.  Where two
    groupings give the same length (N <= 32) every query reads scale 0 under
    either, so the choice does not matter."""
    for g in Q_GROUPS:
        if q_scale.shape[-1] == -(-N // g):
            return g
    raise ValueError(f"q_scale has {q_scale.shape[-1]} scales per head; expected "
                     f"ceil(N / g) for g in {Q_GROUPS} with N = {N}")


def _alloc_qk(B, H, H_kv, N, d, device, q_group=BLKQ, smooth_q=False):
    nq, nk = -(-N // q_group), -(-N // BLKK)
    out = dict(
        q_i8=torch.empty((B, H, N, d), dtype=torch.int8, device=device),
        q_scale=torch.empty((B, H, nq), dtype=torch.float32, device=device),
        k_i8=torch.empty((B, H_kv, N, d), dtype=torch.int8, device=device),
        k_scale=torch.empty((B, H_kv, nk), dtype=torch.float32, device=device),
        k_mean=torch.empty((B, H_kv, d), dtype=torch.float32, device=device),
    )
    if smooth_q:
        out["q_mean"] = torch.empty((B, H, -(-N // BLKQ), d), dtype=torch.float32, device=device)
    return out


def _alloc_v(B, H_kv, N, d, device):
    npad = -(-N // KV_TILE) * KV_TILE
    return dict(
        v_f8=torch.empty((B, H_kv, npad * d), dtype=torch.uint8, device=device),
        v_scale=torch.empty((B, H_kv, d), dtype=torch.float32, device=device),
    )


def sage_quant_qk(q: torch.Tensor, k: torch.Tensor, smooth_k: bool = True, *,
                  q_group: int = BLKQ, smooth_q: bool = False, out=None, workspace=None,
                  stream=None) -> dict:
    """Smooth K (and, with smooth_q, Q by its 128-block means) and quantize Q
    (q_group tokens per scale) and K to INT8 (see sage.h for exact semantics)."""
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d):
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q_group not in Q_GROUPS:
        raise ValueError(f"q_group must be one of {Q_GROUPS}")
    out = out or _alloc_qk(B, H, H_kv, N, d, q.device, q_group, smooth_q)
    if out["q_scale"].numel() != B * H * -(-N // q_group):
        raise ValueError("out['q_scale'] does not hold ceil(N / q_group) scales per head")
    if smooth_q and "q_mean" not in out:
        raise ValueError("smooth_q needs out['q_mean']")
    sizes = sage_buffer_sizes(B, H, H_kv, N, d, q_group)
    _check_sizes("sage_quant_qk", sizes, q_i8=out["q_i8"], q_scale=out["q_scale"],
                 k_i8=out["k_i8"], k_scale=out["k_scale"], k_mean=out["k_mean"],
                 q_mean=out.get("q_mean") if smooth_q else None)
    _need_gpu(q, k, *(t for n, t in out.items() if n != "q_mean" or smooth_q))
    if workspace is None and smooth_k:
        workspace = torch.empty(sizes["ws_quant_qk"], dtype=torch.uint8, device=q.device)
    st = load_library().sage_quant_qk(
        q.data_ptr(), k.data_ptr(), _dt(q.dtype), B, H, H_kv, N, d, q_group, int(bool(smooth_k)),
        int(bool(smooth_q)), out["q_i8"].data_ptr(), out["q_scale"].data_ptr(),
        out["k_i8"].data_ptr(), out["k_scale"].data_ptr(), out["k_mean"].data_ptr(),
        _ptr(out.get("q_mean")) if smooth_q else None, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream, q.device))
    _check(st, "sage_quant_qk")
    return out


def sage_quant_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, smooth_k: bool = True, *,
                   q_group: int = BLKQ, smooth_q: bool = False, out_qk=None, out_v=None,
                   workspace=None, stream=None):
    """sage_quant_qk and sage_quant_v in one call (three launches, bit-identical results);
    returns (qk dict, vq dict)."""
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise TypeError("q, k and v must share a dtype")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d) or v.shape != (B, H_kv, N, d):
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    if q_group not in Q_GROUPS:
        raise ValueError(f"q_group must be one of {Q_GROUPS}")
    out_qk = out_qk or _alloc_qk(B, H, H_kv, N, d, q.device, q_group, smooth_q)
    out_v = out_v or _alloc_v(B, H_kv, N, d, q.device)
    if smooth_q and "q_mean" not in out_qk:
        raise ValueError("smooth_q needs out_qk['q_mean']")
    sizes = sage_buffer_sizes(B, H, H_kv, N, d, q_group)
    _check_sizes("sage_quant_qkv", sizes, q_i8=out_qk["q_i8"], q_scale=out_qk["q_scale"],
                 k_i8=out_qk["k_i8"], k_scale=out_qk["k_scale"], k_mean=out_qk["k_mean"],
                 q_mean=out_qk.get("q_mean") if smooth_q else None, v_f8=out_v["v_f8"],
                 v_scale=out_v["v_scale"])
    _need_gpu(q, k, v, out_v["v_f8"], out_v["v_scale"],
              *(t for n, t in out_qk.items() if n != "q_mean" or smooth_q))
    if workspace is None:
        workspace = torch.empty(max(sizes["ws_quant_qkv"], 16), dtype=torch.uint8, device=q.device)
    st = load_library().sage_quant_qkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q.dtype), B, H, H_kv, N, d, q_group,
        int(bool(smooth_k)), int(bool(smooth_q)), out_qk["q_i8"].data_ptr(),
        out_qk["q_scale"].data_ptr(), out_qk["k_i8"].data_ptr(), out_qk["k_scale"].data_ptr(),
        out_qk["k_mean"].data_ptr(), _ptr(out_qk.get("q_mean")) if smooth_q else None,
        out_v["v_f8"].data_ptr(), out_v["v_scale"].data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st, "sage_quant_qkv")
    return out_qk, out_v


SCRATCH_BYTES = 16 << 20   # SAGE_SCRATCH_BYTES: the library's fixed scratch array


def sage_quant_qk_noalloc(q: torch.Tensor, k: torch.Tensor, smooth_k: bool = True, *,
                          q_group: int = BLKQ, smooth_q: bool = False, out, stream=None) -> dict:
    """sage_quant_qk with the library's fixed scratch array instead of a workspace: the
    entry point allocates nothing (``out`` must hold every output buffer).  Calls that
    overlap on one GPU share that array and race (see sage.h)."""
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d):
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q_group not in Q_GROUPS:
        raise ValueError(f"q_group must be one of {Q_GROUPS}")
    if smooth_q and "q_mean" not in out:
        raise ValueError("smooth_q needs out['q_mean']")
    sizes = sage_buffer_sizes(B, H, H_kv, N, d, q_group)
    _check_sizes("sage_quant_qk_noalloc", sizes, q_i8=out["q_i8"], q_scale=out["q_scale"],
                 k_i8=out["k_i8"], k_scale=out["k_scale"], k_mean=out["k_mean"],
                 q_mean=out.get("q_mean") if smooth_q else None)
    _need_gpu(q, k, *(t for n, t in out.items() if n != "q_mean" or smooth_q))
    st = load_library().sage_quant_qk_noalloc(
        q.data_ptr(), k.data_ptr(), _dt(q.dtype), B, H, H_kv, N, d, q_group, int(bool(smooth_k)),
        int(bool(smooth_q)), out["q_i8"].data_ptr(), out["q_scale"].data_ptr(),
        out["k_i8"].data_ptr(), out["k_scale"].data_ptr(), out["k_mean"].data_ptr(),
        _ptr(out.get("q_mean")) if smooth_q else None, _stream(stream, q.device))
    _check(st, "sage_quant_qk_noalloc")
    return out


def _alloc_v4(B, H_kv, N, d, device):
    nt = -(-N // KV_TILE)
    return dict(
        v_f4=torch.empty((B, H_kv, nt * KV_TILE * d // 2), dtype=torch.uint8, device=device),
        v_e8=torch.empty((B, H_kv, nt * 512), dtype=torch.uint8, device=device),
    )


def sage_quant_v_mxfp4(v: torch.Tensor, *, out=None, stream=None) -> dict:
    """MXFP4 quantization of V (E2M1 codes, E8M0 scale per 32 keys of a channel) into
    the FP4 fragment layout of sage.h."""
    B, H_kv, N, d = v.shape
    out = out or _alloc_v4(B, H_kv, N, d, v.device)
    _check_sizes("sage_quant_v_mxfp4", sage_buffer_sizes(B, H_kv, H_kv, N, d), v_f4=out["v_f4"],
                 v_e8=out["v_e8"])
    _need_gpu(v, out["v_f4"], out["v_e8"])
    st = load_library().sage_quant_v_mxfp4(v.data_ptr(), _dt(v.dtype), B, H_kv, N, d,
                                           out["v_f4"].data_ptr(), out["v_e8"].data_ptr(),
                                           _stream(stream, v.device))
    _check(st, "sage_quant_v_mxfp4")
    return out


def sage_attn_fwd_mxfp4(qk: dict, vq4: dict, *, causal: bool, sm_scale: float,
                        out_dtype=torch.float16, return_lse: bool = False, lse_corr=None,
                        out=None, lse=None, stream=None):
    """Attention with MXFP4 P V; returns O, or (O, lse) with return_lse."""
    q_i8, k_i8 = qk["q_i8"], qk["k_i8"]
    B, H, N, d = q_i8.shape
    H_kv = k_i8.shape[1]
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q_i8.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q_i8.device)
    _check_attn_inputs("sage_attn_fwd_mxfp4", qk, out, v_f4=vq4["v_f4"], v_e8=vq4["v_e8"])
    _need_gpu(q_i8, qk["q_scale"], k_i8, qk["k_scale"], vq4["v_f4"], vq4["v_e8"], out)
    if return_lse:
        _need_gpu(lse)
        _check_tensor("sage_attn_fwd_mxfp4", "lse", lse, (B, H, N), torch.float32)
    if lse_corr is not None:
        _need_gpu(lse_corr)
        if lse_corr.shape != (B, H, N) or lse_corr.dtype != torch.float32:
            raise ValueError("lse_corr must be float32 [B, H, N]")
    st = load_library().sage_attn_fwd_mxfp4(
        q_i8.data_ptr(), qk["q_scale"].data_ptr(), k_i8.data_ptr(), qk["k_scale"].data_ptr(),
        vq4["v_f4"].data_ptr(), vq4["v_e8"].data_ptr(), out.data_ptr(), _dt(out.dtype),
        _ptr(lse) if return_lse else None, _ptr(lse_corr) if return_lse else None, B, H, H_kv, N,
        d, _q_group_of(qk["q_scale"], N), int(bool(causal)), float(sm_scale),
        _stream(stream, q_i8.device))
    _check(st, "sage_attn_fwd_mxfp4")
    return (out, lse) if return_lse else out


def sage_delta_s(k: torch.Tensor, qk: dict, sm_scale: float, *, i0: int = 0,
                 nrows: int | None = None, out=None, stream=None) -> torch.Tensor:
    """Rows of the Delta S term of smooth Q: sm_scale * log2(e) * q_mean . (k - k_mean)
    for the 128-token Q blocks i0 .. i0 + nrows - 1 (default: all) and every key,
    fp32 [B, H, nrows, N] (see sage.h)."""
    _need_gpu(k, qk["k_mean"], qk["q_mean"])
    B, H, nmb, d = qk["q_mean"].shape
    H_kv, N = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, H_kv, N, d) or nmb != -(-N // BLKQ):
        raise ValueError(f"sage_delta_s: k {list(k.shape)} does not match q_mean "
                         f"{list(qk['q_mean'].shape)}")
    if nrows is None:
        nrows = nmb - i0
    if out is None:
        out = torch.empty((B, H, max(nrows, 0), N), dtype=torch.float32, device=k.device)
    _check_tensor("sage_delta_s", "k_mean", qk["k_mean"], (B, H_kv, d), torch.float32)
    _check_tensor("sage_delta_s", "out", out, (B, H, max(nrows, 0), N), torch.float32)
    _need_gpu(out)
    st = load_library().sage_delta_s(k.data_ptr(), _dt(k.dtype), qk["k_mean"].data_ptr(),
                                     qk["q_mean"].data_ptr(), B, H, H_kv, N, d, float(sm_scale),
                                     int(i0), int(nrows), out.data_ptr(),
                                     _stream(stream, k.device))
    _check(st, "sage_delta_s")
    return out


def sage_quant_v(v: torch.Tensor, *, out=None, workspace=None, stream=None) -> dict:
    """Per-channel FP8 E4M3 quantization of V into the fragment layout of sage.h."""
    B, H_kv, N, d = v.shape
    out = out or _alloc_v(B, H_kv, N, d, v.device)
    sizes = sage_buffer_sizes(B, H_kv, H_kv, N, d)
    _check_sizes("sage_quant_v", sizes, v_f8=out["v_f8"], v_scale=out["v_scale"])
    _need_gpu(v, out["v_f8"], out["v_scale"])
    if workspace is None:
        workspace = torch.empty(sizes["ws_quant_v"], dtype=torch.uint8, device=v.device)
    st = load_library().sage_quant_v(
        v.data_ptr(), _dt(v.dtype), B, H_kv, N, d, out["v_f8"].data_ptr(),
        out["v_scale"].data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream, v.device))
    _check(st, "sage_quant_v")
    return out


def sage_attn_fwd(qk: dict, vq: dict, *, causal: bool, sm_scale: float,
                  out_dtype=torch.float16, out=None, stream=None) -> torch.Tensor:
    """Attention on quantized inputs (Q not smoothed); returns O [B, H, N, d] in out_dtype."""
    q_i8, k_i8 = qk["q_i8"], qk["k_i8"]
    B, H, N, d = q_i8.shape
    H_kv = k_i8.shape[1]
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q_i8.device)
    _check_attn_inputs("sage_attn_fwd", qk, out, v_f8=vq["v_f8"], v_scale=vq["v_scale"])
    _no_q_mean("sage_attn_fwd", qk)
    _need_gpu(q_i8, qk["q_scale"], k_i8, qk["k_scale"], vq["v_f8"], vq["v_scale"], out)
    st = load_library().sage_attn_fwd(
        q_i8.data_ptr(), qk["q_scale"].data_ptr(), k_i8.data_ptr(), qk["k_scale"].data_ptr(),
        vq["v_f8"].data_ptr(), vq["v_scale"].data_ptr(), out.data_ptr(), _dt(out.dtype),
        B, H, H_kv, N, d, _q_group_of(qk["q_scale"], N), int(bool(causal)), float(sm_scale),
        _stream(stream, q_i8.device))
    _check(st, "sage_attn_fwd")
    return out


def _check_attn_inputs(where: str, qk: dict, out, **vbufs):
    """Shapes of the quantized inputs and the output against q_i8's [B, H, N, d]."""
    B, H, N, d = qk["q_i8"].shape
    k_i8 = qk["k_i8"]
    if k_i8.dim() != 4 or (k_i8.shape[0], k_i8.shape[2], k_i8.shape[3]) != (B, N, d):
        raise ValueError(f"{where}: k_i8 {list(k_i8.shape)} does not match q_i8 "
                         f"{list(qk['q_i8'].shape)}")
    H_kv = k_i8.shape[1]
    sizes = sage_buffer_sizes(B, H, H_kv, N, d, _q_group_of(qk["q_scale"], N))
    _check_sizes(where, sizes, q_scale=qk["q_scale"], k_scale=qk["k_scale"], **vbufs)
    if tuple(out.shape) != (B, H, N, d):
        raise ValueError(f"{where}: out must be [B, H, N, d] = {[B, H, N, d]}, got "
                         f"{list(out.shape)}")


def _no_q_mean(where: str, qk: dict):
    """Codes of smoothed Q need the Delta S term: only sage_attn_fwd_smooth_q takes them."""
    if qk.get("q_mean") is not None:
        raise ValueError(f"{where}: Q was smoothed (qk has q_mean); use sage_attn_fwd_smooth_q")


def sage_attn_fwd_lse(qk: dict, vq: dict, *, causal: bool, sm_scale: float,
                      out_dtype=torch.float16, lse_corr=None, out=None, lse=None, stream=None):
    """Attention on quantized inputs plus the row log-sum-exp; returns (o, lse).
    lse [B, H, N] fp32 is ln sum_j exp(S_ij) of the scores the softmax used,
    plus lse_corr (the output of sage_lse_correction) when given."""
    q_i8, k_i8 = qk["q_i8"], qk["k_i8"]
    B, H, N, d = q_i8.shape
    H_kv = k_i8.shape[1]
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q_i8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q_i8.device)
    _check_attn_inputs("sage_attn_fwd_lse", qk, out, v_f8=vq["v_f8"], v_scale=vq["v_scale"])
    _check_tensor("sage_attn_fwd_lse", "lse", lse, (B, H, N), torch.float32)
    _no_q_mean("sage_attn_fwd_lse", qk)
    _need_gpu(q_i8, qk["q_scale"], k_i8, qk["k_scale"], vq["v_f8"], vq["v_scale"], out, lse)
    if lse_corr is not None:
        _need_gpu(lse_corr)
        if lse_corr.shape != (B, H, N) or lse_corr.dtype != torch.float32:
            raise ValueError("lse_corr must be float32 [B, H, N]")
    st = load_library().sage_attn_fwd_lse(
        q_i8.data_ptr(), qk["q_scale"].data_ptr(), k_i8.data_ptr(), qk["k_scale"].data_ptr(),
        vq["v_f8"].data_ptr(), vq["v_scale"].data_ptr(), out.data_ptr(), _dt(out.dtype),
        lse.data_ptr(), _ptr(lse_corr), B, H, H_kv, N, d, _q_group_of(qk["q_scale"], N),
        int(bool(causal)), float(sm_scale), _stream(stream, q_i8.device))
    _check(st, "sage_attn_fwd_lse")
    return out, lse


def smooth_q_workspace(B: int, H: int, N: int, d: int, rows: int | None = None,
                       device="cuda") -> torch.Tensor:
    """Workspace of sage_attn_fwd_smooth_q: the library's default (sizes.ws_smooth_q, which
    depends on B*H and N only), or room for `rows` Q blocks of every head's Delta S rows."""
    nbytes = (sage_buffer_sizes(B, H, H, N, d)["ws_smooth_q"] if rows is None
              else B * H * rows * N * 4)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def sage_attn_fwd_smooth_q(qk: dict, vq: dict, k: torch.Tensor, *, causal: bool,
                           sm_scale: float, out_dtype=torch.float16, return_lse: bool = False,
                           lse_corr=None, workspace=None, out=None, lse=None, stream=None):
    """Attention of smoothed Q (sage_quant_qk with smooth_q): the Delta S term
    q_mean . (k - k_mean) is computed a chunk of heads and Q blocks at a time into `workspace`
    (default: smooth_q_workspace) and added to the scores.  k: the original K.
    Returns O, or (O, lse) with return_lse."""
    q_i8, k_i8 = qk["q_i8"], qk["k_i8"]
    B, H, N, d = q_i8.shape
    H_kv = k_i8.shape[1]
    if qk.get("q_mean") is None:
        raise ValueError("sage_attn_fwd_smooth_q: qk has no q_mean (Q was not smoothed)")
    _check_tensor("sage_attn_fwd_smooth_q", "q_mean", qk["q_mean"], (B, H, -(-N // BLKQ), d),
                  torch.float32)
    _check_tensor("sage_attn_fwd_smooth_q", "k_mean", qk["k_mean"], (B, H_kv, d), torch.float32)
    if tuple(k.shape) != (B, H_kv, N, d):
        raise ValueError(f"sage_attn_fwd_smooth_q: k {list(k.shape)} does not match k_i8 "
                         f"{list(k_i8.shape)}")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q_i8.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q_i8.device)
    if not return_lse:
        lse, lse_corr = None, None
    _check_attn_inputs("sage_attn_fwd_smooth_q", qk, out, v_f8=vq["v_f8"], v_scale=vq["v_scale"])
    if lse is not None:
        _check_tensor("sage_attn_fwd_smooth_q", "lse", lse, (B, H, N), torch.float32)
    if lse_corr is not None:
        _check_tensor("sage_attn_fwd_smooth_q", "lse_corr", lse_corr, (B, H, N), torch.float32)
    if workspace is None:
        workspace = smooth_q_workspace(B, H, N, d, device=q_i8.device)
    _need_gpu(q_i8, qk["q_scale"], k_i8, qk["k_scale"], vq["v_f8"], vq["v_scale"], out, k,
              qk["k_mean"], qk["q_mean"], workspace,
              *(t for t in (lse, lse_corr) if t is not None))
    st = load_library().sage_attn_fwd_smooth_q(
        q_i8.data_ptr(), qk["q_scale"].data_ptr(), k_i8.data_ptr(), qk["k_scale"].data_ptr(),
        vq["v_f8"].data_ptr(), vq["v_scale"].data_ptr(), k.data_ptr(), _dt(k.dtype),
        qk["k_mean"].data_ptr(), qk["q_mean"].data_ptr(), out.data_ptr(), _dt(out.dtype),
        _ptr(lse), _ptr(lse_corr), B, H, H_kv, N, d, _q_group_of(qk["q_scale"], N),
        int(bool(causal)), float(sm_scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream, q_i8.device))
    _check(st, "sage_attn_fwd_smooth_q")
    return (out, lse) if return_lse else out


def sage_lse_correction(q: torch.Tensor, k_mean: torch.Tensor, sm_scale: float, *, out=None,
                        stream=None) -> torch.Tensor:
    """sm_scale * q . mean(K) per row, fp32 [B, H, N] (for sage_attn_fwd_lse)."""
    _need_gpu(q, k_mean)
    B, H, N, d = q.shape
    H_kv = k_mean.shape[1]
    _check_tensor("sage_lse_correction", "k_mean", k_mean, (B, H_kv, d), torch.float32)
    if out is None:
        out = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor("sage_lse_correction", "out", out, (B, H, N), torch.float32)
    _need_gpu(out)
    st = load_library().sage_lse_correction(q.data_ptr(), _dt(q.dtype), k_mean.data_ptr(), B, H,
                                            H_kv, N, d, float(sm_scale), out.data_ptr(),
                                            _stream(stream, q.device))
    _check(st, "sage_lse_correction")
    return out


def sage_qk_int32(q_i8: torch.Tensor, k_i8: torch.Tensor, b: int, h: int, *,
                  stream=None) -> torch.Tensor:
    """Exact int32 Q^ K^T of query head (b, h) through the attention kernel's tile routine."""
    _need_gpu(q_i8, k_i8)
    B, H, N, d = q_i8.shape
    H_kv = k_i8.shape[1]
    if tuple(k_i8.shape) != (B, H_kv, N, d):
        raise ValueError(f"sage_qk_int32: k_i8 {list(k_i8.shape)} does not match q_i8 "
                         f"{list(q_i8.shape)}")
    s = torch.empty((N, N), dtype=torch.int32, device=q_i8.device)
    st = load_library().sage_qk_int32(q_i8.data_ptr(), k_i8.data_ptr(), B, H, H_kv, N, d, b, h,
                                      s.data_ptr(), _stream(stream, q_i8.device))
    _check(st, "sage_qk_int32")
    return s


def sageattn(q, k, v, is_causal: bool = False, sm_scale: float | None = None,
             smooth_k: bool = True, return_lse: bool = False, q_group: int = BLKQ,
             smooth_q: bool = False, pv: str = "fp8"):
    """The whole forward pass: quantize Q/K/V, then the attention kernel.
    With return_lse, also the row log-sum-exp of the logits sm_scale q . k
    (corrected for the smoothing of K); returns (o, lse)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    if pv not in ("fp8", "mxfp4"):
        raise ValueError("pv must be 'fp8' or 'mxfp4'")
    if pv == "mxfp4":
        if smooth_q:
            raise ValueError("smooth_q is not combined with MXFP4 P V")
        qk = sage_quant_qk(q, k, smooth_k, q_group=q_group)
        vq4 = sage_quant_v_mxfp4(v)
        corr = sage_lse_correction(q, qk["k_mean"], sm_scale) if return_lse and smooth_k else None
        return sage_attn_fwd_mxfp4(qk, vq4, causal=is_causal, sm_scale=sm_scale,
                                   out_dtype=q.dtype, return_lse=return_lse, lse_corr=corr)
    qk = sage_quant_qk(q, k, smooth_k, q_group=q_group, smooth_q=smooth_q)
    vq = sage_quant_v(v)
    corr = sage_lse_correction(q, qk["k_mean"], sm_scale) if return_lse and smooth_k else None
    if smooth_q:
        return sage_attn_fwd_smooth_q(qk, vq, k, causal=is_causal, sm_scale=sm_scale,
                                      out_dtype=q.dtype, return_lse=return_lse, lse_corr=corr)
    if not return_lse:
        return sage_attn_fwd(qk, vq, causal=is_causal, sm_scale=sm_scale, out_dtype=q.dtype)
    return sage_attn_fwd_lse(qk, vq, causal=is_causal, sm_scale=sm_scale, out_dtype=q.dtype,
                             lse_corr=corr)


MFMA_PEAK_OPS = {0: 32 * 32 * 32 * 2, 1: 32 * 32 * 64 * 2}   # ops per MFMA of each kind


def sage_mfma_peak(kind: int = 0, iters: int = 48000, nwg: int = 256, device="cuda",
                   stream=None):
    """Roofline diagnostic: nwg workgroups of 4 waves, each wave issuing 4 * iters
    back-to-back MFMAs (kind 0: INT8 32x32x32, kind 1: scaled FP8 32x32x64) on
    register operands.  Returns (ops, clocks, sink, wall_khz): the launch's
    algorithmic ops, int64 [nwg*4, 2] per-wave (shader clocks, constant-rate
    clocks), int32 [nwg*256] per-lane accumulator sums (64*32*iters or
    64*64*iters) and the constant-rate clock's kHz.  The caller times the launch."""
    clocks = torch.empty((nwg * 4, 2), dtype=torch.int64, device=device)
    sink = torch.empty(nwg * 256, dtype=torch.int32, device=device)
    khz = ctypes.c_int(0)
    _check(load_library().sage_mfma_peak(int(kind), int(iters), int(nwg), _ptr(clocks),
                                         _ptr(sink), ctypes.byref(khz),
                                         _stream(stream, clocks.device)),
           "sage_mfma_peak")
    ops = nwg * 4 * 4 * iters * MFMA_PEAK_OPS[kind]
    return ops, clocks, sink, khz.value


class SagePlan:
    """Preallocated buffers for repeated calls on fixed shapes (no allocation per call)."""

    def __init__(self, B, H, H_kv, N, d, dtype, causal, sm_scale=None, device="cuda",
                 q_group=BLKQ, smooth_q=False, pv="fp8"):
        if pv not in ("fp8", "mxfp4") or (pv == "mxfp4" and smooth_q):
            raise ValueError("pv must be 'fp8' or 'mxfp4' (and mxfp4 without smooth_q)")
        self.shape = (B, H, H_kv, N, d)
        self.dtype, self.causal, self.q_group = dtype, causal, q_group
        self.smooth_q, self.pv = smooth_q, pv
        self.sm_scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        sz = sage_buffer_sizes(B, H, H_kv, N, d, q_group)
        self.qk = _alloc_qk(B, H, H_kv, N, d, device, q_group, smooth_q)
        self.ws_sq = smooth_q_workspace(B, H, N, d, device=device) if smooth_q else None
        self.k = None   # the original K of the last quant() (read by attn() for smooth Q)
        self.vq = _alloc_v4(B, H_kv, N, d, device) if pv == "mxfp4" else _alloc_v(B, H_kv, N, d, device)
        self.ws_qk = torch.empty(max(sz["ws_quant_qkv"], 16), dtype=torch.uint8, device=device)
        self.ws_v = torch.empty(max(sz["ws_quant_v"], 16), dtype=torch.uint8, device=device)
        self.o = torch.empty((B, H, N, d), dtype=dtype, device=device)

    def quant(self, q, k, v, stream=None):
        if self.pv == "mxfp4":
            sage_quant_qk(q, k, True, q_group=self.q_group, smooth_q=self.smooth_q, out=self.qk,
                          workspace=self.ws_qk, stream=stream)
            self.quant_v(v, stream)
        else:
            sage_quant_qkv(q, k, v, True, q_group=self.q_group, smooth_q=self.smooth_q,
                           out_qk=self.qk, out_v=self.vq, workspace=self.ws_qk, stream=stream)
        self.k = k

    def quant_v(self, v, stream=None):
        if self.pv == "mxfp4":
            sage_quant_v_mxfp4(v, out=self.vq, stream=stream)
        else:
            sage_quant_v(v, out=self.vq, workspace=self.ws_v, stream=stream)

    def attn(self, stream=None):
        if self.pv == "mxfp4":
            return sage_attn_fwd_mxfp4(self.qk, self.vq, causal=self.causal,
                                       sm_scale=self.sm_scale, out_dtype=self.dtype, out=self.o,
                                       stream=stream)
        if self.smooth_q:
            if self.k is None:
                raise RuntimeError("SagePlan.attn: smooth Q needs the original K; call quant() first")
            return sage_attn_fwd_smooth_q(self.qk, self.vq, self.k, causal=self.causal,
                                          sm_scale=self.sm_scale, out_dtype=self.dtype,
                                          workspace=self.ws_sq, out=self.o, stream=stream)
        return sage_attn_fwd(self.qk, self.vq, causal=self.causal, sm_scale=self.sm_scale,
                             out_dtype=self.dtype, out=self.o, stream=stream)

    def __call__(self, q, k, v, stream=None):
        self.quant(q, k, v, stream)
        return self.attn(stream)

    def capture(self, q, k, v):
        """Record one quant() + attn() step on q, k, v as a HIP graph and return it
        (a torch.cuda.CUDAGraph).  graph.replay() reruns the step's launches on the
        same buffers: it reads what q, k and v hold at replay time and writes self.o
        (and the plan's code buffers), so copy new inputs into q, k, v first; q, k, v
        and the plan must stay alive as long as the graph is replayed.  The step's
        launches are this library's kernels only (no memset or copy nodes).  One
        eager step on a side stream comes first, as graph capture requires."""
        side = torch.cuda.Stream(device=self.o.device)
        side.wait_stream(torch.cuda.current_stream(self.o.device))
        with torch.cuda.stream(side):
            self(q, k, v)
        torch.cuda.current_stream(self.o.device).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self(q, k, v)
        return graph
