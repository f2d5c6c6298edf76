"""CPU oracle of the SageAttention-style quantized attention forward pass.

TEST INFRASTRUCTURE ONLY: this is the checker the HIP path is compared with.
Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import it; the product never calls it and it shares no code with the
HIP path.  Plain NumPy in float64 (float32 only where the method's own
arithmetic is float32: the K mean cast, the smoothing subtraction, the scales
and the x/scale divisions that decide integer codes, and the FP8 rounding of
448 * P~, decided on Algorithm 1's float32 softmax values).

Two results are computed:

(i)  ``attn_exact`` -- the plain definition O = softmax(sm_scale Q K^T + mask) V
     in float64 on the unquantized fp16/bf16 inputs.
(ii) ``quantize_qk`` / ``quantize_v`` / ``attn_quant`` -- the quantized
     method step by step, in the order of Algorithm 1 on the SageAttention2
     detail page (with INT8 codes for Q and K; smoothing Q with the Delta S
     compensation is optional: ``smooth_q`` and ``delta_s``).

Where the pages leave a step open the reading taken is stated at the step.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from . import fp8_e4m3
from . import mxfp4

BLKQ = 128        # Q tokens per INT8 scale (Algorithm 1's b_q, detail page sec. 3)
BLKK = 64         # K tokens per INT8 scale (Algorithm 1's b_kv)
INT8_MAX = 127.0
P_SCALE = 448.0   # static scale of P before the FP8 cast (Algorithm 1)
KV_TILE = 128     # keys per online-softmax step of the GPU kernel
LOG2E_F32 = np.float32(1.0 / math.log(2.0))        # log2 e in float32


# ---------------------------------------------------------------------------
# Step 1: Smooth K  (SageAttention synthesis page, the Smooth K paragraph;
# SageAttention2 detail page, Algorithm 1 "Preprocessing": K = K - mean(K)).

def k_sum_exact(k: np.ndarray) -> np.ndarray:
    """Per-channel sum of K over tokens, float64, [..., N, d] -> [..., d].

    Reading: the mean is the exact sum over all N tokens, divided by N and
    rounded to float32.  ``np.sum`` in float64 is exact -- hence equal to the
    correctly rounded sum ``math.fsum`` -- whenever every partial sum is a
    multiple of the smallest quantum present with fewer than 2^53 quanta;
    ``exactness_margin_bits`` checks that condition.
    """
    return np.sum(np.asarray(k, dtype=np.float64), axis=-2)


def exactness_margin_bits(k: np.ndarray) -> float:
    """53 - log2(sum|x| / min quantum) over all columns; > 0 means exact."""
    x = np.abs(np.asarray(k, dtype=np.float64))
    nz = x[x > 0]
    if nz.size == 0:
        return 53.0
    # quantum of a value with 8 (bf16) or 11 (fp16) significant bits is at most
    # 2^(e-10); use the fp16 bound, which is the finer of the two for equal e.
    _, e = np.frexp(nz.min())
    q = 2.0 ** (e - 1 - 10)
    tot = np.sum(x, axis=-2).max()
    return 53.0 - math.log2(max(tot / q, 1.0))


def k_mean(k: np.ndarray) -> np.ndarray:
    """mean32 = float32(sum64 / N), [B, H_kv, N, d] -> [B, H_kv, d]."""
    n = k.shape[-2]
    return (k_sum_exact(k) / n).astype(np.float32)


# ---------------------------------------------------------------------------
# Steps 2-3: per-block INT8 quantization of Q and K (deployment-guide page,
# quantization formula: code = round(x / S); source-analysis page, the
# quantization module: Q/K enter the kernel as INT8 with FP32 scales).
# Reading: scale = float32(amax / 127) by IEEE division, code =
# RNE(float32(x / scale)) clamped to [-127, 127]; an all-zero block has
# scale 0 and codes 0; tail blocks take amax over their valid tokens only.

def quantize_int8_blocks(x32: np.ndarray, block: int):
    """x32: float32 [..., N, d] -> (int8 codes [..., N, d], float32 scales [..., nblk])."""
    assert x32.dtype == np.float32
    *lead, n, d = x32.shape
    nblk = -(-n // block)
    codes = np.zeros(x32.shape, dtype=np.int8)
    scales = np.zeros((*lead, nblk), dtype=np.float32)
    for i in range(nblk):
        xb = x32[..., i * block:(i + 1) * block, :]
        amax = np.max(np.abs(xb), axis=(-2, -1))
        s = (amax / np.float32(INT8_MAX)).astype(np.float32)
        scales[..., i] = s
        safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        y = (xb / safe[..., None, None]).astype(np.float32)       # float32 IEEE division
        c = np.clip(np.rint(y), -INT8_MAX, INT8_MAX)
        c = np.where((s > 0)[..., None, None], c, 0.0)
        codes[..., i * block:(i + 1) * block, :] = c.astype(np.int8)
    return codes, scales


# Q scale granularity.  The detail page's per-thread quantization gives each
# thread of the matrix-core instruction the Q tokens it holds, one scale per
# such group (Figure 4, "Per-thread" paragraph; Table 6 compares per-token,
# per-thread, per-block and per-tensor), and the source-analysis page's
# quantization module lists per-block / per-warp / per-thread Q scales.
# Reading: the groups are runs of consecutive tokens, `q_group` tokens each
# (128 = the per-block scale; 32 = the queries one matrix-core column block
# holds, the per-warp analogue; 1 = one query per scale, the per-thread
# analogue when each lane holds one query).  The scale and code rules are
# those of the block quantizer above, applied per group.
Q_GROUPS = (BLKQ, 32, 1)


# Smooth Q (SageAttention2 detail page, Algorithm 1: q_bar_i = mean(Q_i),
# then Q_i - q_bar_i is quantized; the pipeline figure (Figure 3's stages
# 1-3) smooths Q, computes the Delta S GEMV, then quantizes).  Readings: the
# mean's block is Algorithm 1's b_q = 128 tokens whatever the scale
# granularity (a tail block averages its valid tokens); q_bar =
# float32(exact sum / count), as for K; Q - q_bar is the float32
# subtraction.

def q_block_mean(q32: np.ndarray, block: int = BLKQ) -> np.ndarray:
    """Per-channel mean of each block of `block` tokens, float32
    [..., N, d] -> [..., ceil(N/block), d] (float64 sums: exact for fp16/bf16
    inputs under the same condition as the K mean)."""
    *lead, n, d = q32.shape
    nb = -(-n // block)
    out = np.zeros((*lead, nb, d), dtype=np.float32)
    for i in range(nb):
        xb = np.asarray(q32[..., i * block:(i + 1) * block, :], dtype=np.float64)
        out[..., i, :] = (xb.sum(axis=-2) / xb.shape[-2]).astype(np.float32)
    return out


def quantize_qk(q, k, smooth_k: bool = True, q_group: int = BLKQ, smooth_q: bool = False):
    """Quantize Q per `q_group` tokens and smoothed K per 64 tokens.

    q: [B, H, N, d], k: [B, H_kv, N, d] (fp16/bf16 values as torch or numpy).
    Returns dict(q_i8, q_scale, k_i8, k_scale, k_mean); q_scale has
    ceil(N / q_group) entries per head.  With ``smooth_q`` the codes are of
    Q - q_bar and the dict also holds q_mean [B, H, ceil(N/128), d] float32.
    """
    assert q_group in Q_GROUPS, q_group
    q32 = _f32(q)
    k32 = _f32(k)
    if smooth_k:
        mean = k_mean(k32)
        ks = (k32 - mean[..., None, :]).astype(np.float32)         # float32 RN subtraction
    else:
        mean = np.zeros(k32.shape[:-2] + k32.shape[-1:], dtype=np.float32)
        ks = k32
    if smooth_q:
        qm = q_block_mean(q32)
        n = q32.shape[-2]
        q32 = (q32 - np.repeat(qm, BLKQ, axis=-2)[..., :n, :]).astype(np.float32)
    qc, qs = quantize_int8_blocks(q32, q_group)
    kc, ksc = quantize_int8_blocks(ks, BLKK)
    out = dict(q_i8=qc, q_scale=qs, k_i8=kc, k_scale=ksc, k_mean=mean)
    if smooth_q:
        out["q_mean"] = qm
    return out


# The Delta S compensation (SageAttention2 detail page, Algorithm 1:
# S_ij = dequant(Q^_i K^_j^T) + GEMV(q_bar_i, K_j^T); "GEMV补偿" in its
# line-by-line notes: a 1 x N vector per Q block, for every key).  Reading:
# K_j is the K the quantizer sees (float32(K) - mean32 when K is smoothed,
# float32(K) otherwise), before quantization; the product is exact here.

def delta_s(q_mean, k, k_mean) -> np.ndarray:
    """Delta S[b, h, i, j] = q_bar[b, h, i] . K_s[b, h // (H/H_kv), j], float64
    [B, H, ceil(N/128), N].  k is the original K, k_mean its float32 mean
    (zeros when K is not smoothed)."""
    k32 = _f32(k)
    ks = (k32 - np.asarray(k_mean, dtype=np.float32)[..., None, :]).astype(np.float32)
    qm = np.asarray(q_mean, dtype=np.float64)
    grp = qm.shape[1] // ks.shape[1]
    ks_h = np.repeat(ks.astype(np.float64), grp, axis=1)          # [B, H, N, d]
    return np.einsum("bhic,bhjc->bhij", qm, ks_h)


# ---------------------------------------------------------------------------
# Step 4: per-channel FP8 E4M3 quantization of V (SageAttention2 detail page,
# Algorithm 1 "(delta_V, V^) = psi_V(V)"; source-analysis page, "V 的 FP16/FP8
# 准备": per-channel scale).  Reading: the channel's scale covers all N
# tokens of a (b, kv-head); scale = float32(amax / 448), code =
# E4M3(clamp(float32(v / scale), +-448)) with RNE.

def quantize_v(v):
    """v: [B, H_kv, N, d] -> dict(v_f8 uint8 [B,H_kv,N,d] natural layout, v_scale f32 [B,H_kv,d])."""
    v32 = _f32(v)
    amax = np.max(np.abs(v32), axis=-2)                              # [B, H_kv, d]
    s = (amax / np.float32(fp8_e4m3.E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = (v32 / safe[..., None, :]).astype(np.float32)
    y = np.clip(y, -fp8_e4m3.E4M3_MAX, fp8_e4m3.E4M3_MAX)
    codes = fp8_e4m3.encode(y.astype(np.float64))
    codes = np.where((s > 0)[..., None, :], codes, np.uint8(0)).astype(np.uint8)
    return dict(v_f8=codes, v_scale=s)


# MXFP4 V (the SageAttention3 synthesis page names MXFP4 as the FP4 format
# of MI350-class GPUs; the format is the OCP microscaling standard, see
# ``mxfp4``).  Reading: V's blocks are 32 consecutive keys of one channel,
# the contraction axis of P V; keys past N are zero (a zero block decodes to
# 0 whatever its scale).

def quantize_v_mxfp4(v):
    """v: [B, H_kv, N, d] -> dict(v_f4 E2M1 codes uint8 [B,H_kv,Np,d],
    v_e8 int64 exponents [B,H_kv,Np/32,d]), Np = N rounded up to 32."""
    v32 = _f32(v)
    B, Hk, n, d = v32.shape
    npad = -(-n // mxfp4.MX_BLOCK) * mxfp4.MX_BLOCK
    vp = np.zeros((B, Hk, npad, d))
    vp[:, :, :n] = v32
    codes, e = mxfp4.quantize_blocks(vp, axis=-2)
    return dict(v_f4=codes, v_e8=e)


# ---------------------------------------------------------------------------
# (i) Exact attention: the plain definition, float64.

def attn_exact(q, k, v, *, causal: bool, sm_scale: float, rows=None, heads=None,
               return_lse: bool = False):
    """O = softmax(sm_scale Q K^T + mask) V in float64.

    q [B,H,N,d]; k, v [B,H_kv,N,d]; query head h reads kv head h // (H/H_kv)
    (source-analysis page: num_qo_heads divisible by num_kv_heads).  Causal:
    key j is visible to query i iff j <= i.  ``rows``: optional index array
    of query rows to compute; ``heads``: optional list of (b, h).
    Returns float64 [B,H,len(rows),d] (unselected heads are zero); with
    ``return_lse`` also the row log-sum-exp L_i = ln sum_j exp(s_ij) of the
    logits s = sm_scale q k^T (natural log; the per-row state a forward pass
    keeps in place of P, source-analysis page, FlashAttention section).
    """
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q64.shape
    grp = H // k64.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.zeros((B, H, len(rows), d))
    lse = np.zeros((B, H, len(rows)))
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        hk = h // grp
        s = (q64[b, h, rows] @ k64[b, hk].T) * sm_scale
        if causal:
            s = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, s)
        mx = s.max(axis=1, keepdims=True)
        s = s - mx
        p = np.exp(s)
        ps = p.sum(axis=1, keepdims=True)
        lse[b, h] = (mx + np.log(ps))[:, 0]
        p /= ps
        out[b, h] = p @ v64[b, hk]
    return (out, lse) if return_lse else out


def softmax_rows(q, k, *, causal: bool, sm_scale: float, b=0, h=0, hk=None):
    """Full probability matrix P of one head (float64), for the row-sum check."""
    q64, k64 = _f64(q), _f64(k)
    hk = h if hk is None else hk
    s = (q64[b, h] @ k64[b, hk].T) * sm_scale
    n = s.shape[0]
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# (ii) The quantized attention of Algorithm 1 (SageAttention2 detail page),
# INT8 QK^T and FP8 PV, written as the sums the online recursion produces.
#
# Per query row i and key tile t (tiles of ``kv_tile`` keys, ascending), in
# base 2 (the source-analysis page, "attention kernel 前向": the kernel
# multiplies sm_scale by log2 e, so scores are in log2 units):
#   x_ij  = S^_ij * c_ij   (+ Delta S term with smoothed Q), masked to -inf,
#           S^ the exact int32 dot of the codes, c = dQ dK sm_scale log2 e
#   m_t   = max(m_{t-1}, rowmax_t x)                      (running max)
#   Pt_ij = 2^(x_ij - m_t)                                (P tilde)
#   Pq_ij = E4M3(448 * Pt_ij)                             (static P scale)
#   l     = sum_t 2^(m_t - m_T) rowsum(Pt_t)              (unquantized P tilde)
#   O_i   = [sum_t 2^(m_t - m_T) sum_{j in t} Pq_ij Vdq_j] / (448 l)
# which is what "l = exp(m_old - m_new) l + rowsum(Pt)" and
# "O = diag(exp(m_old - m_new)) O + Pq V" (Algorithm 1 and the online-softmax
# update of the source-analysis page) accumulate to, followed by the final
# rescale O = diag(l)^-1 O / 448 * delta_V.
#
# Precision (reading c25).  The FP8 code of 448 * Pt is a rounding decision,
# so it is taken in the precision the method computes Pt in: float32, the
# precision of the scales, of Algorithm 1's level-2 accumulator and of the
# kernel's softmax registers.  The steps, each a value the pages name and each
# rounded once to float32 (round to nearest even):
#   lam = sm_scale * log2 e                      (the softmax constant)
#   c   = (dQ * dK) * lam                         (psi^-1's scale product, then lam)
#   x   = S^ * c            (with smoothed Q: S^ * c + g, g = Delta S * lam)
#   m   = the running max of x                    (a max: no rounding)
#   a   = x - m                                   (exp's argument; 0 at the max)
#   Pt  = 2^a
#   y   = Pt * 448, then E4M3 round-to-nearest-even of y.
# x is Algorithm 1's S_ij in log2 units, one float32 rounding of its exact
# terms (the scaled integer dot, plus the Delta S term with smoothed Q).
# l, the tile carries 2^(m_t - m_T) and O stay float64 (no decision rides on
# them).  ``quantize_p=False`` keeps the whole path in float64 instead (P is
# not rounded at all): the pin against exact attention on dequantized inputs.

def sm_log2_f32(sm_scale: float) -> np.float32:
    """lam = float32(sm_scale * log2 e), both factors float32 (sm_scale is the
    float the C ABI takes)."""
    return np.float32(np.float32(sm_scale) * LOG2E_F32)


def rn32(x) -> np.ndarray:
    """float64 -> the nearest float32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def rn32_sum(a, b) -> np.ndarray:
    """The float32 nearest (ties to even) to the EXACT sum a + b of two finite
    float64 arrays.  s = a + b is rounded once to float64 first; that can only
    mislead the float32 rounding when s is itself halfway between two float32
    values and the float64 sum was inexact, where the exact residual (Knuth's
    TwoSum) says on which side the true sum lies."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    s = a + b
    bb = s - a
    err = (a - (s - bb)) + (b - bb)                 # a + b = s + err exactly
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    other = np.where(s > r64, up, dn)
    tie = (s != r64) & (2.0 * s == r64 + other.astype(np.float64))
    go = tie & (((err > 0) & (other > r)) | ((err < 0) & (other < r)))
    return np.where(go, other, r).astype(np.float32)


def softmax_f32(sint, c32, g32, valid, kv_tile):
    """Algorithm 1's online softmax on float32 values, for rows of scores.

    sint: exact integer dots (float64) [R, N]; c32: float32 factors c [R, N];
    g32: float32 Delta S terms [R, N] or None; valid: bool [R, N].
    Returns (pt32 float32 [R, N], 0 where not valid; m32 float32 [R, nt], the
    running max after each tile of kv_tile keys).
    """
    R, N = sint.shape
    nt = -(-N // kv_tile)
    prod = np.where(valid, sint, 0.0) * c32.astype(np.float64)  # exact: |S^| < 2^22, c 24 bits
    g = None if g32 is None else np.where(valid, g32, 0).astype(np.float64)
    x32 = rn32(prod) if g is None else rn32_sum(prod, g)
    xp = np.full((R, nt * kv_tile), -np.inf, dtype=np.float32)
    xp[:, :N] = np.where(valid, x32, np.float32(-np.inf))
    m32 = np.maximum.accumulate(xp.reshape(R, nt, kv_tile).max(axis=2), axis=1)
    mk = np.repeat(m32, kv_tile, axis=1)[:, :N].astype(np.float64)
    mk = np.where(valid, mk, 0.0)
    a32 = rn32_sum(np.where(valid, x32, np.float32(0)), -mk)
    pt32 = rn32(np.exp2(a32.astype(np.float64)))
    return np.where(valid, pt32, np.float32(0)), m32


def p_fp8(pt32) -> np.ndarray:
    """(P~ * 448).to(FP8 E4M3): the float32 product, rounded to nearest even
    onto the E4M3 grid; float64 values of the codes."""
    y32 = rn32(np.asarray(pt32, dtype=np.float64) * P_SCALE)   # exact product, one rounding
    return fp8_e4m3.round_to_e4m3(y32.astype(np.float64))


def attn_quant(qc, qs, kc, ks, vc, vs, *, causal: bool, sm_scale: float,
               kv_tile: int = KV_TILE, rows=None, heads=None,
               quantize_p: bool = True, blkq: int = BLKQ, blkk: int = BLKK,
               return_lse: bool = False, delta_s=None, pv: str = "fp8"):
    """Quantized attention, float64 result [B,H,len(rows),d].

    qc int8 [B,H,N,d], qs f32 [B,H,nq]; kc int8 [B,H_kv,N,d], ks f32
    [B,H_kv,nk]; vc uint8 E4M3 codes [B,H_kv,N,d] (natural layout), vs f32
    [B,H_kv,d].  ``quantize_p=False`` skips the FP8 rounding of 448*Pt and keeps
    every step in float64 (the result is then exact attention on the
    dequantized inputs).  With ``return_lse`` also L'_i = ln 2 (m_T + log2 l)
    (natural log) of the dequantized scores the recursion used -- of the
    smoothed K when the codes are of K - mean(K); ``lse_correction`` restores
    the unsmoothed value.  ``delta_s`` ([B,H,ceil(N/128),N], from ``delta_s``):
    with smoothed-Q codes, Delta S[query's 128-block, key] is added to every
    score.  ``pv="mxfp4"``: vc, vs are ``quantize_v_mxfp4``'s codes and
    exponents, and P~ of each 32-key block of a row is MX-quantized (no factor
    448) before the product (the reading stated at ``quantize_v_mxfp4``).
    """
    B, H, N, d = qc.shape
    grp = H // kc.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    nt = -(-N // kv_tile)
    npad = nt * kv_tile
    key_blk = np.arange(N) // blkk
    out = np.zeros((B, H, len(rows), d))
    lse = np.zeros((B, H, len(rows)))
    chunk = max(1, (1 << 23) // npad)               # bound the [rows, keys] temporaries
    mx = pv == "mxfp4"
    assert pv in ("fp8", "mxfp4") and (not mx or kv_tile % mxfp4.MX_BLOCK == 0)
    lam = sm_log2_f32(sm_scale)
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        hk = h // grp
        if mx:
            vdq = mxfp4.dequantize_blocks(vc[b, hk], vs[b, hk], axis=0)[:N]
        else:
            vdq = fp8_e4m3.decode(vc[b, hk]) * vs[b, hk].astype(np.float64)[None, :]
        kf = kc[b, hk].astype(np.float64).T
        dk = ks[b, hk, key_blk].astype(np.float32)
        for r0 in range(0, len(rows), chunk):
            rr = rows[r0:r0 + chunk]
            R = len(rr)
            # exact integer dot products (|partial sums| <= 127^2 d < 2^53)
            sint = qc[b, h, rr].astype(np.float64) @ kf
            valid = np.ones((R, N), dtype=bool)
            if causal:
                valid = np.arange(N)[None, :] <= rr[:, None]
            dq = qs[b, h, rr // blkq].astype(np.float32)
            if not quantize_p:
                # float64 throughout, natural-log units, P not rounded
                s = sint * dq.astype(np.float64)[:, None] * dk.astype(np.float64)[None, :]
                s = s * sm_scale
                if delta_s is not None:
                    s = s + np.asarray(delta_s[b, h], dtype=np.float64)[rr // BLKQ] * sm_scale
                s = np.where(valid, s, -np.inf)
                sp = np.full((R, npad), -np.inf)
                sp[:, :N] = s
                st = sp.reshape(R, nt, kv_tile)
                m_run = np.maximum.accumulate(st.max(axis=2), axis=1)
                carry = np.exp(m_run - m_run[:, -1:])
                pt = np.exp(st - m_run[:, :, None])
                l = np.sum(pt.sum(axis=2) * carry, axis=1)
                w = (P_SCALE * pt * carry[:, :, None]).reshape(R, npad)[:, :N]
                out[b, h, r0:r0 + chunk] = (w @ vdq) / (P_SCALE * l)[:, None]
                lse[b, h, r0:r0 + chunk] = m_run[:, -1] + np.log(l)
                continue
            c32 = rn32(rn32(dq.astype(np.float64)[:, None] * dk.astype(np.float64)[None, :])
                       .astype(np.float64) * np.float64(lam))
            g32 = None
            if delta_s is not None:
                g32 = rn32(np.asarray(delta_s[b, h], dtype=np.float64)[rr // BLKQ] *
                           np.float64(lam))
            pt32, m32 = softmax_f32(sint, c32, g32, valid, kv_tile)
            ptp = np.zeros((R, npad))
            ptp[:, :N] = pt32
            if mx:
                # P~ in MX blocks of 32 consecutive keys; scaled back to 448 * value
                # so the rest of the recursion is shared with the FP8 form
                codes, e = mxfp4.quantize_blocks(ptp, axis=-1)
                pq = P_SCALE * mxfp4.dequantize_blocks(codes, e)
            else:
                pq = p_fp8(ptp)
            carry = np.exp2(m32.astype(np.float64) - np.float64(1) * m32[:, -1:])   # 2^(m_t - m_T)
            l = np.sum(ptp.reshape(R, nt, kv_tile).sum(axis=2) * carry, axis=1)
            w = (pq.reshape(R, nt, kv_tile) * carry[:, :, None]).reshape(R, npad)[:, :N]
            out[b, h, r0:r0 + chunk] = (w @ vdq) / (P_SCALE * l)[:, None]
            lse[b, h, r0:r0 + chunk] = math.log(2.0) * (m32[:, -1].astype(np.float64) +
                                                        np.log2(l))
    return (out, lse) if return_lse else out


def lse_correction(q, k_mean, *, sm_scale: float):
    """sm_scale * q_i . mean(K), float64 [B,H,N]: what smoothing K removed
    from every logit of row i, added back to the log-sum-exp (source-analysis
    page, "smooth_k 与 LSE 校正": the q @ mean(K) term).  q is the original
    fp16/bf16 Q; k_mean the float32 K mean [B,H_kv,d] (query head h uses kv
    head h // (H/H_kv))."""
    q64 = _f64(q)
    km = np.asarray(k_mean, dtype=np.float64)
    grp = q64.shape[1] // km.shape[1]
    km_h = np.repeat(km, grp, axis=1)                       # [B,H,d]
    return np.einsum("bhnc,bhc->bhn", q64, km_h) * sm_scale


def f32_of_fraction(fr: Fraction) -> float:
    """The binary32 value nearest (ties to even) to an exact rational, as a
    Python float (normal and subnormal range; no overflow handling)."""
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^(e-1) < a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                                          # 2^e <= a (or subnormal)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    v = float(k * quantum)
    return -v if neg else v


def attn_quant_recursive(qc, qs, kc, ks, vc, vs, *, causal, sm_scale, kv_tile,
                         b=0, h=0, hk=None, blkq=BLKQ, blkk=BLKK, return_lse=False,
                         delta_s=None, pv="fp8"):
    """Literal online recursion of Algorithm 1 in pure Python loops (tiny sizes).

    Used to pin ``attn_quant``'s closed form: the same steps, one key tile at
    a time, with m, l and O rescaled in place by 2^(m_old - m_new) (and, with
    ``return_lse``, the final ln 2 (m + log2 l) of each row).  The float32
    steps are computed here on exact rationals, each rounded once by
    ``f32_of_fraction`` (an implementation independent of ``rn32_sum``).
    """
    n, d = qc.shape[2], qc.shape[3]
    hk = h if hk is None else hk
    mx = pv == "mxfp4"
    if mx:
        vdq = mxfp4.dequantize_blocks(vc[b, hk], vs[b, hk], axis=0)
    else:
        vdq = fp8_e4m3.decode(vc[b, hk]) * vs[b, hk].astype(np.float64)[None, :]
    out = np.zeros((n, d))
    lse = np.zeros(n)
    lam = Fraction(float(sm_log2_f32(sm_scale)))
    for i in range(n):
        m = None                            # float32 running max (a Python float)
        l = 0.0
        o = [0.0] * d
        dq = Fraction(float(qs[b, h, i // blkq]))
        for t0 in range(0, n, kv_tile):
            keys = [j for j in range(t0, min(t0 + kv_tile, n)) if not (causal and j > i)]
            if not keys:
                continue
            acc, x = {}, {}
            for j in keys:
                acc[j] = sum(int(qc[b, h, i, c]) * int(kc[b, hk, j, c]) for c in range(d))
                dk = Fraction(float(ks[b, hk, j // blkk]))
                cj = Fraction(f32_of_fraction(Fraction(f32_of_fraction(dq * dk)) * lam))
                prod = acc[j] * cj
                if delta_s is not None:
                    g = f32_of_fraction(Fraction(float(delta_s[b, h, i // BLKQ, j])) * lam)
                    x[j] = (prod, f32_of_fraction(prod + Fraction(g)))
                else:
                    x[j] = (prod, f32_of_fraction(prod))
            m_new = max(x32 for _, x32 in x.values())
            if m is not None:
                m_new = max(m, m_new)
                alpha = 2.0 ** (m - m_new)
                l *= alpha
                o = [alpha * v for v in o]
            m = m_new
            pts = {}
            for j in keys:
                a = f32_of_fraction(Fraction(x[j][1]) - Fraction(m))
                pts[j] = float(np.float32(2.0 ** a))
            for j, pt in pts.items():
                l += pt
                if mx:
                    # the shared exponent of j's block of 32 keys (masked keys: 0)
                    j0 = j - j % mxfp4.MX_BLOCK
                    amax = max(pts.get(jj, 0.0) for jj in range(j0, j0 + mxfp4.MX_BLOCK))
                    sc = 2.0 ** int(mxfp4.scale_exponent(amax))
                    pq = P_SCALE * float(mxfp4.decode(mxfp4.encode(pt / sc))) * sc
                else:
                    y = f32_of_fraction(Fraction(pt) * int(P_SCALE))
                    pq = float(fp8_e4m3.round_to_e4m3(y))
                for c in range(d):
                    o[c] += pq * vdq[j, c]
        out[i] = [v / (P_SCALE * l) for v in o]
        lse[i] = math.log(2.0) * (m + math.log2(l))
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------------------
# Metrics (SageAttention2 detail page, Tables 4 and 6 name CosSim, Relative L1
# and RMSE; the definitions are the usual ones, on flattened tensors).

def metrics(a, ref) -> dict:
    a = np.asarray(a, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    return dict(
        cos=float(np.dot(a, r) / math.sqrt(np.dot(a, a) * np.dot(r, r))),
        rel_l1=float(np.abs(a - r).sum() / np.abs(r).sum()),
        rmse=float(math.sqrt(np.mean((a - r) ** 2))),
        max_abs=float(np.abs(a - r).max()),
    )


def round_output(o64, dtype: str):
    """Round the float64 result to the output dtype (RNE), returned as float64.

    torch's CPU cast goes float64 -> float32 -> bf16, so a bf16 tie can be
    double-rounded (one bf16 ulp, rare); the output comparison is toleranced.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(o64, dtype=np.float64))
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    return t.to(tdt).to(torch.float64).numpy()


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float32)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)
