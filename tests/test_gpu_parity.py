"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: K mean, INT8 codes and scales of Q and K, V scales and V codes
(compared by decoded value), int32 QK^T dot products.  Output: max-abs error
<= 2e-2 and cosine >= 0.9995 against the oracle's quantized attention rounded
to the output dtype.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import fp8_e4m3 as F8
from oracle import sage_oracle as O
from tests.sage_testlib import (compare_output, compare_output_mx, lse_tol, to_np, v4_natural,
                                v_natural)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rand_inputs(B, H, H_kv, N, d, dtype, seed, bias=3.0):
    g = np.random.default_rng(seed)
    q = torch.from_numpy(g.standard_normal((B, H, N, d), dtype=np.float32)).to(dtype)
    k = g.standard_normal((B, H_kv, N, d), dtype=np.float32)
    k += (g.standard_normal((B, H_kv, 1, d), dtype=np.float32) * bias)
    k = torch.from_numpy(k).to(dtype)
    v = torch.from_numpy(g.standard_normal((B, H_kv, N, d), dtype=np.float32)).to(dtype)
    return q, k, v


def _check_quant(qa, q, k, v, smooth=True, heads_kv=None, q_group=128):
    qk = qa.sage_quant_qk(q.to(DEV), k.to(DEV), smooth, q_group=q_group)
    vq = qa.sage_quant_v(v.to(DEV))
    torch.cuda.synchronize()
    ref = O.quantize_qk(q, k, smooth_k=smooth, q_group=q_group)
    refv = O.quantize_v(v)
    assert np.array_equal(to_np(qk["k_mean"]), ref["k_mean"])
    assert np.array_equal(to_np(qk["q_scale"]), ref["q_scale"])
    assert np.array_equal(to_np(qk["k_scale"]), ref["k_scale"])
    assert np.array_equal(to_np(qk["q_i8"]), ref["q_i8"])
    assert np.array_equal(to_np(qk["k_i8"]), ref["k_i8"])
    assert np.array_equal(to_np(vq["v_scale"]), refv["v_scale"])
    N, d = q.shape[2], q.shape[3]
    vn, vpad = v_natural(to_np(vq["v_f8"]), N, d)
    assert (vpad == 0).all(), "V padding must be zero codes"
    dec_g, dec_r = F8.decode(vn), F8.decode(refv["v_f8"])
    assert np.array_equal(dec_g, dec_r), np.argwhere(dec_g != dec_r)[:5]
    return qk, vq, ref, refv


def _oracle_o(ref, refv, causal, sm_scale, rows=None, heads=None, q_group=128):
    return O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                        refv["v_f8"], refv["v_scale"], causal=causal, sm_scale=sm_scale,
                        rows=rows, heads=heads, blkq=q_group)


# ------------------------------------------------------------------ small full parity

SMALL = [
    # B, H, H_kv, N, d, dtype, causal
    (1, 2, 2, 256, 64, torch.float16, False),
    (2, 4, 2, 700, 64, torch.bfloat16, True),
    (2, 4, 2, 700, 128, torch.float16, False),
    (1, 4, 1, 385, 128, torch.bfloat16, True),
    (1, 2, 2, 1, 64, torch.float16, False),
    (1, 2, 2, 17, 128, torch.float16, True),
    (1, 2, 1, 130, 64, torch.bfloat16, False),
    (1, 2, 2, 64, 128, torch.float16, True),       # one K block, half a KV tile
    (1, 1, 1, 128, 64, torch.bfloat16, True),      # exactly one tile
    (1, 2, 2, 129, 128, torch.bfloat16, False),    # one key past a tile
    (1, 8, 1, 255, 64, torch.float16, True),       # GQA group of 8, ragged
]


@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", SMALL)
def test_small_full_parity(gpu_lib, B, H, H_kv, N, d, dtype, causal):
    print(f"case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed=N * 7 + d)
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
    sm = 1 / math.sqrt(d)
    o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=sm, out_dtype=dtype)
    torch.cuda.synchronize()
    compare_output(o, _oracle_o(ref, refv, causal, sm))


Q_GROUP_CASES = [SMALL[i] for i in (1, 3, 4, 5, 9, 10)]


@pytest.mark.parametrize("q_group", [32, 1])
@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", Q_GROUP_CASES)
def test_q_group_parity(gpu_lib, B, H, H_kv, N, d, dtype, causal, q_group):
    """Q scales per 32 queries (one wave) or per query (one lane): codes and scales
    bit-exact, output against the oracle with the same grouping."""
    print(f"q_group {q_group} case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal}",
          flush=True)
    q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed=N * 3 + d + q_group)
    # token magnitudes that differ by up to e^3 (scaled up and down), so the groups'
    # scales differ and some rows are sharply peaked
    g = np.random.default_rng(N + q_group)
    q = (q.float() * torch.from_numpy(np.exp(g.uniform(-1.5, 1.5, (B, H, N, 1))).astype(np.float32))
         ).to(dtype)
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v, q_group=q_group)
    assert qk["q_scale"].shape == (B, H, -(-N // q_group))
    sm = 1 / math.sqrt(d)
    o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=sm, out_dtype=dtype)
    torch.cuda.synchronize()
    compare_output(o, _oracle_o(ref, refv, causal, sm, q_group=q_group))


def test_q_group_token_scales_of_very_different_size(gpu_lib):
    """Per-query scales where one query of a wave is 3000 times the others: its scale,
    score factors and running max differ by that much from its neighbours'."""
    q, k, v = _rand_inputs(1, 2, 2, 384, 128, torch.float16, seed=23)
    q = q.float()
    q[:, :, 40] *= 3000.0                     # query 40: wave 1 of the first workgroup
    q = q.clamp(-60000, 60000).half()
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v, q_group=1)
    for causal in (False, True):
        o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=1 / 11.3,
                                  out_dtype=torch.float16)
        torch.cuda.synchronize()
        compare_output(o, _oracle_o(ref, refv, causal, 1 / 11.3, q_group=1))


def test_q_group_lse(gpu_lib):
    q, k, v = _rand_inputs(1, 4, 2, 300, 128, torch.bfloat16, seed=24)
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v, q_group=1)
    sm = 1 / math.sqrt(128)
    o0 = gpu_lib.sage_attn_fwd(qk, vq, causal=True, sm_scale=sm, out_dtype=torch.bfloat16)
    o1, lse = gpu_lib.sage_attn_fwd_lse(qk, vq, causal=True, sm_scale=sm,
                                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
    _, l_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                            refv["v_f8"], refv["v_scale"], causal=True, sm_scale=sm,
                            return_lse=True, blkq=1)
    err = np.abs(to_np(lse).astype(np.float64) - l_ref)
    assert np.all(err <= lse_tol(300, l_ref)), err.max()


@pytest.mark.parametrize("N,d", [(256, 64), (300, 128), (129, 64), (384, 128)])
def test_qk_int32_bit_exact(gpu_lib, N, d):
    q, k, v = _rand_inputs(1, 4, 2, N, d, torch.float16, seed=N + d)
    qk = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV))
    ref = O.quantize_qk(q, k)
    for h in (0, 3):
        s = to_np(gpu_lib.sage_qk_int32(qk["q_i8"], qk["k_i8"], 0, h))
        exact = ref["q_i8"][0, h].astype(np.int64) @ ref["k_i8"][0, h // 2].astype(np.int64).T
        assert np.array_equal(s, exact)


def test_smooth_k_off(gpu_lib):
    q, k, v = _rand_inputs(1, 2, 2, 300, 64, torch.float16, seed=9)
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v, smooth=False)
    assert (to_np(qk["k_mean"]) == 0).all()
    o = gpu_lib.sage_attn_fwd(qk, vq, causal=False, sm_scale=0.125, out_dtype=torch.float16)
    torch.cuda.synchronize()
    compare_output(o, _oracle_o(ref, refv, False, 0.125))


@pytest.mark.parametrize("B,H,H_kv,N,d,dtype", [
    (1, 8, 1, 255, 64, torch.float16),
    (1, 4, 1, 385, 128, torch.bfloat16),
    (1, 4, 2, 1000, 128, torch.float16),
])
def test_causal_parity_over_seeds(gpu_lib, B, H, H_kv, N, d, dtype):
    """The first rows of a causal grid see a handful of keys, so one P~ code decided on
    the other side of an FP8 rounding midpoint would move their output by up to |v| / 12.
    The kernel takes the oracle's float32 steps; every seed must meet the bar."""
    for seed in range(1000, 1008):
        print(f"causal seeds case B{B} H{H}/{H_kv} N{N} d{d} {dtype} seed {seed}", flush=True)
        q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed=seed)
        qk = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV))
        vq = gpu_lib.sage_quant_v(v.to(DEV))
        sm = 1 / math.sqrt(d)
        o = gpu_lib.sage_attn_fwd(qk, vq, causal=True, sm_scale=sm, out_dtype=dtype)
        torch.cuda.synchronize()
        ref, refv = O.quantize_qk(q, k), O.quantize_v(v)
        compare_output(o, _oracle_o(ref, refv, True, sm))


def test_degenerate_inputs(gpu_lib):
    """Zero Q (uniform attention), an all-zero V channel, a zero K block."""
    q, k, v = _rand_inputs(1, 2, 2, 200, 64, torch.float16, seed=11)
    q[:, :, :128] = 0                        # first Q block all zero -> scale 0
    v[:, :, :, 5] = 0                        # zero channel -> V scale 0
    kbar = k[:, 0].float().mean(dim=1, keepdim=True).to(k.dtype)       # [B, 1, d]
    k[:, 0, 64:128] = kbar.expand(-1, 64, -1)  # a K block at the mean: tiny after smoothing
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
    for causal in (False, True):
        o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=0.125, out_dtype=torch.float16)
        torch.cuda.synchronize()
        compare_output(o, _oracle_o(ref, refv, causal, 0.125))


def test_large_magnitudes(gpu_lib):
    """Values near the fp16 range still quantize bit-exactly (scales stay finite)."""
    q, k, v = _rand_inputs(1, 2, 2, 257, 128, torch.float16, seed=12)
    q = (q.float() * 3000).clamp(-60000, 60000).half()
    v = (v.float() * 1e-3).half()
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
    o = gpu_lib.sage_attn_fwd(qk, vq, causal=False, sm_scale=1 / 11.3, out_dtype=torch.float16)
    torch.cuda.synchronize()
    compare_output(o, _oracle_o(ref, refv, False, 1 / 11.3), max_abs=2e-2 * 1e-3 * 4)


def test_largest_head_count(gpu_lib):
    """B*H = 65535, the most heads the ABI accepts (the Delta S pass's grid
    y-dimension), with a ragged N = 3: codes and scales bit-exact over every head,
    and the output of sampled heads (first, middle, last) against the oracle, plain
    and smoothed Q, causal and not."""
    B, H, N, d = 3, 21845, 3, 64
    print(f"largest head count case B{B} H{H} N{N} d{d}", flush=True)
    q, k, v = _rand_inputs(B, H, H, N, d, torch.float16, seed=91)
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
    heads = [(0, 0), (1, H // 2), (2, H - 1)]
    sel = lambda x: np.stack([np.asarray(x[b, h]) for b, h in heads])
    sm = 0.125
    qsq = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV), True, smooth_q=True)
    refsq = O.quantize_qk(q, k, smooth_q=True)
    for n in ("q_i8", "q_scale", "q_mean"):
        assert np.array_equal(to_np(qsq[n]), refsq[n]), n
    ds_ref = O.delta_s(refsq["q_mean"], k, refsq["k_mean"])
    for causal in (False, True):
        o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=sm, out_dtype=torch.float16)
        o_sq = gpu_lib.sage_attn_fwd_smooth_q(qsq, vq, k.to(DEV), causal=causal, sm_scale=sm,
                                              out_dtype=torch.float16)
        torch.cuda.synchronize()
        o_ref = _oracle_o(ref, refv, causal, sm, heads=heads)
        compare_output(torch.stack([o[b, h] for b, h in heads]), sel(o_ref))
        o_ref_sq = O.attn_quant(refsq["q_i8"], refsq["q_scale"], refsq["k_i8"], refsq["k_scale"],
                                refv["v_f8"], refv["v_scale"], causal=causal, sm_scale=sm,
                                heads=heads, delta_s=ds_ref)
        compare_output(torch.stack([o_sq[b, h] for b, h in heads]), sel(o_ref_sq))


def test_quantization_ties_round_to_even(gpu_lib):
    """Every x/scale lands exactly on a rounding midpoint: INT8 codes at k + 1/2 and FP8 codes
    halfway between neighbours must round to even, bit-exactly as the oracle does."""
    N, d = 256, 64
    g = np.random.default_rng(21)
    # Q: each 128-token block has amax 95.25 -> scale 0.75 exactly; the other values are
    # (k + 1/2) * 0.75 for random k, so x / scale = k + 1/2 exactly (fp16 holds them).
    kk = g.integers(-126, 126, size=(1, 2, N, d))
    q = ((kk + 0.5) * 0.75).astype(np.float32)
    q[:, :, ::128, 0] = 95.25
    # V: per-channel amax 448 -> scale 1; values at FP8 midpoints (1 + (2j + 1)/16) * 2^e.
    j = g.integers(0, 8, size=(1, 2, N, d))
    e = g.integers(-3, 7, size=(1, 2, N, d))
    sign = np.where(g.random((1, 2, N, d)) < 0.5, -1.0, 1.0)
    v = (sign * (1 + (2 * j + 1) / 16.0) * 2.0 ** e).astype(np.float32)
    v[:, :, 0, :] = 448.0
    k = g.standard_normal((1, 2, N, d), dtype=np.float32)
    qt, kt, vt = (torch.from_numpy(x).half() for x in (q, k, v))
    assert torch.equal(qt.float(), torch.from_numpy(q)) and torch.equal(vt.float(), torch.from_numpy(v))
    _check_quant(gpu_lib, qt, kt, vt)


def test_one_large_k_block(gpu_lib):
    """One K block with a 400 times larger scale than its neighbours: score factors that
    differ by that much between the K blocks of one tile."""
    q, k, v = _rand_inputs(1, 2, 2, 640, 128, torch.float16, seed=22)
    k = k.float()
    k[:, :, 192:256] *= 400.0
    k = k.clamp(-60000, 60000).half()
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
    for causal in (False, True):
        o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=1 / 11.3, out_dtype=torch.float16)
        torch.cuda.synchronize()
        compare_output(o, _oracle_o(ref, refv, causal, 1 / 11.3))


def test_deterministic(gpu_lib):
    q, k, v = _rand_inputs(2, 4, 2, 700, 128, torch.bfloat16, seed=13)
    outs = []
    for _ in range(3):
        qk = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV))
        vq = gpu_lib.sage_quant_v(v.to(DEV))
        outs.append(gpu_lib.sage_attn_fwd(qk, vq, causal=True, sm_scale=0.09,
                                          out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,q_group,smooth_k,smooth_q", [
    (2, 4, 2, 700, 128, torch.float16, 128, True, False),
    (1, 4, 1, 385, 64, torch.bfloat16, 32, True, True),
    (1, 8, 2, 257, 128, torch.bfloat16, 1, False, True),
    (1, 2, 2, 1, 64, torch.float16, 128, True, False),
    (2, 2, 2, 1000, 64, torch.float16, 1, True, False),
])
def test_quant_qkv_matches_oracle(gpu_lib, B, H, H_kv, N, d, dtype, q_group, smooth_k, smooth_q):
    """The one-call quantization (statistics of K and V in one pass, one launch for all
    codes): every output bit-exact against the oracle, V codes by decoded value."""
    print(f"quant_qkv case B{B} H{H}/{H_kv} N{N} d{d} {dtype} q_group {q_group} "
          f"smooth_k {smooth_k} smooth_q {smooth_q}", flush=True)
    q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed=N * 19 + d)
    qk, vq = gpu_lib.sage_quant_qkv(q.to(DEV), k.to(DEV), v.to(DEV), smooth_k, q_group=q_group,
                                    smooth_q=smooth_q)
    torch.cuda.synchronize()
    ref = O.quantize_qk(q, k, smooth_k=smooth_k, q_group=q_group, smooth_q=smooth_q)
    refv = O.quantize_v(v)
    names = ["q_i8", "q_scale", "k_i8", "k_scale", "k_mean"] + (["q_mean"] if smooth_q else [])
    for n in names:
        assert np.array_equal(to_np(qk[n]), ref[n]), n
    assert np.array_equal(to_np(vq["v_scale"]), refv["v_scale"])
    vn, vpad = v_natural(to_np(vq["v_f8"]), N, d)
    assert (vpad == 0).all()
    assert np.array_equal(F8.decode(vn), F8.decode(refv["v_f8"]))


# ------------------------------------------------------------------ tile choice (c11)

@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", [SMALL[i] for i in (0, 1, 2, 3, 6, 9, 10)])
def test_tile_choice_within_bar(gpu_lib, B, H, H_kv, N, d, dtype, causal):
    """The kernel quantizes P~ against the running max after every 128 keys.  One tile of
    all N keys removes the online effect: the output meets the bar against it (the
    condition the tile reading sets).  Against Algorithm 1's b_kv = 64 it meets the bar on
    every row except, in a causal grid, rows 64..127: they see keys in two 64-key tiles
    but one 128-key tile, so up to half their weights are quantized against a different
    max (oracle against oracle, 64 keys against 128 or N differ there by up to 0.024);
    those rows are held to the cosine bar."""
    print(f"tile choice case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed=N * 17 + d)
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
    sm = 1 / math.sqrt(d)
    o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=sm, out_dtype=dtype)
    torch.cuda.synchronize()
    args = (ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"], refv["v_f8"],
            refv["v_scale"])
    print(f"  kv_tile N: {compare_output(o, O.attn_quant(*args, causal=causal, sm_scale=sm, kv_tile=N))}",
          flush=True)
    o64 = O.attn_quant(*args, causal=causal, sm_scale=sm, kv_tile=64)
    rows = np.arange(N)
    band = (rows >= 64) & (rows < 128) if causal else np.zeros(N, dtype=bool)
    sel = torch.from_numpy(np.flatnonzero(~band)).to(DEV)
    print(f"  kv_tile 64: {compare_output(o[:, :, sel], o64[:, :, ~band])}", flush=True)
    if band.any():
        bsel = torch.from_numpy(np.flatnonzero(band)).to(DEV)
        print(f"  kv_tile 64, rows 64..127: "
              f"{compare_output(o[:, :, bsel], o64[:, :, band], max_abs=np.inf)}", flush=True)


# ------------------------------------------------------------------ peaked rows, plain Q

PEAKED = [
    # N, d, dtype, causal, Q bias (sigma of a channel bias shared by the tokens), seed
    (129, 64, torch.float16, False, 1.5, 3001),
    (129, 128, torch.bfloat16, True, 3.0, 3002),
    (200, 64, torch.bfloat16, False, 2.0, 3003),
    (257, 128, torch.float16, True, 2.5, 3004),
    (300, 64, torch.float16, True, 3.0, 3005),
    (384, 128, torch.bfloat16, False, 1.5, 3006),
    (500, 64, torch.bfloat16, True, 2.0, 3007),
    (640, 128, torch.float16, False, 3.0, 3008),
    (777, 64, torch.float16, False, 2.5, 3009),
    (1000, 128, torch.bfloat16, True, 3.0, 3010),
    (1000, 64, torch.float16, True, 1.5, 3011),
    (1000, 128, torch.float16, False, 2.0, 3012),
]


@pytest.mark.parametrize("N,d,dtype,causal,qbias,seed", PEAKED)
def test_peaked_plain_q_parity(gpu_lib, N, d, dtype, causal, qbias, seed):
    """Q with a channel bias shared by its tokens (the LLM outlier structure of the
    SageAttention2 detail page's Table 4), quantized without smoothing Q: the attention
    rows are peaked on a few keys, so one P~ code decided differently would move an
    output by up to |v| / 12.  Several seeds per shape; every one must meet the bar."""
    sm = 1 / math.sqrt(d)
    for s in range(seed, seed + 4):
        print(f"peaked case N{N} d{d} {dtype} causal={causal} qbias {qbias} seed {s}", flush=True)
        q, k, v = _biased_q_inputs(1, 4, 2, N, d, dtype, seed=s, qbias=qbias)
        qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
        o = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=sm, out_dtype=dtype)
        torch.cuda.synchronize()
        compare_output(o, _oracle_o(ref, refv, causal, sm))


@pytest.mark.parametrize("N,d,dtype,causal,qbias,seed", PEAKED[::3])
def test_peaked_plain_q_mxfp4_parity(gpu_lib, N, d, dtype, causal, qbias, seed):
    """The same peaked rows with MXFP4 P V: the E2M1 codes and block exponents of P~ are
    decided on the same float32 values on both sides."""
    sm = 1 / math.sqrt(d)
    for s in range(seed, seed + 2):
        print(f"peaked mxfp4 case N{N} d{d} {dtype} causal={causal} qbias {qbias} seed {s}",
              flush=True)
        q, k, v = _biased_q_inputs(1, 4, 2, N, d, dtype, seed=s, qbias=qbias)
        qk = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV))
        vq4 = gpu_lib.sage_quant_v_mxfp4(v.to(DEV))
        o = gpu_lib.sage_attn_fwd_mxfp4(qk, vq4, causal=causal, sm_scale=sm, out_dtype=dtype)
        torch.cuda.synchronize()
        ref = O.quantize_qk(q, k)
        ref4 = O.quantize_v_mxfp4(v)
        compare_output_mx(o, O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"],
                                          ref["k_scale"], ref4["v_f4"], ref4["v_e8"],
                                          causal=causal, sm_scale=sm, pv="mxfp4"))


# ------------------------------------------------------------------ smooth Q + Delta S

LOG2E = 1.4426950408889634


def _check_delta_s_table(ds_gpu, ds_ref, q_mean, k, k_mean, sm):
    """One head's table against the oracle's q_bar . K_s (float64): the GPU sums the exact
    products in FP64 and rounds once, so each entry is fp32(q_bar . K_s * sm_log2) with
    sm_log2 = fp32(sm * log2 e).  FP64 sums in another order can only move an entry
    that sits on a float32 rounding boundary, by one float32 step."""
    want = (np.asarray(ds_ref, dtype=np.float64) * np.float64(O.sm_log2_f32(sm))).astype(np.float32)
    got = np.asarray(ds_gpu, dtype=np.float32)
    steps = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert np.all((steps <= 1) | (got == want)), steps.max()
    assert np.count_nonzero(got != want) <= 1e-4 * got.size + 1, np.count_nonzero(got != want)


def _biased_q_inputs(B, H, H_kv, N, d, dtype, seed, qbias=1.5):
    """Inputs whose Q carries a per-(head, channel) bias shared by its tokens (what
    smoothing Q removes)."""
    q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed)
    g = np.random.default_rng(seed + 1)
    bias = torch.from_numpy((g.standard_normal((B, H, 1, d)) * qbias).astype(np.float32))
    return (q.float() + bias).to(dtype), k, v


def _check_smooth_q(qa, q, k, v, sm, q_group=128, smooth_k=True):
    """Quantize with smooth Q on the GPU; check the codes, scales and means bit-exact and
    every Delta S row within its bound.  Returns the GPU buffers and the oracle's."""
    qk = qa.sage_quant_qk(q.to(DEV), k.to(DEV), smooth_k, q_group=q_group, smooth_q=True)
    ds = qa.sage_delta_s(k.to(DEV), qk, sm)
    vq = qa.sage_quant_v(v.to(DEV))
    torch.cuda.synchronize()
    ref = O.quantize_qk(q, k, smooth_k=smooth_k, q_group=q_group, smooth_q=True)
    refv = O.quantize_v(v)
    for n in ("q_mean", "k_mean", "q_scale", "q_i8", "k_scale", "k_i8"):
        assert np.array_equal(to_np(qk[n]), ref[n]), n
    ds_ref = O.delta_s(ref["q_mean"], k, ref["k_mean"])
    B, H = q.shape[:2]
    grp = H // k.shape[1]
    k32 = k.float().numpy()
    ds_g = to_np(ds)
    for b in range(B):
        for h in range(H):
            _check_delta_s_table(ds_g[b, h], ds_ref[b, h], ref["q_mean"][b, h], k32[b, h // grp],
                                 ref["k_mean"][b, h // grp], sm)
    return qk, vq, ds, ref, refv, ds_ref


SQ_CASES = [SMALL[i] for i in (1, 2, 3, 4, 5, 9, 10)]


@pytest.mark.parametrize("q_group", [128, 1])
@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", SQ_CASES)
def test_smooth_q_parity(gpu_lib, B, H, H_kv, N, d, dtype, causal, q_group):
    """Smooth Q: block means, codes and scales bit-exact, the Delta S table within the FP32
    bound, and the output against the oracle with its exact Delta S."""
    print(f"smooth_q q_group {q_group} case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal}",
          flush=True)
    q, k, v = _biased_q_inputs(B, H, H_kv, N, d, dtype, seed=N * 11 + d + q_group)
    sm = 1 / math.sqrt(d)
    qk, vq, ds, ref, refv, ds_ref = _check_smooth_q(gpu_lib, q, k, v, sm, q_group)
    o = gpu_lib.sage_attn_fwd_smooth_q(qk, vq, k.to(DEV), causal=causal, sm_scale=sm,
                                       out_dtype=dtype)
    torch.cuda.synchronize()
    o_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"], refv["v_f8"],
                         refv["v_scale"], causal=causal, sm_scale=sm, blkq=q_group,
                         delta_s=ds_ref)
    compare_output(o, o_ref)


@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", [
    (2, 8, 2, 129, 64, torch.float16, True),
    (2, 8, 2, 300, 64, torch.bfloat16, True),
    (2, 4, 1, 127, 64, torch.bfloat16, True),
])
def test_smooth_q_parity_over_seeds(gpu_lib, B, H, H_kv, N, d, dtype, causal):
    """Smooth Q on Q with a shared bias gives peaked rows, where a Delta S entry a few float32
    ulps off (an FP32 sum in another order) flipped P~ codes.  The table is summed in FP64 and
    rounded once, so every seed meets the bar."""
    sm = 1 / math.sqrt(d)
    for seed in range(2003, 2011):
        print(f"smooth_q seeds case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal} "
              f"seed {seed}", flush=True)
        q, k, v = _biased_q_inputs(B, H, H_kv, N, d, dtype, seed=seed)
        qk, vq, ds, ref, refv, ds_ref = _check_smooth_q(gpu_lib, q, k, v, sm)
        o = gpu_lib.sage_attn_fwd_smooth_q(qk, vq, k.to(DEV), causal=causal, sm_scale=sm,
                                           out_dtype=dtype)
        torch.cuda.synchronize()
        compare_output(o, O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                                       refv["v_f8"], refv["v_scale"], causal=causal, sm_scale=sm,
                                       delta_s=ds_ref))


def test_smooth_q_without_smooth_k(gpu_lib):
    q, k, v = _biased_q_inputs(1, 2, 2, 300, 64, torch.float16, seed=51)
    qk, vq, ds, ref, refv, ds_ref = _check_smooth_q(gpu_lib, q, k, v, 0.125, smooth_k=False)
    assert (to_np(qk["k_mean"]) == 0).all()
    o = gpu_lib.sage_attn_fwd_smooth_q(qk, vq, k.to(DEV), causal=False, sm_scale=0.125,
                                       out_dtype=torch.float16)
    torch.cuda.synchronize()
    compare_output(o, O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                                   refv["v_f8"], refv["v_scale"], causal=False, sm_scale=0.125,
                                   delta_s=ds_ref))


def test_smooth_q_lse(gpu_lib):
    q, k, v = _biased_q_inputs(1, 4, 2, 300, 128, torch.bfloat16, seed=52)
    sm = 1 / math.sqrt(128)
    qk, vq, ds, ref, refv, ds_ref = _check_smooth_q(gpu_lib, q, k, v, sm)
    o0 = gpu_lib.sage_attn_fwd_smooth_q(qk, vq, k.to(DEV), causal=True, sm_scale=sm,
                                        out_dtype=torch.bfloat16)
    o1, lse = gpu_lib.sage_attn_fwd_smooth_q(qk, vq, k.to(DEV), causal=True, sm_scale=sm,
                                             out_dtype=torch.bfloat16, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
    _, l_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                            refv["v_f8"], refv["v_scale"], causal=True, sm_scale=sm,
                            return_lse=True, delta_s=ds_ref)
    # plus the FP32 Delta S error (log2 units -> natural log)
    ks = (k.float().numpy() - ref["k_mean"][:, :, None, :]).astype(np.float32)
    absb = np.einsum("bhic,bhjc->bhij", np.abs(ref["q_mean"]).astype(np.float64),
                     np.repeat(np.abs(ks).astype(np.float64), 2, axis=1))
    ds_err = (128 + 4) * 2.0 ** -24 * sm * absb.max(axis=(2, 3))[..., None]
    err = np.abs(to_np(lse).astype(np.float64) - l_ref)
    assert np.all(err <= lse_tol(300, l_ref) + ds_err), err.max()


@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", [
    (1, 4, 2, 1000, 64, torch.float16, True),
    (2, 2, 1, 2200, 128, torch.bfloat16, False),
    (2, 6, 3, 300, 64, torch.float16, True),
    (1, 32, 16, 300, 64, torch.bfloat16, True),
    (4, 16, 8, 1100, 128, torch.float16, True),
])
def test_smooth_q_chunks_do_not_change_the_result(gpu_lib, B, H, H_kv, N, d, dtype, causal):
    """sage_attn_fwd_smooth_q computes the Delta S rows a chunk at a time in its
    workspace.  Workspaces of 2 to 48 Delta S rows (one group at a time with a range of
    Q blocks; every group with a range of Q blocks; for the 16-group shape at 48 rows,
    8 whole groups at a time), the default and more than the whole table give the same
    output and LSE bit for bit, and the workspace's previous contents do not matter."""
    print(f"smooth_q chunks case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal}",
          flush=True)
    q, k, v = _biased_q_inputs(B, H, H_kv, N, d, dtype, seed=N + d)
    sm = 1 / math.sqrt(d)
    qk = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV), True, smooth_q=True)
    vq = gpu_lib.sage_quant_v(v.to(DEV))
    kd = k.to(DEV)
    nmb = -(-N // 128)
    runs = {}
    for rows in (None, 2, 5, 12, 24, 48, B * H * (nmb + 5)):
        ws = (gpu_lib.smooth_q_workspace(B, H, N, d, device=DEV) if rows is None else
              torch.empty(rows * N * 4, dtype=torch.uint8, device=DEV))
        ws.fill_(0xFF)   # NaN bit patterns: a row the kernel read before writing would show
        runs[rows] = gpu_lib.sage_attn_fwd_smooth_q(qk, vq, kd, causal=causal, sm_scale=sm,
                                                    out_dtype=dtype, return_lse=True,
                                                    workspace=ws)
    torch.cuda.synchronize()
    o0, l0 = runs[None]
    assert torch.isfinite(o0).all() and torch.isfinite(l0).all()
    for rows, (o, lse) in runs.items():
        assert torch.equal(o, o0), rows
        assert torch.equal(lse, l0), rows
    # and the result is the oracle's (sampled rows)
    ref = O.quantize_qk(q, k, smooth_q=True)
    refv = O.quantize_v(v)
    rws = np.array([0, 1, 127, 128, N // 2, N - 1])
    o_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"], refv["v_f8"],
                         refv["v_scale"], causal=causal, sm_scale=sm, rows=rws,
                         delta_s=O.delta_s(ref["q_mean"], k, ref["k_mean"]))
    compare_output(o0[:, :, torch.from_numpy(rws).to(DEV)], o_ref)


@pytest.mark.parametrize("smooth_q,pv,causal", [(False, "fp8", False), (True, "fp8", True),
                                                 (False, "mxfp4", True)])
def test_plan_graph_replays_match_eager(gpu_lib, smooth_q, pv, causal):
    """SagePlan.capture records quant() + attn() as a HIP graph.  Every replay, with eager
    steps on other inputs and synchronizations between the replays, gives the eager
    step's output bit for bit, and a replay reads the inputs' contents at replay time."""
    B, H, H_kv, N, d, dtype = 1, 4, 2, 700, 128, torch.float16
    print(f"graph replay case smooth_q={smooth_q} pv={pv} causal={causal}", flush=True)
    plan = gpu_lib.SagePlan(B, H, H_kv, N, d, dtype, causal, device=DEV, smooth_q=smooth_q,
                            pv=pv)
    q, k, v = (t.to(DEV) for t in _biased_q_inputs(B, H, H_kv, N, d, dtype, seed=5))
    q2, k2, v2 = (t.to(DEV) for t in _biased_q_inputs(B, H, H_kv, N, d, dtype, seed=6))
    o1 = plan(q, k, v).clone()
    o2 = plan(q2, k2, v2).clone()
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and not torch.equal(o1, o2)
    graph = plan.capture(q, k, v)
    torch.cuda.synchronize()
    for i in range(3):
        plan(q2, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(plan.o, o2), i
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.o, o1), i
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(plan.o, o2)


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_peak_loop_runs_every_mfma(gpu_lib, kind):
    """The roofline probe: every lane's accumulator sum is 64 elements x (32 or 64) x iters
    (all operands 1), every wave's clocks are positive, and the shader clock they imply is
    a plausible one."""
    print(f"mfma peak probe kind={kind}", flush=True)
    iters, nwg = 2000, 512
    ops, clocks, sink, khz = gpu_lib.sage_mfma_peak(kind, iters, nwg, device=DEV)
    torch.cuda.synchronize()
    assert ops == nwg * 16 * iters * (65536 if kind == 0 else 131072)
    per = 32 if kind == 0 else 64
    assert torch.all(sink == 64 * per * iters)
    c = clocks.cpu().numpy().astype(np.float64)
    assert (c > 0).all() and khz > 0
    ghz = float(np.median(c[:, 0] / c[:, 1])) * khz / 1e6
    assert 0.5 < ghz < 3.0, ghz


def test_delta_s_row_ranges(gpu_lib):
    """sage_delta_s over a range of Q blocks writes exactly those rows of the whole table."""
    q, k, v = _biased_q_inputs(1, 3, 1, 1100, 64, torch.float16, seed=77)
    qk = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV), True, smooth_q=True)
    kd = k.to(DEV)
    full = gpu_lib.sage_delta_s(kd, qk, 0.125)
    for i0, n in ((0, 1), (2, 3), (8, 1), (0, 9), (5, 4)):
        part = gpu_lib.sage_delta_s(kd, qk, 0.125, i0=i0, nrows=n)
        torch.cuda.synchronize()
        assert torch.equal(part, full[:, :, i0:i0 + n]), (i0, n)


def test_smooth_q_tracks_exact_attention(gpu_lib):
    """End to end (sageattn): on Q with a shared channel bias, smoothing Q brings the
    quantized result closer to exact FP64 attention than quantizing Q directly."""
    q, k, v = _biased_q_inputs(1, 4, 2, 512, 128, torch.float16, seed=53, qbias=3.0)
    sm = 1 / math.sqrt(128)
    ex = O.attn_exact(q, k, v, causal=True, sm_scale=sm)
    rl1 = {}
    for sq in (False, True):
        o = gpu_lib.sageattn(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=True, sm_scale=sm,
                             smooth_q=sq)
        torch.cuda.synchronize()
        m = O.metrics(to_np(o).astype(np.float64), ex)
        rl1[sq] = m["rel_l1"]
        assert m["cos"] >= 0.998, (sq, m)
    assert rl1[True] < rl1[False], rl1


# ------------------------------------------------------------------ MXFP4 P V

def _check_quant_v4(qa, v):
    vq4 = qa.sage_quant_v_mxfp4(v.to(DEV))
    torch.cuda.synchronize()
    ref4 = O.quantize_v_mxfp4(v)
    N, d = v.shape[2], v.shape[3]
    codes, e = v4_natural(to_np(vq4["v_f4"]), to_np(vq4["v_e8"]), N, d)
    np_ = ref4["v_f4"].shape[2]
    assert np.array_equal(codes[:, :, :np_], ref4["v_f4"]), "MXFP4 V codes differ"
    assert (codes[:, :, np_:] == 0).all(), "MXFP4 V padding must be zero codes"
    nb = ref4["v_e8"].shape[2]
    assert np.array_equal(e[:, :, :nb], ref4["v_e8"]), "MXFP4 V exponents differ"
    return vq4, ref4


MX_CASES = [SMALL[i] for i in (0, 1, 3, 5, 9, 10)]


@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", MX_CASES)
def test_mxfp4_parity(gpu_lib, B, H, H_kv, N, d, dtype, causal):
    """MXFP4 P V: V codes and E8M0 exponents bit-exact; the output against the oracle's
    MXFP4 recursion within max-abs 2e-2 and cosine 0.9995."""
    print(f"mxfp4 case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed=N * 13 + d)
    qk = gpu_lib.sage_quant_qk(q.to(DEV), k.to(DEV))
    ref = O.quantize_qk(q, k)
    vq4, ref4 = _check_quant_v4(gpu_lib, v)
    sm = 1 / math.sqrt(d)
    o = gpu_lib.sage_attn_fwd_mxfp4(qk, vq4, causal=causal, sm_scale=sm, out_dtype=dtype)
    torch.cuda.synchronize()
    o_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"], ref4["v_f4"],
                         ref4["v_e8"], causal=causal, sm_scale=sm, pv="mxfp4")
    print(compare_output_mx(o, o_ref), flush=True)


def test_mxfp4_lse_and_exact(gpu_lib):
    """The MXFP4 LSE (no factor 448 in l) against the oracle's, and the output close to
    exact attention (the pages quote CosSim 98.37 % for MXFP4)."""
    q, k, v = _rand_inputs(1, 4, 2, 700, 128, torch.bfloat16, seed=71)
    sm = 1 / math.sqrt(128)
    o, lse = gpu_lib.sageattn(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=True, sm_scale=sm,
                              return_lse=True, pv="mxfp4")
    torch.cuda.synchronize()
    ref = O.quantize_qk(q, k)
    ref4 = O.quantize_v_mxfp4(v)
    _, l_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                            ref4["v_f4"], ref4["v_e8"], causal=True, sm_scale=sm, pv="mxfp4",
                            return_lse=True)
    c_ref = O.lse_correction(q, ref["k_mean"], sm_scale=sm)
    c_abs = O.lse_correction(q.float().abs(), np.abs(ref["k_mean"]), sm_scale=sm)
    err = np.abs(to_np(lse).astype(np.float64) - (l_ref + c_ref))
    assert np.all(err <= lse_tol(700, l_ref, c_abs)), err.max()
    ex = O.attn_exact(q, k, v, causal=True, sm_scale=sm)
    m = O.metrics(to_np(o.float()).astype(np.float64), ex)
    assert m["cos"] >= 0.975, m


@pytest.mark.parametrize("name,heads,nrows", [
    ("llm_prefill", [(0, 9)], 96),
    ("video_dit", [(0, 20)], 64),
])
def test_workload_parity_mxfp4(gpu_lib, name, heads, nrows):
    w = W.get(name)
    print(f"workload {name} mxfp4: generating", flush=True)
    t = W.generate(w)
    plan = gpu_lib.SagePlan(w.B, w.H, w.H_kv, w.N, w.d, w.torch_dtype, w.causal, pv="mxfp4")
    o = plan(t["q"].to(DEV), t["k"].to(DEV), t["v"].to(DEV))
    torch.cuda.synchronize()
    grp = w.H // w.H_kv
    for b, h in heads:
        hk = h // grp
        ref = O.quantize_qk(t["q"][b:b + 1, h:h + 1], t["k"][b:b + 1, hk:hk + 1])
        ref4 = O.quantize_v_mxfp4(t["v"][b:b + 1, hk:hk + 1])
        codes, e = v4_natural(to_np(plan.vq["v_f4"][b:b + 1, hk:hk + 1]),
                              to_np(plan.vq["v_e8"][b:b + 1, hk:hk + 1]), w.N, w.d)
        assert np.array_equal(codes[:, :, :ref4["v_f4"].shape[2]], ref4["v_f4"])
        assert np.array_equal(e[:, :, :ref4["v_e8"].shape[2]], ref4["v_e8"])
        g = np.random.default_rng(b * 100 + h)
        rows = np.unique(np.concatenate([g.choice(w.N, size=nrows, replace=False), [0, w.N - 1]]))
        o_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                             ref4["v_f4"], ref4["v_e8"], causal=w.causal, sm_scale=w.sm_scale,
                             rows=rows, pv="mxfp4")
        m = compare_output_mx(o[b, h, torch.from_numpy(rows).to(DEV)], o_ref[0, 0])
        print(f"workload {name} mxfp4 head {(b, h)}: {m}", flush=True)


# ------------------------------------------------------------------ the workloads

def _workload_check(gpu_lib, name, heads, nrows, seed=0, q_group=128, smooth_q=False):
    w = W.get(name)
    print(f"workload {name} q_group {q_group} smooth_q {smooth_q}: generating", flush=True)
    t = W.generate(w)
    plan = gpu_lib.SagePlan(w.B, w.H, w.H_kv, w.N, w.d, w.torch_dtype, w.causal,
                            q_group=q_group, smooth_q=smooth_q)
    qd, kd, vd = t["q"].to(DEV), t["k"].to(DEV), t["v"].to(DEV)
    o = plan(qd, kd, vd)
    torch.cuda.synchronize()
    print(f"workload {name}: gpu done", flush=True)
    # bit-exact quantities on the sampled heads (all tokens)
    hk_set = sorted({(b, h // (w.H // w.H_kv)) for b, h in heads})
    sub = lambda x, hs: np.stack([x[b, h] for b, h in hs])
    qsel = torch.stack([t["q"][b, h] for b, h in heads])[None]
    ksel = torch.stack([t["k"][b, h] for b, h in hk_set])[None]
    vsel = torch.stack([t["v"][b, h] for b, h in hk_set])[None]
    ref = O.quantize_qk(qsel, ksel, q_group=q_group, smooth_q=smooth_q)
    refv = O.quantize_v(vsel)
    if smooth_q:
        assert np.array_equal(sub(to_np(plan.qk["q_mean"]), heads), ref["q_mean"][0])
    assert np.array_equal(sub(to_np(plan.qk["k_mean"]), hk_set), ref["k_mean"][0])
    assert np.array_equal(sub(to_np(plan.qk["q_i8"]), heads), ref["q_i8"][0])
    assert np.array_equal(sub(to_np(plan.qk["q_scale"]), heads), ref["q_scale"][0])
    assert np.array_equal(sub(to_np(plan.qk["k_i8"]), hk_set), ref["k_i8"][0])
    assert np.array_equal(sub(to_np(plan.qk["k_scale"]), hk_set), ref["k_scale"][0])
    assert np.array_equal(sub(to_np(plan.vq["v_scale"]), hk_set), refv["v_scale"][0])
    vn, _ = v_natural(sub(to_np(plan.vq["v_f8"]), hk_set)[None], w.N, w.d)
    assert np.array_equal(F8.decode(vn), F8.decode(refv["v_f8"]))
    # output on sampled rows (ragged tail and, if causal, the first rows included)
    g = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([g.choice(w.N, size=min(nrows, w.N), replace=False),
                                     [0, 1, w.N - 1]]))
    # re-index the selected heads as a small (1, len(heads)) problem with its own GQA map
    qsel_i8 = ref["q_i8"]
    kv_index = [hk_set.index((b, h // (w.H // w.H_kv))) for b, h in heads]
    o_ref = np.zeros((len(heads), len(rows), w.d))
    if smooth_q:
        # Delta S rows of two Q blocks (the attention computes its own, chunk by chunk)
        i0 = (-(-w.N // 128)) // 2
        ds_rows = to_np(gpu_lib.sage_delta_s(kd, plan.qk, w.sm_scale, i0=i0, nrows=2))
    for j, (b, h) in enumerate(heads):
        kvj = kv_index[j]
        ds = None
        if smooth_q:
            ds = O.delta_s(ref["q_mean"][:, j:j + 1], ksel[:, kvj:kvj + 1],
                           ref["k_mean"][:, kvj:kvj + 1])
            _check_delta_s_table(ds_rows[b, h], ds[0, 0, i0:i0 + 2], ref["q_mean"][0, j],
                                 ksel[0, kvj].float().numpy(), ref["k_mean"][0, kvj], w.sm_scale)
        o1 = O.attn_quant(qsel_i8[:, j:j + 1], ref["q_scale"][:, j:j + 1],
                          ref["k_i8"][:, kvj:kvj + 1], ref["k_scale"][:, kvj:kvj + 1],
                          refv["v_f8"][:, kvj:kvj + 1], refv["v_scale"][:, kvj:kvj + 1],
                          causal=w.causal, sm_scale=w.sm_scale, rows=rows, blkq=q_group,
                          delta_s=ds)
        o_ref[j] = o1[0, 0]
    o_gpu = torch.stack([o[b, h, torch.from_numpy(rows).to(DEV)] for b, h in heads])
    m = compare_output(o_gpu, o_ref)
    print(f"workload {name}: {m}", flush=True)


@pytest.mark.parametrize("name,heads,nrows", [
    ("tiny", [(0, 0), (0, 1)], 256),
    ("llm_prefill", [(0, 0), (0, 17), (0, 31)], 192),
    ("video_dit", [(0, 0), (0, 47)], 128),
    ("sweep@N1024", [(0, 0), (3, 31)], 192),
    ("sweep@N2048", [(2, 5)], 128),
    ("sweep@N4096", [(1, 7)], 128),
    ("sweep@N8192", [(0, 19)], 96),
    ("sweep@N16384", [(3, 2)], 64),
    ("sweep@N32768", [(3, 30)], 64),
    ("gqa_long", [(0, 0), (0, 3), (0, 29)], 48),
])
def test_workload_parity(gpu_lib, name, heads, nrows):
    _workload_check(gpu_lib, name, heads, nrows)


@pytest.mark.parametrize("name,heads,nrows,q_group", [
    ("llm_prefill", [(0, 0), (0, 31)], 128, 1),
    ("video_dit", [(0, 5)], 96, 32),
    ("sweep@N4096", [(2, 9)], 96, 1),
    ("gqa_long", [(0, 6)], 32, 32),
])
def test_workload_parity_q_group(gpu_lib, name, heads, nrows, q_group):
    _workload_check(gpu_lib, name, heads, nrows, q_group=q_group)


@pytest.mark.parametrize("name,heads,nrows,q_group", [
    ("llm_prefill", [(0, 3)], 128, 128),
    ("video_dit", [(0, 11), (0, 40)], 64, 1),
    ("sweep@N4096", [(3, 2)], 96, 128),
])
def test_workload_parity_smooth_q(gpu_lib, name, heads, nrows, q_group):
    _workload_check(gpu_lib, name, heads, nrows, q_group=q_group, smooth_q=True)


# ------------------------------------------------------------------ log-sum-exp (LSE)

@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal", [
    (1, 2, 2, 256, 64, torch.float16, False),
    (2, 4, 2, 700, 128, torch.bfloat16, True),
    (1, 8, 1, 255, 64, torch.float16, True),
    (1, 2, 2, 129, 128, torch.float16, False),
])
def test_lse_parity(gpu_lib, B, H, H_kv, N, d, dtype, causal):
    """sage_attn_fwd_lse: O identical to sage_attn_fwd; lse = ln sum exp of the scores used
    (+ the q . mean(K) correction) against the oracle's m_T + ln l (+ lse_correction)."""
    print(f"lse case B{B} H{H}/{H_kv} N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = _rand_inputs(B, H, H_kv, N, d, dtype, seed=N * 5 + d)
    qk, vq, ref, refv = _check_quant(gpu_lib, q, k, v)
    sm = 1 / math.sqrt(d)
    o0 = gpu_lib.sage_attn_fwd(qk, vq, causal=causal, sm_scale=sm, out_dtype=dtype)
    corr = gpu_lib.sage_lse_correction(q.to(DEV), qk["k_mean"], sm)
    o1, lse = gpu_lib.sage_attn_fwd_lse(qk, vq, causal=causal, sm_scale=sm, out_dtype=dtype,
                                        lse_corr=corr)
    _, lse_raw = gpu_lib.sage_attn_fwd_lse(qk, vq, causal=causal, sm_scale=sm, out_dtype=dtype)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
    _, l_ref = O.attn_quant(ref["q_i8"], ref["q_scale"], ref["k_i8"], ref["k_scale"],
                            refv["v_f8"], refv["v_scale"], causal=causal, sm_scale=sm,
                            return_lse=True)
    c_ref = O.lse_correction(q, ref["k_mean"], sm_scale=sm)
    c_gpu = to_np(corr).astype(np.float64)
    # FP32 dot product of d terms: within (d + 2) * 2^-24 * sm * sum |q_c mean_c|
    c_abs = O.lse_correction(q.float().abs(), np.abs(ref["k_mean"]), sm_scale=sm)
    c_err = np.abs(c_gpu - c_ref)
    assert np.all(c_err <= (d + 2) * 2.0 ** -24 * c_abs + 1e-9), c_err.max()
    tol = lse_tol(N, l_ref, c_abs)
    err = np.abs(to_np(lse).astype(np.float64) - (l_ref + c_ref))
    assert np.all(err <= tol), (err.max(), np.unravel_index(err.argmax(), err.shape))
    err_raw = np.abs(to_np(lse_raw).astype(np.float64) - l_ref)
    assert np.all(err_raw <= lse_tol(N, l_ref)), err_raw.max()


def test_lse_tracks_exact_lse(gpu_lib):
    """End to end (sageattn with return_lse): the corrected LSE of the quantized method is
    close to the exact FP64 LSE of the original inputs (quantization error only), for a
    workload with a large shared K bias (the correction is many units)."""
    q, k, v = _rand_inputs(1, 4, 2, 512, 128, torch.float16, seed=41, bias=3.0)
    o, lse = gpu_lib.sageattn(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=True,
                              sm_scale=1 / math.sqrt(128), return_lse=True)
    torch.cuda.synchronize()
    _, l_exact = O.attn_exact(q, k, v, causal=True, sm_scale=1 / math.sqrt(128), return_lse=True)
    assert np.abs(to_np(lse).astype(np.float64) - l_exact).max() < 0.05
