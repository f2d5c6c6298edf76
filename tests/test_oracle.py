"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: each checks a worked value, a
closed form, an invariant, a library routine or a brute-force loop.
"""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import fp8_e4m3 as F8
from oracle import mxfp4 as MX
from oracle import sage_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------- FP8 codec

def test_fp8_golden_points():
    for line in open(os.path.join(GOLD, "fp8_e4m3_points.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        val, code = line.split()
        assert int(F8.encode(float(val))) == int(code, 16), line
        if abs(float(val)) <= 448 and "e" not in val:
            # points that are grid values decode back exactly
            r = F8.decode(np.uint8(int(code, 16)))
            assert r == F8.round_to_e4m3(float(val))


def test_fp8_exhaustive_roundtrip():
    codes = np.arange(256, dtype=np.uint8)
    vals = F8.decode(codes)
    ok = ~np.isnan(vals)
    assert ok.sum() == 254                       # only S.1111.111 is NaN
    assert np.nanmax(vals) == 448.0 and np.nanmin(vals) == -448.0
    assert (F8.encode(vals[ok]) == codes[ok]).all()


def test_fp8_midpoints_round_to_even():
    vals = np.unique(F8.decode(np.arange(0, 0x7F, dtype=np.uint8)))   # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    got = F8.encode(mids)
    lo = F8.encode(vals[:-1])
    hi = F8.encode(vals[1:])
    even = np.where(lo % 2 == 0, lo, hi)
    assert (got == even).all()
    # just off the midpoint goes to the nearer neighbour
    assert (F8.encode(mids * (1 - 1e-9)) == lo).all()
    assert (F8.encode(mids * (1 + 1e-9)) == hi).all()


def test_fp8_matches_torch_in_range():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * 10 ** g.uniform(-4, 2.6, 20000),
                        g.uniform(-448, 448, 20000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]            # torch's cast does not saturate; compare in range
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F8.encode(x.astype(np.float64))
    same = (F8.decode(got) == F8.decode(ref))
    assert same.all(), x[~same][:10]


def test_fp8_saturates():
    assert (F8.encode([449.0, 464.0, 479.0, 1e30]) == 0x7E).all()
    assert (F8.encode([-449.0, -1e30]) == 0xFE).all()


# --------------------------------------------------------------------- INT8 quant

def _read_sections(path):
    sec, out = None, {}
    for line in open(path):
        line = line.strip()
        if line.startswith("# section:"):
            sec = line.split(":", 1)[1].strip()
            out[sec] = []
        elif line and not line.startswith("#"):
            out[sec].append([float(t) for t in line.split()])
    return out


def test_int8_worked_example():
    s = _read_sections(os.path.join(GOLD, "int8_block_example.txt"))
    x = np.array(s["input"], dtype=np.float32)[None]
    codes, scales = O.quantize_int8_blocks(x, 128)
    assert scales[0, 0] == np.float32(s["scale"][0][0])
    assert (codes[0] == np.array(s["codes"])).all()


def test_int8_invariants_random_blocks():
    g = np.random.default_rng(1)
    x = (g.standard_normal((3, 300, 64)) * np.exp(g.uniform(-20, 20, (3, 1, 1)))).astype(np.float32)
    codes, scales = O.quantize_int8_blocks(x, 64)
    assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= 127
    for h in range(3):
        for i in range(scales.shape[1]):
            xb = x[h, i * 64:(i + 1) * 64].astype(np.float64)
            cb = codes[h, i * 64:(i + 1) * 64].astype(np.float64)
            s = float(scales[h, i])
            assert np.abs(cb).max() == 127                     # the block's amax hits 127
            assert abs(np.abs(xb).max() / s - 127) < 127 * 2 ** -22
            err = np.abs(xb - cb * s)
            assert (err <= s / 2 * (1 + 2 ** -20)).all()      # nearest code


def test_int8_zero_block_and_tail():
    x = np.zeros((1, 150, 8), dtype=np.float32)
    x[0, 130:] = 3.0
    codes, scales = O.quantize_int8_blocks(x, 128)
    assert scales[0, 0] == 0 and (codes[0, :128] == 0).all()
    assert scales.shape == (1, 2)
    assert (codes[0, 130:] == 127).all() and (codes[0, 128:130] == 0).all()


def test_int8_ties_go_to_even():
    # amax 127 -> scale exactly 1.0; x = k + 0.5 hits ties
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]], dtype=np.float32)[None]
    codes, scales = O.quantize_int8_blocks(x, 128)
    assert scales[0, 0] == 1.0
    assert codes[0, 0].tolist() == [127, 0, 2, 2, 0, -2, -2, 4]


@pytest.mark.parametrize("q_group", [1, 32])
def test_q_group_scales_cover_their_runs(q_group):
    # each scale belongs to exactly the q_group consecutive tokens it covers:
    # its group's amax lands on code 127, and changing a token moves only
    # its own group's scale
    g = np.random.default_rng(11)
    n = 100
    q = torch.from_numpy((g.standard_normal((1, 2, n, 64)) *
                          np.exp(g.uniform(-3, 3, (1, 2, n, 1)))).astype(np.float32)).half()
    k = torch.from_numpy(g.standard_normal((1, 2, n, 64)).astype(np.float32)).half()
    z = O.quantize_qk(q, k, q_group=q_group)
    qs = z["q_scale"]
    assert qs.shape == (1, 2, -(-n // q_group))
    q32 = q.float().numpy()
    for h in range(2):
        for i in range(qs.shape[2]):
            rows = slice(i * q_group, min((i + 1) * q_group, n))
            c = z["q_i8"][0, h, rows].astype(np.int64)
            assert np.abs(c).max() == 127
            assert abs(np.abs(q32[0, h, rows]).max() / float(qs[0, h, i]) - 127) < 127 * 2 ** -22
    q2 = q.clone()
    q2[0, 1, 70] = 500.0          # above every |q| of the input: its group's new amax
    z2 = O.quantize_qk(q2, k, q_group=q_group)
    changed = np.nonzero(z2["q_scale"] != qs)
    assert set(zip(*changed)) == {(0, 1, 70 // q_group)}


def test_q_group_128_is_the_block_quantizer():
    g = np.random.default_rng(12)
    q = torch.from_numpy(g.standard_normal((1, 1, 300, 64)).astype(np.float32)).half()
    k = torch.from_numpy(g.standard_normal((1, 1, 300, 64)).astype(np.float32)).half()
    a = O.quantize_qk(q, k)
    b = O.quantize_qk(q, k, q_group=128)
    assert (a["q_i8"] == b["q_i8"]).all() and (a["q_scale"] == b["q_scale"]).all()
    with pytest.raises(AssertionError):
        O.quantize_qk(q, k, q_group=16)


def test_q_group_score_error_ordering():
    # Table 6 of the detail page: finer Q groups quantize more accurately
    # (per-token/per-thread below per-block).  On queries whose magnitudes
    # vary from token to token, the dequantized scores' relative L1 error
    # falls strictly as the group shrinks from 128 to 32 to 1 token.
    g = np.random.default_rng(13)
    n, d = 256, 64
    q = torch.from_numpy((g.standard_normal((1, 1, n, d)) *
                          np.exp(g.uniform(-2, 2, (1, 1, n, 1)))).astype(np.float32)).half()
    k = torch.from_numpy(g.standard_normal((1, 1, n, d)).astype(np.float32)).half()
    s_ref = q.double().numpy()[0, 0] @ k.double().numpy()[0, 0].T
    err = {}
    for qg in (128, 32, 1):
        z = O.quantize_qk(q, k, smooth_k=False, q_group=qg)
        qd = z["q_i8"][0, 0].astype(np.float64) * z["q_scale"][0, 0, np.arange(n) // qg, None]
        kd = z["k_i8"][0, 0].astype(np.float64) * z["k_scale"][0, 0, np.arange(n) // 64, None]
        err[qg] = np.abs(qd @ kd.T - s_ref).sum() / np.abs(s_ref).sum()
    assert err[1] < err[32] < err[128]
    assert err[1] < 0.5 * err[128]


# --------------------------------------------------------------------- Smooth K

def test_k_mean_equals_fsum():
    t = W.generate(W.get("tiny"))
    k = t["k"].float().numpy()
    assert O.exactness_margin_bits(k) > 0
    got = O.k_sum_exact(k)
    for h in range(k.shape[1]):
        for c in range(k.shape[3]):
            assert got[0, h, c] == math.fsum(k[0, h, :, c].astype(np.float64).tolist())
    mean = O.k_mean(k)
    assert mean.dtype == np.float32


def test_smoothing_invariance_exact_attention():
    """Softmax is shift invariant along a row: K and K - mean give the same O."""
    w = W.get("tiny")
    t = W.generate(w)
    k64 = t["k"].double()
    ks = k64 - k64.mean(dim=2, keepdim=True)
    for causal in (False, True):
        a = O.attn_exact(t["q"], k64, t["v"], causal=causal, sm_scale=w.sm_scale)
        b = O.attn_exact(t["q"], ks, t["v"], causal=causal, sm_scale=w.sm_scale)
        assert np.abs(a - b).max() <= 1e-6


def test_smoothing_removes_a_shared_bias_exactly():
    """K + c (c exact per channel) smooths to the same K - mean, so same codes."""
    g = np.random.default_rng(2)
    # k on a 1/16 grid, c on an 8 grid, N a power of two: k + c is exact in
    # fp16, and the sums, the mean and k - mean are all exact in float32/64
    k = (g.integers(-64, 64, (1, 2, 256, 16)) / 16.0).astype(np.float32)
    c = (g.integers(-4, 5, (1, 2, 1, 16)) * 8.0).astype(np.float32)
    q = g.standard_normal((1, 2, 256, 16)).astype(np.float32)
    a = O.quantize_qk(q, torch.from_numpy(k).half())
    b = O.quantize_qk(q, torch.from_numpy(k + c).half())
    assert (a["k_i8"] == b["k_i8"]).all() and (a["k_scale"] == b["k_scale"]).all()
    assert np.allclose(b["k_mean"] - a["k_mean"], c[:, :, 0], atol=0)
    # without smoothing the bias leaks into the codes
    n = O.quantize_qk(q, torch.from_numpy(k + c).half(), smooth_k=False)
    assert not (n["k_i8"] == a["k_i8"]).all()


# --------------------------------------------------------------------- exact attention

def _brute_attention(q, k, v, causal, sm_scale, grp):
    B, H, N, d = q.shape
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(H):
            hk = h // grp
            for i in range(N):
                sc = []
                for j in range(N):
                    if causal and j > i:
                        continue
                    sc.append((j, sm_scale * sum(float(q[b, h, i, c]) * float(k[b, hk, j, c]) for c in range(d))))
                mx = max(s for _, s in sc)
                den = sum(math.exp(s - mx) for _, s in sc)
                for c in range(d):
                    out[b, h, i, c] = sum(math.exp(s - mx) * float(v[b, hk, j, c]) for j, s in sc) / den
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2)])
def test_exact_attention_brute_force(causal, H, H_kv):
    g = np.random.default_rng(3)
    q = g.standard_normal((1, H, 12, 8))
    k = g.standard_normal((1, H_kv, 12, 8)) + 2
    v = g.standard_normal((1, H_kv, 12, 8))
    ref = _brute_attention(q, k, v, causal, 0.4, H // H_kv)
    got = O.attn_exact(q, k, v, causal=causal, sm_scale=0.4)
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_exact_attention_matches_sdpa(causal):
    w = W.get("tiny")
    t = W.generate(w)
    ref = torch.nn.functional.scaled_dot_product_attention(
        t["q"].double(), t["k"].double(), t["v"].double(), is_causal=causal,
        scale=w.sm_scale).numpy()
    got = O.attn_exact(t["q"], t["k"], t["v"], causal=causal, sm_scale=w.sm_scale)
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    w = W.get("tiny")
    t = W.generate(w)
    p = O.softmax_rows(t["q"], t["k"], causal=causal, sm_scale=w.sm_scale, h=1)
    assert np.abs(p.sum(axis=1) - 1).max() <= 1e-12
    if causal:
        assert (np.triu(p, 1) == 0).all()


# --------------------------------------------------------------------- quantized attention

def _quant_all(t, smooth=True):
    qz = O.quantize_qk(t["q"], t["k"], smooth_k=smooth)
    vz = O.quantize_v(t["v"])
    return qz, vz


def _aq(qz, vz, **kw):
    return O.attn_quant(qz["q_i8"], qz["q_scale"], qz["k_i8"], qz["k_scale"],
                        vz["v_f8"], vz["v_scale"], **kw)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("grp", [1, 2])
def test_closed_form_matches_literal_recursion(causal, grp):
    g = np.random.default_rng(4)
    n, d, H = 45, 8, 2 * grp
    q = torch.from_numpy(g.standard_normal((1, H, n, d)).astype(np.float32) * 2).half()
    k = torch.from_numpy(g.standard_normal((1, 2, n, d)).astype(np.float32) + 3).half()
    v = torch.from_numpy(g.standard_normal((1, 2, n, d)).astype(np.float32)).half()
    qz = O.quantize_qk(q, k)
    vz = O.quantize_v(v)
    kw = dict(causal=causal, sm_scale=0.35, kv_tile=16, blkq=16, blkk=8)
    qz16 = dict(q_i8=qz["q_i8"], k_i8=qz["k_i8"])
    # per-16 / per-8 scales so several scale blocks fall in one run
    _, qs = O.quantize_int8_blocks(q.float().numpy(), 16)
    qc, _ = O.quantize_int8_blocks(q.float().numpy(), 16)
    ks32 = (k.float().numpy() - qz["k_mean"][:, :, None, :]).astype(np.float32)
    kc, kss = O.quantize_int8_blocks(ks32, 8)
    a = O.attn_quant(qc, qs, kc, kss, vz["v_f8"], vz["v_scale"], **kw)
    for h in range(H):
        r = O.attn_quant_recursive(qc, qs, kc, kss, vz["v_f8"], vz["v_scale"],
                                   causal=causal, sm_scale=0.35, kv_tile=16, h=h,
                                   hk=h // grp, blkq=16, blkk=8)
        assert np.abs(a[0, h] - r).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_dequantized_v(causal):
    w = W.get("tiny")
    t = W.generate(w)
    t["q"] = torch.zeros_like(t["q"])
    qz, vz = _quant_all(t)
    assert (qz["q_scale"] == 0).all()
    o = _aq(qz, vz, causal=causal, sm_scale=w.sm_scale)
    vdq = F8.decode(vz["v_f8"]) * vz["v_scale"][:, :, None, :].astype(np.float64)
    if causal:
        ref = np.cumsum(vdq, axis=2) / np.arange(1, w.N + 1)[None, None, :, None]
    else:
        ref = np.broadcast_to(vdq.mean(axis=2, keepdims=True), vdq.shape)
    assert np.abs(o - ref).max() < 1e-12


def test_constant_v_returns_it():
    w = W.get("tiny")
    t = W.generate(w)
    row = torch.linspace(-3, 3, w.d).half()
    t["v"] = row.expand_as(t["v"]).contiguous()
    qz, vz = _quant_all(t)
    o = _aq(qz, vz, causal=True, sm_scale=w.sm_scale)
    vdq = F8.decode(vz["v_f8"][0, 0, 0]) * vz["v_scale"][0, 0].astype(np.float64)
    # weights sum to l * 448 up to the FP8 rounding of P, so O is v times a
    # factor within the P-rounding error of 1
    ratio = o / vdq[None, None, None, :]
    fin = np.isfinite(ratio) & (np.abs(vdq) > 0)[None, None, None, :]
    assert np.abs(ratio[fin] - 1).max() < 2 ** -4


def test_one_dominant_key():
    g = np.random.default_rng(5)
    n, d = 64, 16
    k = g.standard_normal((1, 1, n, d)).astype(np.float32)
    q = np.zeros((1, 1, n, d), dtype=np.float32)
    q[..., :] = 40 * k[0, 0, 17]                        # every query aligns with key 17
    v = g.standard_normal((1, 1, n, d)).astype(np.float32)
    qz = O.quantize_qk(torch.from_numpy(q).half(), torch.from_numpy(k).half(), smooth_k=False)
    vz = O.quantize_v(torch.from_numpy(v).half())
    o = _aq(qz, vz, causal=False, sm_scale=1.0)
    vdq = F8.decode(vz["v_f8"][0, 0, 17]) * vz["v_scale"][0, 0]
    assert np.abs(o[0, 0] - vdq[None, :]).max() < 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_unrounded_p_equals_exact_attention_on_dequantized_inputs(causal):
    w = W.get("tiny")
    t = W.generate(w)
    qz, vz = _quant_all(t)
    got = _aq(qz, vz, causal=causal, sm_scale=w.sm_scale, quantize_p=False)
    qd = qz["q_i8"].astype(np.float64) * np.repeat(qz["q_scale"], 128, axis=-1)[..., :w.N, None]
    kd = qz["k_i8"].astype(np.float64) * np.repeat(qz["k_scale"], 64, axis=-1)[..., :w.N, None]
    vd = F8.decode(vz["v_f8"]) * vz["v_scale"][:, :, None, :].astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qd), torch.from_numpy(kd), torch.from_numpy(vd),
        is_causal=causal, scale=w.sm_scale).numpy()
    assert np.abs(got - ref).max() < 1e-12


def test_tile_choice_changes_little():
    w = W.get("tiny")
    t = W.generate(w)
    qz, vz = _quant_all(t)
    a = _aq(qz, vz, causal=False, sm_scale=w.sm_scale, kv_tile=128)
    b = _aq(qz, vz, causal=False, sm_scale=w.sm_scale, kv_tile=w.N)
    m = O.metrics(a, b)
    assert m["max_abs"] < 2e-2 and m["cos"] > 0.9995


# --------------------------------------------------------------------- accuracy self-check

def _sample_check(name, heads, nrows, seed):
    w = W.get(name)
    t = W.generate(w, heads=heads)
    qz, vz = _quant_all(t)
    g = np.random.default_rng(seed)
    rows = np.sort(g.choice(w.N, size=min(nrows, w.N), replace=False))
    if w.causal:
        rows = np.unique(np.concatenate([rows, [0, 1, w.N - 1]]))
    oq = _aq(qz, vz, causal=w.causal, sm_scale=w.sm_scale, rows=rows, heads=heads)
    oe = O.attn_exact(t["q"], t["k"], t["v"], causal=w.causal, sm_scale=w.sm_scale,
                      rows=rows, heads=heads)
    sel = np.array([[b, h] for b, h in heads])
    m = O.metrics(oq[sel[:, 0], sel[:, 1]], oe[sel[:, 0], sel[:, 1]])
    assert m["cos"] >= 0.998, m
    return m


@pytest.mark.parametrize("causal", [False, True])
def test_per_token_q_scales_closed_form_matches_recursion(causal):
    # the dequantization reads the scale of the query's own group: with one
    # scale per token the closed form and the literal recursion agree
    g = np.random.default_rng(14)
    n, d = 40, 8
    q = torch.from_numpy((g.standard_normal((1, 2, n, d)) *
                          np.exp(g.uniform(-2, 2, (1, 2, n, 1)))).astype(np.float32)).half()
    k = torch.from_numpy(g.standard_normal((1, 2, n, d)).astype(np.float32) + 1).half()
    v = torch.from_numpy(g.standard_normal((1, 2, n, d)).astype(np.float32)).half()
    qz = O.quantize_qk(q, k, q_group=1)
    vz = O.quantize_v(v)
    kw = dict(causal=causal, sm_scale=0.4, kv_tile=16, blkq=1)
    a = O.attn_quant(qz["q_i8"], qz["q_scale"], qz["k_i8"], qz["k_scale"], vz["v_f8"],
                     vz["v_scale"], **kw)
    for h in range(2):
        r = O.attn_quant_recursive(qz["q_i8"], qz["q_scale"], qz["k_i8"], qz["k_scale"],
                                   vz["v_f8"], vz["v_scale"], h=h, **kw)
        assert np.abs(a[0, h] - r).max() < 1e-12


# ------------------------------------------------------------ smooth Q + Delta S

def _biased_q(shape, seed, bias=3.0):
    """Q with a per-(head, channel) bias shared by all tokens: the outlier
    structure smoothing Q removes (SageAttention2 detail page, Table 4)."""
    g = np.random.default_rng(seed)
    B, H, N, d = shape
    x = g.standard_normal(shape) + g.standard_normal((B, H, 1, d)) * bias
    return torch.from_numpy(x.astype(np.float32)).half()


def test_q_block_mean_equals_fsum():
    q = _biased_q((1, 2, 300, 16), 31)
    qm = O.q_block_mean(q.float().numpy())
    assert qm.shape == (1, 2, 3, 16) and qm.dtype == np.float32
    for h in range(2):
        for i in range(3):
            rows = q[0, h, i * 128:(i + 1) * 128].double().numpy()
            for c in range(16):
                assert qm[0, h, i, c] == np.float32(math.fsum(rows[:, c]) / rows.shape[0])


@pytest.mark.parametrize("smooth_k", [True, False])
def test_smooth_q_delta_s_restores_the_scores(smooth_k):
    # (Q - q_bar) K_s^T + Delta S = Q K_s^T: the compensation belongs to the
    # query's own 128-block and to every key, with GQA's head mapping
    g = np.random.default_rng(32)
    B, H, H_kv, N, d = 1, 4, 2, 300, 32
    q = _biased_q((B, H, N, d), 33)
    k = torch.from_numpy((g.standard_normal((B, H_kv, N, d)) + 2).astype(np.float32)).half()
    z = O.quantize_qk(q, k, smooth_k=smooth_k, smooth_q=True)
    ds = O.delta_s(z["q_mean"], k, z["k_mean"])
    assert ds.shape == (B, H, 3, N)
    q32 = q.float().numpy()
    qs = (q32 - np.repeat(z["q_mean"], 128, axis=-2)[..., :N, :]).astype(np.float32)
    ks = (k.float().numpy() - z["k_mean"][..., None, :]).astype(np.float32).astype(np.float64)
    for h in range(H):
        hk = h // 2
        recon = qs[0, h].astype(np.float64) @ ks[0, hk].T + ds[0, h][np.arange(N) // 128]
        exact = q32[0, h].astype(np.float64) @ ks[0, hk].T
        # only the float32 rounding of Q - q_bar separates the two
        bound = np.abs(q32[0, h]).astype(np.float64) @ np.abs(ks[0, hk]).T * 2.0 ** -23
        assert (np.abs(recon - exact) <= bound + 1e-12).all()


def test_smooth_q_lowers_the_score_error():
    # Table 4's direction: on Q with a shared channel bias, quantizing Q - q_bar
    # and adding Delta S back gives smaller score errors than quantizing Q
    g = np.random.default_rng(34)
    n, d = 512, 64
    q = _biased_q((1, 1, n, d), 35, bias=4.0)
    k = torch.from_numpy(g.standard_normal((1, 1, n, d)).astype(np.float32)).half()
    err = {}
    for sq in (False, True):
        z = O.quantize_qk(q, k, smooth_q=sq)
        ks = (k.float().numpy() - z["k_mean"][..., None, :]).astype(np.float32)
        exact = q.double().numpy()[0, 0] @ ks[0, 0].astype(np.float64).T
        qd = z["q_i8"][0, 0].astype(np.float64) * z["q_scale"][0, 0, np.arange(n) // 128, None]
        kd = z["k_i8"][0, 0].astype(np.float64) * z["k_scale"][0, 0, np.arange(n) // 64, None]
        s = qd @ kd.T
        if sq:
            s = s + O.delta_s(z["q_mean"], k, z["k_mean"])[0, 0][np.arange(n) // 128]
        err[sq] = np.abs(s - exact).sum() / np.abs(exact).sum()
    assert err[True] < 0.5 * err[False], err


@pytest.mark.parametrize("causal", [False, True])
def test_smooth_q_closed_form_matches_recursion(causal):
    g = np.random.default_rng(36)
    n, d = 150, 8
    q = _biased_q((1, 2, n, d), 37)
    k = torch.from_numpy((g.standard_normal((1, 1, n, d)) + 1).astype(np.float32)).half()
    v = torch.from_numpy(g.standard_normal((1, 1, n, d)).astype(np.float32)).half()
    z = O.quantize_qk(q, k, smooth_q=True, q_group=32)
    vz = O.quantize_v(v)
    ds = O.delta_s(z["q_mean"], k, z["k_mean"])
    kw = dict(causal=causal, sm_scale=0.3, kv_tile=32, blkq=32)
    args = (z["q_i8"], z["q_scale"], z["k_i8"], z["k_scale"], vz["v_f8"], vz["v_scale"])
    a, la = O.attn_quant(*args, delta_s=ds, return_lse=True, **kw)
    for h in range(2):
        r, lr = O.attn_quant_recursive(*args, h=h, hk=0, delta_s=ds, return_lse=True, **kw)
        assert np.abs(a[0, h] - r).max() < 1e-12
        assert np.abs(la[0, h] - lr).max() < 1e-12


def test_smooth_q_quantized_tracks_exact_attention():
    # with Delta S the smoothed-Q method is still attention on the original
    # inputs: close to exact attention, and closer than without smoothing Q
    g = np.random.default_rng(38)
    n, d = 384, 64
    q = _biased_q((1, 2, n, d), 39, bias=4.0)
    k = torch.from_numpy((g.standard_normal((1, 2, n, d)) + 2).astype(np.float32)).half()
    v = torch.from_numpy(g.standard_normal((1, 2, n, d)).astype(np.float32)).half()
    ex = O.attn_exact(q, k, v, causal=True, sm_scale=0.125)
    vz = O.quantize_v(v)
    rl1 = {}
    for sq in (False, True):
        z = O.quantize_qk(q, k, smooth_q=sq)
        ds = O.delta_s(z["q_mean"], k, z["k_mean"]) if sq else None
        o = O.attn_quant(z["q_i8"], z["q_scale"], z["k_i8"], z["k_scale"], vz["v_f8"],
                         vz["v_scale"], causal=True, sm_scale=0.125, delta_s=ds)
        rl1[sq] = O.metrics(o, ex)["rel_l1"]
    assert O.metrics(o, ex)["cos"] >= 0.998
    assert rl1[True] < rl1[False], rl1


# ------------------------------------------------------------------ MXFP4 PV

_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_golden_table():
    rows = [l.split() for l in open(os.path.join(GOLD, "e2m1_codes.txt"))
            if l.strip() and not l.startswith("#")]
    for c, v in rows:
        got = MX.decode(int(c))
        assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), (c, v)
    # every code survives encode(decode(.)), -0 included (the sign is copied)
    codes = np.arange(16)
    assert (MX.encode(MX.decode(codes)) == codes).all()
    assert (MX.encode(np.array([-0.1, -0.0, 0.0, 0.2])) == [8, 8, 0, 0]).all()


def test_e2m1_encode_is_nearest_with_ties_to_even():
    g = np.random.default_rng(61)
    grid = np.array(sorted(set([-v for v in _E2M1] + _E2M1)))
    x = np.concatenate([g.uniform(-7, 7, 20000),
                        (np.array(_E2M1[1:]) + np.array(_E2M1[:-1])) / 2,       # midpoints
                        -(np.array(_E2M1[1:]) + np.array(_E2M1[:-1])) / 2])
    v = MX.decode(MX.encode(x))
    xc = np.clip(x, -6, 6)
    d = np.abs(grid[None, :] - xc[:, None])
    best = d.min(axis=1)
    assert np.allclose(np.abs(v - xc), best)                       # nearest (after saturation)
    # ties: the chosen code is even (mantissa bit 0)
    tie = (np.sort(d, axis=1)[:, 1] - best) < 1e-12
    assert tie.sum() >= 14
    assert (MX.encode(x[tie]) & 1 == 0).all()
    assert (MX.encode(np.array([7.0, 100.0, -9.0])) == [7, 7, 15]).all()   # saturation


def test_mx_scale_rule():
    g = np.random.default_rng(62)
    x = g.standard_normal((50, 64)) * np.exp(g.uniform(-30, 30, (50, 1)))
    codes, e = MX.quantize_blocks(x, axis=-1)
    assert e.shape == (50, 2)
    amax = np.abs(x.reshape(50, 2, 32)).max(axis=-1)
    r = amax / np.exp2(e.astype(np.float64))
    assert ((r >= 4) & (r < 8)).all()                  # amax lands in E2M1's top binade
    dq = MX.dequantize_blocks(codes, e, axis=-1)
    # within half a grid step of x / 2^e (saturation only above 6)
    step = np.where(np.abs(x / np.exp2(np.repeat(e, 32, axis=-1))) <= 2, 0.25,
                    np.where(np.abs(x / np.exp2(np.repeat(e, 32, axis=-1))) <= 4, 0.5, 1.0))
    err = np.abs(dq - x) / np.exp2(np.repeat(e, 32, axis=-1))
    sat = np.abs(x / np.exp2(np.repeat(e, 32, axis=-1))) > 6
    assert (err[~sat] <= step[~sat] + 1e-12).all()
    z, ez = MX.quantize_blocks(np.zeros((1, 32)))
    assert (z == 0).all() and ez[0, 0] == -127
    assert MX.scale_exponent(1.0) == -2 and MX.scale_exponent(6.0) == 0
    assert MX.scale_exponent(3.999) == -1 and MX.scale_exponent(2.0 ** -140) == -127


@pytest.mark.parametrize("causal", [False, True])
def test_mxfp4_pv_closed_form_matches_recursion(causal):
    g = np.random.default_rng(63)
    n, d = 100, 8
    q = torch.from_numpy(g.standard_normal((1, 2, n, d)).astype(np.float32) * 2).half()
    k = torch.from_numpy((g.standard_normal((1, 1, n, d)) + 1).astype(np.float32)).half()
    v = torch.from_numpy(g.standard_normal((1, 1, n, d)).astype(np.float32)).half()
    z = O.quantize_qk(q, k)
    v4 = O.quantize_v_mxfp4(v)
    assert v4["v_f4"].shape == (1, 1, 128, d) and v4["v_e8"].shape == (1, 1, 4, d)
    kw = dict(causal=causal, sm_scale=0.35, kv_tile=64, pv="mxfp4")
    args = (z["q_i8"], z["q_scale"], z["k_i8"], z["k_scale"], v4["v_f4"], v4["v_e8"])
    a, la = O.attn_quant(*args, return_lse=True, **kw)
    for h in range(2):
        r, lr = O.attn_quant_recursive(*args, h=h, hk=0, return_lse=True, **kw)
        assert np.abs(a[0, h] - r).max() < 1e-12
        assert np.abs(la[0, h] - lr).max() < 1e-12


def test_mxfp4_pv_constant_v_and_accuracy():
    # constant V is represented exactly by MX blocks, so O = v * sum(Pq) / l
    # with l the unquantized sum; on random data MXFP4 PV is close to exact
    # attention but less accurate than FP8 PV (the pages rank MXFP4 below
    # finer formats)
    w = W.get("tiny")
    t = W.generate(w)
    qz = O.quantize_qk(t["q"], t["k"])
    ex = O.attn_exact(t["q"], t["k"], t["v"], causal=False, sm_scale=w.sm_scale)
    v4 = O.quantize_v_mxfp4(t["v"])
    vz = O.quantize_v(t["v"])
    args = (qz["q_i8"], qz["q_scale"], qz["k_i8"], qz["k_scale"])
    o4 = O.attn_quant(*args, v4["v_f4"], v4["v_e8"], causal=False, sm_scale=w.sm_scale,
                      pv="mxfp4")
    o8 = O.attn_quant(*args, vz["v_f8"], vz["v_scale"], causal=False, sm_scale=w.sm_scale)
    m4, m8 = O.metrics(o4, ex), O.metrics(o8, ex)
    # the SageAttention3 synthesis page quotes CosSim 98.37 % for MXFP4
    assert m4["cos"] >= 0.975 and m8["rel_l1"] < m4["rel_l1"], (m4, m8)
    vc = torch.full_like(t["v"], 1.5)
    vc4 = O.quantize_v_mxfp4(vc)
    oc = O.attn_quant(*args, vc4["v_f4"], vc4["v_e8"], causal=True, sm_scale=w.sm_scale,
                      pv="mxfp4")
    # O = 1.5 * sum(Pq) / sum(P~): each E2M1 rounding (and the saturation of
    # the [6, 8) top of a block) moves an element by at most 1/4 of itself
    assert np.abs(oc - 1.5).max() <= 0.25 * 1.5


def test_quantized_vs_exact_tiny_full():
    w = W.get("tiny")
    t = W.generate(w)
    qz, vz = _quant_all(t)
    m = O.metrics(_aq(qz, vz, causal=False, sm_scale=w.sm_scale),
                  O.attn_exact(t["q"], t["k"], t["v"], causal=False, sm_scale=w.sm_scale))
    assert m["cos"] >= 0.998


@pytest.mark.parametrize("name,heads", [
    ("llm_prefill", [(0, 0), (0, 31)]),
    ("video_dit", [(0, 7)]),
    ("sweep@N1024", [(3, 5)]),
    ("gqa_long", [(0, 13)]),
])
def test_quantized_vs_exact_sampled(name, heads):
    _sample_check(name, heads, 96, 7)


# ---------------------------------------------------------------- log-sum-exp (LSE)

@pytest.mark.parametrize("causal", [False, True])
def test_exact_lse_matches_logsumexp(causal):
    """attn_exact's LSE equals scipy's logsumexp of the masked logits and a plain
    math.log(sum(math.exp)) loop on a few rows."""
    from scipy.special import logsumexp
    g = np.random.default_rng(31)
    q = torch.from_numpy(g.standard_normal((1, 2, 37, 16), dtype=np.float32)).half()
    k = torch.from_numpy(g.standard_normal((1, 1, 37, 16), dtype=np.float32) * 2).half()
    v = torch.zeros((1, 1, 37, 16), dtype=torch.float16)
    _, lse = O.attn_exact(q, k, v, causal=causal, sm_scale=0.3, return_lse=True)
    s = np.einsum("hnc,mc->hnm", q[0].double().numpy(), k[0, 0].double().numpy()) * 0.3
    if causal:
        s = np.where(np.arange(37)[None, None, :] > np.arange(37)[None, :, None], -np.inf, s)
    assert np.allclose(lse[0], logsumexp(s, axis=2), rtol=0, atol=1e-12)
    for i in (0, 5, 36):
        n = i + 1 if causal else 37
        ref = math.log(sum(math.exp(s[1, i, j]) for j in range(n)))
        assert abs(lse[0, 1, i] - ref) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_quant_lse_matches_literal_recursion(causal):
    """The closed form's m_T + ln l equals the final state of the literal recursion."""
    g = np.random.default_rng(32)
    q = torch.from_numpy(g.standard_normal((1, 1, 40, 32), dtype=np.float32)).half()
    k = torch.from_numpy(g.standard_normal((1, 1, 40, 32), dtype=np.float32) + 2).half()
    v = torch.from_numpy(g.standard_normal((1, 1, 40, 32), dtype=np.float32)).half()
    z, zv = O.quantize_qk(q, k), O.quantize_v(v)
    args = (z["q_i8"], z["q_scale"], z["k_i8"], z["k_scale"], zv["v_f8"], zv["v_scale"])
    _, l1 = O.attn_quant(*args, causal=causal, sm_scale=0.2, kv_tile=16, return_lse=True)
    _, l2 = O.attn_quant_recursive(*args, causal=causal, sm_scale=0.2, kv_tile=16,
                                   return_lse=True)
    assert np.allclose(l1[0, 0], l2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_quant_lse_of_zero_q(causal):
    """Q = 0: every logit is 0, so L_i = ln(number of visible keys) exactly."""
    N = 200
    q = torch.zeros((1, 1, N, 64), dtype=torch.float16)
    g = np.random.default_rng(33)
    k = torch.from_numpy(g.standard_normal((1, 1, N, 64), dtype=np.float32)).half()
    z, zv = O.quantize_qk(q, k), O.quantize_v(k)
    _, lse = O.attn_quant(z["q_i8"], z["q_scale"], z["k_i8"], z["k_scale"], zv["v_f8"],
                          zv["v_scale"], causal=causal, sm_scale=0.125, return_lse=True)
    nvis = np.arange(1, N + 1) if causal else np.full(N, N)
    assert np.allclose(lse[0, 0], np.log(nvis), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_correction_restores_unsmoothed_lse(causal):
    """Smoothing shifts every logit of row i by sm_scale q_i . mean(K); the quantized LSE of
    the smoothed scores plus lse_correction matches the exact LSE of the original inputs
    within the quantization error, and is far from it without the correction (a shared
    K bias of sigma 3 makes the shift large).  Also with GQA (two query heads per kv head)."""
    g = np.random.default_rng(34)
    B, H, Hk, N, d = 1, 4, 2, 300, 64
    q = torch.from_numpy(g.standard_normal((B, H, N, d), dtype=np.float32)).half()
    k = g.standard_normal((B, Hk, N, d), dtype=np.float32)
    k += g.standard_normal((B, Hk, 1, d), dtype=np.float32) * 3
    k = torch.from_numpy(k).half()
    v = torch.from_numpy(g.standard_normal((B, Hk, N, d), dtype=np.float32)).half()
    _, lx = O.attn_exact(q, k, v, causal=causal, sm_scale=0.125, return_lse=True)
    z, zv = O.quantize_qk(q, k, smooth_k=True), O.quantize_v(v)
    _, ls = O.attn_quant(z["q_i8"], z["q_scale"], z["k_i8"], z["k_scale"], zv["v_f8"],
                         zv["v_scale"], causal=causal, sm_scale=0.125, return_lse=True)
    corr = O.lse_correction(q, z["k_mean"], sm_scale=0.125)
    assert np.abs(ls + corr - lx).max() < 0.05
    assert np.abs(ls - lx).max() > 1.0


@pytest.mark.parametrize("with_ds,causal", [(False, False), (False, True), (True, True)])
def test_p_codes_f32_differ_from_float64_only_at_midpoints(with_ds, causal):
    """The E4M3 code of 448 * P~ is taken on float32 values (reading c25).  Against the
    same steps in float64 (scores S dQ dK sm log2 e (+ Delta S), the running max per
    128-key tile, 448 * 2^(x - m)), a code may differ only where the float64 value lies
    within a few float32 ulps of an E4M3 rounding midpoint, and only rarely.  A wrong
    factor, max, tile or Delta S term would move codes far from any midpoint."""
    g = np.random.default_rng(31)
    n, d = 300, 64
    q = torch.from_numpy(g.standard_normal((1, 1, n, d)).astype(np.float32) * 1.5).half()
    k = torch.from_numpy(g.standard_normal((1, 1, n, d)).astype(np.float32) + 2).half()
    qz = O.quantize_qk(q, k, smooth_q=with_ds)
    sm = 0.125
    ds = O.delta_s(qz["q_mean"], k, qz["k_mean"]) if with_ds else None
    rows = np.arange(n)
    sint = qz["q_i8"][0, 0].astype(np.float64) @ qz["k_i8"][0, 0].astype(np.float64).T
    qs = qz["q_scale"][0, 0][rows // O.BLKQ].astype(np.float64)
    ks = qz["k_scale"][0, 0][np.arange(n) // O.BLKK].astype(np.float64)
    valid = (np.arange(n)[None, :] <= rows[:, None]) if causal else np.ones((n, n), bool)
    lam = O.sm_log2_f32(sm)
    c32 = O.rn32(O.rn32(qs[:, None] * ks[None, :]).astype(np.float64) * np.float64(lam))
    g32 = O.rn32(ds[0, 0][rows // O.BLKQ] * np.float64(lam)) if with_ds else None
    pt32, m32 = O.softmax_f32(sint, c32, g32, valid, O.KV_TILE)
    got = O.p_fp8(pt32)
    # float64: the same scores and running max without any float32 rounding
    x = sint * qs[:, None] * ks[None, :] * sm / math.log(2)
    if with_ds:
        x = x + ds[0, 0][rows // O.BLKQ] * sm / math.log(2)
    x = np.where(valid, x, -np.inf)
    nt = -(-n // O.KV_TILE)
    xp = np.full((n, nt * O.KV_TILE), -np.inf)
    xp[:, :n] = x
    m = np.maximum.accumulate(xp.reshape(n, nt, O.KV_TILE).max(axis=2), axis=1)
    p64 = np.where(valid, O.P_SCALE * np.exp2(x - np.repeat(m, O.KV_TILE, axis=1)[:, :n]), 0.0)
    want = F8.round_to_e4m3(p64)
    diff = np.argwhere(got != want)
    assert len(diff) <= 1e-3 * valid.sum(), len(diff)
    for i, j in diff:
        mid = 0.5 * (got[i, j] + want[i, j])
        # both codes are neighbours, and p64 sits next to the midpoint between them
        assert abs(got[i, j] - want[i, j]) <= 0.13 * max(got[i, j], want[i, j])
        assert abs(p64[i, j] - mid) <= 2.0 ** -19 * (1 + abs(x[i, j])) * p64[i, j], (i, j)
    # the row max element has P~ = 1 exactly (x - m = 0), so its code is 448
    for i in range(n):
        jm = np.argmax(np.where(valid[i], x[i], -np.inf))
        if m[i, jm // O.KV_TILE] == m[i, -1]:
            assert pt32[i, jm] == 1.0 and got[i, jm] == 448.0
    # the decisions are not trivially equal to the float64 ones by construction:
    # the float32 x carries rounding (else this test would not exercise anything)
    assert np.any(c32.astype(np.float64) != qs[:, None] * ks[None, :] * sm / math.log(2))


def _exact_f32(fr):
    """Brute-force nearest float32 of a rational: scan the float32 neighbours of its
    float64 approximation and keep the closest (ties to the even significand)."""
    from fractions import Fraction
    c = np.float32(float(fr))
    best = None
    for k in range(-3, 4):
        v = c
        for _ in range(abs(k)):
            v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(-np.inf))
        dist = abs(Fraction(float(v)) - fr)
        even = (int(np.array(v).view(np.int32)) & 1) == 0
        key = (dist, not even)
        if best is None or key < best[0]:
            best = (key, v)
    return float(best[1])


def test_float32_rounding_helpers_are_exact():
    """rn32_sum (float64 sum + TwoSum residual) and f32_of_fraction (rational
    arithmetic) both give the nearest float32 of an exact sum; checked against a
    brute-force search over float32 neighbours, on random sums and on sums built to land
    exactly on a float32 midpoint in float64 while the exact value is just off it."""
    from fractions import Fraction
    g = np.random.default_rng(77)
    # the oracle's use: (integer dot * float32 factor) + float32 term
    a = g.integers(-2 ** 21, 2 ** 21, 400).astype(np.float64) * \
        g.standard_normal(400).astype(np.float32).astype(np.float64)
    b = (g.standard_normal(400) * np.exp(g.uniform(-8, 8, 400))).astype(np.float32).astype(np.float64)
    # ties: a float32 midpoint m, split as m = a + b with a tiny residual beyond float64
    mids, lows = [], []
    for _ in range(200):
        # a float32 midpoint just above 1 (mid = 1 + (2k + 1) 2^-24), split as
        # b = 2^e and a = mid - b + tiny with tiny below float64's resolution of the
        # sum: the float64 sum is exactly mid, the exact sum is just off it
        e = int(g.integers(0, 3))
        kk = int(g.integers(0, 2 ** 12))
        mid = (1.0 + (2 * kk + 1) * 2.0 ** -24) * 2.0 ** e
        tiny = 2.0 ** (e - 62) * g.choice([-1.0, 1.0])
        a_part = mid - 2.0 ** e + tiny
        assert a_part - tiny == mid - 2.0 ** e and a_part + 2.0 ** e == mid
        mids.append(a_part)
        lows.append(2.0 ** e)
    a = np.concatenate([a, np.array(mids)])
    b = np.concatenate([b, np.array(lows)])
    got = O.rn32_sum(a, b)
    for x, y, r in zip(a, b, got):
        want = _exact_f32(Fraction(x) + Fraction(y))
        assert float(r) == want, (x, y, r, want)
        assert O.f32_of_fraction(Fraction(x) + Fraction(y)) == want
    # on float64 values the rational rounding agrees with numpy's float64 -> float32 cast
    x = g.standard_normal(2000) * np.exp(g.uniform(-95, 80, 2000))    # subnormal .. 1e35
    assert all(O.f32_of_fraction(Fraction(v)) == float(np.float32(v)) for v in x)


# --------------------------------------------------------------------- per-channel FP8 V

def _read_hex_sections(path):
    out, sec = {}, None
    for line in open(path):
        line = line.strip()
        if line.startswith("# section:"):
            sec = line.split(":", 1)[1].strip()
            out[sec] = []
        elif line and not line.startswith("#"):
            out[sec].append([int(t, 0) if t.startswith("0x") else float(t) for t in line.split()])
    return out


def test_quantize_v_worked_example():
    s = _read_hex_sections(os.path.join(GOLD, "v_fp8_channel_example.txt"))
    v = torch.tensor(s["input"], dtype=torch.float16)[None, None]         # [1, 1, 4, 3]
    assert torch.equal(v.float()[0, 0], torch.tensor(s["input"]))       # exact in fp16
    z = O.quantize_v(v)
    assert np.array_equal(z["v_scale"][0, 0], np.array(s["scale"][0], dtype=np.float32))
    assert np.array_equal(z["v_f8"][0, 0], np.array(s["codes"], dtype=np.uint8))


def test_quantize_v_scale_is_per_channel():
    """The scale runs over the tokens of one channel: each nonzero channel's largest
    |v| maps to the code of +-448, changing one token of channel c moves only channel c's
    scale and codes, and scaling a channel by a power of two scales only its scale."""
    g = np.random.default_rng(81)
    B, Hk, N, d = 2, 2, 130, 16
    v = torch.from_numpy((g.standard_normal((B, Hk, N, d)) *
                          np.exp(g.uniform(-3, 3, (B, Hk, 1, d)))).astype(np.float32)).half()
    z = O.quantize_v(v)
    assert z["v_scale"].shape == (B, Hk, d) and z["v_f8"].shape == (B, Hk, N, d)
    vv = v.float().numpy()
    amax_at = np.abs(vv).argmax(axis=2)                                   # [B, Hk, d]
    top = np.take_along_axis(z["v_f8"], amax_at[:, :, None, :], axis=2)[:, :, 0, :]
    assert np.all((top & 0x7F) == 0x7E)
    # reconstruction within half an E4M3 step of each value (relative 1/16, or the
    # subnormal quantum 2^-9 of the scaled value)
    dq = F8.decode(z["v_f8"]) * z["v_scale"][:, :, None, :].astype(np.float64)
    step = np.maximum(np.abs(vv) / 16, 2.0 ** -10 * z["v_scale"][:, :, None, :])
    assert np.all(np.abs(dq - vv) <= step * (1 + 1e-6))
    # one token of channel 5 of head (1, 0) made the channel's largest
    v2 = v.clone()
    v2[1, 0, 77, 5] = float(np.abs(vv[1, 0, :, 5]).max() * 3)
    z2 = O.quantize_v(v2)
    diff_s = np.argwhere(z2["v_scale"] != z["v_scale"])
    assert diff_s.tolist() == [[1, 0, 5]]
    diff_c = np.argwhere(z2["v_f8"] != z["v_f8"])
    assert set(map(tuple, diff_c[:, [0, 1, 3]])) == {(1, 0, 5)}
    # a power-of-two rescale of one channel scales its scale exactly, codes unchanged
    v3 = v.clone()
    v3[:, :, :, 2] *= 4
    z3 = O.quantize_v(v3)
    assert np.array_equal(z3["v_f8"], z["v_f8"])
    assert np.array_equal(z3["v_scale"][..., 2], z["v_scale"][..., 2] * 4)
