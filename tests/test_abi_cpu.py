"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, computes buffer sizes, and rejects bad arguments before
touching the device."""
import ctypes
import math
import os
import re

import pytest

import quantized_attention_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")
FAKE = 0x10000          # an aligned, never-dereferenced pointer value


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = qa.load_library()
    names = _declared()
    assert {"sage_quant_qk", "sage_quant_v", "sage_attn_fwd", "sage_attn_fwd_lse",
            "sage_lse_correction", "sage_buffer_sizes", "sage_qk_int32", "sage_status_str",
            "sage_delta_s", "sage_quant_v_mxfp4", "sage_attn_fwd_mxfp4",
            "sage_abi_version", "sage_quant_qk_noalloc", "sage_quant_qkv",
            "sage_attn_fwd_smooth_q", "sage_mfma_peak"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.sage_abi_version() == 10


def test_status_strings():
    lib = qa.load_library()
    for s in range(11):
        assert lib.sage_status_str(s)
    assert lib.sage_status_str(0) == b"ok"


@pytest.mark.parametrize("q_group", [128, 32, 1])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 256, 64), (4, 32, 8, 17550, 128),
                                          (1, 1, 1, 1, 64), (2, 6, 3, 129, 128)])
def test_buffer_sizes(B, H, H_kv, N, d, q_group):
    s = qa.sage_buffer_sizes(B, H, H_kv, N, d, q_group)
    assert s["q_i8"] == B * H * N * d
    assert s["q_scale"] == 4 * B * H * math.ceil(N / q_group)
    assert s["k_i8"] == B * H_kv * N * d
    assert s["k_scale"] == 4 * B * H_kv * math.ceil(N / 64)
    assert s["k_mean"] == s["v_scale"] == 4 * B * H_kv * d
    assert s["v_f8"] == B * H_kv * math.ceil(N / 128) * 128 * d
    assert s["o"] == 2 * B * H * N * d
    assert s["ws_quant_qk"] == 8 * B * H_kv * math.ceil(N / 256) * d
    assert s["ws_quant_v"] == 4 * B * H_kv * math.ceil(N / 256) * d
    assert s["ws_quant_qkv"] == s["ws_quant_qk"] + s["ws_quant_v"]
    assert s["q_mean"] == 4 * B * H * math.ceil(N / 128) * d
    assert s["ws_smooth_q"] == 4 * B * H * _smooth_q_default_rows(B * H, N) * N
    assert s["v_f4"] == B * H_kv * math.ceil(N / 128) * 64 * d
    assert s["v_e8"] == B * H_kv * math.ceil(N / 128) * 512


def _even_rows(total, rmax):
    n = -(-total // rmax)
    r = -(-total // n)
    r16 = -(-r // 16) * 16
    return r16 if r16 <= rmax else r


def _smooth_q_chunk(nbk, G, M, R):
    """(groups, Q blocks) of one sage_attn_fwd_smooth_q chunk for a workspace of R Delta
    S rows, by the rule sage.h states."""
    g = R // (G * M)
    if g >= nbk:
        return nbk, M
    if R < nbk * G:
        return 1, _even_rows(M, R // G)
    rows = _even_rows(M, R // (nbk * G))
    g -= g % 8
    if g >= 8 and g * G * M >= nbk * G * rows:
        n = -(-nbk // g)
        return min(g, -(-(-(-nbk // n)) // 8) * 8), M
    return nbk, rows


def _smooth_q_default_rows(bh, N):
    """Default Q blocks per head of sage_attn_fwd_smooth_q's workspace (sage.h's rule)."""
    r = max(32, 16 * math.ceil(math.ceil(2048 / bh) / 16))
    return min(math.ceil(N / 128), r)


@pytest.mark.parametrize("nbk,G,M,R,want", [
    (128, 1, 256, 4096, (16, 256)),    # sweep N=32K default: 16 whole heads per chunk
    (48, 1, 138, 2304, (48, 48)),      # video-DiT default: 16 heads (2208 rows) < 48 x 48
    (8, 4, 800, 2048, (8, 64)),        # GQA long default: every group, 64 Q blocks
    (48, 1, 138, 1104, (8, 138)),      # 8 heads (1104 rows) = 48 x 23 rows: whole heads
    (48, 1, 138, 4416, (24, 138)),     # 32 heads fit (4416 > 48 x 80): evened to 24 + 24
    (40, 1, 256, 4096, (16, 256)),     # 16 + 16 + 8
    (2, 2, 8, 4, (2, 1)), (2, 2, 8, 12, (2, 3)), (2, 2, 8, 64, (2, 8)),
    (2, 2, 8, 3, (1, 1)),
    (2, 2, 18, 40, (2, 9)), (3, 1, 1, 7, (3, 1)), (6, 2, 3, 12, (6, 1)),
])
def test_smooth_q_chunk_rule(nbk, G, M, R, want):
    """The chunk rule in closed cases."""
    assert _smooth_q_chunk(nbk, G, M, R) == want


def test_largest_head_fits_32_bit_buffer_ranges():
    """One head's K codes are read through a 32-bit buffer range: N*d just below 2^32
    is accepted, the next 128 keys are not."""
    n = (1 << 25) - 128
    assert qa.sage_buffer_sizes(1, 1, 1, n, 128)["k_i8"] == n * 128
    with pytest.raises(qa.SageError):
        qa.sage_buffer_sizes(1, 1, 1, n + 1, 128)


def test_smooth_q_workspace_is_linear_in_n():
    """The default smooth-Q workspace holds a bounded number of Delta S rows: it grows
    linearly with N (the whole table, B*H*ceil(N/128)*N floats, grows as N^2)."""
    per_n = set()
    for N in (1 << 16, 1 << 18, 1 << 20):
        s = qa.sage_buffer_sizes(1, 32, 8, N, 128)
        per_n.add(s["ws_smooth_q"] / N)
        assert s["ws_smooth_q"] * 8 <= 4 * 32 * math.ceil(N / 128) * N
    assert len(per_n) == 1
    # sequence sweep at N = 32K: 128 heads x 32 Q blocks x 32768 keys (512 MiB, not 4 GiB)
    assert qa.sage_buffer_sizes(4, 32, 32, 32768, 128)["ws_smooth_q"] == 4 * 128 * 32 * 32768


@pytest.mark.parametrize("args,code", [
    ((0, 2, 2, 256, 64), 2), ((1, 2, 2, 0, 64), 2), ((1, 0, 1, 256, 64), 2),
    ((1, 2, 2, 256, 96), 3), ((1, 2, 2, 256, 256), 3), ((1, 6, 4, 256, 64), 4),
    ((1, 70000, 1, 16, 64), 2), ((64, 512, 512, 1 << 30, 128), 2),
    ((1, 1, 1, 1 << 25, 128), 2), ((1, 1, 1, 1 << 26, 64), 2),
    ((1, 2, 2, 256, 64, 64), 6), ((1, 2, 2, 256, 64, 0), 6), ((1, 2, 2, 256, 64, -32), 6),
])
def test_buffer_sizes_rejects(args, code):
    with pytest.raises(qa.SageError) as e:
        qa.sage_buffer_sizes(*args)
    assert e.value.status == code


def _qk(lib, **kw):
    a = dict(q=FAKE, k=FAKE, dt=0, B=1, H=2, H_kv=2, N=256, d=64, qg=128, smooth=1, sq=0,
             q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, k_mean=FAKE, q_mean=None, ws=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.sage_quant_qk(*a.values())


def _v(lib, **kw):
    a = dict(v=FAKE, dt=0, B=1, H_kv=2, N=256, d=64, v_f8=FAKE, v_scale=FAKE, ws=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.sage_quant_v(*a.values())


def _attn(lib, **kw):
    a = dict(q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, v_f8=FAKE, v_scale=FAKE,
             o=FAKE, dt=0, B=1, H=2, H_kv=2, N=256, d=64, qg=128, causal=0, sm_scale=0.125,
             stream=None)
    a.update(kw)
    return lib.sage_attn_fwd(*a.values())


def _attn_lse(lib, **kw):
    a = dict(q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, v_f8=FAKE, v_scale=FAKE,
             o=FAKE, dt=0, lse=FAKE, corr=None, B=1, H=2, H_kv=2, N=256, d=64, qg=128, causal=0,
             sm_scale=0.125, stream=None)
    a.update(kw)
    return lib.sage_attn_fwd_lse(*a.values())


def _attn_sq(lib, **kw):
    a = dict(q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, v_f8=FAKE, v_scale=FAKE, k=FAKE,
             k_dt=0, k_mean=FAKE, q_mean=FAKE, o=FAKE, dt=0, lse=None, corr=None, B=1, H=2,
             H_kv=2, N=256, d=64, qg=128, causal=0, sm_scale=0.125, ws=FAKE,
             ws_bytes=256 * 4, stream=None)
    a.update(kw)
    return lib.sage_attn_fwd_smooth_q(*a.values())


def _lse_corr(lib, **kw):
    a = dict(q=FAKE, dt=0, k_mean=FAKE, B=1, H=2, H_kv=2, N=256, d=64, sm_scale=0.125, corr=FAKE,
             stream=None)
    a.update(kw)
    return lib.sage_lse_correction(*a.values())


def _ds(lib, **kw):
    a = dict(k=FAKE, dt=0, k_mean=FAKE, q_mean=FAKE, B=1, H=2, H_kv=2, N=256, d=64,
             sm_scale=0.125, i0=0, nrows=2, out=FAKE, stream=None)
    a.update(kw)
    return lib.sage_delta_s(*a.values())


def _qv4(lib, **kw):
    a = dict(v=FAKE, dt=0, B=1, H_kv=2, N=256, d=64, v_f4=FAKE, v_e8=FAKE, stream=None)
    a.update(kw)
    return lib.sage_quant_v_mxfp4(*a.values())


def _attn4(lib, **kw):
    a = dict(q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, v_f4=FAKE, v_e8=FAKE, o=FAKE,
             dt=0, lse=None, corr=None, B=1, H=2, H_kv=2, N=256, d=64, qg=128, causal=0,
             sm_scale=0.125, stream=None)
    a.update(kw)
    return lib.sage_attn_fwd_mxfp4(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), 1), (dict(v_e8=None), 1), (dict(N=0), 2), (dict(d=32), 3), (dict(dt=5), 5),
    (dict(v_f4=FAKE + 4), 9), (dict(v_e8=FAKE + 1), 9),
])
def test_quant_v_mxfp4_rejects(kw, code):
    assert _qv4(qa.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(v_f4=None), 1), (dict(o=None), 1), (dict(B=0), 2), (dict(d=96), 3),
    (dict(H=4, H_kv=3), 4), (dict(dt=3), 5), (dict(qg=8), 6), (dict(causal=2), 6),
    (dict(sm_scale=-1.0), 6), (dict(v_e8=FAKE + 2), 9),
])
def test_attn_fwd_mxfp4_rejects(kw, code):
    assert _attn4(qa.load_library(), **kw) == code


def _qk32(lib, **kw):
    a = dict(q_i8=FAKE, k_i8=FAKE, B=1, H=2, H_kv=2, N=256, d=64, b=0, h=0, s=FAKE, stream=None)
    a.update(kw)
    return lib.sage_qk_int32(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k_mean=None), 1), (dict(B=0), 2), (dict(N=-5), 2),
    (dict(d=32), 3), (dict(H=3), 4), (dict(dt=2), 5), (dict(smooth=2), 6),
    (dict(q=FAKE + 8), 9), (dict(k_i8=FAKE + 4), 9), (dict(ws=None), 7), (dict(ws_bytes=1023), 7),
    (dict(qg=64), 6), (dict(qg=0), 6), (dict(qg=2), 6), (dict(sq=2), 6), (dict(sq=1), 1),
    (dict(sq=-1), 6),
])
def test_quant_qk_rejects(kw, code):
    assert _qk(qa.load_library(), **kw) == code


def test_quant_qk_no_workspace_needed_without_smoothing_is_validated_first():
    # smooth_k = 0 needs no workspace, but a bad shape still fails first
    assert _qk(qa.load_library(), smooth=0, ws=None, ws_bytes=0, d=80) == 3


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), 1), (dict(v_scale=None), 1), (dict(N=0), 2), (dict(d=100), 3),
    (dict(dt=-1), 5), (dict(v_f8=FAKE + 1), 9), (dict(ws=None), 7), (dict(ws_bytes=511), 7),
])
def test_quant_v_rejects(kw, code):
    assert _v(qa.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), 1), (dict(v_scale=None), 1), (dict(H_kv=0), 2), (dict(d=16), 3),
    (dict(H=4, H_kv=3), 4), (dict(dt=7), 5), (dict(causal=3), 6), (dict(sm_scale=0.0), 6),
    (dict(sm_scale=-1.0), 6), (dict(sm_scale=float("inf")), 6), (dict(sm_scale=float("nan")), 6),
    (dict(o=FAKE + 2), 9), (dict(qg=16), 6), (dict(qg=-1), 6), (dict(v_f8=FAKE + 4), 9),
])
def test_attn_fwd_rejects(kw, code):
    assert _attn(qa.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), 1), (dict(o=None), 1), (dict(B=0), 2), (dict(d=96), 3),
    (dict(H=4, H_kv=3), 4), (dict(dt=3), 5), (dict(causal=2), 6), (dict(sm_scale=0.0), 6),
    (dict(sm_scale=float("nan")), 6), (dict(k_i8=FAKE + 4), 9), (dict(qg=256), 6),
])
def test_attn_fwd_lse_rejects(kw, code):
    assert _attn_lse(qa.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k_mean=None), 1), (dict(corr=None), 1), (dict(N=0), 2),
    (dict(d=48), 3), (dict(H=3), 4), (dict(dt=9), 5), (dict(sm_scale=-2.0), 6),
    (dict(q=FAKE + 2), 9),
])
def test_lse_correction_rejects(kw, code):
    assert _lse_corr(qa.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), 1), (dict(k_mean=None), 1), (dict(q_mean=None), 1), (dict(out=None), 1),
    (dict(B=0), 2), (dict(d=96), 3), (dict(H=3), 4), (dict(dt=4), 5), (dict(sm_scale=0.0), 6),
    (dict(sm_scale=float("inf")), 6), (dict(q_mean=FAKE + 8), 9), (dict(out=FAKE + 4), 9),
    (dict(B=8, H=512, H_kv=512, N=1 << 20, nrows=1024), 2), (dict(i0=-1), 6), (dict(nrows=0), 6),
    (dict(i0=1, nrows=2), 6), (dict(nrows=3), 6),
])
def test_delta_s_rejects(kw, code):
    assert _ds(qa.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q_i8=None), 1), (dict(k=None), 1), (dict(k_mean=None), 1), (dict(q_mean=None), 1),
    (dict(o=None), 1), (dict(N=0), 2), (dict(d=96), 3), (dict(H=3), 4), (dict(k_dt=2), 5),
    (dict(dt=7), 5), (dict(qg=64), 6), (dict(causal=2), 6), (dict(sm_scale=0.0), 6),
    (dict(corr=FAKE), 6), (dict(k=FAKE + 2), 9), (dict(q_mean=FAKE + 4), 9),
    (dict(ws=None), 7), (dict(ws_bytes=256 * 4 - 1), 7), (dict(ws=FAKE + 8), 9),
    (dict(H=4, H_kv=2, ws_bytes=2 * 256 * 4 - 1), 7),
])
def test_attn_fwd_smooth_q_rejects(kw, code):
    assert _attn_sq(qa.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(s=None), 1), (dict(b=1), 6), (dict(h=2), 6), (dict(h=-1), 6), (dict(d=48), 3),
    (dict(N=200000), 2),
])
def test_qk_int32_rejects(kw, code):
    assert _qk32(qa.load_library(), **kw) == code


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 64, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        qa.sage_quant_qk(q, q)
    with pytest.raises(ValueError):
        qa.sage_quant_v(q)


def test_q_group_inferred_from_scale_length():
    import torch
    for N in (1, 17, 32, 33, 129, 17550):
        for g in qa.Q_GROUPS:
            qs = torch.zeros(1, 2, -(-N // g))
            got = qa._q_group_of(qs, N)
            # the inferred group indexes every query to the same scale as g
            assert all(i // got == i // g for i in range(min(N, 300)))
    with pytest.raises(ValueError):
        qa._q_group_of(torch.zeros(1, 2, 5), 300)


def _cpu_qk_vq(B=1, H=4, H_kv=2, N=200, d=64, q_group=128):
    import torch
    qk = qa._alloc_qk(B, H, H_kv, N, d, "cpu", q_group)
    vq = qa._alloc_v(B, H_kv, N, d, "cpu")
    return qk, vq


def test_binding_rejects_short_or_mismatched_buffers_before_any_launch():
    """A buffer shorter than the shapes need would be read or written past its
    end by the kernels; the binding refuses it (on the host, before the device
    check, so this runs without a GPU)."""
    import torch
    qk, vq = _cpu_qk_vq()
    short = dict(vq, v_f8=vq["v_f8"][..., :-1])
    with pytest.raises(ValueError, match="v_f8"):
        qa.sage_attn_fwd(qk, short, causal=False, sm_scale=0.125)
    with pytest.raises(ValueError, match="v_scale"):
        qa.sage_attn_fwd(qk, dict(vq, v_scale=vq["v_scale"][..., :-1]), causal=False,
                         sm_scale=0.125)
    with pytest.raises(ValueError, match="k_scale"):
        qa.sage_attn_fwd_lse(dict(qk, k_scale=qk["k_scale"][..., :-1]), vq, causal=False,
                             sm_scale=0.125)
    # K for another sequence length
    other, _ = _cpu_qk_vq(N=100)
    with pytest.raises(ValueError, match="k_i8"):
        qa.sage_attn_fwd(dict(qk, k_i8=other["k_i8"]), vq, causal=False, sm_scale=0.125)
    with pytest.raises(ValueError, match="out"):
        qa.sage_attn_fwd(qk, vq, causal=False, sm_scale=0.125,
                         out=torch.empty(1, 4, 199, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="lse"):
        qa.sage_attn_fwd_lse(qk, vq, causal=False, sm_scale=0.125,
                             lse=torch.empty(1, 4, 199))
    v4 = qa._alloc_v4(1, 2, 200, 64, "cpu")
    with pytest.raises(ValueError, match="v_e8"):
        qa.sage_attn_fwd_mxfp4(qk, dict(v4, v_e8=v4["v_e8"][..., :-1]), causal=False,
                               sm_scale=0.125)
    v = torch.zeros(1, 2, 200, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="v_f8"):
        qa.sage_quant_v(v, out=short)
    with pytest.raises(ValueError, match="v_f4"):
        qa.sage_quant_v_mxfp4(v, out=dict(v4, v_f4=v4["v_f4"][..., :-1]))
    q = torch.zeros(1, 4, 200, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="k_i8"):
        qa.sage_quant_qk(q, v, out=dict(qk, k_i8=qk["k_i8"][..., :-1]))
    # well-formed buffers get as far as the device check
    with pytest.raises(ValueError, match="CUDA"):
        qa.sage_attn_fwd(qk, vq, causal=False, sm_scale=0.125)


def _qk_noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, dt=0, B=1, H=2, H_kv=2, N=256, d=64, qg=128, smooth=1, sq=0,
             q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, k_mean=FAKE, q_mean=None,
             stream=None)
    a.update(kw)
    return lib.sage_quant_qk_noalloc(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k_mean=None), 1), (dict(sq=1), 1), (dict(B=0), 2), (dict(d=32), 3),
    (dict(H=3), 4), (dict(dt=2), 5), (dict(smooth=2), 6), (dict(qg=64), 6), (dict(sq=-1), 6),
    (dict(q=FAKE + 8), 9),
    # B * H_kv * ceil(N/256) * d * 8 bytes of K column sums above the 16 MiB array
    (dict(B=1, H=64, H_kv=64, N=65536 + 256, d=128), 10),
])
def test_quant_qk_noalloc_rejects(kw, code):
    """The no-allocation entry point validates like sage_quant_qk and refuses shapes whose
    scratch exceeds its fixed array, before any HIP call."""
    assert _qk_noalloc(qa.load_library(), **kw) == code
    assert qa.sage_buffer_sizes(1, 64, 64, 65536, 128)["ws_quant_qk"] == qa.SCRATCH_BYTES


def _qkv(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=0, B=1, H=2, H_kv=2, N=256, d=64, qg=128, smooth=1, sq=0,
             q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, k_mean=FAKE, q_mean=None,
             v_f8=FAKE, v_scale=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.sage_quant_qkv(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(v=None), 1), (dict(v_scale=None), 1), (dict(sq=1), 1),
    (dict(B=0), 2), (dict(d=32), 3), (dict(H=3), 4), (dict(dt=2), 5), (dict(smooth=2), 6),
    (dict(qg=64), 6), (dict(v=FAKE + 8), 9), (dict(v_f8=FAKE + 4), 9), (dict(ws=None), 7),
    (dict(ws_bytes=1024 + 511), 7),
])
def test_quant_qkv_rejects(kw, code):
    """The one-call quantization validates like sage_quant_qk and sage_quant_v together
    (its workspace holds both scratch areas: 1024 + 512 bytes at these shapes)."""
    assert _qkv(qa.load_library(), **kw) == code


def test_smooth_q_entry_points_refuse_the_wrong_codes():
    """Codes of smoothed Q need the Delta S term: the plain attention entry points refuse
    them and the smooth-Q one refuses plain codes (on the host, before any launch)."""
    import torch
    qk_sq = qa._alloc_qk(1, 2, 2, 256, 64, "cpu", smooth_q=True)
    qk = qa._alloc_qk(1, 2, 2, 256, 64, "cpu")
    vq = qa._alloc_v(1, 2, 256, 64, "cpu")
    k = torch.zeros(1, 2, 256, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="smooth_q"):
        qa.sage_attn_fwd(qk_sq, vq, causal=False, sm_scale=0.125)
    with pytest.raises(ValueError, match="smooth_q"):
        qa.sage_attn_fwd_lse(qk_sq, vq, causal=False, sm_scale=0.125)
    with pytest.raises(ValueError, match="q_mean"):
        qa.sage_attn_fwd_smooth_q(qk, vq, k, causal=False, sm_scale=0.125)
    plan = qa.SagePlan(1, 2, 2, 256, 64, torch.float16, False, device="cpu", smooth_q=True)
    with pytest.raises(RuntimeError, match="quant"):
        plan.attn()


def _mfma_peak(lib, kind=0, iters=100, nwg=4, clocks=FAKE, sink=FAKE):
    khz = ctypes.c_int(0)
    return lib.sage_mfma_peak(kind, iters, nwg, clocks, sink, ctypes.byref(khz), None)


@pytest.mark.parametrize("kw,code", [
    (dict(clocks=None), 1), (dict(sink=None), 1), (dict(kind=2), 6), (dict(kind=-1), 6),
    (dict(iters=0), 6), (dict(iters=(1 << 18) + 1), 6), (dict(nwg=0), 6), (dict(nwg=65537), 6),
    (dict(clocks=FAKE + 8), 9), (dict(sink=FAKE + 4), 9),
])
def test_mfma_peak_rejects(kw, code):
    """The roofline probe checks its arguments before touching a device."""
    assert _mfma_peak(qa.load_library(), **kw) == code
