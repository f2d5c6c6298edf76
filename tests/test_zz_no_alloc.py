"""The entry point that allocates nothing (sage_quant_qk_noalloc), called raw
through the C ABI, against sage_quant_qk with a caller workspace: every
output bit-identical, on two calls in a row (the second smaller, so it reads
scratch the first call left behind), plus smooth Q and per-query scales."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(B, H, H_kv, N, d, dtype, seed):
    g = np.random.default_rng(seed)
    q = torch.from_numpy(g.standard_normal((B, H, N, d), dtype=np.float32) * 2).to(dtype)
    k = g.standard_normal((B, H_kv, N, d), dtype=np.float32)
    k += g.standard_normal((B, H_kv, 1, d), dtype=np.float32) * 3
    return q.to(DEV), torch.from_numpy(k).to(dtype).to(DEV)


def _alloc(B, H, H_kv, N, d, q_group, smooth_q):
    nq, nk = -(-N // q_group), -(-N // 64)
    out = dict(q_i8=torch.empty((B, H, N, d), dtype=torch.int8, device=DEV),
               q_scale=torch.empty((B, H, nq), dtype=torch.float32, device=DEV),
               k_i8=torch.empty((B, H_kv, N, d), dtype=torch.int8, device=DEV),
               k_scale=torch.empty((B, H_kv, nk), dtype=torch.float32, device=DEV),
               k_mean=torch.empty((B, H_kv, d), dtype=torch.float32, device=DEV))
    if smooth_q:
        out["q_mean"] = torch.empty((B, H, -(-N // 128), d), dtype=torch.float32, device=DEV)
    return out


CALLS = [
    # B, H, H_kv, N, d, dtype, q_group, smooth_q
    (2, 8, 4, 3000, 128, torch.float16, 128, False),
    (1, 4, 2, 300, 64, torch.bfloat16, 1, True),
]


def test_quant_qk_noalloc_matches_workspace_entry_point(gpu_lib):
    lib = gpu_lib.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    for i, (B, H, H_kv, N, d, dtype, qg, sq) in enumerate(CALLS):
        print(f"noalloc call {i}: B{B} H{H}/{H_kv} N{N} d{d} {dtype} q_group {qg} smooth_q {sq}",
              flush=True)
        q, k = _inputs(B, H, H_kv, N, d, dtype, seed=90 + i)
        ref = gpu_lib.sage_quant_qk(q, k, True, q_group=qg, smooth_q=sq)
        out = _alloc(B, H, H_kv, N, d, qg, sq)
        for t in out.values():
            t.fill_(0x55 if t.dtype == torch.int8 else 7.0)
        st = lib.sage_quant_qk_noalloc(
            q.data_ptr(), k.data_ptr(), 1 if dtype == torch.bfloat16 else 0, B, H, H_kv, N, d,
            qg, 1, int(sq), out["q_i8"].data_ptr(), out["q_scale"].data_ptr(),
            out["k_i8"].data_ptr(), out["k_scale"].data_ptr(), out["k_mean"].data_ptr(),
            out["q_mean"].data_ptr() if sq else None, ctypes.c_void_p(stream))
        assert st == 0, lib.sage_status_str(st)
        torch.cuda.synchronize()
        for name, t in out.items():
            assert torch.equal(t, ref[name]), (i, name)
