"""Seeded synthetic inputs for the quantized attention forward pass.

This module only draws random tensors; it holds none of the method's
arithmetic (no smoothing, quantization or attention).  Both the CPU oracle
(``oracle/``) and the GPU binding's tests and benchmark take their inputs from
here, so the two sides always see identical bits.

Workload shapes follow the pages' kernel benchmarks and model workloads
(SageAttention2 detail page, "Deep Analysis (kernel)": head dims 64 and 128,
long sequences; CogVideoX ~17K-token attention on the SageAttention page;
Llama3.1 100K-token prefill in SageAttention2 Table 8).  The real model
activations are not available, so K carries a per-channel bias shared by all
tokens: that is the channel-outlier structure smoothing K is meant to remove
(SageAttention page, the Smooth K paragraph).

Recipe (every config): standard normals are drawn in float32 from
``np.random.default_rng(SeedSequence([seed, tensor_id, b, head]))`` one
(b, head) slice at a time, then cast to fp16/bf16 with round-to-nearest-even
(torch CPU cast).  tensor_id: Q=0, K=1, V=2, K-bias=3.  The K bias is drawn
per (b, kv-head) as N(0, bias_var) per channel; ``outlier_channels`` channels
(indices drawn once from the config seed) have their bias multiplied by
``outlier_mult``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "generate", "sweep"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    H_kv: int
    N: int
    d: int
    causal: bool
    dtype: str  # "fp16" | "bf16"
    bias_var: float
    seed: int
    outlier_channels: int = 0
    outlier_mult: float = 1.0
    description: str = ""

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16

    def ops(self) -> float:
        """4*B*H*N^2*d, halved when causal (the pages' TOPS convention)."""
        o = 4.0 * self.B * self.H * self.N * self.N * self.d
        return o / 2 if self.causal else o

    def with_n(self, n: int, seed: int | None = None) -> "Workload":
        return replace(self, N=n, name=f"{self.name.split('@')[0]}@N{n}",
                       seed=self.seed if seed is None else seed)


WORKLOADS = {
    "tiny": Workload(
        "tiny", B=1, H=2, H_kv=2, N=256, d=64, causal=False, dtype="fp16",
        bias_var=9.0, seed=1,
        description="tiny non-causal attention B1 H2 N256 d64 fp16"),
    "llm_prefill": Workload(
        "llm_prefill", B=1, H=32, H_kv=32, N=4096, d=128, causal=True,
        dtype="fp16", bias_var=9.0, seed=2, outlier_channels=4,
        outlier_mult=10.0,
        description="LLM prefill B1 H32 N4096 d128 fp16 causal, 4 outlier K channels x10"),
    "video_dit": Workload(
        "video_dit", B=1, H=48, H_kv=48, N=17550, d=64, causal=False,
        dtype="bf16", bias_var=4.0, seed=3,
        description="video-DiT self-attention B1 H48 N17550 d64 bf16"),
    "sweep": Workload(
        "sweep", B=4, H=32, H_kv=32, N=32768, d=128, causal=False,
        dtype="fp16", bias_var=9.0, seed=40,
        description="sequence sweep B4 H32 d128 fp16 non-causal"),
    "gqa_long": Workload(
        "gqa_long", B=1, H=32, H_kv=8, N=102400, d=128, causal=True,
        dtype="bf16", bias_var=9.0, seed=5,
        description="long-context GQA prefill B1 H32/8 N102400 d128 bf16 causal"),
}

SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768)


def sweep(n: int) -> Workload:
    """The sequence-sweep workload at sequence length n (seed 40+i)."""
    i = SWEEP_N.index(n)
    return WORKLOADS["sweep"].with_n(n, seed=40 + i)


def get(name: str) -> Workload:
    if "@N" in name:
        base, n = name.split("@N")
        assert base == "sweep"
        return sweep(int(n))
    return WORKLOADS[name]


def _rng(seed: int, tensor_id: int, b: int, head: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id, b, head]))


def _outlier_idx(w: Workload) -> np.ndarray:
    if w.outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    g = np.random.default_rng(np.random.SeedSequence([w.seed, 99]))
    return np.sort(g.choice(w.d, size=w.outlier_channels, replace=False))


def k_bias(w: Workload, b: int, hk: int) -> np.ndarray:
    """The per-channel K bias of kv-head (b, hk), float32 [d]."""
    g = _rng(w.seed, 3, b, hk)
    bias = g.standard_normal(w.d, dtype=np.float32) * np.float32(math.sqrt(w.bias_var))
    idx = _outlier_idx(w)
    bias[idx] *= np.float32(w.outlier_mult)
    return bias


def _slice(w: Workload, tensor_id: int, b: int, head: int, n: int) -> torch.Tensor:
    g = _rng(w.seed, tensor_id, b, head)
    x = g.standard_normal((n, w.d), dtype=np.float32)
    if tensor_id == 1:
        x += k_bias(w, b, head)[None, :]
    return torch.from_numpy(x).to(w.torch_dtype)


def generate(w: Workload, tensors=("q", "k", "v"), heads=None, threads: int | None = None):
    """Return a dict of CPU torch tensors q [B,H,N,d], k/v [B,H_kv,N,d].

    ``heads``: optional list of (b, h) query heads; then only those query
    heads (and the kv heads they map to) are filled, the rest is left zero.
    Generation is per (b, head) slice, so any subset is bit-identical to the
    same slice of the full tensor.
    """
    ids = {"q": 0, "k": 1, "v": 2}
    out = {}
    grp = w.H // w.H_kv
    threads = threads or min(16, os.cpu_count() or 1)
    jobs = []
    for name in tensors:
        nh = w.H if name == "q" else w.H_kv
        t = torch.zeros((w.B, nh, w.N, w.d), dtype=w.torch_dtype)
        out[name] = t
        if heads is None:
            sel = [(b, h) for b in range(w.B) for h in range(nh)]
        elif name == "q":
            sel = sorted(set(heads))
        else:
            sel = sorted({(b, h // grp) for b, h in heads})
        for b, h in sel:
            jobs.append((name, b, h))

    def run(job):
        name, b, h = job
        out[name][b, h] = _slice(w, ids[name], b, h, w.N)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, jobs))
    return out
