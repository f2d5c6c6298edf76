"""Host-side contracts: bench.py measures one GPU only and has no CPU fallback, its
workloads exist, and the binding and smoke() refuse to run without a GPU."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, env=env, cwd=ROOT)


@pytest.mark.parametrize("args,env", [(("--gpus", "2"), None), ((), {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused_with_a_message(args, env):
    r = _bench(*args, env_extra=env)
    assert r.returncode == 2, r.stderr
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""          # no result line


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_means_no_result_rather_than_a_cpu_fallback():
    r = _bench("--steps", "1", "--warmup", "0", "--no-cpu")
    assert r.returncode != 0
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_every_workload_the_benchmark_names_exists():
    import workloads as W
    names = ["tiny", "llm_prefill", "video_dit", "gqa_long"] + [
        f"sweep@N{n}" for n in (1024, 2048, 4096, 8192, 16384, 32768)]
    for name in names:
        w = W.get(name)
        assert w.N > 0 and w.d in (64, 128) and w.H % w.H_kv == 0, name
    assert W.get("sweep@N32768").N == 32768


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_binding_refuses_host_tensors():
    import quantized_attention_amd as qa
    q = torch.randn(1, 2, 64, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="CUDA"):
        qa.sageattn(q, q, q)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_smoke_refuses_a_host_without_a_gpu():
    import __graft_entry__ as g
    with pytest.raises(AssertionError, match="needs a GPU"):
        g.smoke()
