"""The Python binding on the CPU: it refuses tensors it cannot hand to the C
ABI (wrong device, shape, dtype, layout) with a clear error before any
device call, and the package fails loudly when libfa.so is missing (there is
no CPU fallback)."""

import os
import subprocess
import sys

import pytest
import torch

import tiled_attention_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def cpu(*shape, dtype=torch.float16):
    return torch.zeros(shape, dtype=dtype)


def test_host_tensors_are_refused():
    q = cpu(1, 2, 64, 64)
    with pytest.raises(ValueError, match="HIP device"):
        fa.fa_forward(q, q, q, torch.empty_like(q))
    with pytest.raises(ValueError, match="HIP device"):
        fa.fa_forward_strided(q, q, q, torch.empty_like(q))


@pytest.mark.parametrize("bad,match", [
    (lambda q: cpu(2, 64, 64), "must be \\[B, H, N, D\\]"),
    (lambda q: cpu(1, 2, 64, 128).transpose(2, 3), "contiguous"),
    (lambda q: cpu(1, 2, 64, 64, dtype=torch.bfloat16), "must match q"),
    (lambda q: cpu(1, 3, 64, 64), "must match q"),
])
def test_malformed_tensors_are_refused(bad, match):
    q = cpu(1, 2, 64, 64)
    with pytest.raises(ValueError, match=match):
        fa.fa_forward(q, q, bad(q), torch.empty_like(q))


def test_strided_shape_rules():
    q = cpu(1, 4, 64, 64)
    kv = cpu(1, 2, 64, 64)
    with pytest.raises(ValueError, match="contiguous last dimension"):
        fa.fa_forward_strided(q, kv.transpose(2, 3), kv, torch.empty_like(q))
    with pytest.raises(ValueError, match="shapes must be"):
        fa.fa_forward_strided(q, kv, cpu(1, 2, 32, 64), torch.empty_like(q))


def test_unsupported_dtype_code():
    with pytest.raises(TypeError, match="unsupported tensor dtype"):
        fa._lib._dtype_code(torch.zeros(1, dtype=torch.float64))


def test_missing_library_fails_loudly(tmp_path):
    """A copy of the package without libfa.so: loading raises ImportError
    with the build instructions instead of falling back to anything."""
    pkg = tmp_path / "tiled_attention_fa_amd"
    pkg.mkdir()
    for name in ("__init__.py", "_lib.py"):
        (pkg / name).write_text(open(os.path.join(ROOT, "tiled_attention_fa_amd", name)).read())
    code = ("import tiled_attention_fa_amd as fa\n"
            "try:\n    fa.load_library()\nexcept ImportError as e:\n    print('refused:', e)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert "refused:" in out.stdout and "not built" in out.stdout
