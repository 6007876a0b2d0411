"""The example host program on the C ABI (the article's aclnn call sequence,
section 调用方式一 aclnn API, written for HIP) runs to completion on the GPU
and its own checks pass: rows sum to 1 with the library's lse, and values
appear only at selected columns."""

import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "sparse_mla_attention_02_amd", "smla_example")


def test_c_example_program():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "build the library first (__graft_entry__.build())"
    print("[c-example] running the example program", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=90)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "smla_example: OK" in r.stdout
