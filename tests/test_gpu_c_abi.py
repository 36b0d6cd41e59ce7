"""The C ABI driven from a plain C program (tests/c/abi_example.c, built with
gcc): pack_ternary and lowbit_gemm on the GPU, outputs printed and compared
with the oracle. The program's inputs are exact in FP32 at every step (codes
in {-1, 0, 1}, activations that are multiples of 1/8, power-of-two scales), so
the comparison is bit for bit."""
import subprocess

import numpy as np
import pytest

import oracle
from gpu_util import banner
from test_abi import build_c_example

pytestmark = pytest.mark.gpu


def _inputs(M, N, K):
    """The program's inputs, from the same 32-bit LCG in the same order."""
    state = [12345]

    def nxt():
        state[0] = (state[0] * 1664525 + 1013904223) & 0xFFFFFFFF
        return state[0] >> 8
    t = np.array([nxt() % 3 - 1 for _ in range(N * K)], dtype=np.int8).reshape(N, K)
    xv = np.array([(nxt() % 17) - 8 for _ in range(M * K)], dtype=np.float32).reshape(M, K) / 8
    xbits = (xv.view(np.uint32) >> 16).astype(np.uint16)
    s = np.array([0x3000 + 0x400 * (nxt() % 4) for _ in range(N * K // 128)], dtype=np.uint16)
    return t, xbits, s.view(np.float16).reshape(N, K // 128)


@pytest.mark.parametrize("M,N,K", [(37, 300, 384), (4, 520, 1024)])
def test_c_program_matches_the_oracle(tmp_path, M, N, K):
    banner(f"C ABI program {M}x{N}x{K}")
    exe = build_c_example(str(tmp_path))
    r = subprocess.run([exe, str(M), str(N), str(K)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    y = np.array([float(v) for v in r.stdout.split()], dtype=np.float64).reshape(M, N)
    t, xbits, s = _inputs(M, N, K)
    A = oracle.linear(xbits, "bf16", t, s)
    assert np.array_equal(y, A.astype(np.float32).astype(np.float64))
