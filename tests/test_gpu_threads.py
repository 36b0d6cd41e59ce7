"""The library from several host threads at once: each thread runs its own
problems on its own stream with its own workspace (calls that can overlap
must not share one), interleaving with the other threads' calls on the host
(the binding's ctypes calls release the interpreter lock). Every result must
equal, bit for bit, the same call made alone; the library's only shared
state is its per-device property cache."""
import threading

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import banner, dev_bits, dev_weights

pytestmark = pytest.mark.gpu

PROBLEMS = [  # (fmt, M, N, K): thin, column tiles with split K, large M
    ("ternary", 16, 3072, 3072),
    ("binary", 16, 3072, 9216),
    ("ternary", 300, 2048, 1024),
    ("binary", 4, 9216, 3072),
]


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def test_concurrent_host_threads(lb):
    banner("host threads")
    ops = []
    for i, (fmt, M, N, K) in enumerate(PROBLEMS):
        lin = wl.make_linear(f"thr{i}", fmt, M, N, K, seed=990 + i, p0=0.35)
        x = dev_bits(lin.x, "bf16")
        p, s = dev_weights(fmt, lin.codes, lin.scales)
        ref = lb.gemm(x, p, s, fmt, workspace=lb.new_workspace(lb.workspace_bytes(fmt, M, N, K)))
        ops.append((fmt, M, N, K, x, p, s, ref))
    torch.cuda.synchronize()
    errors = []

    def worker(tid):
        try:
            st = torch.cuda.Stream()
            # zeroed on the stream that uses them
            wss = [lb.new_workspace(lb.workspace_bytes(fmt, M, N, K), stream=st) for fmt, M, N, K, *_ in ops]
            with torch.cuda.stream(st):
                outs = []
                for r in range(12):
                    j = (tid + r) % len(ops)
                    fmt, M, N, K, x, p, s, ref = ops[j]
                    outs.append((j, lb.gemm(x, p, s, fmt, workspace=wss[j], stream=st)))
            st.synchronize()
            for j, y in outs:
                if not torch.equal(y.view(torch.int16), ops[j][7].view(torch.int16)):
                    errors.append(f"thread {tid}, problem {j}: differs from the single call")
        except Exception as e:                       # reported below, in the main thread
            errors.append(f"thread {tid}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
