"""Helpers shared by the GPU tests: move host inputs to the device, call the
library, bring results back as float64 for the oracle's check."""
import sys

import numpy as np
import torch

import bit_weight_gemm_int2_amd as lb
import oracle

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def banner(msg: str):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_bits(bits: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 host pattern -> device tensor of the 16-bit float dtype (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.cuda().view(TORCH_DT[dtype])


def to_host64(y: torch.Tensor) -> np.ndarray:
    if y.dtype == torch.float32:
        return y.cpu().numpy().astype(np.float64)
    bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.decode(bits, "f16" if y.dtype == torch.float16 else "bf16")


def dev_weights(fmt: str, codes: np.ndarray, scales: np.ndarray):
    c = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    packed = lb.pack_ternary(c) if fmt == "ternary" else lb.pack_binary(c)
    s = torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).cuda().view(torch.float16)
    return packed, s


def run_linear(lin, x_bits=None, activation=None, out_dtype=None, bias=True):
    """Run one workloads.Linear on the GPU; return (Y float64, packed)."""
    xb = lin.x if x_bits is None else x_bits
    x = dev_bits(xb, lin.x_dtype)
    packed, s = dev_weights(lin.fmt, lin.codes, lin.scales)
    b = None
    if bias and lin.bias is not None:
        b = torch.from_numpy(lin.bias.view(np.int16)).cuda().view(torch.float16)
    y = lb.gemm(x, packed, s, lin.fmt, bias=b, out_dtype=out_dtype or TORCH_DT[lin.y_dtype],
                activation=activation)
    torch.cuda.synchronize()
    return to_host64(y), packed


def oracle_linear(lin, x_bits=None, bias=True):
    xb = lin.x if x_bits is None else x_bits
    b = lin.bias if bias else None
    A = oracle.linear(xb, lin.x_dtype, lin.codes, lin.scales, b)
    Mg = oracle.magnitude(xb, lin.x_dtype, lin.codes, lin.scales, b)
    return A, Mg
