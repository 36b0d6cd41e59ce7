"""Python binding of ``liblowbit.so``, the gfx950 low-bit-weight GEMM library.

Argument marshalling only: every step runs in the HIP kernels of the library.
PyTorch supplies device memory (``torch.empty`` on the GPU) and the current
HIP stream. If the library is not built, or no gfx950 GPU is present, calls
raise; there is no fallback implementation.

    packed = pack_ternary(codes_int8_cuda)            # [N, K/4] uint8
    y = gemm(x_bf16_cuda, packed, scales_f16_cuda, "ternary", bias=None)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblowbit.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_GROUP, ERR_WORKSPACE, ERR_DEVICE, ERR_HIP, ERR_OVERLAP = range(10)
F16, BF16, F32, NONE = 0, 1, 2, 3
BINARY, TERNARY, BASE3, INT4 = 1, 2, 3, 4
ACT_NONE, ACT_GELU = 0, 1
GROUP = 128

_FMT = {"ternary": TERNARY, "binary": BINARY, "base3": BASE3, "int4": INT4, TERNARY: TERNARY, BINARY: BINARY,
        BASE3: BASE3, INT4: INT4}
_DT = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
_ACT = {None: ACT_NONE, "none": ACT_NONE, "gelu": ACT_GELU, ACT_NONE: ACT_NONE, ACT_GELU: ACT_GELU}

_lib = None

# (name, restype, argtypes) for every entry point of include/lowbit.h
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = [
    ("lowbit_abi_version", _I32, []),
    ("lowbit_status_string", ctypes.c_char_p, [_I32]),
    ("lowbit_init", _I32, []),
    ("lowbit_debug_force_variant", _I32, [ctypes.c_char_p]),
    ("lowbit_packed_bytes", _I64, [_I32, _I64, _I64]),
    ("lowbit_scale_count", _I64, [_I64, _I64, _I32]),
    ("pack_ternary", _I32, [_P, _I64, _I64, _P, _P, _P]),
    ("pack_binary", _I32, [_P, _I64, _I64, _P, _P, _P]),
    ("pack_base3", _I32, [_P, _I64, _I64, _P, _P, _P]),
    ("unpack_lowbit", _I32, [_I32, _P, _I64, _I64, _P, _P, _P]),
    ("base3_to_int2", _I32, [_P, _I64, _I64, _P, _P, _P]),
    ("lowbit_gemm_workspace_bytes", _SZ, [_I32, _I64, _I64, _I64]),
    ("lowbit_gemm", _I32, [_I32, _P, _I32, _I64, _I64, _I64, _P, _P, _I32, _I64,
                           _P, _I32, _P, _I32, _I64, _I32, _P, _SZ, _P]),
    ("lowbit_gelu", _I32, [_P, _P, _I32, _I64, _P]),
    ("lowbit_gemm_grouped", _I32, [_I32, _I32, _P, _I32, _I64, _I64, _I64, _P, _P, _I32, _I64,
                                   _P, _I32, _P, _I32, _I64, _I32, _P, _SZ, _P]),
    ("lowbit_gemm_grouped_workspace_bytes", _SZ, [_I32, _I32, _I64, _I64, _I64]),
    ("lowbit_gemm_noalloc", _I32, [_I32, _P, _I32, _I64, _I64, _I64, _P, _P, _I32, _I64,
                                   _P, _I32, _P, _I32, _I64, _I32, _P]),
    ("pack_int4", _I32, [_P, _I64, _I64, _P, _P, _P]),
    ("lowbit_gemm_int4_workspace_bytes", _SZ, [_I64, _I64, _I64]),
    ("lowbit_gemm_int4", _I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _I64,
                                _P, _I32, _P, _I32, _I64, _I32, _P, _SZ, _P]),
    ("lowbit_quantize", _I32, [_I32, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
]
MAX_GROUP = 8


class LowbitError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load liblowbit.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m bit_weight_gemm_int2_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lowbit_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise LowbitError(status, what)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _cuda(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def packed_bytes(fmt, N: int, K: int) -> int:
    return int(lib().lowbit_packed_bytes(_FMT[fmt], N, K))


def workspace_bytes(fmt, M: int, N: int, K: int) -> int:
    return int(lib().lowbit_gemm_workspace_bytes(_FMT[fmt], M, N, K))


def force_variant(name=None):
    """Test hook: force one kernel family ("large", "small", "large-wide",
    "large-pair", "small-split"; for the ternary quantiser "quant-eighth",
    "quant-lane": eight or one lane per group) for every later call of the process, or restore the
    automatic choice with None / "auto"."""
    _check(lib().lowbit_debug_force_variant(None if name is None else name.encode()), "lowbit_debug_force_variant")


_WORKSPACES = {}


def new_workspace(nbytes: int, device=None, stream=None) -> torch.Tensor:
    """A workspace for lowbit_gemm: zeroed device bytes (the library returns
    its counters to zero after every call, so it stays reusable). The zeros
    are written on `stream` (default: the current stream), the stream the
    workspace is then used on."""
    dev = torch.device(device or "cuda")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(st):
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
        ws.zero_()
    return ws


def _shared_workspace(device: torch.device, nbytes: int, stream) -> torch.Tensor:
    """A workspace per (device, stream), reused by every call on that stream
    that passes none: calls on one stream never overlap, and calls on two
    streams never share one. It is zeroed on the stream it serves, and grows
    when a larger problem needs more (the buffer it replaces is kept alive
    until the work queued on the stream so far is done); grow it before any
    HIP graph capture by running the largest problem once."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    st = stream if stream is not None else torch.cuda.current_stream(idx)
    key = (idx, st.cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            ws.record_stream(st)
        ws = new_workspace(max(nbytes, 1 << 20), torch.device("cuda", idx), st)
        _WORKSPACES[key] = ws
    return ws


def _row_bytes(fmt: int, K: int) -> int:
    if fmt == BASE3:
        return (K + 4) // 5
    return K // {TERNARY: 4, BINARY: 8, INT4: 2}[fmt]


def _counted(fn, src: torch.Tensor, N: int, K: int, out: torch.Tensor, check: bool, stream, what: str):
    cnt = torch.empty(1, dtype=torch.int32, device=src.device) if check else None
    _check(fn(src.data_ptr(), N, K, out.data_ptr(), _ptr(cnt), _stream(stream)), fn.__name__)
    if check:
        bad = int(cnt.item())
        if bad:
            raise ValueError(f"{bad} {what}")
    return out


def _pack(fn, codes: torch.Tensor, fmt: int, check: bool, stream) -> torch.Tensor:
    _cuda(codes, "codes")
    want = torch.uint8 if fmt == INT4 else torch.int8
    if codes.dtype != want or codes.dim() != 2:
        raise ValueError(f"codes must be a 2-D {want} tensor")
    codes = codes.contiguous()
    N, K = codes.shape
    out = torch.empty((N, _row_bytes(fmt, K)), dtype=torch.uint8, device=codes.device)
    return _counted(fn, codes, N, K, out, check, stream, "code(s) outside the allowed set")


def pack_ternary(codes: torch.Tensor, check: bool = True, stream=None) -> torch.Tensor:
    """int8 codes [N, K] in {-1,0,+1} -> packed uint8 [N, K/4] (K % 16 == 0)."""
    return _pack(lib().pack_ternary, codes, TERNARY, check, stream)


def pack_binary(codes: torch.Tensor, check: bool = True, stream=None) -> torch.Tensor:
    """int8 codes [N, K] in {-1,+1} -> packed uint8 [N, K/8] (K % 32 == 0)."""
    return _pack(lib().pack_binary, codes, BINARY, check, stream)


def pack_int4(codes: torch.Tensor, check: bool = True, stream=None) -> torch.Tensor:
    """uint8 codes [N, K] in 0..15 -> packed uint8 [N, K/2] (K % 8 == 0)."""
    return _pack(lib().pack_int4, codes, INT4, check, stream)


def gemm_int4(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
              bias: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None, activation=None,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """Y = act(X W^T + bias) with W = s * (q - z) from 4-bit codes (lowbit_gemm_int4).

    x: [M, K] fp16/bf16; packed: [N, K/2] uint8; scales, zeros: fp16 [N, K/128].
    A workspace for the row sums is allocated per call unless one is given."""
    for t, nm in ((x, "x"), (packed, "packed"), (scales, "scales"), (zeros, "zeros")):
        _cuda(t, nm)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    M, K = x.shape
    N = packed.shape[0]
    packed, scales, zeros = packed.contiguous(), scales.contiguous(), zeros.contiguous()
    _check_packed(INT4, packed, N, K)
    for t, nm in ((scales, "scales"), (zeros, "zeros")):
        if t.dtype != torch.float16 or tuple(t.shape) != (N, K // GROUP):
            raise ValueError(f"{nm} must be float16 [{N}, {K // GROUP}]")
    if bias is not None:
        _cuda(bias, "bias")
        bias = bias.contiguous()
        if bias.numel() != N or bias.dtype not in _DT:
            raise ValueError(f"bias must hold {N} float16, bfloat16 or float32 values")
    odt = out_dtype or x.dtype
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=x.device)
    elif tuple(out.shape) != (M, N) or out.stride(1) != 1 or out.dtype not in _DT:
        raise ValueError(f"out must be [{M}, {N}] with unit stride along N")
    need = int(lib().lowbit_gemm_int4_workspace_bytes(M, N, K))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"lowbit_gemm_int4 needs {need}")
    _check(lib().lowbit_gemm_int4(
        x.data_ptr(), _DT[x.dtype], M, K, x.stride(0), packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
        GROUP, N, _ptr(bias), NONE if bias is None else _DT[bias.dtype], out.data_ptr(), _DT[out.dtype],
        out.stride(0), _ACT[activation], workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)), "lowbit_gemm_int4")
    return out


def quantize(w: torch.Tensor, fmt, check: bool = True, out=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Dense FP16 weights [N, K] (row stride may exceed K) -> (packed uint8
    [N, K/4] or [N, K/8], fp16 scales [N, K/128]) by lowbit_quantize, into
    `out` = (packed, scales) when given. With check, waits for the device and
    raises on NaN or infinite weights."""
    _cuda(w, "w")
    if w.dtype != torch.float16 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D float16 tensor with unit stride along K")
    fmt = _FMT[fmt]
    N, K = w.shape
    if fmt not in (TERNARY, BINARY) or K % GROUP:
        raise ValueError("quantize makes ternary or binary codes; K must be a multiple of 128")
    if out is None:
        packed = torch.empty((N, _row_bytes(fmt, K)), dtype=torch.uint8, device=w.device)
        scales = torch.empty((N, K // GROUP), dtype=torch.float16, device=w.device)
    else:
        packed, scales = out
        if (packed.dtype != torch.uint8 or tuple(packed.shape) != (N, _row_bytes(fmt, K))
                or not packed.is_contiguous() or scales.dtype != torch.float16
                or tuple(scales.shape) != (N, K // GROUP) or not scales.is_contiguous()):
            raise ValueError("out must be contiguous (uint8 packed [N, row bytes], float16 scales [N, K/128])")
    cnt = torch.empty(1, dtype=torch.int32, device=w.device) if check else None
    _check(lib().lowbit_quantize(fmt, w.data_ptr(), N, K, w.stride(0), packed.data_ptr(), scales.data_ptr(),
                                 _ptr(cnt), _stream(stream)), "lowbit_quantize")
    if check:
        bad = int(cnt.item())
        if bad:
            raise ValueError(f"{bad} non-finite weight(s)")
    return packed, scales


def pack_base3(codes: torch.Tensor, check: bool = True, stream=None) -> torch.Tensor:
    """int8 codes [N, K] in {-1,0,+1} -> base-3 uint8 [N, ceil(K/5)] (any K >= 1)."""
    return _pack(lib().pack_base3, codes, BASE3, check, stream)


def base3_to_int2(packed: torch.Tensor, K: int, check: bool = True, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """base-3 uint8 [N, ceil(K/5)] -> INT2 uint8 [N, K/4] for gemm (K % 16 == 0).
    With check, waits for the device and raises on invalid base-3 bytes."""
    _cuda(packed, "packed")
    if packed.dtype != torch.uint8 or packed.dim() != 2 or packed.shape[1] != (K + 4) // 5:
        raise ValueError("packed must be a 2-D uint8 tensor of ceil(K/5) bytes per row")
    packed = packed.contiguous()
    N = packed.shape[0]
    if out is None:
        out = torch.empty((N, K // 4), dtype=torch.uint8, device=packed.device)
    elif out.dtype != torch.uint8 or tuple(out.shape) != (N, K // 4) or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 tensor [N, K/4]")
    return _counted(lib().base3_to_int2, packed, N, K, out, check, stream, "invalid base-3 value(s)")


def _check_packed(fmt, packed: torch.Tensor, N: int, K: int):
    """The library reads N x (bytes per row) packed bytes: check the tensor holds them."""
    if packed.dtype != torch.uint8 or packed.dim() != 2:
        raise ValueError("packed must be a 2-D uint8 tensor")
    row = _row_bytes(_FMT[fmt], K)
    if tuple(packed.shape) != (N, row):
        raise ValueError(f"packed must be [{N}, {row}] for K = {K}, got {list(packed.shape)}")


def unpack(fmt, packed: torch.Tensor, K: int, stream=None) -> Tuple[torch.Tensor, int]:
    """packed [N, K/4, K/8, ceil(K/5) or K/2] -> (codes [N, K], number of invalid codes);
    int8 codes, uint8 for the 4-bit format."""
    _cuda(packed, "packed")
    packed = packed.contiguous()
    N = packed.shape[0]
    _check_packed(fmt, packed, N, K)
    codes = torch.empty((N, K), dtype=torch.uint8 if _FMT[fmt] == INT4 else torch.int8, device=packed.device)
    cnt = torch.empty(1, dtype=torch.int32, device=packed.device)
    _check(lib().unpack_lowbit(_FMT[fmt], packed.data_ptr(), N, K, codes.data_ptr(), cnt.data_ptr(),
                               _stream(stream)), "unpack_lowbit")
    return codes, int(cnt.item())


def gemm(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, fmt, bias: Optional[torch.Tensor] = None,
         out_dtype: Optional[torch.dtype] = None, activation=None, out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = act(X W^T + bias) with W = scale_g * t from packed codes.

    x: [M, K] fp16/bf16 (row stride may exceed K); packed: [N, K/4] (ternary) or
    [N, K/8] (binary) uint8; scales: fp16 [N, K/128]; bias: [N] or None.
    Output dtype defaults to x's dtype."""
    for t, nm in ((x, "x"), (packed, "packed"), (scales, "scales")):
        _cuda(t, nm)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    M, K = x.shape
    N = packed.shape[0]
    packed = packed.contiguous()
    scales = scales.contiguous()
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be float16 or bfloat16")
    _check_packed(fmt, packed, N, K)
    if scales.dtype != torch.float16 or tuple(scales.shape) != (N, K // GROUP):
        raise ValueError(f"scales must be float16 [{N}, {K // GROUP}]")
    if bias is not None:
        _cuda(bias, "bias")
        bias = bias.contiguous()
        if bias.numel() != N or bias.dtype not in _DT:
            raise ValueError(f"bias must hold {N} float16, bfloat16 or float32 values")
    odt = out_dtype or x.dtype
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=x.device)
    elif tuple(out.shape) != (M, N) or out.dim() != 2 or out.stride(1) != 1 or out.dtype not in _DT:
        raise ValueError(f"out must be [{M}, {N}] with unit stride along N")
    ws_need = workspace_bytes(fmt, M, N, K)
    if ws_need and workspace is None:
        workspace = _shared_workspace(x.device, ws_need, stream)
    elif ws_need and workspace.numel() * workspace.element_size() < ws_need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"lowbit_gemm needs {ws_need}")
    st = lib().lowbit_gemm(
        _FMT[fmt], x.data_ptr(), _DT[x.dtype], M, K, x.stride(0),
        packed.data_ptr(), scales.data_ptr(), GROUP, N,
        _ptr(bias), NONE if bias is None else _DT[bias.dtype],
        out.data_ptr(), _DT[out.dtype], out.stride(0), _ACT[activation],
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "lowbit_gemm")
    return out


def _ptr_array(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def gemm_grouped(xs, packeds, scales, fmt, biases=None, out_dtype: Optional[torch.dtype] = None,
                 activation=None, outs=None, workspace: Optional[torch.Tensor] = None,
                 stream=None):
    """Several independent linears of one shape in one launch (small M):
    ys[z] = act(xs[z] W[z]^T + biases[z]). Every x shares shape, dtype and row
    stride; every packed / scales pair shares shape. Returns the list of outputs."""
    count = len(xs)
    if not 1 <= count <= MAX_GROUP or len(packeds) != count or len(scales) != count:
        raise ValueError(f"1 .. {MAX_GROUP} problems, with one packed and one scales tensor each")
    if biases is not None and len(biases) != count:
        raise ValueError("one bias per problem")
    x0 = xs[0]
    for t in list(xs) + list(packeds) + list(scales):
        _cuda(t, "operand")
    if x0.dim() != 2 or any(x.shape != x0.shape or x.stride() != x0.stride() or x.dtype != x0.dtype for x in xs):
        raise ValueError("every x must have the shape, stride and dtype of the first")
    if x0.stride(1) != 1:
        raise ValueError("x must have unit stride along K")
    M, K = x0.shape
    packeds = [p.contiguous() for p in packeds]
    scales = [s_.contiguous() for s_ in scales]
    N = packeds[0].shape[0]
    for p in packeds:
        _check_packed(fmt, p, N, K)
    if any(s_.dtype != torch.float16 or tuple(s_.shape) != (N, K // GROUP) for s_ in scales):
        raise ValueError(f"scales must be float16 [{N}, {K // GROUP}]")
    odt = out_dtype or x0.dtype
    if outs is None:
        outs = [torch.empty((M, N), dtype=odt, device=x0.device) for _ in range(count)]
    elif len(outs) != count or any(tuple(y.shape) != (M, N) or y.stride(1) != 1 or y.dtype != outs[0].dtype
                                   or y.stride(0) != outs[0].stride(0) for y in outs):
        raise ValueError(f"outs: {count} tensors [{M}, {N}] of one dtype and row stride")
    bdt = NONE
    if biases is not None:
        biases = [b.contiguous() for b in biases]
        if any(b.numel() != N or b.dtype != biases[0].dtype for b in biases):
            raise ValueError(f"biases: {count} tensors of {N} values and one dtype")
        bdt = _DT[biases[0].dtype]
    need = int(lib().lowbit_gemm_grouped_workspace_bytes(count, _FMT[fmt], M, N, K))
    if need and workspace is None:
        workspace = _shared_workspace(x0.device, need, stream)
    elif need and workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"lowbit_gemm_grouped needs {need}")
    st = lib().lowbit_gemm_grouped(
        count, _FMT[fmt], _ptr_array([x.data_ptr() for x in xs]), _DT[x0.dtype], M, K, x0.stride(0),
        _ptr_array([p.data_ptr() for p in packeds]), _ptr_array([s_.data_ptr() for s_ in scales]), GROUP, N,
        None if biases is None else _ptr_array([b.data_ptr() for b in biases]), bdt,
        _ptr_array([y.data_ptr() for y in outs]), _DT[outs[0].dtype], outs[0].stride(0), _ACT[activation],
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "lowbit_gemm_grouped")
    return outs


def gelu(x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Exact-erf GELU (x * Phi(x)) in FP32, stored in x's dtype."""
    _cuda(x, "x")
    x = x.contiguous()
    out = torch.empty_like(x) if out is None else out
    _check(lib().lowbit_gelu(x.data_ptr(), out.data_ptr(), _DT[x.dtype], x.numel(), _stream(stream)),
           "lowbit_gelu")
    return out
