"""The C-ABI library loads and exports every entry point include/lowbit.h declares;
host-only calls (sizes, status strings, argument checks that fail before any
device work) behave as documented. CPU only: no kernel is launched here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowbit.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s+(\w+)\s*\(", text, flags=re.M)))


# Tests that pass made-up device addresses: every call in them must fail a
# host-side check, so on a machine with a GPU (where a call that passed every
# check would launch a kernel on those addresses) they are skipped.
made_up_addresses = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                                       reason="made-up device addresses; CPU-only checks")


@pytest.fixture(scope="module")
def L():
    import bit_weight_gemm_int2_amd as b
    if not os.path.exists(b.LIB_PATH):
        b_build = __import__("bit_weight_gemm_int2_amd.build", fromlist=["build"])
        b_build.build()
    return b.lib()


def test_header_declares_expected_entry_points():
    names = _declared()
    for want in ("pack_ternary", "pack_binary", "pack_base3", "unpack_lowbit", "base3_to_int2",
                 "lowbit_gemm", "lowbit_gemm_grouped", "lowbit_gemm_grouped_workspace_bytes",
                 "lowbit_gemm_workspace_bytes", "lowbit_packed_bytes", "lowbit_scale_count",
                 "lowbit_status_string", "lowbit_abi_version", "lowbit_init", "lowbit_gelu",
                 "lowbit_debug_force_variant", "lowbit_gemm_noalloc", "pack_int4", "lowbit_gemm_int4",
                 "lowbit_gemm_int4_workspace_bytes", "lowbit_quantize"):
        assert want in names


def test_every_declared_symbol_is_exported(L):
    import bit_weight_gemm_int2_amd as b
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in exported, name
        assert hasattr(L, name)
    # the Python binding declares a signature for every one of them
    assert sorted(n for n, _, _ in b.SIGNATURES) == _declared()


def test_host_only_queries(L):
    import bit_weight_gemm_int2_amd as b
    assert L.lowbit_abi_version() == 1
    assert L.lowbit_packed_bytes(b.TERNARY, 3072, 3072) == 3072 * 3072 // 4
    assert L.lowbit_packed_bytes(b.BINARY, 9216, 3072) == 9216 * 3072 // 8
    assert L.lowbit_packed_bytes(b.TERNARY, 4, 24) == -1       # K % 16
    assert L.lowbit_packed_bytes(b.BINARY, 4, 48) == -1        # K % 32
    assert L.lowbit_packed_bytes(7, 4, 128) == -1
    # base-3: ceil(K/5) bytes a row, any K >= 1
    assert L.lowbit_packed_bytes(b.BASE3, 3072, 3072) == 3072 * 615
    assert L.lowbit_packed_bytes(b.BASE3, 2, 1) == 2
    assert L.lowbit_packed_bytes(b.BASE3, 5, 7) == 10
    assert L.lowbit_packed_bytes(b.BASE3, 1, 0) == -1
    assert L.lowbit_packed_bytes(b.BASE3, 1, 1 << 31) == -1
    assert L.lowbit_packed_bytes(b.INT4, 2560, 9728) == 2560 * 4864
    assert L.lowbit_packed_bytes(b.INT4, 4, 12) == -1          # K % 8
    # 4-bit row sums: one float per 128-group and padded row
    assert L.lowbit_gemm_int4_workspace_bytes(4608, 9216, 3072) == 24 * (4608 + 128) * 4
    # with a K split (no GPU here: a 256-CU device is assumed): 80 tiles of
    # 64 x 256 at M = 512, N = 2560 take three splits; the planes follow the
    # row sums from the next 256-byte boundary
    sums = 76 * (512 + 128) * 4
    assert L.lowbit_gemm_int4_workspace_bytes(512, 2560, 9728) == (sums + 255) // 256 * 256 + 3 * 512 * 2560 * 4
    assert L.lowbit_gemm_int4_workspace_bytes(1, 64, 256) == 2 * 256 * 4
    assert L.lowbit_gemm_int4_workspace_bytes(1, 64, 200) == 0
    assert L.lowbit_scale_count(3072, 9216, 128) == 3072 * 72
    assert L.lowbit_scale_count(3072, 9216, 64) == -1
    for s in range(10):
        assert len(L.lowbit_status_string(s)) > 0
    assert L.lowbit_status_string(99) == b"unknown status"


@made_up_addresses
def test_argument_errors_before_any_device_work(L):
    """Every status that the host check returns before touching the device."""
    import bit_weight_gemm_int2_amd as b
    P = 1 << 20            # fake, 16-byte-aligned non-NULL "device" addresses, far apart
    PX, PW, PS, PY, PB = (k << 36 for k in range(1, 6))
    good = dict(fmt=b.TERNARY, X=PX, xd=b.BF16, M=16, K=256, ldx=256, W=PW, S=PS, group=128, N=64,
                bias=None, bd=b.NONE, Y=PY, yd=b.BF16, ldy=64, act=0, ws=None, wsb=0)

    def call(**kw):
        a = dict(good, **kw)
        return L.lowbit_gemm(a["fmt"], a["X"], a["xd"], a["M"], a["K"], a["ldx"], a["W"], a["S"],
                             a["group"], a["N"], a["bias"], a["bd"], a["Y"], a["yd"], a["ldy"],
                             a["act"], a["ws"], a["wsb"], None)

    assert call(fmt=b.BASE3) == b.ERR_DTYPE                   # the GEMM reads INT2 only
    assert call(fmt=7) == b.ERR_DTYPE
    assert call(xd=b.F32) == b.ERR_DTYPE
    assert call(yd=b.NONE) == b.ERR_DTYPE
    assert call(bd=9) == b.ERR_DTYPE
    assert call(act=5) == b.ERR_DTYPE
    assert call(group=64) == b.ERR_GROUP
    assert call(X=None) == b.ERR_NULL
    assert call(W=None) == b.ERR_NULL
    assert call(bd=b.F16) == b.ERR_NULL                       # bias dtype without bias
    assert call(bias=P) == b.ERR_DTYPE                        # bias without dtype
    assert call(K=200, ldx=200) == b.ERR_SHAPE                # K % 128
    assert call(M=0) == b.ERR_SHAPE
    assert call(N=0) == b.ERR_SHAPE
    assert call(ldx=128) == b.ERR_SHAPE                       # ldx < K
    assert call(ldy=32) == b.ERR_SHAPE
    assert call(ldx=1 << 31) == b.ERR_SHAPE                  # ldx >= 2^31
    assert call(ldy=1 << 31) == b.ERR_SHAPE
    # packed weights spanning 4 GiB (32-bit column offsets): N * K / 4 bytes
    assert call(N=1 << 20, ldy=1 << 20, K=1 << 14, ldx=1 << 14) == b.ERR_SHAPE
    assert call(fmt=b.BINARY, N=1 << 20, ldy=1 << 20, K=1 << 15, ldx=1 << 15) == b.ERR_SHAPE
    # M > 16 whose X row chunks under 4 GiB would be 16 rows or fewer
    assert call(M=64, ldx=(1 << 27) + 8) == b.ERR_SHAPE
    assert call(X=P + 8) == b.ERR_ALIGN
    assert call(ldx=260) == b.ERR_ALIGN
    assert call(Y=P + 2, yd=b.F32) == b.ERR_ALIGN
    assert call(S=P + 1) == b.ERR_ALIGN
    assert L.pack_ternary(None, 4, 16, P, None, None) == b.ERR_NULL
    assert L.pack_ternary(P, 4, 24, P, None, None) == b.ERR_SHAPE
    assert L.pack_binary(P + 4, 4, 32, P, None, None) == b.ERR_ALIGN
    assert L.unpack_lowbit(5, P, 4, 32, P, None, None) == b.ERR_DTYPE
    assert L.pack_base3(P, 4, 0, P, None, None) == b.ERR_SHAPE
    assert L.pack_base3(P, 4, 7, None, None, None) == b.ERR_NULL
    assert L.pack_base3(P, 4, 7, P, P + 2, None) == b.ERR_ALIGN   # counter not 4-byte aligned
    assert L.unpack_lowbit(b.BASE3, P, 0, 7, P, None, None) == b.ERR_SHAPE
    assert L.base3_to_int2(None, 4, 32, P, None, None) == b.ERR_NULL
    assert L.base3_to_int2(P, 4, 40, P, None, None) == b.ERR_SHAPE       # INT2 needs K % 16
    assert L.base3_to_int2(P, 4, 32, P + 4, None, None) == b.ERR_ALIGN
    assert L.base3_to_int2(P + 1, 4, 32, P, None, None) == b.ERR_ALIGN
    assert L.lowbit_gelu(None, P, b.BF16, 10, None) == b.ERR_NULL
    # grouped: host arrays of device pointers
    arr = lambda *ptrs: (ctypes.c_void_p * len(ptrs))(*ptrs)

    def grouped(count=2, X=None, W=None, S=None, Y=None, bias=None, bd=b.NONE, fmt=b.TERNARY, M=16):
        X = arr(PX, PX) if X is None else X           # inputs may be shared
        W = arr(PW, PW) if W is None else W
        S = arr(PS, PS) if S is None else S
        Y = arr(PY, PY + (1 << 30)) if Y is None else Y
        return L.lowbit_gemm_grouped(count, fmt, X, b.BF16, M, 256, 256, W, S, 128, 64, bias, bd,
                                     Y, b.BF16, 64, 0, None, 0, None)
    assert grouped(count=0) == b.ERR_SHAPE
    assert grouped(count=9) == b.ERR_SHAPE
    assert grouped(fmt=b.BASE3) == b.ERR_DTYPE
    assert grouped(Y=arr(P, None)) == b.ERR_NULL                 # one problem's output missing
    assert grouped(X=arr(P, P + 8)) == b.ERR_ALIGN               # one problem's X misaligned
    assert grouped(bd=b.F16) == b.ERR_NULL                       # bias dtype without biases
    assert L.lowbit_gemm_grouped(2, b.TERNARY, None, b.BF16, 16, 256, 256, arr(P, P), arr(P, P), 128, 64,
                                 None, b.NONE, arr(P, P), b.BF16, 64, 0, None, 0, None) == b.ERR_NULL
    assert grouped(Y=arr(PY, PY + 64)) == b.ERR_OVERLAP            # two outputs share bytes
    assert grouped(Y=arr(PY, PX)) == b.ERR_OVERLAP                 # an output on an input
    # outputs overlapping inputs, everywhere
    assert call(Y=PX) == b.ERR_OVERLAP
    assert call(Y=PX + 256 * 2 * 15) == b.ERR_OVERLAP             # into X's last row
    assert call(Y=PW + 1024) == b.ERR_OVERLAP
    assert call(Y=PS) == b.ERR_OVERLAP
    assert call(bias=PY + 64, bd=b.F16) == b.ERR_OVERLAP
    assert L.pack_ternary(PX, 4, 16, PX + 32, None, None) == b.ERR_OVERLAP
    assert L.pack_base3(PX, 4, 16, PX + 48, None, None) == b.ERR_OVERLAP
    assert L.unpack_lowbit(b.TERNARY, PX, 4, 16, PX, None, None) == b.ERR_OVERLAP
    assert L.base3_to_int2(PX, 4, 16, PX, None, None) == b.ERR_OVERLAP
    assert L.pack_ternary(PX, 4, 16, PW, PX + 2, None) == b.ERR_ALIGN    # counter checked for alignment first
    assert L.pack_ternary(PX, 4, 16, PW, PX + 16, None) == b.ERR_OVERLAP  # then for overlap
    assert L.lowbit_gelu(PX, PX + 16, b.BF16, 100, None) == b.ERR_OVERLAP
    # a workspace may share no byte with any operand (its declared size is checked)
    for where in (PX, PX + 256 * 2 * 15, PW + 512, PS, PY + 64):
        assert call(ws=where - 256, wsb=512) == b.ERR_OVERLAP, hex(where)
    assert call(ws=PB, wsb=256, bias=PB + 128, bd=b.F32) == b.ERR_OVERLAP
    for z in (0, 1):
        for where in (PX, PW, PS):
            ins = [PX + (1 << 30), PX + (2 << 30)]
            ins[z] = where
            kw = dict(X=arr(*ins)) if where == PX else dict(W=arr(*ins)) if where == PW else dict(S=arr(*ins))
            X = kw.get("X", arr(PX + (1 << 30), PX + (2 << 30)))
            W = kw.get("W", arr(PW, PW))
            S = kw.get("S", arr(PS, PS))
            assert L.lowbit_gemm_grouped(2, b.TERNARY, X, b.BF16, 16, 256, 256, W, S, 128, 64, None, b.NONE,
                                         arr(PY, PY + (1 << 30)), b.BF16, 64, 0, where, 256, None) == b.ERR_OVERLAP
        assert L.lowbit_gemm_grouped(2, b.TERNARY, arr(PX, PX), b.BF16, 16, 256, 256, arr(PW, PW), arr(PS, PS), 128,
                                     64, None, b.NONE, arr(PY, PY + (1 << 30)), b.BF16, 64, 0,
                                     [PY, PY + (1 << 30)][z] + 32, 64, None) == b.ERR_OVERLAP
    assert L.lowbit_gemm_grouped_workspace_bytes(0, b.TERNARY, 16, 64, 256) == 0
    assert L.lowbit_gemm_grouped_workspace_bytes(9, b.TERNARY, 16, 64, 256) == 0
    assert L.lowbit_gelu(P, P, b.NONE, 10, None) == b.ERR_DTYPE


@made_up_addresses
def test_int4_argument_errors_before_any_device_work(L):
    """lowbit_gemm_int4 runs every check of lowbit_gemm, then its own: zero
    points present and aligned, K/2 bytes a packed row, the row-sum
    workspace present, large enough, aligned and apart from every operand."""
    import bit_weight_gemm_int2_amd as b
    P = 1 << 20
    PX, PW, PS, PY, PB, PZ, PWS = (k << 36 for k in range(1, 8))
    need = L.lowbit_gemm_int4_workspace_bytes(16, 64, 256)
    good = dict(X=PX, xd=b.BF16, M=16, K=256, ldx=256, W=PW, S=PS, Z=PZ, group=128, N=64, bias=None, bd=b.NONE,
                Y=PY, yd=b.BF16, ldy=64, act=0, ws=PWS, wsb=need)

    def call(**kw):
        a = dict(good, **kw)
        return L.lowbit_gemm_int4(a["X"], a["xd"], a["M"], a["K"], a["ldx"], a["W"], a["S"], a["Z"], a["group"],
                                  a["N"], a["bias"], a["bd"], a["Y"], a["yd"], a["ldy"], a["act"], a["ws"],
                                  a["wsb"], None)

    assert call(Z=None) == b.ERR_NULL
    assert call(X=None) == b.ERR_NULL
    assert call(xd=b.F32) == b.ERR_DTYPE
    assert call(group=64) == b.ERR_GROUP
    assert call(K=200, ldx=200) == b.ERR_SHAPE
    assert call(M=0) == b.ERR_SHAPE
    # packed 4-bit weights spanning 4 GiB: N * K / 2 bytes (2^20 * 2^13 / 2 = 2^32)
    assert call(N=1 << 20, ldy=1 << 20, K=1 << 13, ldx=1 << 13) == b.ERR_SHAPE
    assert call(Z=PZ + 1) == b.ERR_ALIGN
    assert call(ws=None) == b.ERR_WORKSPACE
    assert call(wsb=need - 4) == b.ERR_WORKSPACE
    assert call(ws=PWS + 16) == b.ERR_ALIGN
    assert call(Y=PW + 64 * 100) == b.ERR_OVERLAP                 # into the second half of the K/2-byte rows
    assert call(Y=PZ) == b.ERR_OVERLAP
    for where in (PX, PW + 64 * 100, PS, PZ, PY + 64):
        assert call(ws=(where & ~255) - 256, wsb=max(need, 512)) == b.ERR_OVERLAP, hex(where)
    assert call(ws=PB, wsb=need, bias=PB + need - 4, bd=b.F32) == b.ERR_OVERLAP
    assert L.pack_int4(None, 4, 16, P, None, None) == b.ERR_NULL
    assert L.pack_int4(P, 4, 12, P << 1, None, None) == b.ERR_SHAPE
    assert L.pack_int4(PX, 4, 16, PX + 16, None, None) == b.ERR_OVERLAP


@made_up_addresses
def test_quantize_argument_errors_before_any_device_work(L):
    """lowbit_quantize: format, NULLs, the K and ldw rules, alignment of each
    pointer and of the row stride, and overlaps between W and each output."""
    import bit_weight_gemm_int2_amd as b
    PW, PP, PS, PC = (k << 36 for k in range(1, 5))
    good = dict(f=b.TERNARY, W=PW, N=64, K=256, ldw=256, P=PP, S=PS, C=PC)

    def call(**kw):
        a = dict(good, **kw)
        return L.lowbit_quantize(a["f"], a["W"], a["N"], a["K"], a["ldw"], a["P"], a["S"], a["C"], None)

    assert call(f=b.BASE3) == b.ERR_DTYPE
    assert call(f=b.INT4) == b.ERR_DTYPE
    assert call(W=None) == b.ERR_NULL
    assert call(P=None) == b.ERR_NULL
    assert call(S=None) == b.ERR_NULL
    assert call(K=192, ldw=192) == b.ERR_SHAPE                   # K % 128
    assert call(K=0, ldw=8) == b.ERR_SHAPE
    assert call(N=0) == b.ERR_SHAPE
    assert call(ldw=128) == b.ERR_SHAPE                          # ldw < K
    assert call(ldw=260) == b.ERR_ALIGN                          # ldw % 8
    assert call(W=PW + 8) == b.ERR_ALIGN
    assert call(P=PP + 4) == b.ERR_ALIGN
    assert call(S=PS + 1) == b.ERR_ALIGN
    assert call(C=PC + 2) == b.ERR_ALIGN
    # W spans (63 * 256 + 256) * 2 = 32 KiB: outputs inside it are refused
    assert call(P=PW + 32768 - 16) == b.ERR_OVERLAP
    assert call(S=PW + 100) == b.ERR_OVERLAP
    assert call(S=PP + 64 * 64 - 2) == b.ERR_OVERLAP             # scales into the packed bytes
    assert call(C=PS + 4) == b.ERR_OVERLAP
    # a wider row stride widens the span W covers
    assert call(ldw=512, P=PW + 40000) == b.ERR_OVERLAP
    # (that an output just past W is accepted is checked only without a GPU,
    # in test_valid_call_without_a_gpu_reports_no_device: with a GPU such a
    # call would launch on these made-up addresses)


def test_variant_hook_names(L):
    """The test hook takes exactly the documented names; an unknown one is
    refused and leaves the setting alone."""
    import bit_weight_gemm_int2_amd as b
    for name in (b"large", b"small", b"large-wide", b"large-pair", b"small-split", b"quant-eighth",
                 b"quant-lane", b"auto", None):
        assert L.lowbit_debug_force_variant(name) == b.OK
    assert L.lowbit_debug_force_variant(b"bogus") == b.ERR_DTYPE
    b.force_variant(None)


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="checks the no-GPU answer")
def test_valid_call_without_a_gpu_reports_no_device(L):
    """Every host check passes, then the device check answers LOWBIT_ERR_DEVICE."""
    import bit_weight_gemm_int2_amd as b
    PX, PW, PS, PY = (k << 36 for k in range(1, 5))
    assert L.lowbit_init() == b.ERR_DEVICE
    assert L.lowbit_gemm(b.TERNARY, PX, b.BF16, 16, 256, 256, PW, PS, 128, 64, None, b.NONE,
                         PY, b.BF16, 64, 0, None, 0, None) == b.ERR_DEVICE
    assert L.pack_ternary(PX, 4, 16, PW, None, None) == b.ERR_DEVICE
    assert L.lowbit_quantize(b.TERNARY, PX, 4, 128, 128, PW, PS, None, None) == b.ERR_DEVICE
    # outputs that start just past W's span (4 rows of 256: 2 KiB) pass the overlap check
    assert L.lowbit_quantize(b.TERNARY, PX, 4, 256, 256, PX + 2048, PX + 2048 + 256, None, None) == b.ERR_DEVICE
    assert L.lowbit_quantize(b.BINARY, PX, 4, 256, 256, PX + 2048, PX + 2048 + 128, None, None) == b.ERR_DEVICE
    assert L.lowbit_gelu(PX, PX, b.BF16, 100, None) == b.ERR_DEVICE     # in place is allowed
    assert L.lowbit_gemm_workspace_bytes(b.TERNARY, 16, 3072, 9216) == 0


C_EXAMPLE = os.path.join(ROOT, "tests", "c", "abi_example.c")


def build_c_example(out_dir):
    """Compile the plain C user of the ABI with gcc against include/ and the
    in-tree library; returns the executable's path."""
    import bit_weight_gemm_int2_amd as b
    exe = os.path.join(out_dir, "abi_example")
    libdir = os.path.dirname(b.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-o", exe, C_EXAMPLE,
           "-L", libdir, "-llowbit", "-L/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_builds_against_the_header(L, tmp_path):
    """The ABI is usable from C alone: a C99 program includes lowbit.h and
    links liblowbit.so with gcc, no C++ and no Python."""
    assert os.path.exists(build_c_example(str(tmp_path)))
