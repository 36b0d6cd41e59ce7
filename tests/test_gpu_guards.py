"""Guard bands: every launch path writes exactly its output and nothing
around it. Y sits inside a larger buffer, with its rows padded (ldy > N); the
guard regions before and after it and the padding are filled with a NaN
pattern that no output can take, and must keep their bits; Y itself is
pre-filled with that pattern too, so an element left unwritten shows up. The
workspace is followed by sentinel bytes that must stay untouched as well.
The packers and the base-3 transcoder are checked the same way."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import TORCH_DT, banner, dev_bits, dev_weights, oracle_linear, to_host64

pytestmark = pytest.mark.gpu

GUARD = 4096                   # elements before and after Y
SENTINEL = {"bf16": 0x7FA5, "f16": 0x7E5A, "f32": 0x7FC0A5A5}


@pytest.fixture(scope="module")
def lb():
    import bit_weight_gemm_int2_amd as b
    b.lib()
    return b


def _guarded_out(M, N, pad, yd):
    """(whole buffer, Y view [M, N] with row stride N + pad, ldy); the
    sentinels are positive in the signed type, so torch.full takes them."""
    ldy = N + pad
    it = torch.int32 if yd == "f32" else torch.int16
    raw = torch.full((2 * GUARD + M * ldy,), SENTINEL[yd], dtype=it, device="cuda")
    y = raw[GUARD:GUARD + M * ldy].view(M, ldy).view(TORCH_DT[yd])[:, :N]
    return raw, y, ldy


def _check_guards(raw, M, N, ldy, yd):
    h = raw.cpu().numpy().view(np.uint32 if yd == "f32" else np.uint16)
    s = SENTINEL[yd]
    assert (h[:GUARD] == s).all(), "guard before Y written"
    assert (h[GUARD + M * ldy:] == s).all(), "guard after Y written"
    body = h[GUARD:GUARD + M * ldy].reshape(M, ldy)
    assert (body[:, N:] == s).all(), "row padding written"
    assert not (body[:, :N] == s).any(), "an output element left unwritten"


CASES = [  # (forced variant, fmt, M, N, K, y dtype, row padding)
    (None, "ternary", 13, 1001, 1152, "bf16", 7),         # thin, ragged N
    (None, "binary", 1, 33, 128, "f32", 3),               # thin, one group, one row
    ("small-split", "ternary", 16, 4100, 9216, "bf16", 8),  # column tiles, K split across workgroups
    (None, "binary", 9, 9000, 3072, "f16", 5),            # column tiles
    ("large-pair", "ternary", 257, 1030, 1152, "bf16", 2),  # large M, 16-byte stores through LDS (ldy % 8 == 0)
    ("large-wide", "binary", 130, 2100, 384, "bf16", 3),  # large M, element stores (ldy % 8 != 0)
    ("large-wide", "ternary", 100, 300, 1024, "f32", 4),  # large M, narrow wide tiles, f32
]


@pytest.mark.parametrize("variant,fmt,M,N,K,yd,pad", CASES)
def test_gemm_writes_only_its_output(lb, variant, fmt, M, N, K, yd, pad):
    banner(f"guards {variant} {fmt} {M}x{N}x{K} -> {yd}")
    if variant:
        lb.force_variant(variant)
    else:
        lb.force_variant(None)
    try:
        lin = wl.make_linear("guard", fmt, M, N, K, seed=950 + M, p0=0.35, with_bias=True)
        x = dev_bits(lin.x, "bf16")
        packed, s = dev_weights(fmt, lin.codes, lin.scales)
        b = torch.from_numpy(lin.bias.view(np.int16)).cuda().view(torch.float16)
        need = lb.workspace_bytes(fmt, M, N, K)
        if variant == "small-split":
            assert need > 0
        ws = torch.zeros(need + 65536, dtype=torch.uint8, device="cuda")
        ws[need:] = 0xA5
        raw, y, ldy = _guarded_out(M, N, pad, yd)
        lb.gemm(x, packed, s, fmt, bias=b, out=y, workspace=ws[:need] if need else None)
        torch.cuda.synchronize()
        _check_guards(raw, M, N, ldy, yd)
        assert int((ws[need:] != 0xA5).sum()) == 0, "bytes past the workspace written"
        A, Mg = oracle_linear(lin)
        ok, worst, nfail = oracle.check(to_host64(y.contiguous()), A, Mg, yd)
        assert ok, f"{nfail} outside the bound"
    finally:
        lb.force_variant(None)


def test_grouped_writes_only_its_outputs(lb):
    banner("guards grouped")
    count, M, N, K, yd, pad = 3, 16, 2000, 9216, "bf16", 8
    lins = [wl.make_linear(f"gg{z}", "ternary", M, N, K, seed=960 + z, p0=0.35) for z in range(count)]
    xs = [dev_bits(l.x, "bf16") for l in lins]
    ws_ = [dev_weights("ternary", l.codes, l.scales) for l in lins]
    outs = [_guarded_out(M, N, pad, yd) for _ in range(count)]
    need = int(lb.lib().lowbit_gemm_grouped_workspace_bytes(count, lb.TERNARY, M, N, K))
    wsp = torch.zeros(need + 65536, dtype=torch.uint8, device="cuda")
    wsp[need:] = 0xA5
    lb.gemm_grouped(xs, [w[0] for w in ws_], [w[1] for w in ws_], "ternary", outs=[o[1] for o in outs],
                    workspace=wsp[:need] if need else None)
    torch.cuda.synchronize()
    for (raw, y, ldy), l in zip(outs, lins):
        _check_guards(raw, M, N, ldy, yd)
        A, Mg = oracle_linear(l)
        assert oracle.check(to_host64(y.contiguous()), A, Mg, yd)[0]
    assert int((wsp[need:] != 0xA5).sum()) == 0, "bytes past the workspace written"


@pytest.mark.parametrize("what", ["pack_ternary", "pack_binary", "pack_base3", "base3_to_int2"])
def test_packers_write_only_their_output(lb, what):
    banner(f"guards {what}")
    N, K = 37, 1008 if what != "pack_binary" else 1024
    g = wl.generator(970)
    t = wl.binary_codes(g, N, K) if what == "pack_binary" else wl.ternary_codes(g, N, K, 0.35)
    L = lb.lib()
    if what == "base3_to_int2":
        src = torch.from_numpy(oracle.pack_base3(t)).cuda()
        nbytes = N * K // 4
        ref = oracle.pack_ternary(t)
    else:
        src = torch.from_numpy(t).cuda()
        fmt = {"pack_ternary": lb.TERNARY, "pack_binary": lb.BINARY, "pack_base3": lb.BASE3}[what]
        nbytes = int(L.lowbit_packed_bytes(fmt, N, K))
        ref = {"pack_ternary": oracle.pack_ternary, "pack_binary": oracle.pack_binary,
               "pack_base3": oracle.pack_base3}[what](t)
    raw = torch.full((nbytes + 2 * GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = raw[GUARD:GUARD + nbytes]
    st = torch.cuda.current_stream().cuda_stream
    assert getattr(L, what)(src.data_ptr(), N, K, dst.data_ptr(), None, st) == 0
    torch.cuda.synchronize()
    h = raw.cpu().numpy()
    assert (h[:GUARD] == 0xA5).all() and (h[GUARD + nbytes:] == 0xA5).all()
    assert np.array_equal(h[GUARD:GUARD + nbytes], ref.reshape(-1))
