"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes

import pytest

from exact_io_aware_tiled_amd import attn as A

F = 16  # a fake, 16-byte aligned, non-null "device" address; never dereferenced


@pytest.fixture(scope="module")
def lib():
    return A.load_library()


def test_exports_every_declared_function(lib):
    names = A.header_functions()
    assert set(names) == {"attn_fwd", "attn_bwd", "attn_bwd_stage", "attn_bwd_workspace_bytes",
                          "attn_bwd_noalloc",
                          "attn_fwd_dropout", "attn_bwd_dropout", "attn_bwd_dropout_stage",
                          "attn_decode", "attn_decode_stage", "attn_decode_workspace_bytes",
                          "attn_quant_fp8", "attn_fwd_fp8", "attn_quant_fp8_v", "attn_fwd_fp8_pv",
                          "attn_status_string",
                          "attn_last_error", "attn_abi_version"}
    for name in names:
        assert hasattr(lib, name), name
    assert lib.attn_abi_version() == 6


def test_status_strings(lib):
    assert lib.attn_status_string(0) == b"EIAT_OK"
    assert lib.attn_status_string(1) == b"EIAT_ERR_INVALID_ARG"
    assert lib.attn_status_string(2) == b"EIAT_ERR_UNSUPPORTED"
    assert lib.attn_status_string(3) == b"EIAT_ERR_HIP"
    assert lib.attn_status_string(99) == b"EIAT_UNKNOWN_STATUS"


def test_workspace_bytes(lib):
    assert lib.attn_bwd_workspace_bytes(4, 16, 8192) == 4 * 16 * 8192 * 4
    assert lib.attn_bwd_workspace_bytes(0, 16, 8192) == 0


def fwd(lib, q=F, k=F * 2**20, v=F * 2**21, o=F * 2**22, lse=F * 2**23, B=1, H=1, n=64, d=64,
        dv=64, dtype=2, scale=0.125, mask=1, window=0):
    return lib.attn_fwd(q, k, v, o, lse, B, H, n, d, dv, dtype, scale, mask, window, None)


def bwd(lib, ws_bytes=None, **kw):
    args = dict(q=F, k=F * 2**20, v=F * 2**21, o=F * 2**22, do=F * 2**23, lse=F * 2**24,
                dq=F * 2**25, dk=F * 2**26, dv=F * 2**27, ws=F * 2**28, B=1, H=1, n=64, d=64,
                dv_=64, dtype=2, scale=0.125, mask=1, window=0)
    args.update(kw)
    if ws_bytes is None:
        ws_bytes = args["B"] * args["H"] * args["n"] * 4
    return lib.attn_bwd(args["q"], args["k"], args["v"], args["o"], args["do"], args["lse"],
                        args["dq"], args["dk"], args["dv"], args["ws"], ws_bytes, args["B"],
                        args["H"], args["n"], args["d"], args["dv_"], args["dtype"],
                        args["scale"], args["mask"], args["window"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(lse=0), 1), (dict(B=-1), 1), (dict(n=-5), 1), (dict(d=0), 1),
    (dict(dtype=7), 1), (dict(mask=3), 1), (dict(mask=2, window=0), 1),
    (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1), (dict(q=F + 2), 1),
    (dict(o=F), 1),  # output overlaps q
    (dict(d=32, dv=32), 2), (dict(d=64, dv=128), 2), (dict(d=256, dv=256), 2),
    (dict(scale=3e38), 1),  # c * log2(e) overflows float32
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert lib.attn_last_error() != b""


def test_fwd_empty_is_ok_without_gpu(lib):
    # nothing to do: returns before touching pointers or the GPU
    assert fwd(lib, n=0, q=0, k=0, v=0, o=0, lse=0) == 0
    assert fwd(lib, B=0) == 0
    assert lib.attn_last_error() == b""


@pytest.mark.parametrize("kw,code", [
    (dict(ws=0), 1), (dict(do=0), 1), (dict(dv_=16), 2), (dict(mask=2, window=-3), 1),
    (dict(dq=F), 1),  # overlaps q
    (dict(dk=F * 2**25), 1),  # overlaps dq
    (dict(lse=F * 2**24 + 4), 1),  # misaligned
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_bwd_stage_rejects_unknown_stage(lib):
    args = [F, F * 2**20, F * 2**21, F * 2**22, F * 2**23, F * 2**24, F * 2**25, F * 2**26,
            F * 2**27, F * 2**28, 256, 1, 1, 64, 64, 64, 2, 0.125, 1, 0, None]
    assert lib.attn_bwd_stage(3, *args) == 1
    assert lib.attn_bwd_stage(-1, *args) == 1
    assert b"stage" in lib.attn_last_error()
    assert lib.attn_bwd_stage(1, *args[:12], -1, *args[13:]) == 1  # n < 0


def test_bwd_small_workspace(lib):
    assert bwd(lib, ws_bytes=64 * 4 - 1) == 1
    assert b"workspace" in lib.attn_last_error()


def test_python_binding_requires_gpu_tensors():
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.attn_fwd(q, q, q)


def dec(lib, ws_bytes=None, **kw):
    args = dict(q=F, k=F * 2**20, v=F * 2**21, o=F * 2**22, lse=F * 2**23, ws=F * 2**24, B=2, H=8,
                Hkv=2, nq=3, nk=100, d=64, dv=64, dtype=2, scale=0.125, mask=1, window=0)
    args.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_workspace_bytes(args["B"], args["H"], args["Hkv"], args["nq"],
                                                   args["nk"], args["dv"])
    return lib.attn_decode(args["q"], args["k"], args["v"], args["o"], args["lse"], args["ws"],
                           ws_bytes, args["B"], args["H"], args["Hkv"], args["nq"], args["nk"],
                           args["d"], args["dv"], args["dtype"], args["scale"], args["mask"],
                           args["window"], None)


def test_decode_workspace_bytes(lib):
    # units * ranges * rows * (dv + 2) floats; ranges: ~2048 single-wave workgroups in all
    assert lib.attn_decode_workspace_bytes(16, 32, 32, 1, 4096, 128) == 512 * 4 * 1 * 130 * 4
    assert lib.attn_decode_workspace_bytes(1, 32, 8, 1, 65536, 128) == 8 * 256 * 4 * 130 * 4
    assert lib.attn_decode_workspace_bytes(1, 1, 1, 1, 1, 64) == 1 * 1 * 1 * 66 * 4
    assert lib.attn_decode_workspace_bytes(0, 8, 2, 1, 10, 64) == 0
    assert lib.attn_decode_workspace_bytes(1, 6, 4, 1, 10, 64) == 0  # 6 heads do not split over 4


@pytest.mark.parametrize("kw,code", [
    (dict(H=6, Hkv=4), 1), (dict(Hkv=0), 1), (dict(nq=101), 1), (dict(nk=-1), 1),
    (dict(mask=2, window=0), 1), (dict(dtype=5), 1), (dict(scale=float("nan")), 1),
    (dict(q=0), 1), (dict(ws=0), 1), (dict(lse=F * 2**23 + 8), 1),
    (dict(o=F), 1),  # overlaps q
    (dict(ws=F * 2**22), 1),  # overlaps o
    (dict(dtype=0), 2), (dict(d=16, dv=16), 2), (dict(d=128, dv=64), 2),
    (dict(H=64, Hkv=2, nq=2), 2),  # 64 rows per key/value head
])
def test_decode_rejects(lib, kw, code):
    assert dec(lib, **kw) == code
    assert lib.attn_last_error() != b""


def test_decode_small_workspace_and_empty(lib):
    need = lib.attn_decode_workspace_bytes(2, 8, 2, 3, 100, 64)
    assert dec(lib, ws_bytes=need - 1) == 1
    assert b"workspace" in lib.attn_last_error()
    assert dec(lib, B=0, q=0, k=0, v=0, o=0, lse=0, ws=0, ws_bytes=0) == 0
    assert dec(lib, nq=0, ws_bytes=0) == 0


def test_decode_stage_rejects_unknown_stage(lib):
    need = lib.attn_decode_workspace_bytes(2, 8, 2, 3, 100, 64)
    args = [F, F * 2**20, F * 2**21, F * 2**22, F * 2**23, F * 2**24, need, 2, 8, 2, 3, 100, 64,
            64, 2, 0.125, 1, 0, None]
    assert lib.attn_decode_stage(2, *args) == 1
    assert lib.attn_decode_stage(-1, *args) == 1
    assert b"stage" in lib.attn_last_error()


@pytest.mark.parametrize("p", [-0.1, 1.0, 1.5, float("nan"), float("inf")])
def test_dropout_rejects_probability(lib, p):
    args = [F, F * 2**20, F * 2**21, F * 2**22, F * 2**23, 1, 1, 64, 64, 64, 2, 0.125, 1, 0]
    assert lib.attn_fwd_dropout(*args, p, 7, None) == 1
    assert b"p_drop" in lib.attn_last_error()
    bargs = [F, F * 2**20, F * 2**21, F * 2**22, F * 2**23, F * 2**24, F * 2**25, F * 2**26,
             F * 2**27, F * 2**28, 256, 1, 1, 64, 64, 64, 2, 0.125, 1, 0]
    assert lib.attn_bwd_dropout(*bargs, p, 7, None) == 1
    assert lib.attn_bwd_dropout_stage(1, *bargs, p, 7, None) == 1


def test_dropout_checks_shapes_like_base(lib):
    args = [F, F * 2**20, F * 2**21, F * 2**22, F * 2**23, 1, 1, 64, 32, 32, 2, 0.125, 1, 0]
    assert lib.attn_fwd_dropout(*args, 0.1, 7, None) == 2  # d = 32 has no kernel
    args = [F, F * 2**20, F * 2**21, F * 2**22, F * 2**23, 1, 1, 0, 64, 64, 2, 0.125, 1, 0]
    assert lib.attn_fwd_dropout(*args, 0.1, 7, None) == 0  # empty: nothing to do



def quant(lib, x=F, signs=None, codes=F * 2**20, scales=F * 2**21, rows=100, d=64, dtype=2):
    return lib.attn_quant_fp8(x, signs, codes, scales, rows, d, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), 1), (dict(codes=0), 1), (dict(scales=0), 1), (dict(rows=-1), 1), (dict(d=0), 1),
    (dict(dtype=5), 1), (dict(x=F + 4), 1), (dict(signs=F * 2**22 + 8), 1),
    (dict(codes=F), 1),  # codes overlap x
    (dict(scales=F * 2**20 + 16), 1),  # scales overlap codes
    (dict(d=32), 2), (dict(d=256), 2), (dict(d=48), 2),
])
def test_quant_fp8_rejects(lib, kw, code):
    assert quant(lib, **kw) == code
    assert lib.attn_last_error() != b""


def test_quant_fp8_no_rows_is_ok_without_gpu(lib):
    assert quant(lib, rows=0, x=0, codes=0, scales=0) == 0


def fwd8(lib, q=F, qs=F * 2**20, k=F * 2**21, ks=F * 2**22, v=F * 2**23, o=F * 2**24,
         lse=F * 2**25, B=1, H=1, n=64, d=64, dv=64, dtype=2, scale=0.125, mask=1, window=0):
    return lib.attn_fwd_fp8(q, qs, k, ks, v, o, lse, B, H, n, d, dv, dtype, scale, mask, window,
                            None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(qs=0), 1), (dict(ks=0), 1), (dict(B=-1), 1), (dict(mask=4), 1),
    (dict(mask=2, window=0), 1), (dict(scale=float("nan")), 1), (dict(qs=F * 2**20 + 1), 1),
    (dict(o=F * 2**21), 1),  # output overlaps k
    (dict(dtype=0), 2),  # float32 values: no FP8 kernel
    (dict(d=16, dv=16), 2), (dict(d=64, dv=128), 2), (dict(d=32, dv=32), 2),
])
def test_fwd_fp8_rejects(lib, kw, code):
    assert fwd8(lib, **kw) == code
    assert lib.attn_last_error() != b""


def test_fwd_fp8_empty_is_ok_without_gpu(lib):
    assert fwd8(lib, n=0, q=0, qs=0, k=0, ks=0, v=0, o=0, lse=0) == 0


def quantv(lib, v=F, codes=F * 2**20, scales=F * 2**21, BH=2, n=100, dv=64, dtype=2):
    return lib.attn_quant_fp8_v(v, codes, scales, BH, n, dv, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(v=0), 1), (dict(codes=0), 1), (dict(scales=0), 1), (dict(BH=-1), 1), (dict(n=-3), 1),
    (dict(dv=0), 1), (dict(dtype=4), 1), (dict(v=F + 8), 1),
    (dict(codes=F), 1),  # codes overlap v
    (dict(scales=F * 2**20 + 64), 1),  # scales overlap codes
    (dict(dv=32), 2), (dict(dv=96), 2),
])
def test_quant_fp8_v_rejects(lib, kw, code):
    assert quantv(lib, **kw) == code
    assert lib.attn_last_error() != b""


def test_quant_fp8_v_empty_is_ok_without_gpu(lib):
    assert quantv(lib, n=0, v=0, codes=0, scales=0) == 0
    assert quantv(lib, BH=0, v=0, codes=0, scales=0) == 0


def fwd8pv(lib, q=F, qs=F * 2**20, k=F * 2**21, ks=F * 2**22, v=F * 2**23, vs=F * 2**24,
           o=F * 2**25, lse=F * 2**26, B=1, H=1, n=64, d=64, dv=64, dtype=2, scale=0.125, mask=1,
           window=0):
    return lib.attn_fwd_fp8_pv(q, qs, k, ks, v, vs, o, lse, B, H, n, d, dv, dtype, scale, mask,
                               window, None)


@pytest.mark.parametrize("kw,code", [
    (dict(vs=0), 1), (dict(v=0), 1), (dict(q=0), 1), (dict(vs=F * 2**24 + 2), 1),
    (dict(o=F * 2**23 + 1024), 1),  # output overlaps the value codes
    (dict(dtype=0), 2), (dict(d=16, dv=16), 2), (dict(d=64, dv=128), 2),
])
def test_fwd_fp8_pv_rejects(lib, kw, code):
    assert fwd8pv(lib, **kw) == code
    assert lib.attn_last_error() != b""


def bwd_noalloc(lib, **kw):
    args = dict(q=F, k=F * 2**20, v=F * 2**21, o=F * 2**22, do=F * 2**23, lse=F * 2**24,
                dq=F * 2**25, dk=F * 2**26, dv=F * 2**27, B=1, H=1, n=64, d=64, dv_=64, dtype=2,
                scale=0.125, mask=1, window=0)
    args.update(kw)
    return lib.attn_bwd_noalloc(args["q"], args["k"], args["v"], args["o"], args["do"],
                                args["lse"], args["dq"], args["dk"], args["dv"], args["B"],
                                args["H"], args["n"], args["d"], args["dv_"], args["dtype"],
                                args["scale"], args["mask"], args["window"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(dk=0), 1), (dict(B=-1), 1), (dict(mask=2, window=0), 1),
    (dict(dq=F), 1),  # output overlaps q
    (dict(d=32, dv_=32), 2),
    # beyond the scratch: B * H * n > 4,194,304 rows, rejected before any HIP call
    (dict(B=2, H=32, n=65537), 2), (dict(B=1, H=1, n=(1 << 22) + 1), 2),
])
def test_bwd_noalloc_rejects(lib, kw, code):
    assert bwd_noalloc(lib, **kw) == code
    assert lib.attn_last_error() != b""


def test_bwd_noalloc_limit_message_and_empty(lib):
    assert bwd_noalloc(lib, B=4, H=16, n=65536 + 1) == 2
    assert b"no-allocation scratch" in lib.attn_last_error()
    assert bwd_noalloc(lib, n=0, q=0, k=0) == 0  # nothing to do, no GPU touched
