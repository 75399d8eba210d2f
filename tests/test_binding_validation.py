"""The Python binding checks every tensor it hands to the C ABI (inputs and
outputs: shape, dtype, contiguity, device) and raises ValueError before any
launch.  These run on CPU tensors: every check before the device check is
reached without a GPU, and a fully consistent set of CPU tensors is refused
for its device."""
import pytest
import torch

from exact_io_aware_tiled_amd import attn as A

B, H, n, d = 1, 2, 8, 64
bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def qkv():
    return t(B, H, n, d), t(B, H, n, d), t(B, H, n, d)


@pytest.mark.parametrize("case,msg", [
    ("k_short", "k has shape"),
    ("v_rows", "v has shape"),
    ("k_dtype", "k has dtype"),
    ("out_short", "out has shape"),
    ("out_dtype", "out has dtype"),
    ("lse_dtype", "lse has dtype"),
    ("lse_shape", "lse has shape"),
    ("out_noncontig", "out must be contiguous"),
    ("q_int", "q has dtype"),
    ("cpu", "must be a GPU tensor"),
])
def test_fwd_validation(case, msg):
    q, k, v = qkv()
    kw = {}
    if case == "k_short":
        k = t(B, H, n - 1, d)
    elif case == "v_rows":
        v = t(B, H, n + 1, d)
    elif case == "k_dtype":
        k = t(B, H, n, d, dtype=torch.float16)
    elif case == "out_short":
        kw["out"] = t(B, H, n - 1, d)
    elif case == "out_dtype":
        kw["out"] = t(B, H, n, d, dtype=torch.float32)
    elif case == "lse_dtype":
        kw["lse"] = t(B, H, n, dtype=bf)
    elif case == "lse_shape":
        kw["lse"] = t(B, H, n - 1, dtype=torch.float32)
    elif case == "out_noncontig":
        kw["out"] = t(B, H, d, n).transpose(2, 3)
    elif case == "q_int":
        q = t(B, H, n, d, dtype=torch.int32)
    with pytest.raises(ValueError, match=msg):
        A.attn_fwd(q, k, v, **kw)


@pytest.mark.parametrize("name", ["k", "v", "o", "do", "dq", "dk", "dv"])
def test_bwd_validation_shapes(name):
    q, k, v = qkv()
    ts = {"q": q, "k": k, "v": v, "o": t(B, H, n, d), "do": t(B, H, n, d),
          "lse": t(B, H, n, dtype=torch.float32)}
    kw = {}
    short = t(B, H, n - 1, d)
    if name in ("dq", "dk", "dv"):
        kw[name] = short
    else:
        ts[name] = short
    with pytest.raises(ValueError, match=f"{name} has shape"):
        A.attn_bwd(ts["q"], ts["k"], ts["v"], ts["o"], ts["lse"], ts["do"], **kw)


def test_bwd_validation_lse_and_device():
    q, k, v = qkv()
    o, do = t(B, H, n, d), t(B, H, n, d)
    with pytest.raises(ValueError, match="lse has dtype"):
        A.attn_bwd(q, k, v, o, t(B, H, n, dtype=bf), do)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        A.attn_bwd(q, k, v, o, t(B, H, n, dtype=torch.float32), do)


def test_decode_validation():
    q = t(2, 8, 3, d)
    k = t(2, 2, 100, d)
    v = t(2, 2, 100, d)
    with pytest.raises(ValueError, match="k has shape"):
        A.attn_decode(q, t(2, 2, 100, 32), v)
    with pytest.raises(ValueError, match="v has shape"):
        A.attn_decode(q, k, t(2, 2, 99, d))
    with pytest.raises(ValueError, match="out has shape"):
        A.attn_decode(q, k, v, out=t(2, 8, 2, d))
    with pytest.raises(ValueError, match="lse has dtype"):
        A.attn_decode(q, k, v, lse=t(2, 8, 3, dtype=bf))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        A.attn_decode(q, k, v)


def test_fp8_validation():
    u8 = torch.uint8
    q8, k8 = t(B, H, n, d, dtype=u8), t(B, H, n, d, dtype=u8)
    qs, ks = t(B, H, n, d // 32, dtype=u8), t(B, H, n, d // 32, dtype=u8)
    v = t(B, H, n, d)
    with pytest.raises(ValueError, match="k_scale has shape"):
        A.attn_fwd_fp8(q8, qs, k8, t(B, H, n, 1, dtype=u8), v, 0.1)
    with pytest.raises(ValueError, match="q has dtype"):
        A.attn_fwd_fp8(t(B, H, n, d), qs, k8, ks, v, 0.1)
    with pytest.raises(ValueError, match="v has dtype"):
        A.attn_fwd_fp8(q8, qs, k8, ks, t(B, H, n, d, dtype=torch.float32), 0.1)
    with pytest.raises(ValueError, match="codes has shape"):
        A.attn_quant_fp8(v, codes=t(B, H, n, d - 1, dtype=u8))
    with pytest.raises(ValueError, match="signs has dtype"):
        A.attn_quant_fp8(v, signs=t(d, dtype=torch.int32))
    nt = 1
    v8, vsc = t(B, H, nt, d, 64, dtype=u8), t(B, H, nt, d, 2, dtype=u8)
    with pytest.raises(ValueError, match="v_scale has shape"):
        A.attn_fwd_fp8_pv(q8, qs, k8, ks, v8, t(B, H, nt, d, 1, dtype=u8), 0.1)
    with pytest.raises(ValueError, match="scales has shape"):
        A.attn_quant_fp8_v(v, scales=t(B, H, nt, d, 1, dtype=u8))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        A.attn_fwd_fp8_pv(q8, qs, k8, ks, v8, vsc, 0.1)
