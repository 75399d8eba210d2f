"""Python binding of the C ABI in include/eiat_attn.h (argument marshalling only).

``attn_fwd`` and ``attn_bwd`` carry the C entry points' names.  PyTorch supplies
device memory and the stream; every step of the computation runs in the HIP
kernels of ``libeiat_attn.so``.  There is no fallback: if the library is not
built, or the tensors are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libeiat_attn.so")
HEADER = os.path.join(ROOT, "include", "eiat_attn.h")

DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
MASK_CODES = {"none": 0, "causal": 1, "window": 2}
STATUS = {0: "EIAT_OK", 1: "EIAT_ERR_INVALID_ARG", 2: "EIAT_ERR_UNSUPPORTED", 3: "EIAT_ERR_HIP"}


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def header_functions() -> list[str]:
    """Names of the functions declared in include/eiat_attn.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"EIAT_API[^;(]*?\b(attn_[a-z0-9_]+)\s*\(", text)


def load_library():
    """Load libeiat_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def load_check_library(name: str):
    """One of the check builds (``poison``, ``alt`` or ``timing``, see
    build.CHECK_BUILDS): the same C ABI compiled with a checking macro, for
    tests and the workgroup timeline only."""
    return _open(os.path.join(HERE, f"libeiat_attn_{name}.so"))


def _open(path: str):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python exact_io_aware_tiled_amd/build.py`")
    lib = ctypes.CDLL(path, mode=os.RTLD_LOCAL)
    vp, i64, c_int, c_float = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, c_int, c_float, c_int,
                             i64, vp]
    lib.attn_fwd.restype = c_int
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64,
                             i64, i64, i64, c_int, c_float, c_int, i64, vp]
    lib.attn_bwd.restype = c_int
    lib.attn_bwd_noalloc.argtypes = [vp] * 9 + [i64, i64, i64, i64, i64, c_int, c_float, c_int,
                                                i64, vp]
    lib.attn_bwd_noalloc.restype = c_int
    lib.attn_bwd_stage.argtypes = [c_int] + lib.attn_bwd.argtypes
    lib.attn_bwd_stage.restype = c_int
    lib.attn_fwd_dropout.argtypes = lib.attn_fwd.argtypes[:-1] + [c_float, ctypes.c_uint64, vp]
    lib.attn_fwd_dropout.restype = c_int
    lib.attn_bwd_dropout.argtypes = lib.attn_bwd.argtypes[:-1] + [c_float, ctypes.c_uint64, vp]
    lib.attn_bwd_dropout.restype = c_int
    lib.attn_bwd_dropout_stage.argtypes = [c_int] + lib.attn_bwd_dropout.argtypes
    lib.attn_bwd_dropout_stage.restype = c_int
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, i64,
                                i64, i64, c_int, c_float, c_int, i64, vp]
    lib.attn_decode.restype = c_int
    lib.attn_decode_stage.argtypes = [c_int] + lib.attn_decode.argtypes
    lib.attn_decode_stage.restype = c_int
    lib.attn_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    u8p = ctypes.c_void_p
    lib.attn_quant_fp8.argtypes = [vp, vp, u8p, u8p, i64, i64, c_int, vp]
    lib.attn_quant_fp8.restype = c_int
    lib.attn_fwd_fp8.argtypes = [u8p, u8p, u8p, u8p, vp, vp, vp, i64, i64, i64, i64, i64, c_int,
                                 c_float, c_int, i64, vp]
    lib.attn_fwd_fp8.restype = c_int
    lib.attn_quant_fp8_v.argtypes = [vp, u8p, u8p, i64, i64, i64, c_int, vp]
    lib.attn_quant_fp8_v.restype = c_int
    lib.attn_fwd_fp8_pv.argtypes = [u8p, u8p, u8p, u8p, u8p, u8p, vp, vp, i64, i64, i64, i64, i64,
                                    c_int, c_float, c_int, i64, vp]
    lib.attn_fwd_fp8_pv.restype = c_int
    lib.attn_status_string.argtypes = [c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = c_int
    return lib


def _check(status: int):
    if status != 0:
        raise AttnError(status, load_library().attn_last_error().decode())


def _stream_handle(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dims(q: torch.Tensor, v: torch.Tensor):
    if not isinstance(q, torch.Tensor) or not isinstance(v, torch.Tensor) or q.dim() != 4 \
            or v.dim() != 4:
        raise ValueError("expected [B, H, n, d] tensors")
    B, H, n, d = q.shape
    return B, H, n, d, v.shape[-1]


def _validate(specs):
    """Check every tensor a call hands to the library, outputs included, before
    any launch: ``specs`` is a list of (name, tensor, shape, dtype), where shape
    is a tuple (or None to skip) and dtype a torch dtype, a tuple of allowed
    dtypes, or None.  Shapes and dtypes are checked first, then contiguity,
    then that every tensor sits on the same GPU; the first mismatch raises
    ValueError.  The C ABI receives raw pointers and the sizes derived from
    the inputs, so a short or mistyped buffer here would otherwise become
    out-of-bounds device accesses."""
    for name, t, shape, dtype in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None:
            allowed = dtype if isinstance(dtype, tuple) else (dtype,)
            if t.dtype not in allowed:
                raise ValueError(f"{name} has dtype {t.dtype}, expected "
                                 + " or ".join(str(a) for a in allowed))
    for name, t, _, _ in specs:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dev = None
    for name, t, _, _ in specs:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


FLOAT_TYPES = tuple(DTYPE_CODES)
HALF_TYPES = (torch.float16, torch.bfloat16)


def _float_dtype(t: torch.Tensor, name: str, allowed=FLOAT_TYPES):
    if t.dtype not in allowed:
        raise ValueError(f"{name} has dtype {t.dtype}, expected "
                         + " or ".join(str(a) for a in allowed))
    return t.dtype


def _workspace(ws, name="workspace"):
    if not isinstance(ws, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    return (name, ws, None, None)


def attn_fwd(q, k, v, scale: Optional[float] = None, mask: str = "causal", window: int = 0,
             out=None, lse=None, stream=None, p_drop: float = 0.0, seed: int = 0):
    """O, LSE = attention forward.  q, k: [B, H, n, d]; v: [B, H, n, dv] (same dtype).

    p_drop > 0 applies dropout to the weights (attn_fwd_dropout; mask keyed on seed)."""
    lib = load_library()
    B, H, n, d, dv = _dims(q, v)
    dt = _float_dtype(q, "q")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty(B, H, n, dv, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, n, dtype=torch.float32, device=q.device)
    _validate([("q", q, (B, H, n, d), dt), ("k", k, (B, H, n, d), dt), ("v", v, (B, H, n, dv), dt),
               ("out", out, (B, H, n, dv), dt), ("lse", lse, (B, H, n), torch.float32)])
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, n, d,
            dv, DTYPE_CODES[q.dtype], float(scale), MASK_CODES[mask], int(window))
    if p_drop:
        _check(lib.attn_fwd_dropout(*args, float(p_drop), int(seed), _stream_handle(stream)))
    else:
        _check(lib.attn_fwd(*args, _stream_handle(stream)))
    return out, lse


def attn_quant_fp8(x, signs=None, codes=None, scales=None, stream=None):
    """(codes, scales) of rows x [..., d] (attn_quant_fp8): uint8 e4m3 codes
    [..., d] and E8M0 scale bytes [..., d / 32]; ``signs`` (int8 [d] of +-1 on
    the GPU) rotates the rows as H (signs * x) first."""
    lib = load_library()
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise ValueError("x must be a tensor of rows [..., d]")
    _float_dtype(x, "x")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device)
    specs = [("x", x, None, None), ("codes", codes, tuple(x.shape), torch.uint8),
             ("scales", scales, tuple(x.shape[:-1]) + (d // 32,), torch.uint8)]
    if signs is not None:
        specs.append(("signs", signs, (d,), torch.int8))
    _validate(specs)
    _check(lib.attn_quant_fp8(x.data_ptr(), None if signs is None else signs.data_ptr(),
                              codes.data_ptr(), scales.data_ptr(), rows, d, DTYPE_CODES[x.dtype],
                              _stream_handle(stream)))
    return codes, scales


def attn_fwd_fp8(q, q_scale, k, k_scale, v, scale: float, mask: str = "causal", window: int = 0,
                 out=None, lse=None, stream=None):
    """O, LSE with FP8 scores (attn_fwd_fp8).  q, k: uint8 e4m3 codes [B, H, n, d];
    q_scale, k_scale: uint8 [B, H, n, d / 32]; v: [B, H, n, dv] f16/bf16.  ``scale``
    multiplies the dequantized products (c / d for rows rotated by attn_quant_fp8)."""
    lib = load_library()
    B, H, n, d, dv = _dims(q, v)
    dt = _float_dtype(v, "v", HALF_TYPES)
    u8 = torch.uint8
    if out is None:
        out = torch.empty(B, H, n, dv, dtype=v.dtype, device=v.device)
    if lse is None:
        lse = torch.empty(B, H, n, dtype=torch.float32, device=v.device)
    _validate([("q", q, (B, H, n, d), u8), ("q_scale", q_scale, (B, H, n, d // 32), u8),
               ("k", k, (B, H, n, d), u8), ("k_scale", k_scale, (B, H, n, d // 32), u8),
               ("v", v, (B, H, n, dv), dt), ("out", out, (B, H, n, dv), dt),
               ("lse", lse, (B, H, n), torch.float32)])
    _check(lib.attn_fwd_fp8(q.data_ptr(), q_scale.data_ptr(), k.data_ptr(), k_scale.data_ptr(),
                            v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, n, d, dv,
                            DTYPE_CODES[v.dtype], float(scale), MASK_CODES[mask], int(window),
                            _stream_handle(stream)))
    return out, lse


def attn_quant_fp8_v(v, codes=None, scales=None, stream=None):
    """(codes, scales) of values v [B, H, n, dv] quantized along the keys
    (attn_quant_fp8_v): uint8 [B, H, nt, dv, 64] and [B, H, nt, dv, 2], nt =
    ceil(n / 64), in the tile-major key order the FP8 value product reads."""
    lib = load_library()
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("expected v of shape [B, H, n, dv]")
    _float_dtype(v, "v")
    B, H, n, dv = v.shape
    nt = (n + 63) // 64
    if codes is None:
        codes = torch.empty(B, H, nt, dv, 64, dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.empty(B, H, nt, dv, 2, dtype=torch.uint8, device=v.device)
    _validate([("v", v, None, None), ("codes", codes, (B, H, nt, dv, 64), torch.uint8),
               ("scales", scales, (B, H, nt, dv, 2), torch.uint8)])
    _check(lib.attn_quant_fp8_v(v.data_ptr(), codes.data_ptr(), scales.data_ptr(), B * H, n, dv,
                                DTYPE_CODES[v.dtype], _stream_handle(stream)))
    return codes, scales


def attn_fwd_fp8_pv(q, q_scale, k, k_scale, v, v_scale, scale: float, mask: str = "causal",
                    window: int = 0, out=None, lse=None, dtype=torch.bfloat16, stream=None):
    """O, LSE with FP8 scores and FP8 weights/values (attn_fwd_fp8_pv): q, k,
    q_scale, k_scale as attn_fwd_fp8; v, v_scale from attn_quant_fp8_v; O in
    ``dtype`` (float16 or bfloat16)."""
    lib = load_library()
    if (not isinstance(q, torch.Tensor) or not isinstance(v, torch.Tensor) or q.dim() != 4
            or v.dim() != 5):
        raise ValueError("expected q [B, H, n, d] and v [B, H, nt, dv, 64]")
    B, H, n, d = q.shape
    dv = v.shape[-2]
    nt = (n + 63) // 64
    u8 = torch.uint8
    if out is None:
        if dtype not in HALF_TYPES:
            raise ValueError(f"dtype {dtype} must be float16 or bfloat16")
        out = torch.empty(B, H, n, dv, dtype=dtype, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, n, dtype=torch.float32, device=q.device)
    _validate([("q", q, (B, H, n, d), u8), ("q_scale", q_scale, (B, H, n, d // 32), u8),
               ("k", k, (B, H, n, d), u8), ("k_scale", k_scale, (B, H, n, d // 32), u8),
               ("v", v, (B, H, nt, dv, 64), u8), ("v_scale", v_scale, (B, H, nt, dv, 2), u8),
               ("out", out, (B, H, n, dv), HALF_TYPES), ("lse", lse, (B, H, n), torch.float32)])
    _check(lib.attn_fwd_fp8_pv(q.data_ptr(), q_scale.data_ptr(), k.data_ptr(), k_scale.data_ptr(),
                               v.data_ptr(), v_scale.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                               H, n, d, dv, DTYPE_CODES[out.dtype], float(scale), MASK_CODES[mask],
                               int(window), _stream_handle(stream)))
    return out, lse


def attn_bwd_workspace_bytes(B: int, H: int, n: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, H, n))


def attn_bwd(q, k, v, o, lse, do, scale: Optional[float] = None, mask: str = "causal",
             window: int = 0, dq=None, dk=None, dv=None, workspace=None, stream=None,
             stage: Optional[int] = None, p_drop: float = 0.0, seed: int = 0):
    """dQ, dK, dV of sum(dO * O) given the forward's O and LSE.

    stage=None runs attn_bwd (dQ with delta, then dK and dV); stage 0, 1 or 2
    runs attn_bwd_stage (delta into `workspace`; dK and dV, reading delta; dQ,
    also writing delta) -- pass the same workspace to all.
    p_drop > 0 replays the dropout of attn_fwd(..., p_drop, seed) (same values).
    """
    lib = load_library()
    B, H, n, d, dvd = _dims(q, v)
    dt = _float_dtype(q, "q")
    qs, vs = (B, H, n, d), (B, H, n, dvd)
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = attn_bwd_workspace_bytes(B, H, n)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    _validate([("q", q, qs, dt), ("k", k, qs, dt), ("v", v, vs, dt), ("o", o, vs, dt),
               ("lse", lse, (B, H, n), torch.float32), ("do", do, vs, dt),
               ("dq", dq, qs, dt), ("dk", dk, qs, dt), ("dv", dv, vs, dt), _workspace(workspace)])
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), B, H, n, d, dvd, DTYPE_CODES[q.dtype],
            float(scale), MASK_CODES[mask], int(window))
    sh = _stream_handle(stream)
    if p_drop:
        extra = (float(p_drop), int(seed), sh)
        if stage is None:
            _check(lib.attn_bwd_dropout(*args, *extra))
        else:
            _check(lib.attn_bwd_dropout_stage(int(stage), *args, *extra))
    elif stage is None:
        _check(lib.attn_bwd(*args, sh))
    else:
        _check(lib.attn_bwd_stage(int(stage), *args, sh))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale: Optional[float] = None,
                     mask: str = "causal", window: int = 0, stream=None):
    """attn_bwd_noalloc: dQ, dK, dV into the caller's dq, dk, dv, with the
    per-row delta in the library's own per-GPU scratch (no workspace, nothing
    allocated by this call; B * H * n up to 4,194,304 rows).  Calls that
    overlap on one GPU race on that scratch."""
    lib = load_library()
    B, H, n, d, dvd = _dims(q, v)
    dt = _float_dtype(q, "q")
    qs, vs = (B, H, n, d), (B, H, n, dvd)
    _validate([("q", q, qs, dt), ("k", k, qs, dt), ("v", v, vs, dt), ("o", o, vs, dt),
               ("lse", lse, (B, H, n), torch.float32), ("do", do, vs, dt),
               ("dq", dq, qs, dt), ("dk", dk, qs, dt), ("dv", dv, vs, dt)])
    if scale is None:
        scale = d ** -0.5
    _check(lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), B, H, n, d, dvd, DTYPE_CODES[q.dtype], float(scale),
                                MASK_CODES[mask], int(window), _stream_handle(stream)))
    return dq, dk, dv


def attn_decode_workspace_bytes(B: int, H: int, Hkv: int, nq: int, nk: int, dv: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, H, Hkv, nq, nk, dv))


def attn_decode(q, k, v, scale: Optional[float] = None, mask: str = "none", window: int = 0,
                out=None, lse=None, workspace=None, stream=None, stage: Optional[int] = None):
    """O, LSE for nq new rows against a key/value cache.

    q: [B, H, nq, d] (the last nq positions); k: [B, Hkv, nk, d]; v: [B, Hkv, nk, dv];
    H a multiple of Hkv (query head h reads key/value head h // (H // Hkv)).
    stage=None runs attn_decode; stage 0 / 1 runs attn_decode_stage (range
    summaries into `workspace`; their merge into out, lse) -- pass the same workspace.
    """
    lib = load_library()
    if any(not isinstance(t, torch.Tensor) or t.dim() != 4 for t in (q, k, v)):
        raise ValueError("q, k, v must be 4-d tensors")
    B, H, nq, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    dv = v.shape[-1]
    dt = _float_dtype(q, "q")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty(B, H, nq, dv, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, nq, dtype=torch.float32, device=q.device)
    ws_bytes = attn_decode_workspace_bytes(B, H, Hkv, nq, nk, dv)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    _validate([("q", q, (B, H, nq, d), dt), ("k", k, (B, Hkv, nk, d), dt),
               ("v", v, (B, Hkv, nk, dv), dt), ("out", out, (B, H, nq, dv), dt),
               ("lse", lse, (B, H, nq), torch.float32), _workspace(workspace)])
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), B, H, Hkv, nq, nk,
            d, dv, DTYPE_CODES[q.dtype], float(scale), MASK_CODES[mask], int(window),
            _stream_handle(stream))
    if stage is None:
        _check(lib.attn_decode(*args))
    else:
        _check(lib.attn_decode_stage(int(stage), *args))
    return out, lse
