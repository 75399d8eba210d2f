"""fp64 CPU oracle for exact masked row-softmax attention (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  It wraps ``oracle.c`` (plain C, IEEE double, OpenMP
over rows) through ctypes and shares no code with the HIP library.

What each function follows (page title, then the named item on it):

* ``fwd``        -- alphabetamath, "Exact tiled attention and memory-aware
  differentiation", Theorem "Tiled attention and its recomputed reverse pass
  are exact": the dense masked attention row, max-shifted as in proof step 2.1.
* ``bwd``        -- the same page, Algorithm "Exact tiled softmax attention with
  block-recomputed vector-Jacobian products", reverse procedure, written per
  output element as in proof steps 4.1-6.1.
* ``summary`` / ``merge`` -- the same page, Definition "Stable summary of an
  attention key block" (the summary and its merge).
* ``fwd_tiled``  -- the Algorithm's forward procedure with key-block size b.
  ``broken=True`` plants the mistake of Night School "Fused attention",
  section "Forget one step" (no shrink of the running total).
* ``mx_quant`` / ``mx_dequant`` / ``e4m3_*`` / ``fwht_f32`` -- webturing.com.tr
  Principia, "Bellek Duvarinin Fizigi", section on FlashAttention-3: FP8
  scores with block scaling and incoherent processing (random sign
  multipliers); the block layout and code format are those of the OCP
  microscaling FP8 (e4m3) format.

Inputs are numpy arrays (any float dtype; converted to float64, which is exact
for fp16/bf16/fp32 values), shaped ``[..., n, d]`` with leading dims flattened
into independent heads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MASKS = {"none": 0, "causal": 1, "window": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, baseline x86-64: no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, dbl, ip = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_fwd.argtypes = [i64, i64, i64, i64, ip, ip, ip, dbl, ctypes.c_int, i64, ip,
                                   i64, ip, ip, ip, ip]
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [i64, i64, i64, i64, ip, ip, ip, ip, dbl, ctypes.c_int, i64,
                                   ip, ip, ip, ip, ip, ip]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_summary.argtypes = [i64, i64, ip, ip, ip, ip, ip]
        lib.oracle_summary.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [i64, dbl, dbl, ip, dbl, dbl, ip, ctypes.c_int, ip, ip, ip]
        lib.oracle_merge.restype = ctypes.c_int
        lib.oracle_fwd_tiled.argtypes = [i64, i64, i64, i64, ip, ip, ip, dbl, ctypes.c_int, i64,
                                         i64, ctypes.c_int, ip, ip, ip]
        lib.oracle_fwd_tiled.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [i64, i64, i64, i64, i64, i64, i64, ip, ip, ip, dbl,
                                      ctypes.c_int, i64, ip, ip]
        lib.oracle_decode.restype = ctypes.c_int
        u64 = ctypes.c_uint64
        lib.oracle_fwd_drop.argtypes = [i64, i64, i64, i64, ip, ip, ip, dbl, ctypes.c_int, i64,
                                        u64, ctypes.c_int, i64, ip, ip]
        lib.oracle_fwd_drop.restype = ctypes.c_int
        lib.oracle_bwd_drop.argtypes = [i64, i64, i64, i64, ip, ip, ip, ip, dbl, ctypes.c_int,
                                        i64, u64, ctypes.c_int, i64, ip, ip, ip, ip, ip, ip]
        lib.oracle_bwd_drop.restype = ctypes.c_int
        lib.oracle_dropout_keep.argtypes = [u64, ctypes.c_int, i64, i64, i64,
                                            ctypes.POINTER(ctypes.c_int)]
        lib.oracle_dropout_keep.restype = ctypes.c_int
        lib.oracle_xxh32_words.argtypes = [ip, ctypes.c_int, ctypes.c_uint32,
                                           ctypes.POINTER(ctypes.c_uint32)]
        lib.oracle_xxh32_words.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = dbl
        lib.oracle_e4m3_encode.argtypes = [dbl]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_fwht_f32.argtypes = [i64, ip]
        lib.oracle_fwht_f32.restype = ctypes.c_int
        lib.oracle_mx_quant.argtypes = [i64, i64, ip, ip, ip, ip]
        lib.oracle_mx_quant.restype = ctypes.c_int
        lib.oracle_mx_dequant.argtypes = [i64, i64, ip, ip, ip]
        lib.oracle_mx_dequant.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _mask_code(mask) -> int:
    return MASKS[mask] if isinstance(mask, str) else int(mask)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def fwd(q, k, v, scale: float, mask="none", window: int = 0, rows=None):
    """Dense forward. Returns (Y, M, L, LSE); Y is [..., len(rows), dv]."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    if rows is None:
        rows_arr, nrows, rp = None, n, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows, rp = len(rows_arr), _ptr(rows_arr)
    y = np.empty((nh, nrows, dv))
    m = np.empty((nh, nrows))
    l = np.empty((nh, nrows))
    lse = np.empty((nh, nrows))
    _check(lib.oracle_fwd(nh, n, d, dv, _ptr(q), _ptr(k), _ptr(v), float(scale), _mask_code(mask),
                          int(window), rp, nrows, _ptr(y), _ptr(m), _ptr(l), _ptr(lse)), "fwd")
    shp = lead + (nrows,)
    return y.reshape(shp + (dv,)), m.reshape(shp), l.reshape(shp), lse.reshape(shp)


def decode(q, k, v, scale: float, mask="none", window: int = 0):
    """Decode-shaped forward: q [B, H, nq, d] are the last nq positions of a
    sequence whose keys/values k, v [B, Hkv, nk, d|dv] are all cached; H must be
    a multiple of Hkv.  Returns (Y [B, H, nq, dv], LSE [B, H, nq])."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, nq, d = q.shape
    _, Hkv, nk, _ = k.shape
    dv = v.shape[-1]
    y = np.empty((B, H, nq, dv))
    lse = np.empty((B, H, nq))
    _check(lib.oracle_decode(B, H, Hkv, nq, nk, d, dv, _ptr(q), _ptr(k), _ptr(v), float(scale),
                             _mask_code(mask), int(window), _ptr(y), _ptr(lse)), "decode")
    return y, lse


def xxh32_words(words, seed: int) -> int:
    """XXH32 of the little-endian 32-bit words (at most 3) with a 32-bit seed."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    out = ctypes.c_uint32()
    _check(_load().oracle_xxh32_words(_ptr(w), len(w), seed & 0xFFFFFFFF, ctypes.byref(out)),
           "xxh32")
    return out.value


def dropout_keep(seed: int, thr: int, bh: int, i: int, j: int) -> bool:
    """keep_ij of the realized dropout mask (seed, drop threshold thr / 256)."""
    out = ctypes.c_int()
    _check(_load().oracle_dropout_keep(seed, thr, bh, i, j, ctypes.byref(out)), "dropout_keep")
    return bool(out.value)


def fwd_drop(q, k, v, scale: float, mask="none", window: int = 0, seed: int = 0, thr: int = 0,
             bh0: int = 0):
    """Dense forward with dropout on the weights; q, k, v [..., n, d]; the flat
    leading index plus bh0 is the head index bh of the mask.  Returns (Y, LSE)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    y = np.empty((nh, n, dv))
    lse = np.empty((nh, n))
    _check(lib.oracle_fwd_drop(nh, n, d, dv, _ptr(q), _ptr(k), _ptr(v), float(scale),
                               _mask_code(mask), int(window), seed, thr, int(bh0), _ptr(y),
                               _ptr(lse)), "fwd_drop")
    return y.reshape(lead + (n, dv)), lse.reshape(lead + (n,))


def bwd_drop(q, k, v, g, scale: float, mask="none", window: int = 0, seed: int = 0, thr: int = 0,
             bh0: int = 0):
    """VJP of sum(G * Y) for the forward with dropout (same mask replayed).
    Returns (dQ, dK, dV, Y, delta, LSE)."""
    lib = _load()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    dq, dk = np.empty((nh, n, d)), np.empty((nh, n, d))
    dvv, y = np.empty((nh, n, dv)), np.empty((nh, n, dv))
    delta, lse = np.empty((nh, n)), np.empty((nh, n))
    _check(lib.oracle_bwd_drop(nh, n, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), float(scale),
                               _mask_code(mask), int(window), seed, thr, int(bh0), _ptr(dq),
                               _ptr(dk), _ptr(dvv), _ptr(y), _ptr(delta), _ptr(lse)), "bwd_drop")
    sh = lead + (n,)
    return (dq.reshape(sh + (d,)), dk.reshape(sh + (d,)), dvv.reshape(sh + (dv,)),
            y.reshape(sh + (dv,)), delta.reshape(sh), lse.reshape(sh))


def e4m3_decode(code: int) -> float:
    """Value of one FP8 e4m3 code (NaN for 0x7F / 0xFF)."""
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(x: float) -> int:
    """The e4m3 code nearest to x (|x| <= 448), ties to the even code."""
    return int(_load().oracle_e4m3_encode(float(x)))


def fwht_f32(x) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform of one float32 vector, butterfly
    stages of span 1, 2, ..., n/2, every sum rounded to float32."""
    a = np.ascontiguousarray(x, dtype=np.float32).copy()
    _check(_load().oracle_fwht_f32(a.size, _ptr(a)), "fwht_f32")
    return a


def mx_quant(x, signs=None):
    """Block-scaled FP8 codes of rows x [..., d]: with ``signs`` (d values of
    +-1) the rows are first rotated as H (signs * x) (incoherent processing);
    then every 32 consecutive values share the scale 2^e, e the least with
    max |x| <= 448 2^e.  Returns (codes uint8 [..., d], scale bytes e + 127
    uint8 [..., ceil(d / 32)])."""
    x = _f64(x)
    d = x.shape[-1]
    rows = x.size // d if d else 0
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros(x.shape[:-1] + ((d + 31) // 32,), dtype=np.uint8)
    sg = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    if sg is not None and sg.shape != (d,):
        raise ValueError("signs must have d entries")
    _check(_load().oracle_mx_quant(rows, d, _ptr(x), None if sg is None else _ptr(sg),
                                   _ptr(codes), _ptr(scales)), "mx_quant")
    return codes, scales


def mx_dequant(codes, scales) -> np.ndarray:
    """Values of block-scaled codes (float64, exact)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    d = codes.shape[-1]
    if scales.shape != codes.shape[:-1] + ((d + 31) // 32,):
        raise ValueError("scales must be [..., ceil(d / 32)]")
    out = np.zeros(codes.shape, dtype=np.float64)
    _check(_load().oracle_mx_dequant(codes.size // d if d else 0, d, _ptr(codes), _ptr(scales),
                                     _ptr(out)), "mx_dequant")
    return out


def bwd(q, k, v, g, scale: float, mask="none", window: int = 0):
    """Dense VJP of Phi = sum(G * Y). Returns (dQ, dK, dV, Y, delta, LSE)."""
    lib = _load()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    dq, dk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    y = np.empty_like(v)
    delta = np.empty(lead + (n,))
    lse = np.empty(lead + (n,))
    _check(lib.oracle_bwd(nh, n, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), float(scale),
                          _mask_code(mask), int(window), _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(y),
                          _ptr(delta), _ptr(lse)), "bwd")
    return dq, dk, dvv, y, delta, lse


def summary(s, vrows):
    """Sigma(S) = (m, l, z) of one nonempty block of scores s with value rows vrows [k, dv]."""
    lib = _load()
    s = _f64(s).reshape(-1)
    vrows = _f64(vrows).reshape(len(s), -1)
    dv = vrows.shape[1]
    m, l = ctypes.c_double(), ctypes.c_double()
    z = np.empty(dv)
    _check(lib.oracle_summary(len(s), dv, _ptr(s), _ptr(vrows), ctypes.byref(m), ctypes.byref(l),
                              _ptr(z)), "summary")
    return m.value, l.value, z


def merge(a, b, broken: bool = False):
    """Sigma(S) * Sigma(T) for summaries a = (mS, lS, zS), b = (mT, lT, zT)."""
    lib = _load()
    zS, zT = _f64(a[2]).reshape(-1), _f64(b[2]).reshape(-1)
    m, l = ctypes.c_double(), ctypes.c_double()
    z = np.empty(len(zS))
    _check(lib.oracle_merge(len(zS), float(a[0]), float(a[1]), _ptr(zS), float(b[0]), float(b[1]),
                            _ptr(zT), int(broken), ctypes.byref(m), ctypes.byref(l), _ptr(z)),
           "merge")
    return m.value, l.value, z


def fwd_tiled(q, k, v, scale: float, mask="none", window: int = 0, block: int = 16,
              broken: bool = False):
    """The Algorithm's tiled forward procedure. Returns (Y, M, L)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    y = np.empty((nh, n, dv))
    m = np.empty((nh, n))
    l = np.empty((nh, n))
    _check(lib.oracle_fwd_tiled(nh, n, d, dv, _ptr(q), _ptr(k), _ptr(v), float(scale),
                                _mask_code(mask), int(window), int(block), int(broken), _ptr(y),
                                _ptr(m), _ptr(l)), "fwd_tiled")
    shp = lead + (n,)
    return y.reshape(shp + (dv,)), m.reshape(shp), l.reshape(shp)
