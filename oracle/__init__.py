"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg may import this
package.  It is built from oracle.c with gcc (no fast-math, no FP contraction)
and shares no code with the GPU library.  Each wrapper below names the C
function it calls; the C file cites the passages each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_c_i64 = ctypes.c_longlong
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_longlong)
_up = ctypes.POINTER(ctypes.c_ulonglong)

_libs: dict = {}
_active = None  # path of the library the module-level functions use


def compile_library(src: str, out: str) -> str:
    """gcc build of an oracle source file into a shared library."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-pthread", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(_LIB):
        compile_library(_SRC, _LIB)
    return _LIB


class use_library:
    """Context manager: route the module functions to another build of the
    oracle source (used by the planted-mistake tests)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _active
        self.prev, _active = _active, self.path
        return self

    def __exit__(self, *exc):
        global _active
        _active = self.prev
        return False


def _load():
    path = _active or _LIB
    if path in _libs:
        return _libs[path]
    if path == _LIB and (not os.path.exists(_LIB)
                         or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(path)
    lib.orc_attention.argtypes = [_fp, _fp, _fp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                  ctypes.c_int, ctypes.c_double, _ip, _c_i64, _dp, _dp,
                                  ctypes.c_int]
    lib.orc_attention.restype = ctypes.c_int
    lib.orc_attention_probs.argtypes = [_fp, _fp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                        _c_i64, ctypes.c_int, ctypes.c_double, _c_i64, _c_i64,
                                        _c_i64, _dp]
    lib.orc_attention_probs.restype = ctypes.c_int
    lib.orc_pcast.argtypes = [_fp, _fp, _fp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                              ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                              ctypes.c_int, _c_i64, _ip, _c_i64, _dp, _dp, _up, ctypes.c_int]
    lib.orc_pcast.restype = ctypes.c_int
    lib.orc_attention_bwd.argtypes = [_fp, _fp, _fp, _fp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      _c_i64, ctypes.c_int, ctypes.c_double, _dp, _dp, _dp, _dp,
                                      _dp, _dp, ctypes.c_int]
    lib.orc_attention_bwd.restype = ctypes.c_int
    lib.orc_quant_e4m3.argtypes = [_fp, _c_i64, _c_i64, _c_i64, _c_i64, _fp, ctypes.c_int,
                                   ctypes.c_int, ctypes.POINTER(ctypes.c_ubyte), _fp]
    lib.orc_quant_e4m3.restype = ctypes.c_int
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint]
    lib.orc_e4m3_decode.restype = ctypes.c_float
    for name in ("orc_Phi", "orc_delta_c", "orc_dp"):
        getattr(lib, name).restype = ctypes.c_double
    lib.orc_Phi.argtypes = [ctypes.c_double]
    lib.orc_delta_c.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.orc_dp.argtypes = [ctypes.c_double]
    lib.orc_F.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.orc_F.restype = ctypes.c_double
    lib.orc_expected_max_gauss.argtypes = [ctypes.c_int]
    lib.orc_expected_max_gauss.restype = ctypes.c_double
    _libs[path] = lib
    return lib


def default_threads() -> int:
    """Worker threads: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when that is set, and at 16."""
    try:
        n = max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return min(n, 16)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _rows_arg(rows, B, H, Nq):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.ndim == 1:
        r = np.broadcast_to(r, (B * H, r.shape[0])).copy()
    r = r.reshape(B * H, -1)
    return r, r.shape[1]


def attention(q, k, v, causal: bool, scale: float, rows=None, nthreads: int | None = None):
    """orc_attention: exact O [B,H,R,d] (float64) and LSE [B,H,R].

    q: [B,H,Nq,d], k/v: [B,Hkv,Nk,d], given as float32 arrays holding the exact
    values handed to the GPU (bf16/fp16 widen exactly).  rows: None (all Nq
    rows), a 1-D row list used for every (b,h), or a [B*H, R] array.
    """
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    r, R = _rows_arg(rows, B, H, Nq)
    if r is None:
        R = Nq
    o = np.zeros((B, H, R, d), dtype=np.float64)
    lse = np.zeros((B, H, R), dtype=np.float64)
    rc = lib.orc_attention(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), B, H, Hkv, Nq, Nk, d,
                           int(bool(causal)), float(scale),
                           None if r is None else _ptr(r, _ip), R, _ptr(o, _dp),
                           _ptr(lse, _dp), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"orc_attention rejected its arguments (rc={rc})")
    return o, lse


def attention_bwd(q, k, v, dout, causal: bool, scale: float, abs_sums: bool = False,
                  nthreads: int | None = None):
    """orc_attention_bwd: (dq, dk, dv) in float64 for the loss gradient dout = dL/dO.

    q, dout: [B,H,Nq,d]; k, v: [B,Hkv,Nk,d] (float32 arrays with the exact
    values handed to the GPU).  With abs_sums=True also returns the absolute
    sums (adq, adk, adv) of the terms of each gradient element.
    """
    lib = _load()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    dq = np.zeros((B, H, Nq, d), dtype=np.float64)
    dk = np.zeros((B, Hkv, Nk, d), dtype=np.float64)
    dv = np.zeros((B, Hkv, Nk, d), dtype=np.float64)
    ab = [np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)] if abs_sums else [None] * 3
    rc = lib.orc_attention_bwd(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), _ptr(dout, _fp), B, H,
                               Hkv, Nq, Nk, d, int(bool(causal)), float(scale), _ptr(dq, _dp),
                               _ptr(dk, _dp), _ptr(dv, _dp),
                               *[None if a is None else _ptr(a, _dp) for a in ab],
                               nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"orc_attention_bwd rejected its arguments (rc={rc})")
    return (dq, dk, dv, *ab) if abs_sums else (dq, dk, dv)


def attention_probs(q, k, causal: bool, scale: float, b: int, h: int, i: int) -> np.ndarray:
    """orc_attention_probs: the probability row of query (b,h,i), length Nk."""
    lib = _load()
    q, k = _f32(q), _f32(k)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    p = np.zeros(Nk, dtype=np.float64)
    rc = lib.orc_attention_probs(_ptr(q, _fp), _ptr(k, _fp), B, H, Hkv, Nq, Nk, d,
                                 int(bool(causal)), float(scale), b, h, i, _ptr(p, _dp))
    if rc != 0:
        raise ValueError("orc_attention_probs rejected its arguments")
    return p


def pcast_emulate(q, k, v, causal: bool, scale: float, kv_tile: int, p_scale: float,
                  reverse: bool, n_sink: int = 0, rows=None, nthreads: int | None = None,
                  tile_local: bool = False):
    """orc_pcast: E4M3 P-cast emulation (tile_local: P relative to each tile's
    own maximum instead of the running one -- the ablation).

    Returns (O, LSE, counts) with counts = [casts, zeros] over keys >= n_sink
    followed by [casts, zeros] over keys outside the KV tiles holding a sink.
    """
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    r, R = _rows_arg(rows, B, H, Nq)
    if r is None:
        R = Nq
    o = np.zeros((B, H, R, d), dtype=np.float64)
    lse = np.zeros((B, H, R), dtype=np.float64)
    counts = np.zeros(4, dtype=np.uint64)
    rc = lib.orc_pcast(_ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), B, H, Hkv, Nq, Nk, d,
                       int(bool(causal)), float(np.float32(scale)), int(kv_tile),
                       float(np.float32(p_scale)), int(bool(reverse)) | (int(bool(tile_local)) << 1),
                       int(n_sink),
                       None if r is None else _ptr(r, _ip), R, _ptr(o, _dp), _ptr(lse, _dp),
                       _ptr(counts, _up), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"orc_pcast rejected its arguments (rc={rc})")
    return o, lse, [int(c) for c in counts]


def quant_e4m3(x, signs=None, layout: str = "rows32", whole: bool = False):
    """orc_quant_e4m3: E4M3 codes (uint8, x's shape) and power-of-two scales.

    x: [B,H,N,d] (float32 array of the exact input values).  signs: None or a
    length-d array of +-1 (random-sign Hadamard rotation before quantising).
    layout "rows32": scales [B,H,ceil(N/32)]; "channels": scales [B,H,d].
    whole=True: one scale for the whole tensor, repeated in that layout.
    """
    lib = _load()
    x = _f32(x)
    B, H, N, d = x.shape
    lay = {"rows32": 0, "channels": 1}[layout]
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros((B, H, (N + 31) // 32 if lay == 0 else d), dtype=np.float32)
    sg = None if signs is None else _f32(signs)
    rc = lib.orc_quant_e4m3(_ptr(x, _fp), B, H, N, d, None if sg is None else _ptr(sg, _fp), lay,
                            int(bool(whole)), codes.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)),
                            _ptr(scales, _fp))
    if rc != 0:
        raise ValueError(f"orc_quant_e4m3 rejected its arguments (rc={rc})")
    return codes, scales


def dequant_e4m3(codes, scales, layout: str = "rows32") -> np.ndarray:
    """The values the codes stand for: decode(code) * scale of its group (float32, exact)."""
    vals = e4m3_decode_table()[np.asarray(codes, dtype=np.int64)]
    sc = np.asarray(scales, dtype=np.float32)
    if layout == "rows32":
        N = vals.shape[2]
        s = np.repeat(sc, 32, axis=2)[:, :, :N, None]
    else:
        s = sc[:, :, None, :]
    return (vals * s).astype(np.float32)


def e4m3_decode_table() -> np.ndarray:
    """decode() of all 256 codes (float32)."""
    return e4m3_decode(np.arange(256))


def e4m3_encode(x) -> np.ndarray:
    lib = _load()
    xs = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.orc_e4m3_encode(float(t)) for t in xs], dtype=np.uint8).reshape(
        np.shape(x))


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    cs = np.asarray(codes, dtype=np.int64).ravel()
    return np.array([lib.orc_e4m3_decode(int(c)) for c in cs], dtype=np.float32).reshape(
        np.shape(codes))


def Phi(x: float) -> float:
    return _load().orc_Phi(float(x))


def F_closed_form(delta: float, S: float, delta_k: float) -> float:
    return _load().orc_F(float(delta), float(S), float(delta_k))


def delta_c(S: float, delta_k: float) -> float:
    return _load().orc_delta_c(float(S), float(delta_k))


def expected_max_gauss(k: int) -> float:
    return _load().orc_expected_max_gauss(int(k))


def dp(S: float) -> float:
    return _load().orc_dp(float(S))


def pcast_bound(a_rows, v_rows, S: float, slack: float = 2e-5) -> np.ndarray:
    """The stated per-element error bound of the E4M3 P-cast (the analysis of
    gist.science "Resumen Tecnico: Precision de P-Cast en la Atencion FP8",
    sections "Marco Teorico" and "Optimizacion 2"), around exact attention.

    a_rows: [R, Nk] exact weights (rows of the softmax); v_rows: [Nk, d] (or
    [R, Nk, d]).  Returns the bound [R, d] on |O_pcast - O_exact|.

    With p_j = a_j / max(a) the probability relative to the row's final
    maximum, casting S*p to E4M3 with round-to-nearest-even moves each weight
    by a relative amount r_j:
      r_j = 2^-4                    if S*p_j >= 2^-6 (normal: half an ulp of a
                                    3-bit mantissa),
      r_j = min(1, 2^-10 / (S*p_j)) otherwise (subnormal grid 2^-9, half step
                                    2^-10; a flushed value loses all of it).
    A running maximum never exceeds the final one, so the p a kernel casts is
    at least p_j and the same r_j bounds its error.  The normaliser is the sum
    of the uncast p, so |O_pcast - O| <= sum_j a_j r_j |v_j| per element;
    `slack` covers fp32 rounding of logits, exponentials and sums.  The stated
    MSE bound is the mean of the squared per-element bounds.
    """
    a_rows = np.asarray(a_rows, dtype=np.float64)
    mx = a_rows.max(axis=1, keepdims=True)
    p = np.divide(a_rows, mx, out=np.zeros_like(a_rows), where=mx > 0)
    sp = S * p
    with np.errstate(divide="ignore"):
        r = np.where(sp >= 2.0 ** -6, 2.0 ** -4, np.minimum(1.0, 2.0 ** -10 / sp))
    r = np.where(a_rows > 0, r, 0.0)
    av = np.abs(np.asarray(v_rows, dtype=np.float64))
    if av.ndim == 2:
        core = (a_rows * r) @ av
        scl = a_rows @ av
    else:
        core = np.einsum("rj,rjc->rc", a_rows * r, av)
        scl = np.einsum("rj,rjc->rc", a_rows, av)
    return core + slack * scl + 1e-7


def pcast_bound_rows(q, k, v, causal: bool, scale: float, S: float, b: int, h: int,
                     rows) -> np.ndarray:
    """pcast_bound for the given query rows of (b, h): the exact weights come
    from orc_attention_probs, the value rows from v's KV head.  [R, d]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    H, Hkv = q.shape[1], k.shape[1]
    a = np.stack([attention_probs(q, k, causal, scale, b, h, int(i)) for i in rows])
    return pcast_bound(a, v[b, h // (H // Hkv)], S)
