"""CPU oracle for the group-scaled INT8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never links, loads or
calls it, and it never calls the HIP library: the two share no code.

The arithmetic lives in ``i8gs_oracle.c`` (plain C loops, built with gcc);
this module only builds it, marshals numpy arrays and names the functions.
Every function cites the page passage it follows (see the C source header).

Parity pins: every function here is pinned by a CPU test against something
other than itself (closed forms, exact rational arithmetic, brute force,
float64 BLAS on integer-valued matrices, special cases); none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "i8gs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_i8gs.so")
GROUP = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (IEEE arithmetic: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _configure(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_quant_act_per_token.argtypes = [P, I, I, I, P, P]
    lib.oracle_gptq_unpack.argtypes = [P, ctypes.c_int, I, I, P]
    lib.oracle_gptq_dequant.argtypes = [P, P, ctypes.c_int, I, I, P]
    lib.oracle_gptq_quantize_rtn.argtypes = [P, ctypes.c_int, I, I, P, P]
    lib.oracle_group_partials.argtypes = [P, P, I, I, I, P]
    lib.oracle_gemm_w8a8_g128.argtypes = [P, P, P, P, I, I, I, P, I, P, P]
    lib.oracle_gemm_w4a16_g128.argtypes = [P, I, P, P, I, I, I, P, I, P, P]
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_bf16_from_double_array.argtypes = [P, I, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    for f in ("oracle_quant_act_per_token", "oracle_gptq_unpack", "oracle_gptq_dequant",
              "oracle_gptq_quantize_rtn", "oracle_group_partials", "oracle_gemm_w8a8_g128",
              "oracle_gemm_w4a16_g128"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def use_library(path):
    """Point this module at another build of the oracle source (used by the
    planted-mistake tests); ``None`` restores the regular build.  Returns the
    previous handle."""
    global _lib
    prev = _lib
    _lib = None if path is None else _configure(ctypes.CDLL(path))
    return prev


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def quant_act_per_token(x_bf16: np.ndarray):
    """Per-token symmetric INT8 quantisation of bf16 bit patterns [M, K] -> (qa int8 [M,K], a_scale fp32 [M])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    qa = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    _check(_load().oracle_quant_act_per_token(_ptr(x), M, K, K, _ptr(qa), _ptr(s)), "quant")
    return qa, s


def gptq_unpack(qweight: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Signed weight codes int8 [K, N] from GPTQ int32 words [K/(32/bits), N]."""
    qw = np.ascontiguousarray(qweight, dtype=np.int32)
    N = qw.shape[1]
    assert qw.shape[0] * (32 // bits) == K
    q = np.empty((K, N), dtype=np.int8)
    _check(_load().oracle_gptq_unpack(_ptr(qw), bits, K, N, _ptr(q)), "unpack")
    return q


def gptq_dequant(qweight: np.ndarray, w_scale: np.ndarray, bits: int, K: int) -> np.ndarray:
    """fp32 [K, N] = fl32(w_scale[k/128, n] * q[k, n])."""
    qw = np.ascontiguousarray(qweight, dtype=np.int32)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    N = qw.shape[1]
    w = np.empty((K, N), dtype=np.float32)
    _check(_load().oracle_gptq_dequant(_ptr(qw), _ptr(ws), bits, K, N, _ptr(w)), "dequant")
    return w


def gptq_quantize_rtn(w: np.ndarray, bits: int):
    """RTN G128 symmetric quantisation of fp32 [K, N] -> (qweight int32 [K/(32/bits), N], w_scale fp32 [K/128, N])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    qw = np.empty((K // (32 // bits), N), dtype=np.int32)
    ws = np.empty((K // GROUP, N), dtype=np.float32)
    _check(_load().oracle_gptq_quantize_rtn(_ptr(w), bits, K, N, _ptr(qw), _ptr(ws)), "rtn")
    return qw, ws


def group_partials(qa: np.ndarray, q: np.ndarray) -> np.ndarray:
    """int32 P [M, K/128, N] of per-group integer dot products."""
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = qa.shape
    N = q.shape[1]
    P = np.empty((M, K // GROUP, N), dtype=np.int32)
    _check(_load().oracle_group_partials(_ptr(qa), _ptr(q), M, N, K, _ptr(P)), "partials")
    return P


def _rows_arg(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.shape[0])


def gemm_w8a8_g128(qa, a_scale, q, w_scale, rows=None):
    """(y, T) fp64 [nrows, N]: exact W8A8 G128 output and its fp32-fold magnitude bound."""
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.int8)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = qa.shape
    N = q.shape[1]
    r, nrows = _rows_arg(rows, M)
    y = np.empty((nrows, N), dtype=np.float64)
    T = np.empty((nrows, N), dtype=np.float64)
    _check(_load().oracle_gemm_w8a8_g128(_ptr(qa), _ptr(a_scale), _ptr(q), _ptr(ws), M, N, K,
                                         None if r is None else _ptr(r), nrows, _ptr(y), _ptr(T)),
           "gemm_w8a8")
    return y, T


def gemm_w4a16_g128(x_bf16, q, w_scale, rows=None):
    """(y, T) fp64 [nrows, N]: exact W4A16 g128 output and its magnitude bound."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = x.shape
    N = q.shape[1]
    r, nrows = _rows_arg(rows, M)
    y = np.empty((nrows, N), dtype=np.float64)
    T = np.empty((nrows, N), dtype=np.float64)
    _check(_load().oracle_gemm_w4a16_g128(_ptr(x), K, _ptr(q), _ptr(ws), M, N, K,
                                          None if r is None else _ptr(r), nrows, _ptr(y), _ptr(T)),
           "gemm_w4a16")
    return y, T


def bf16_from_double(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp64 values, nearest-even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_bf16_from_double_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_from_double_scalar(v: float) -> int:
    return int(_load().oracle_bf16_from_double(float(v)))
