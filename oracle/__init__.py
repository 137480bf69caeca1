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
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_gemm_weight_only.argtypes = [P, I, P, P, I, I, I, I, P, I, P, P]
    lib.oracle_gptq_quantize_rtn_group.argtypes = [P, ctypes.c_int, I, I, I, P, P]
    lib.oracle_rmsnorm_bf16.argtypes = [P, I, P, ctypes.c_double, I, I, P]
    lib.oracle_attn_qk_int8.argtypes = [P, P, P, P, ctypes.c_double, I, I, I, I, P, P]
    lib.oracle_attn_pv_int8.argtypes = [P, P, P, I, I, I, I, P, P, P, P]
    for f in ("oracle_quant_act_per_token", "oracle_gptq_unpack", "oracle_gptq_dequant",
              "oracle_gptq_quantize_rtn", "oracle_group_partials", "oracle_gemm_w8a8_g128",
              "oracle_gemm_w4a16_g128", "oracle_gemm_weight_only", "oracle_gptq_quantize_rtn_group",
              "oracle_rmsnorm_bf16", "oracle_attn_qk_int8", "oracle_attn_pv_int8"):
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


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on (timing of the CPU baseline)."""
    _load().oracle_set_num_threads(int(n))


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


def gemm_weight_only(x_bf16, q, w_scale, group: int, rows=None):
    """(y, T) fp64 [nrows, N]: exact weight-only output with one scale per `group` K values
    (W8A16 at group 128 or 32; W4A16 at group 128) and its fp32 magnitude bound."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = x.shape
    N = q.shape[1]
    r, nrows = _rows_arg(rows, M)
    y = np.empty((nrows, N), dtype=np.float64)
    T = np.empty((nrows, N), dtype=np.float64)
    _check(_load().oracle_gemm_weight_only(_ptr(x), K, _ptr(q), _ptr(ws), group, M, N, K,
                                           None if r is None else _ptr(r), nrows, _ptr(y), _ptr(T)),
           "gemm_weight_only")
    return y, T


def gptq_quantize_rtn_group(w: np.ndarray, bits: int, group: int):
    """RTN symmetric quantisation with `group` K values per scale -> (qweight int32, w_scale fp32 [K/group, N])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    qw = np.empty((K // (32 // bits), N), dtype=np.int32)
    ws = np.empty((K // group, N), dtype=np.float32)
    _check(_load().oracle_gptq_quantize_rtn_group(_ptr(w), bits, group, K, N, _ptr(qw), _ptr(ws)), "rtn_group")
    return qw, ws


def rmsnorm_bf16(x_bf16, gamma_bf16, eps: float) -> np.ndarray:
    """bf16 bit patterns [M, K] of bf16(gamma * bf16(x / sqrt(mean(x^2) + eps)))."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    g = np.ascontiguousarray(gamma_bf16, dtype=np.uint16)
    M, K = x.shape
    h = np.empty((M, K), dtype=np.uint16)
    _check(_load().oracle_rmsnorm_bf16(_ptr(x), K, _ptr(g), float(eps), M, K, _ptr(h)), "rmsnorm")
    return h


def kv_quant_block128(kv_bf16: np.ndarray):
    """The block-g128 INT8 KV codec: codes int8 [..., 128] and one fp32 scale per 128-wide
    block [...], by the per-token quantiser applied to every 128-wide row."""
    kv = np.ascontiguousarray(kv_bf16, dtype=np.uint16)
    assert kv.shape[-1] == 128
    lead = kv.shape[:-1]
    qa, s = quant_act_per_token(kv.reshape(-1, 128))
    return qa.reshape(*lead, 128), s.reshape(lead)


def attn_qk_int8(qq, qs, kq, ks, scale: float):
    """(s fp64 [Hq, Mq, T], dots int32 [Hq, Mq, T]) of the INT8 QK product; qq int8 [Mq, Hq, 128],
    qs fp32 [Mq, Hq], kq int8 [T, Hkv, 128], ks fp32 [T, Hkv]."""
    qq = np.ascontiguousarray(qq, dtype=np.int8)
    qs = np.ascontiguousarray(qs, dtype=np.float32)
    kq = np.ascontiguousarray(kq, dtype=np.int8)
    ks = np.ascontiguousarray(ks, dtype=np.float32)
    Mq, Hq, _ = qq.shape
    T, Hkv, _ = kq.shape
    s = np.empty((Hq, Mq, T), dtype=np.float64)
    d = np.empty((Hq, Mq, T), dtype=np.int32)
    _check(_load().oracle_attn_qk_int8(_ptr(qq), _ptr(qs), _ptr(kq), _ptr(ks), float(scale), Mq, T, Hq, Hkv,
                                       _ptr(s), _ptr(d)), "attn_qk")
    return s, d


def attn_pv_int8(p, vq, vs):
    """(out fp64 [Hq, Mq, 128], mag fp64 [Hq, Mq, 128], pq int8 [Hq, Mq, T], ps fp32 [Hq, Mq, ceil(T/128)])
    of the INT8 PV product; p fp32 [Hq, Mq, T], vq int8 [T, Hkv, 128], vs fp32 [T, Hkv]."""
    p = np.ascontiguousarray(p, dtype=np.float32)
    vq = np.ascontiguousarray(vq, dtype=np.int8)
    vs = np.ascontiguousarray(vs, dtype=np.float32)
    Hq, Mq, T = p.shape
    Hkv = vq.shape[1]
    B = (T + 127) // 128
    out = np.empty((Hq, Mq, 128), dtype=np.float64)
    mag = np.empty((Hq, Mq, 128), dtype=np.float64)
    pq = np.empty((Hq, Mq, T), dtype=np.int8)
    ps = np.empty((Hq, Mq, B), dtype=np.float32)
    _check(_load().oracle_attn_pv_int8(_ptr(p), _ptr(vq), _ptr(vs), Mq, T, Hq, Hkv, _ptr(out), _ptr(mag), _ptr(pq),
                                       _ptr(ps)), "attn_pv")
    return out, mag, pq, ps
