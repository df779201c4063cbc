"""CPU oracle for the block-quantized decode mat-vec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``routed_moe_matvec_amd``) never imports it, and it never imports the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation, one 32-weight
block dequantized at a time; fp32 only in the activation quantizer, whose
result is defined by fp32 rounding).  This module only builds that library and
marshals numpy arrays into it.

Every function here is pinned by ``tests/test_oracle.py`` against something
other than itself (closed forms, integer special cases checked with numpy
int64 matmul, library conversions, brute force and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FMT_Q8_0 = 0
FMT_Q4K = 1
FMT_FP8_B128 = 2  # FP8 E4M3 codes, UE8M0 scale per 128 x 128 block
FMT_FP4_MX = 3    # FP4 E2M1 codes (two per byte, low nibble first), UE8M0 scale per 1 x 32
BAD_EXPERT = 1  # status code for an expert id outside [0, E)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.oracle_half_to_double.restype = dbl
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = dbl
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_to_double.restype = dbl
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_to_double.restype = dbl
    lib.oracle_e2m1_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_ue8m0_to_double.restype = dbl
    lib.oracle_ue8m0_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_row_bytes.restype = i64
    lib.oracle_row_bytes.argtypes = [ctypes.c_int, i64]
    lib.oracle_matrix_bytes.restype = i64
    lib.oracle_matrix_bytes.argtypes = [ctypes.c_int, i64, i64]
    lib.oracle_dequant.restype = ctypes.c_int
    lib.oracle_dequant.argtypes = [ctypes.c_int, vp, i64, i64, vp]
    lib.oracle_quantize_act_q8.restype = None
    lib.oracle_quantize_act_q8.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.oracle_gemv.restype = ctypes.c_int
    lib.oracle_gemv.argtypes = [ctypes.c_int, vp, i64, i64, vp, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_gemv_fx.restype = ctypes.c_int
    lib.oracle_gemv_fx.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_block_isums.restype = ctypes.c_int
    lib.oracle_block_isums.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, vp]
    lib.oracle_moe_table.restype = ctypes.c_int
    lib.oracle_moe_table.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.oracle_silu.restype = dbl
    lib.oracle_silu.argtypes = [dbl]
    lib.oracle_moe_routed.restype = ctypes.c_int
    lib.oracle_moe_routed.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_int]
    lib.oracle_moe_routed_fmt.restype = ctypes.c_int
    lib.oracle_moe_routed_fmt.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                          vp, vp, ctypes.c_int]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def max_threads() -> int:
    return _load().oracle_max_threads()


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(int(bits) & 0xFFFF)


def e4m3_to_double(code: int) -> float:
    return _load().oracle_e4m3_to_double(int(code) & 0xFF)


def e2m1_to_double(code: int) -> float:
    return _load().oracle_e2m1_to_double(int(code) & 0x0F)


def ue8m0_to_double(code: int) -> float:
    return _load().oracle_ue8m0_to_double(int(code) & 0xFF)


def row_bytes(fmt: int, K: int) -> int:
    """Bytes of one row (for FP8 / FP4: of its codes only)."""
    return int(_load().oracle_row_bytes(fmt, K))


def matrix_bytes(fmt: int, N: int, K: int) -> int:
    """Bytes of a whole N x K matrix, scales included."""
    return int(_load().oracle_matrix_bytes(fmt, N, K))


def dequant(fmt: int, W: np.ndarray, N: int, K: int) -> np.ndarray:
    """Dequantized [N, K] float64 matrix."""
    W = _c(W, np.uint8)
    assert W.size == matrix_bytes(fmt, N, K)
    out = np.empty((N, K), np.float64)
    _check(_load().oracle_dequant(fmt, _ptr(W), N, K, _ptr(out)), "dequant")
    return out


def quantize_act_q8(x: np.ndarray):
    """x fp32 [M, K] -> (qx int8 [M, K], dx fp32 [M, K/32], sx int32 [M, K/32])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    assert K % 32 == 0
    qx = np.empty((M, K), np.int8)
    dx = np.empty((M, K // 32), np.float32)
    sx = np.empty((M, K // 32), np.int32)
    _load().oracle_quantize_act_q8(_ptr(x), M, K, _ptr(qx), _ptr(dx), _ptr(sx))
    return qx, dx, sx


def gemv(fmt: int, W: np.ndarray, N: int, K: int, qx: np.ndarray, dx: np.ndarray, nthreads: int = 1):
    """(y, bound), both float64 [M, N]."""
    W = _c(W, np.uint8)
    qx = _c(qx, np.int8).reshape(-1, K)
    M = qx.shape[0]
    dx = _c(dx, np.float32).reshape(M, K // 32)
    assert W.size == matrix_bytes(fmt, N, K)
    y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    _check(_load().oracle_gemv(fmt, _ptr(W), N, K, _ptr(qx), _ptr(dx), M, _ptr(y), _ptr(bound), nthreads),
           "gemv")
    return y, bound


def gemv_fx(fmt: int, W: np.ndarray, N: int, K: int, x: np.ndarray, nthreads: int = 1):
    """(y, bound) float64 [M, N] of the weights against the fp32 activation x as given."""
    W = _c(W, np.uint8)
    x = _c(x, np.float32).reshape(-1, K)
    M = x.shape[0]
    assert W.size == matrix_bytes(fmt, N, K)
    y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    _check(_load().oracle_gemv_fx(fmt, _ptr(W), N, K, _ptr(x), M, _ptr(y), _ptr(bound), nthreads), "gemv_fx")
    return y, bound


def block_isums(fmt: int, W: np.ndarray, N: int, K: int, qx: np.ndarray) -> np.ndarray:
    """int32 [M, N, K/32] per-block integer dot products of raw quants."""
    W = _c(W, np.uint8)
    qx = _c(qx, np.int8).reshape(-1, K)
    M = qx.shape[0]
    out = np.empty((M, N, K // 32), np.int32)
    _check(_load().oracle_block_isums(fmt, _ptr(W), N, K, _ptr(qx), M, _ptr(out)), "block_isums")
    return out


def moe_table(ids: np.ndarray, E: int):
    """Compact selected-expert table: dict(uniq, n_uniq, slot, pair_off, pairs, status)."""
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    P = T * topk
    cap = max(1, min(P, E))
    uniq = np.full(cap, -1, np.int32)
    n_uniq = np.zeros(1, np.int32)
    slot = np.empty(max(P, 1), np.int32)
    pair_off = np.zeros(cap + 1, np.int32)
    pairs = np.full(max(P, 1), -1, np.int32)
    status = np.zeros(1, np.int32)
    _check(_load().oracle_moe_table(_ptr(ids), T, topk, E, _ptr(uniq), _ptr(n_uniq), _ptr(slot), _ptr(pair_off),
                                    _ptr(pairs), _ptr(status)), "moe_table")
    U = int(n_uniq[0])
    npairs = int(pair_off[U])
    return dict(uniq=uniq[:U].copy(), n_uniq=U, slot=slot[:P].reshape(T, topk).copy(),
                pair_off=pair_off[:U + 1].copy(), pairs=pairs[:npairs].copy(), status=int(status[0]))


def silu(z: float) -> float:
    return _load().oracle_silu(float(z))


def moe_routed(qx, dx, ids, rw, gate, up, down, D: int, F: int, nthreads: int = 1, fmt: int = FMT_Q4K):
    """End-to-end routed MoE from scratch.  gate/up/down: lists of E uint8 arrays in format fmt.

    Returns (y, bound, status) with y, bound float64 [T, D].
    """
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    qx = _c(qx, np.int8).reshape(T, D)
    dx = _c(dx, np.float32).reshape(T, D // 32)
    rw = _c(rw, np.float32).reshape(T, topk)
    E = len(gate)
    assert len(up) == E and len(down) == E
    mats = [[_c(m, np.uint8) for m in lst] for lst in (gate, up, down)]
    ptr_arrays = []
    for lst in mats:
        arr = (ctypes.c_void_p * E)(*[m.ctypes.data for m in lst])
        ptr_arrays.append(arr)
    y = np.empty((T, D), np.float64)
    bound = np.empty((T, D), np.float64)
    status = np.zeros(1, np.int32)
    _check(_load().oracle_moe_routed_fmt(fmt, _ptr(qx), _ptr(dx), T, D, F, E, topk, _ptr(ids), _ptr(rw),
                                     ctypes.cast(ptr_arrays[0], ctypes.c_void_p),
                                     ctypes.cast(ptr_arrays[1], ctypes.c_void_p),
                                     ctypes.cast(ptr_arrays[2], ctypes.c_void_p),
                                     _ptr(y), _ptr(bound), _ptr(status), nthreads), "moe_routed")
    del mats
    return y, bound, int(status[0])


def prefill(fmt: int, W: np.ndarray, N: int, K: int, xbf16: np.ndarray, nthreads: int = 1):
    """(Y, bound) float64 [M, N] for bf16 activations given as uint16 bits [M, K]."""
    W = _c(W, np.uint8)
    xbf16 = _c(xbf16, np.uint16).reshape(-1, K)
    M = xbf16.shape[0]
    Y = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    _check(_load().oracle_prefill(fmt, _ptr(W), N, K, _ptr(xbf16), M, _ptr(Y), _ptr(bound), nthreads),
           "prefill")
    return Y, bound
