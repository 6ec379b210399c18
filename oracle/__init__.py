"""CPU oracle for the W4A16 decode GEMV -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg may import this package.
The product (the HIP library and its Python binding) never imports, links or runs it,
and the two share no code: this side is plain single-threaded C in float64
(w4a16_oracle.c), loaded through ctypes, with numpy wrappers below.

It computes y[n] = sum_k q[n,k] * s[n, k/128] * x[k] exactly as that sum reads (float64),
plus mag[n] = sum_k |q s x|, the basis of the per-element tolerance
|err| <= 1e-3 * mag + 1e-5. For the expert tail it also computes the SwiGLU of the grouped
gate+up product (h = silu(g) * u, rounded to bfloat16) and the router-weighted sum of the
grouped down projection, out = sum_t w[t] * W_down[ids[t]] h[t], and the step before the path:
symmetric round-to-nearest quantisation of bf16 weights into the packed format (codes and fp16
scales decided in float32, so they are exact targets). See w4a16_oracle.c for
the storage format and the passage of the local-kimi README it follows.

Pins (tests/test_oracle_pins.py) tie it to facts other than itself: hand-computed worked
examples, IEEE decodes checked against numpy's own conversions over every bit pattern,
unit-vector probes with chosen nibbles and scales, zero-scale groups, linearity in x and
negation, and exact closed forms for constant rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "w4a16_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

TOL_REL = 1e-3
TOL_ABS = 1e-5


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source with gcc (-O2, no fast-math) into a shared object."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build() -> str:
    return compile_source(SOURCE, _LIB)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _experts(qw: np.ndarray, num_experts: Optional[int]) -> int:
    """Expert count passed to the oracle: qw's leading size unless a smaller one is asked for."""
    if num_experts is None:
        return qw.shape[0]
    if not 1 <= num_experts <= qw.shape[0]:
        raise ValueError("num_experts must lie in [1, experts held]")
    return int(num_experts)


def _rows(rows, N):
    if rows is None:
        return None, N
    r = _c(rows, np.int64)
    return r, r.size


class Oracle:
    """numpy front end over one compiled copy of the oracle."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_unpack.argtypes = [P, P, i64, i64]
        lib.oracle_gemv.argtypes = [P, P, P, i64, i64, i32, P, i64, P, P]
        lib.oracle_gemv_batched.argtypes = [P, P, P, i64, i32, i64, i64, i32, P, i64, P, P]
        lib.oracle_moe_gemv.argtypes = [P, P, P, i32, i32, P, i64, i64, i32, P, i64, P, P]
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_moe_swiglu.argtypes = [P, P, P, i32, i32, P, i64, i64, i32,
                                          P, P, P, P, P, P]
        lib.oracle_moe_down_combine.argtypes = [P, P, P, P, i32, i32, P, i64, i64, i32, P, i64,
                                                P, P]
        lib.oracle_unpack3.argtypes = [P, P, i64, i64]
        lib.oracle_moe_gemv3.argtypes = [P, P, P, i32, i32, P, i64, i64, i32, P, i64, P, P]
        lib.oracle_float_to_f16_sat.argtypes = [ctypes.c_float]
        lib.oracle_float_to_f16_sat.restype = ctypes.c_uint16
        lib.oracle_quantize_pack.argtypes = [P, i64, i64, i64, i32, P, P]
        lib.oracle_moe_gemv_batched.argtypes = [P, P, P, i32, i32, i32, P, i64, i64, i64, i32,
                                                P, i64, P, P]
        for f in (lib.oracle_unpack, lib.oracle_gemv, lib.oracle_gemv_batched,
                  lib.oracle_moe_gemv, lib.oracle_moe_swiglu, lib.oracle_moe_down_combine,
                  lib.oracle_quantize_pack, lib.oracle_moe_gemv_batched):
            f.restype = ctypes.c_int
        self.lib = lib

    def f16_to_double(self, bits: int) -> float:
        return self.lib.oracle_f16_to_double(int(bits))

    def bf16_to_double(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_double(int(bits))

    def unpack(self, qweight: np.ndarray, K: int) -> np.ndarray:
        """int8 [N][K] signed values of packed uint32 [N][K/8] words."""
        qw = _c(qweight, np.uint32)
        N = qw.shape[0] if qw.ndim == 2 else 1
        out = np.empty((N, K), np.int8)
        if self.lib.oracle_unpack(_ptr(qw), _ptr(out), N, K):
            raise ValueError("oracle_unpack: bad arguments")
        return out

    def gemv(self, qweight, scales, x, K: int, group: int = 128,
             rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """(y, mag) as float64 for the listed rows (all rows by default)."""
        qw, sc, xx = _c(qweight, np.uint32), _c(scales, np.uint16), _c(x, np.uint16).reshape(-1)
        N = qw.shape[0]
        if xx.size < K:
            raise ValueError("x shorter than K")
        r, nr = _rows(rows, N)
        y, mag = np.empty(nr), np.empty(nr)
        if self.lib.oracle_gemv(_ptr(qw), _ptr(sc), _ptr(xx), N, K, group, _ptr(r), nr,
                                _ptr(y), _ptr(mag)):
            raise ValueError("oracle_gemv: bad arguments")
        return y, mag

    def gemv_batched(self, qweight, scales, X, K: int, group: int = 128,
                     rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """(Y, mag) as float64 [M][rows] for activation rows X [M][ldx]."""
        qw, sc, XX = _c(qweight, np.uint32), _c(scales, np.uint16), _c(X, np.uint16)
        if XX.ndim == 1:
            XX = XX.reshape(1, -1)
        M, ldx = XX.shape
        N = qw.shape[0]
        r, nr = _rows(rows, N)
        Y, mag = np.empty((M, nr)), np.empty((M, nr))
        if self.lib.oracle_gemv_batched(_ptr(qw), _ptr(sc), _ptr(XX), ldx, M, N, K, group,
                                        _ptr(r), nr, _ptr(Y), _ptr(mag)):
            raise ValueError("oracle_gemv_batched: bad arguments")
        return Y, mag

    def moe_gemv(self, qweight, scales, ids, x, K: int, group: int = 128,
                 rows: Optional[Sequence[int]] = None,
                 num_experts: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """(y, mag) as float64 [topk][rows] for experts ids over qweight [E][N][K/8].
        num_experts (default: qweight's leading size) is the E the oracle is told; a smaller
        value leaves spare experts in memory past the last valid one."""
        qw, sc = _c(qweight, np.uint32), _c(scales, np.uint16)
        ii, xx = _c(ids, np.int32).reshape(-1), _c(x, np.uint16).reshape(-1)
        E, N = _experts(qw, num_experts), qw.shape[1]
        r, nr = _rows(rows, N)
        y, mag = np.empty((ii.size, nr)), np.empty((ii.size, nr))
        if self.lib.oracle_moe_gemv(_ptr(qw), _ptr(sc), _ptr(ii), ii.size, E, _ptr(xx), N, K,
                                    group, _ptr(r), nr, _ptr(y), _ptr(mag)):
            raise ValueError("oracle_moe_gemv: bad arguments")
        return y, mag

    def double_to_bf16(self, v: float) -> int:
        return int(self.lib.oracle_double_to_bf16(float(v)))

    def silu(self, g: float) -> float:
        return self.lib.oracle_silu(float(g))

    def moe_swiglu(self, qweight, scales, ids, x, K: int, group: int = 128,
                   num_experts: Optional[int] = None) -> dict:
        """Gate+up product of the selected experts (qweight [E][2I][K/8]) and SwiGLU.
        Returns float64 [topk][I] arrays h, g, u, mag_g, mag_u and uint16 h_bf16."""
        qw, sc = _c(qweight, np.uint32), _c(scales, np.uint16)
        ii, xx = _c(ids, np.int32).reshape(-1), _c(x, np.uint16).reshape(-1)
        E, N2 = _experts(qw, num_experts), qw.shape[1]
        if N2 % 2:
            raise ValueError("gate+up weights need an even row count")
        I, T = N2 // 2, ii.size
        out = {k: np.empty((T, I)) for k in ("h", "g", "u", "mag_g", "mag_u")}
        out["h_bf16"] = np.empty((T, I), np.uint16)
        if self.lib.oracle_moe_swiglu(_ptr(qw), _ptr(sc), _ptr(ii), T, E, _ptr(xx), I, K, group,
                                      _ptr(out["h"]), _ptr(out["h_bf16"]), _ptr(out["g"]),
                                      _ptr(out["u"]), _ptr(out["mag_g"]), _ptr(out["mag_u"])):
            raise ValueError("oracle_moe_swiglu: bad arguments")
        return out

    def moe_down_combine(self, qweight, scales, ids, weights, h, group: int = 128,
                         rows: Optional[Sequence[int]] = None,
                         num_experts: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """(out, mag) float64 [rows]: sum_t w[t] * W_down[ids[t]] h[t], qweight [E][H][I/8]."""
        qw, sc = _c(qweight, np.uint32), _c(scales, np.uint16)
        ii, ww = _c(ids, np.int32).reshape(-1), _c(weights, np.float32).reshape(-1)
        hh = _c(h, np.uint16)
        E, H, I = _experts(qw, num_experts), qw.shape[1], qw.shape[2] * 8
        if ww.size != ii.size or hh.shape != (ii.size, I):
            raise ValueError("ids, weights and h disagree")
        r, nr = _rows(rows, H)
        out, mag = np.empty(nr), np.empty(nr)
        if self.lib.oracle_moe_down_combine(_ptr(qw), _ptr(sc), _ptr(ii), _ptr(ww), ii.size, E,
                                            _ptr(hh), H, I, group, _ptr(r), nr, _ptr(out),
                                            _ptr(mag)):
            raise ValueError("oracle_moe_down_combine: bad arguments")
        return out, mag


    def moe_gemv_batched(self, qweight, scales, ids, X, K: int, group: int = 128,
                         rows: Optional[Sequence[int]] = None,
                         num_experts: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """(Y, mag) float64 [M][topk][rows]: token m times expert ids[m][t], qweight [E][N][K/8]."""
        qw, sc = _c(qweight, np.uint32), _c(scales, np.uint16)
        ii, XX = _c(ids, np.int32), _c(X, np.uint16)
        if XX.ndim == 1:
            XX = XX.reshape(1, -1)
        M, ldx = XX.shape
        ii = ii.reshape(M, -1)
        topk = ii.shape[1]
        E, N = _experts(qw, num_experts), qw.shape[1]
        r, nr = _rows(rows, N)
        Y, mag = np.empty((M, topk, nr)), np.empty((M, topk, nr))
        if self.lib.oracle_moe_gemv_batched(_ptr(qw), _ptr(sc), _ptr(ii), M, topk, E, _ptr(XX),
                                            ldx, N, K, group, _ptr(r), nr, _ptr(Y), _ptr(mag)):
            raise ValueError("oracle_moe_gemv_batched: bad arguments")
        return Y, mag

    def unpack3(self, qweight3, K: int) -> np.ndarray:
        """Signed three-bit codes int8 [N][K] of qweight3 uint32 [N][3K/32]."""
        qw = _c(qweight3, np.uint32)
        N = qw.shape[0] if qw.ndim == 2 else 1
        out = np.empty((N, K), np.int8)
        if self.lib.oracle_unpack3(_ptr(qw), _ptr(out), N, K):
            raise ValueError("oracle_unpack3: bad arguments")
        return out

    def moe_gemv3(self, qweight3, scales, ids, x, K: int, group: int = 128,
                  rows: Optional[Sequence[int]] = None,
                  num_experts: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """(y, mag) float64 [topk][rows] for three-bit experts qweight3 [E][N][3K/32]."""
        qw, sc = _c(qweight3, np.uint32), _c(scales, np.uint16)
        ii, xx = _c(ids, np.int32).reshape(-1), _c(x, np.uint16).reshape(-1)
        E, N = _experts(qw, num_experts), qw.shape[1]
        r, nr = _rows(rows, N)
        y, mag = np.empty((ii.size, nr)), np.empty((ii.size, nr))
        if self.lib.oracle_moe_gemv3(_ptr(qw), _ptr(sc), _ptr(ii), ii.size, E, _ptr(xx), N, K,
                                     group, _ptr(r), nr, _ptr(y), _ptr(mag)):
            raise ValueError("oracle_moe_gemv3: bad arguments")
        return y, mag

    def float_to_f16_sat(self, v: float) -> int:
        return int(self.lib.oracle_float_to_f16_sat(float(v)))

    def quantize_pack(self, w_bf16, K: int, group: int = 128) -> Tuple[np.ndarray, np.ndarray]:
        """(qweight uint32 [N][K/8], scales uint16 fp16 bits [N][K/G]) of bf16 bits [N][ldw]."""
        ww = _c(w_bf16, np.uint16)
        if ww.ndim == 1:
            ww = ww.reshape(1, -1)
        N, ldw = ww.shape
        qw = np.zeros((N, K // 8), np.uint32)
        sc = np.zeros((N, K // group), np.uint16)
        if self.lib.oracle_quantize_pack(_ptr(ww), ldw, N, K, group, _ptr(qw), _ptr(sc)):
            raise ValueError("oracle_quantize_pack: bad arguments")
        return qw, sc


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle compiled from w4a16_oracle.c (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(_LIB)
    return _default


def f16_to_double(bits):
    return default().f16_to_double(bits)


def bf16_to_double(bits):
    return default().bf16_to_double(bits)


def unpack(qweight, K):
    return default().unpack(qweight, K)


def gemv(*a, **kw):
    return default().gemv(*a, **kw)


def gemv_batched(*a, **kw):
    return default().gemv_batched(*a, **kw)


def moe_gemv(*a, **kw):
    return default().moe_gemv(*a, **kw)


def double_to_bf16(v):
    return default().double_to_bf16(v)


def silu(g):
    return default().silu(g)


def moe_swiglu(*a, **kw):
    return default().moe_swiglu(*a, **kw)


def moe_down_combine(*a, **kw):
    return default().moe_down_combine(*a, **kw)


def moe_gemv_batched(*a, **kw):
    return default().moe_gemv_batched(*a, **kw)


def unpack3(qweight3, K):
    return default().unpack3(qweight3, K)


def moe_gemv3(*a, **kw):
    return default().moe_gemv3(*a, **kw)


def quantize_pack(*a, **kw):
    return default().quantize_pack(*a, **kw)


def bound(mag: np.ndarray) -> np.ndarray:
    """Per-element allowance: 1e-3 * sum|q s x| + 1e-5."""
    return TOL_REL * np.asarray(mag) + TOL_ABS
