"""CPU oracle for the k-quant decode matvec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library neither links nor
calls it, and it shares no code with the HIP path.

The arithmetic lives in ``kq_oracle.c`` (plain C, binary64), compiled with
gcc into ``oracle/_build/libkqoracle.so``; this module is argument
marshalling only.  ``oracle.exact`` is an independent exact-rational
re-statement used to pin the C oracle on tiny inputs.

What is computed: muser-book Ch 13 section 13.1, y_i = sum_j W[i,j] x[j],
with W decoded per muser-book Ch 6 sections 6.2-6.4; and the embedding
lookup of Ch 6 section 6.7, out[t] = row ids[t] of the dequantized table.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kq_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libkqoracle.so")

Q4_K, Q5_K, Q6_K = 12, 13, 14
FORMATS = (Q4_K, Q5_K, Q6_K)

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP for row splits)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-fopenmp", "-Wall", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.oracle_block_bytes.argtypes = [ctypes.c_int]
        L.oracle_block_bytes.restype = ctypes.c_int
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_decode_block.argtypes = [ctypes.c_int, u8p, i32p, i32p, i32p, f64p, f64p]
        L.oracle_decode_block.restype = ctypes.c_int
        L.oracle_dequant.argtypes = [ctypes.c_int, u8p, ctypes.c_int64, ctypes.c_int64, f64p]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_matvec.argtypes = [ctypes.c_int, u8p, ctypes.c_int64, ctypes.c_int64, f32p,
                                    ctypes.c_int64, ctypes.c_int32, i64p, ctypes.c_int64,
                                    f64p, f64p, ctypes.c_int32]
        L.oracle_matvec.restype = ctypes.c_int
        L.oracle_embed.argtypes = [ctypes.c_int, u8p, ctypes.c_int64, ctypes.c_int64, i32p, ctypes.c_int64, f64p]
        L.oracle_embed.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def block_bytes(fmt: int) -> int:
    return lib().oracle_block_bytes(fmt)


def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(bits)


def decode_block(fmt: int, block) -> dict:
    """Integer decode of one super-block (see kq_oracle.c oracle_decode_block)."""
    b = np.ascontiguousarray(np.frombuffer(bytes(block), dtype=np.uint8))
    if b.size != block_bytes(fmt):
        raise ValueError("block has %d bytes, format %d needs %d" % (b.size, fmt, block_bytes(fmt)))
    codes = np.zeros(256, np.int32)
    scale = np.zeros(16, np.int32)
    minv = np.zeros(16, np.int32)
    d = ctypes.c_double()
    dmin = ctypes.c_double()
    rc = lib().oracle_decode_block(fmt, _ptr(b, ctypes.c_uint8), _ptr(codes, ctypes.c_int32),
                                   _ptr(scale, ctypes.c_int32), _ptr(minv, ctypes.c_int32),
                                   ctypes.byref(d), ctypes.byref(dmin))
    if rc:
        raise ValueError("unknown format %r" % fmt)
    return {"codes": codes, "scale": scale, "min": minv, "d": d.value, "dmin": dmin.value}


def dequant(fmt: int, w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Exact dequantized weights, float64 [rows, cols]."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    need = rows * (cols // 256) * block_bytes(fmt)
    if w.size < need:
        raise ValueError("weight buffer too small")
    out = np.empty((rows, cols), np.float64)
    rc = lib().oracle_dequant(fmt, _ptr(w, ctypes.c_uint8), rows, cols, _ptr(out, ctypes.c_double))
    if rc:
        raise ValueError("bad format or cols")
    return out


def embed(fmt: int, w: np.ndarray, rows: int, cols: int, ids) -> np.ndarray:
    """Embedding rows, float64 [n, cols]: row ids[t] of the dequantized
    table, element by element (muser-book Ch 6 section 6.7); NaN rows for
    ids outside [0, rows)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    ids = np.ascontiguousarray(np.atleast_1d(ids), dtype=np.int32)
    need = rows * (cols // 256) * block_bytes(fmt)
    if w.size < need:
        raise ValueError("weight buffer too small")
    out = np.empty((ids.size, cols), np.float64)
    rc = lib().oracle_embed(fmt, _ptr(w, ctypes.c_uint8), rows, cols, _ptr(ids, ctypes.c_int32), ids.size,
                            _ptr(out, ctypes.c_double))
    if rc:
        raise ValueError("bad format, rows or cols")
    return out


def matvec(fmt: int, w: np.ndarray, rows: int, cols: int, x: np.ndarray,
           row_idx=None, nthreads: int = 1):
    """(y, s) float64 [ntok, n_out]: y = W x and s = sum |W_ij x_j| per row.

    ``x`` is float32 [ntok, cols] (or [cols]); ``row_idx`` selects rows
    (default: all rows)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    ntok = x.shape[0]
    if x.shape[1] != cols:
        raise ValueError("x has %d columns, expected %d" % (x.shape[1], cols))
    need = rows * (cols // 256) * block_bytes(fmt)
    if w.size < need:
        raise ValueError("weight buffer too small")
    if row_idx is None:
        idx_p = None
        n_out = rows
    else:
        idx = np.ascontiguousarray(row_idx, dtype=np.int64)
        idx_p = _ptr(idx, ctypes.c_int64)
        n_out = idx.size
    y = np.empty((ntok, n_out), np.float64)
    s = np.empty((ntok, n_out), np.float64)
    rc = lib().oracle_matvec(fmt, _ptr(w, ctypes.c_uint8), rows, cols, _ptr(x, ctypes.c_float),
                             cols, ntok, idx_p, n_out, _ptr(y, ctypes.c_double),
                             _ptr(s, ctypes.c_double), int(nthreads))
    if rc:
        raise ValueError("oracle_matvec failed with %d" % rc)
    return y, s
