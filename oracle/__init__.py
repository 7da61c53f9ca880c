"""CPU oracle of the 3LC codec: plain C, single-threaded, fp32 IEEE arithmetic.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never links, loads or calls it, and it shares no code with the GPU path.

The C source (``tlc_oracle.c``) follows the 3LC review page ("3LC:
Lightweight and Effective Traffic Compression for Distributed Machine
Learning", section "Proposed method"): error accumulation and ternary
quantization with a sparsity multiplier, quartic encoding, zero-run encoding,
and the reverse path.  This module only builds the shared object with gcc and
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tlc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# fp32 must stay binary32 with no contraction: the oracle's results are
# compared bit for bit.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Werror"]

OK = 0
ERR_INVALID_ARG = 1
ERR_CAPACITY = 2
ERR_CORRUPT = 5
ERR_RANGE = 6


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle error code {code}")
        self.code = code


def build(extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile tlc_oracle.c with gcc into liboracle.so (or ``out``)."""
    out = out or _LIB
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
                or os.path.getmtime(_LIB) < os.path.getmtime(os.path.join(_HERE, "tlc_oracle.h"))):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        U64 = ctypes.c_uint64
        F = ctypes.c_float
        sigs = {
            "tlco_quartic_len": (U64, [U64]),
            "tlco_quantize": (ctypes.c_int, [P, P, U64, F, P, P]),
            "tlco_quartic_pack": (ctypes.c_int, [P, U64, P]),
            "tlco_quartic_unpack": (ctypes.c_int, [P, U64, P]),
            "tlco_zre_encode": (ctypes.c_int, [P, U64, P, U64, P]),
            "tlco_zre_decode": (ctypes.c_int, [P, U64, P, U64]),
            "tlco_compress": (ctypes.c_int, [P, P, U64, F, P, U64, P, P]),
            "tlco_decompress": (ctypes.c_int, [P, U64, F, U64, F, P]),
            "tlco_decompress_accumulate": (ctypes.c_int, [P, U64, F, U64, F, P]),
            "tlco_server_compress": (ctypes.c_int, [P, ctypes.c_uint32, P, U64, F, P, U64, P, P]),
            "tlco_fixed_len": (U64, [U64, ctypes.c_int]),
            "tlco_pack_fixed": (ctypes.c_int, [P, U64, ctypes.c_int, P]),
            "tlco_unpack_fixed": (ctypes.c_int, [P, U64, ctypes.c_int, P]),
            "tlco_compress_fixed": (ctypes.c_int, [P, P, U64, F, ctypes.c_int, P, U64, P]),
            "tlco_decompress_fixed": (ctypes.c_int, [P, F, U64, F, ctypes.c_int, P]),
            "tlco_quartic_pack_planes": (ctypes.c_int, [P, U64, P]),
            "tlco_quartic_unpack_planes": (ctypes.c_int, [P, U64, P]),
            "tlco_compress_planes": (ctypes.c_int, [P, P, U64, F, P, U64, P, P]),
            "tlco_decompress_planes": (ctypes.c_int, [P, U64, F, U64, F, P]),
            "tlco_wire_pack": (ctypes.c_int, [P, P, P, P, ctypes.c_uint32, P, U64, P]),
            "tlco_wire_unpack": (ctypes.c_int, [P, U64, ctypes.c_uint32, P, P, P, P, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(rc, what)


def _f32(a, writable=False) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if writable and not a.flags.writeable:
        a = a.copy()
    return a


def quartic_len(n: int) -> int:
    return int(lib().tlco_quartic_len(n))


def quantize(x, err, s: float):
    """Returns (q int8[n], M float32, err_new float32[n]); inputs are not modified."""
    x = _f32(x)
    e = _f32(err).copy()
    q = np.empty(x.size, dtype=np.int8)
    M = ctypes.c_float()
    _check(lib().tlco_quantize(_ptr(x), _ptr(e), x.size, s, _ptr(q), ctypes.byref(M)), "quantize")
    return q, np.float32(M.value), e


def quartic_pack(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    b = np.empty(quartic_len(q.size), dtype=np.uint8)
    _check(lib().tlco_quartic_pack(_ptr(q), q.size, _ptr(b)), "quartic_pack")
    return b


def quartic_unpack(b, n: int) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    if b.size < quartic_len(n):
        raise ValueError("byte array shorter than ceil(n/5)")
    q = np.empty(n, dtype=np.int8)
    _check(lib().tlco_quartic_unpack(_ptr(b), n, _ptr(q)), "quartic_unpack")
    return q


def zre_encode(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(max(b.size, 1), dtype=np.uint8)
    L = ctypes.c_uint64()
    _check(lib().tlco_zre_encode(_ptr(b), b.size, _ptr(out), out.size, ctypes.byref(L)), "zre_encode")
    return out[: L.value].copy()


def zre_decode(stream, B: int) -> np.ndarray:
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    out = np.empty(max(B, 1), dtype=np.uint8)
    _check(lib().tlco_zre_decode(_ptr(stream), stream.size, _ptr(out), B), "zre_decode")
    return out[:B].copy()


def compress(x, err, s: float):
    """Returns (stream uint8[L], M float32, err_new float32[n]); inputs are not modified."""
    x = _f32(x)
    e = _f32(err).copy()
    cap = quartic_len(x.size)
    out = np.empty(max(cap, 1), dtype=np.uint8)
    L = ctypes.c_uint64()
    M = ctypes.c_float()
    _check(lib().tlco_compress(_ptr(x), _ptr(e), x.size, s, _ptr(out), cap,
                               ctypes.byref(L), ctypes.byref(M)), "compress")
    return out[: L.value].copy(), np.float32(M.value), e


def compress_inplace(x: np.ndarray, err: np.ndarray, s: float, out: np.ndarray):
    """Allocation-free form for timing: err and out are updated in place.  Returns (L, M)."""
    L = ctypes.c_uint64()
    M = ctypes.c_float()
    _check(lib().tlco_compress(_ptr(x), _ptr(err), x.size, s, _ptr(out), out.size,
                               ctypes.byref(L), ctypes.byref(M)), "compress")
    return int(L.value), np.float32(M.value)


def decompress(stream, M, n: int, s: float, out: np.ndarray | None = None) -> np.ndarray:
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    y = np.empty(n, dtype=np.float32) if out is None else out
    _check(lib().tlco_decompress(_ptr(stream), stream.size, float(M), n, s, _ptr(y)), "decompress")
    return y


def decompress_accumulate(stream, M, n: int, s: float, acc: np.ndarray) -> np.ndarray:
    """acc (float32, contiguous) is updated in place and returned."""
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    if acc.dtype != np.float32 or not acc.flags.c_contiguous or acc.size != n:
        raise ValueError("acc must be a contiguous float32 array of n elements")
    _check(lib().tlco_decompress_accumulate(_ptr(stream), stream.size, float(M), n, s, _ptr(acc)),
           "decompress_accumulate")
    return acc


def server_compress(acc, workers: int, err, s: float):
    """Model-delta direction: compress of acc / workers with the server's error buffer.
    Returns (stream uint8[L], M float32, err_new float32[n]); inputs are not modified."""
    acc = _f32(acc)
    e = _f32(err).copy()
    cap = quartic_len(acc.size)
    out = np.empty(max(cap, 1), dtype=np.uint8)
    L = ctypes.c_uint64()
    M = ctypes.c_float()
    _check(lib().tlco_server_compress(_ptr(acc), workers, _ptr(e), acc.size, s, _ptr(out), cap,
                                      ctypes.byref(L), ctypes.byref(M)), "server_compress")
    return out[: L.value].copy(), np.float32(M.value), e


ENC_QUARTIC = 1  # quartic bytes without zero-run encoding
ENC_TWOBIT = 2   # 2-bit fields, four values per byte


def fixed_len(n: int, encoding: int) -> int:
    return int(lib().tlco_fixed_len(n, encoding))


def pack_fixed(q, encoding: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    out = np.empty(max(fixed_len(q.size, encoding), 1), dtype=np.uint8)
    _check(lib().tlco_pack_fixed(_ptr(q), q.size, encoding, _ptr(out)), "pack_fixed")
    return out[: fixed_len(q.size, encoding)].copy()


def unpack_fixed(b, n: int, encoding: int) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    q = np.empty(max(n, 1), dtype=np.int8)
    _check(lib().tlco_unpack_fixed(_ptr(b), n, encoding, _ptr(q)), "unpack_fixed")
    return q[:n].copy()


def compress_fixed(x, err, s: float, encoding: int):
    """Fixed-length encoding of the quantized codes (no zero-run encoding).
    Returns (bytes uint8[fixed_len], M float32, err_new float32[n])."""
    x = _f32(x)
    e = _f32(err).copy()
    nb = fixed_len(x.size, encoding)
    out = np.empty(max(nb, 1), dtype=np.uint8)
    M = ctypes.c_float()
    _check(lib().tlco_compress_fixed(_ptr(x), _ptr(e), x.size, s, encoding, _ptr(out), nb, ctypes.byref(M)),
           "compress_fixed")
    return out[:nb].copy(), np.float32(M.value), e


def decompress_fixed(stream, M, n: int, s: float, encoding: int) -> np.ndarray:
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    if stream.size < fixed_len(n, encoding):
        raise ValueError("stream shorter than the fixed length")
    y = np.empty(n, dtype=np.float32)
    _check(lib().tlco_decompress_fixed(_ptr(stream), float(M), n, s, encoding, _ptr(y)), "decompress_fixed")
    return y


def rc_of(fn_name: str, *args) -> int:
    """Raw return code of an oracle entry point (for error-path tests)."""
    return int(getattr(lib(), fn_name)(*args))


# Five-plane layout (the other reading of which five values share a byte):
# byte k holds elements k + j*B, j = 0..4, as digit j; B = ceil(n/5).

def quartic_pack_planes(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    b = np.empty(quartic_len(q.size), dtype=np.uint8)
    _check(lib().tlco_quartic_pack_planes(_ptr(q), q.size, _ptr(b)), "quartic_pack_planes")
    return b


def quartic_unpack_planes(b, n: int) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    if b.size < quartic_len(n):
        raise ValueError("byte array shorter than ceil(n/5)")
    q = np.empty(n, dtype=np.int8)
    _check(lib().tlco_quartic_unpack_planes(_ptr(b), n, _ptr(q)), "quartic_unpack_planes")
    return q


def compress_planes(x, err, s: float):
    """As compress, with the five-plane byte layout.  Returns (stream, M, err_new)."""
    x = _f32(x)
    e = _f32(err).copy()
    cap = quartic_len(x.size)
    out = np.empty(max(cap, 1), dtype=np.uint8)
    L = ctypes.c_uint64()
    M = ctypes.c_float()
    _check(lib().tlco_compress_planes(_ptr(x), _ptr(e), x.size, s, _ptr(out), cap,
                                      ctypes.byref(L), ctypes.byref(M)), "compress_planes")
    return out[: L.value].copy(), np.float32(M.value), e


def decompress_planes(stream, M, n: int, s: float) -> np.ndarray:
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    y = np.empty(n, dtype=np.float32)
    _check(lib().tlco_decompress_planes(_ptr(stream), stream.size, float(M), n, s, _ptr(y)), "decompress_planes")
    return y


# Wire message of a group (what one worker would send): count headers of
# 8 bytes (L_t as little-endian uint32, M_t as little-endian fp32), then the
# streams back to back.  A layout of this library, not of the pages.

def wire_pack(streams, Ms) -> np.ndarray:
    """The wire message of tensors whose streams and scales are given."""
    count = len(streams)
    lens = np.array([np.asarray(st).size for st in streams], dtype=np.uint64)
    offs = np.zeros(count, dtype=np.uint64)
    if count > 1:
        offs[1:] = np.cumsum(lens)[:-1]
    flat = np.concatenate([np.asarray(st, dtype=np.uint8) for st in streams] + [np.zeros(1, np.uint8)])
    M = np.ascontiguousarray(Ms, dtype=np.float32)
    cap = 8 * count + int(lens.sum())
    wire = np.zeros(max(cap, 1), dtype=np.uint8)
    wl = ctypes.c_uint64(0)
    _check(lib().tlco_wire_pack(_ptr(flat), _ptr(offs), _ptr(lens), _ptr(M), count, _ptr(wire), cap,
                                ctypes.byref(wl)), "wire_pack")
    return wire[:wl.value]


def wire_unpack(wire, sizes):
    """(streams, Ms) of a wire message for tensors of the given sizes; raises
    OracleError(ERR_CORRUPT) on a malformed message."""
    count = len(sizes)
    caps = np.array([quartic_len(int(n)) for n in sizes], dtype=np.uint64)
    offs = np.zeros(count, dtype=np.uint64)
    if count > 1:
        offs[1:] = np.cumsum(caps)[:-1]
    out = np.zeros(int(caps.sum()) + 1, dtype=np.uint8)
    lens = np.zeros(count, dtype=np.uint64)
    M = np.zeros(count, dtype=np.float32)
    w = np.ascontiguousarray(wire, dtype=np.uint8)
    w1 = w if w.size else np.zeros(1, np.uint8)
    _check(lib().tlco_wire_unpack(_ptr(w1), w.size, count, _ptr(caps), _ptr(out), _ptr(offs), _ptr(lens), _ptr(M)),
           "wire_unpack")
    streams = [out[int(o):int(o) + int(l)].copy() for o, l in zip(offs, lens)]
    return streams, M
