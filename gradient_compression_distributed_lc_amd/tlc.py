"""Python binding of libtlc.so (the C ABI in include/tlc.h).

Argument marshalling only: PyTorch allocates device memory and provides the
HIP stream; every step of the codec runs in the library's HIP kernels.  The
entry points have the same names as the C functions without the ``tlc_``
prefix.  If the library is missing this module raises instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from . import build as _build

OK = 0
ERR_INVALID_ARG = 1
ERR_CAPACITY = 2
ERR_WORKSPACE = 3
ERR_HIP = 4
ERR_CORRUPT = 5
ERR_INTERNAL = 6
ERR_TOO_LARGE = 7


class TLCError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} (code {code})")
        self.code = code


class GroupInfo(ctypes.Structure):
    _fields_ = [("count", ctypes.c_uint64), ("total_elems", ctypes.c_uint64),
                ("stream_bytes", ctypes.c_uint64), ("table_bytes", ctypes.c_uint64),
                ("workspace_bytes", ctypes.c_uint64), ("tiles", ctypes.c_uint64),
                ("chunks", ctypes.c_uint64), ("spans", ctypes.c_uint64)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_uint64), ("total_ms", ctypes.c_double)]


_lib = None

_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_F = ctypes.c_float
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_U32 = ctypes.c_uint32

_SIGS = {
    "tlc_status_string": (ctypes.c_char_p, [_I]),
    "tlc_version": (ctypes.c_char_p, []),
    "tlc_compress_bound": (_U64, [_U64]),
    "tlc_workspace_size": (_SZ, [_U64]),
    "tlc_compress": (_I, [_P, _P, _U64, _F, _P, _U64, _P, _P, _P, _SZ, _P, _P]),
    "tlc_compress_static": (_I, [_P, _P, _U64, _F, _P, _U64, _P, _P, _P, _P]),
    "tlc_compress_static_max_n": (_U64, []),
    "tlc_server_compress": (_I, [_P, _U32, _P, _U64, _F, _P, _U64, _P, _P, _P, _SZ, _P, _P]),
    "tlc_fixed_len": (_U64, [_U64, _I]),
    "tlc_compress_fixed": (_I, [_P, _P, _U64, _F, _I, _P, _U64, _P, _P, _SZ, _P, _P]),
    "tlc_decompress_fixed": (_I, [_P, _P, _U64, _F, _I, _P, _P, _P]),
    "tlc_compress_fixed_group": (_I, [ctypes.POINTER(GroupInfo), _P, _I, _P, _P, _F, _P, _P, _P, _P, _SZ, _P, _P]),
    "tlc_decompress_fixed_group": (_I, [ctypes.POINTER(GroupInfo), _P, _I, _P, _P, _P, _F, _P, _P, _P]),
    "tlc_decompress": (_I, [_P, _P, _P, _U64, _F, _P, _P, _SZ, _P, _P, _P]),
    "tlc_decompress_accumulate": (_I, [_P, _P, _P, _U64, _F, _P, _P, _SZ, _P, _P]),
    "tlc_group_plan": (_I, [_P, _U64, ctypes.POINTER(GroupInfo), _P, _SZ, _P]),
    "tlc_compress_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _P, _F, _P, _P, _P, _P, _SZ, _P, _P]),
    "tlc_server_compress_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _U32, _P, _F, _P, _P, _P, _P, _SZ,
                                       _P, _P]),
    "tlc_decompress_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _P, _P, _F, _P, _P, _SZ, _P, _P, _P]),
    "tlc_decompress_accumulate_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _P, _P, _F, _P, _P, _SZ,
                                             _P, _P]),
    "tlc_accumulate_many_workspace_size": (_U64, [ctypes.POINTER(GroupInfo), _U32]),
    "tlc_decompress_accumulate_many_group": (_I, [ctypes.POINTER(GroupInfo), _P, _U32, _P, _U64, _P, _P, _F, _P,
                                                  _P, _SZ, _P, _P, _P]),
    "tlc_wire_bound": (_U64, [ctypes.POINTER(GroupInfo)]),
    "tlc_wire_workspace_size": (_U64, [ctypes.POINTER(GroupInfo)]),
    "tlc_wire_pack_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _P, _P, _P, _U64, _P, _P, _SZ, _P, _P]),
    "tlc_wire_unpack_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _U64, _P, _P, _P, _P, _SZ, _P, _P]),
    "tlc_wire_pack_ranges_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _U32, _P, _P, _P, _P, _U64, _P, _P, _SZ,
                                        _P, _P]),
    "tlc_wire_unpack_ranges_group": (_I, [ctypes.POINTER(GroupInfo), _P, _P, _U32, _P, _U64, _P, _P, _P, _P, _SZ,
                                          _P, _P]),
    "tlc_planes_gather": (_I, [_P, _P, _P, _P, _P, _U32, _U64, _P]),
    "tlc_planes_scatter": (_I, [_P, _P, _P, _P, _P, _U32, _U64, _P]),
    "tlc_gather_probe": (_I, [_P, _P, _U64, _P, _P]),
    "tlc_copy_probe": (_I, [_P, _P, _U64, _P]),
    "tlc_profile_enable": (_I, [_I]),
    "tlc_profile_read": (_I, [ctypes.POINTER(KernelTime), _I, ctypes.POINTER(_I)]),
    "tlc_profile_only": (_I, [ctypes.c_char_p]),
}


def library_path() -> str:
    return _build.LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m gradient_compression_distributed_lc_amd.build`"
                               " (or __graft_entry__.build())")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(code: int) -> str:
    try:
        return lib().tlc_status_string(int(code)).decode()
    except RuntimeError:
        return f"status {code}"


def _check(rc: int, what: str):
    if rc != OK:
        raise TLCError(rc, what)


def _ptr(t: torch.Tensor | None, dtype: torch.dtype | None = None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def path_hint() -> torch.Tensor:
    """A decompress path hint word: one uint32 (held as int32) in pinned host
    memory, starting at 0 (the sparse sequence).  Pass the same tensor to
    every decompress of a stream of steps; the device keeps it up to date."""
    return torch.zeros(1, dtype=torch.int32, pin_memory=True)


def _hint_ptr(h: torch.Tensor | None):
    if h is None:
        return None
    if h.is_cuda or not h.is_pinned():
        raise ValueError("path_hint must be a pinned host tensor (tlc.path_hint())")
    if h.dtype != torch.int32 or h.numel() < 1 or not h.is_contiguous():
        raise ValueError("path_hint must hold one contiguous int32")
    return ctypes.c_void_p(h.data_ptr())


def _need(t: torch.Tensor | None, count: int, name: str):
    """Raise unless t holds at least `count` elements (checked before any
    pointer is handed to the library, so an undersized buffer never reaches a
    kernel)."""
    if t is not None and t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {count}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def compress_bound(n: int) -> int:
    return int(lib().tlc_compress_bound(n))


def workspace_size(n: int) -> int:
    return int(lib().tlc_workspace_size(n))


def version() -> str:
    return lib().tlc_version().decode()


@dataclass
class Compressed:
    """A compressed tensor.  ``out`` has capacity ``ceil(n/5)``; the stream is
    ``out[:length]`` where ``length`` is the device scalar ``out_len``."""
    out: torch.Tensor       # uint8[ceil(n/5)]
    out_len: torch.Tensor   # int64[1] (the C side writes a uint64)
    scale: torch.Tensor     # float32[1]
    status: torch.Tensor    # int32[1]
    n: int
    s: float

    def stream(self) -> torch.Tensor:
        return self.out[: int(self.out_len.item())]


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return workspace


def compress(x: torch.Tensor, err: torch.Tensor, s: float, *, out=None, out_len=None, scale=None,
             workspace=None, status=None, stream=None) -> Compressed:
    n = x.numel()
    dev = x.device
    if err.numel() != n:
        raise ValueError("err must have as many elements as x")
    out = out if out is not None else torch.empty(max(compress_bound(n), 1), dtype=torch.uint8, device=dev)
    out_len = out_len if out_len is not None else torch.empty(1, dtype=torch.int64, device=dev)
    scale = scale if scale is not None else torch.zeros(1, dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
    _need(out_len, 1, "out_len")
    _need(scale, 1, "scale")
    _need(status, 1, "status")
    workspace = _workspace(workspace_size(n), dev, workspace)
    rc = lib().tlc_compress(_ptr(x, torch.float32, "x"), _ptr(err, torch.float32, "err"), n, s,
                            _ptr(out, torch.uint8, "out"), out.numel(), _ptr(out_len, torch.int64, "out_len"),
                            _ptr(scale, torch.float32, "scale"), _ptr(workspace, torch.uint8, "workspace"),
                            workspace.numel(), _ptr(status, torch.int32, "status"), _stream(stream))
    _check(rc, "tlc_compress")
    return Compressed(out, out_len, scale, status, n, s)


def compress_static_max_n() -> int:
    return int(lib().tlc_compress_static_max_n())


def compress_static(x: torch.Tensor, err: torch.Tensor, s: float, *, out=None, out_len=None, scale=None,
                    status=None, stream=None) -> Compressed:
    """tlc_compress_static: tlc_compress with the library's fixed scratch array
    instead of a workspace (for callers that cannot allocate).  Buffers the
    caller does not pass are allocated here, by torch; pass them all to keep
    the call free of allocation."""
    n = x.numel()
    dev = x.device
    if err.numel() != n:
        raise ValueError("err must have as many elements as x")
    out = out if out is not None else torch.empty(max(compress_bound(n), 1), dtype=torch.uint8, device=dev)
    out_len = out_len if out_len is not None else torch.empty(1, dtype=torch.int64, device=dev)
    scale = scale if scale is not None else torch.zeros(1, dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
    _need(out_len, 1, "out_len")
    _need(scale, 1, "scale")
    _need(status, 1, "status")
    rc = lib().tlc_compress_static(_ptr(x, torch.float32, "x"), _ptr(err, torch.float32, "err"), n, s,
                                   _ptr(out, torch.uint8, "out"), out.numel(),
                                   _ptr(out_len, torch.int64, "out_len"), _ptr(scale, torch.float32, "scale"),
                                   _ptr(status, torch.int32, "status"), _stream(stream))
    _check(rc, "tlc_compress_static")
    return Compressed(out, out_len, scale, status, n, s)


def server_compress(acc: torch.Tensor, workers: int, err: torch.Tensor, s: float, *, out=None, out_len=None,
                    scale=None, workspace=None, status=None, stream=None) -> Compressed:
    """Model-delta direction: compress the workers' mean acc / workers with the
    server's error buffer err (updated in place)."""
    n = acc.numel()
    dev = acc.device
    if err.numel() != n:
        raise ValueError("err must have as many elements as acc")
    out = out if out is not None else torch.empty(max(compress_bound(n), 1), dtype=torch.uint8, device=dev)
    out_len = out_len if out_len is not None else torch.empty(1, dtype=torch.int64, device=dev)
    scale = scale if scale is not None else torch.zeros(1, dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
    _need(out_len, 1, "out_len")
    _need(scale, 1, "scale")
    _need(status, 1, "status")
    workspace = _workspace(workspace_size(n), dev, workspace)
    rc = lib().tlc_server_compress(_ptr(acc, torch.float32, "acc"), workers, _ptr(err, torch.float32, "err"), n,
                                   s, _ptr(out, torch.uint8, "out"), out.numel(),
                                   _ptr(out_len, torch.int64, "out_len"), _ptr(scale, torch.float32, "scale"),
                                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                   _ptr(status, torch.int32, "status"), _stream(stream))
    _check(rc, "tlc_server_compress")
    return Compressed(out, out_len, scale, status, n, s)


ENC_QUARTIC = 1  # quartic bytes without zero-run encoding, ceil(n/5) bytes
ENC_TWOBIT = 2   # 2-bit fields, four values per byte, ceil(n/4) bytes


def fixed_len(n: int, encoding: int) -> int:
    return int(lib().tlc_fixed_len(n, encoding))


def compress_fixed(x: torch.Tensor, err: torch.Tensor, s: float, encoding: int, *, out=None, scale=None,
                   workspace=None, status=None, stream=None):
    """Fixed-length encoding of the codes (no zero-run encoding).  Returns (out, scale, status)."""
    n = x.numel()
    dev = x.device
    if err.numel() != n:
        raise ValueError("err must have as many elements as x")
    nb = fixed_len(n, encoding)
    if nb == 0:
        raise ValueError("bad size or encoding")
    out = out if out is not None else torch.empty(nb, dtype=torch.uint8, device=dev)
    scale = scale if scale is not None else torch.zeros(1, dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
    _need(scale, 1, "scale")
    _need(status, 1, "status")
    workspace = _workspace(workspace_size(n), dev, workspace)
    rc = lib().tlc_compress_fixed(_ptr(x, torch.float32, "x"), _ptr(err, torch.float32, "err"), n, s, encoding,
                                  _ptr(out, torch.uint8, "out"), out.numel(), _ptr(scale, torch.float32, "scale"),
                                  _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                  _ptr(status, torch.int32, "status"), _stream(stream))
    _check(rc, "tlc_compress_fixed")
    return out, scale, status


def decompress_fixed(inp: torch.Tensor, scale: torch.Tensor, n: int, s: float, encoding: int, *, y=None,
                     status=None, stream=None):
    """Returns (y, status)."""
    dev = inp.device
    y = y if y is not None else torch.empty(n, dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
    nb = fixed_len(n, encoding)
    if nb == 0:
        raise ValueError("bad size or encoding")
    _need(inp, nb, "in")
    _need(scale, 1, "scale")
    _need(y, n, "y")
    _need(status, 1, "status")
    rc = lib().tlc_decompress_fixed(_ptr(inp, torch.uint8, "in"), _ptr(scale, torch.float32, "scale"), n, s,
                                    encoding, _ptr(y, torch.float32, "y"), _ptr(status, torch.int32, "status"),
                                    _stream(stream))
    _check(rc, "tlc_decompress_fixed")
    return y, status


def decompress(inp: torch.Tensor, in_len: torch.Tensor, scale: torch.Tensor, n: int, s: float, *, y=None,
               workspace=None, status=None, path_hint=None, stream=None):
    """Returns (y, status).  inp holds at least ceil(n/5) bytes (the capacity
    tlc_compress writes into), so that no device length can send a read past
    its end.  path_hint: None (sparse sequence) or a tensor from
    tlc.path_hint(), read on entry and rewritten by the device."""
    dev = inp.device
    y = y if y is not None else torch.empty(n, dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
    _need(inp, compress_bound(n), "in")
    _need(in_len, 1, "in_len")
    _need(scale, 1, "scale")
    _need(y, n, "y")
    _need(status, 1, "status")
    workspace = _workspace(workspace_size(n), dev, workspace)
    rc = lib().tlc_decompress(_ptr(inp, torch.uint8, "in"), _ptr(in_len, torch.int64, "in_len"),
                              _ptr(scale, torch.float32, "scale"), n, s, _ptr(y, torch.float32, "y"),
                              _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                              _ptr(status, torch.int32, "status"), _hint_ptr(path_hint), _stream(stream))
    _check(rc, "tlc_decompress")
    return y, status


def decompress_accumulate(inp: torch.Tensor, in_len: torch.Tensor, scale: torch.Tensor, n: int, s: float,
                          acc: torch.Tensor, *, workspace=None, status=None, stream=None):
    """acc is updated in place.  Returns (acc, status).  inp holds at least
    ceil(n/5) bytes, as for decompress."""
    dev = inp.device
    status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
    _need(inp, compress_bound(n), "in")
    _need(in_len, 1, "in_len")
    _need(scale, 1, "scale")
    _need(acc, n, "acc")
    _need(status, 1, "status")
    workspace = _workspace(workspace_size(n), dev, workspace)
    rc = lib().tlc_decompress_accumulate(_ptr(inp, torch.uint8, "in"), _ptr(in_len, torch.int64, "in_len"),
                                         _ptr(scale, torch.float32, "scale"), n, s,
                                         _ptr(acc, torch.float32, "acc"),
                                         _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                         _ptr(status, torch.int32, "status"), _stream(stream))
    _check(rc, "tlc_decompress_accumulate")
    return acc, status


def group_plan(sizes) -> tuple[GroupInfo, bytes, list[int]]:
    """Host-only: (info, table bytes, stream offsets) for tensors of the given sizes."""
    count = len(sizes)
    arr = (ctypes.c_uint64 * max(count, 1))(*[int(v) for v in sizes])
    info = GroupInfo()
    _check(lib().tlc_group_plan(arr, count, ctypes.byref(info), None, 0, None), "tlc_group_plan")
    table = ctypes.create_string_buffer(int(info.table_bytes))
    offs = (ctypes.c_uint64 * max(count, 1))()
    _check(lib().tlc_group_plan(arr, count, ctypes.byref(info), table, len(table), offs), "tlc_group_plan")
    return info, table.raw, [int(v) for v in offs[:count]]


class Group:
    """Tensors packed back to back in one flat fp32 buffer (a gradient bucket),
    compressed with one launch sequence.  M, error state and stream are per
    tensor; stream t lives at ``out[offsets[t]:]``."""

    def __init__(self, sizes, device="cuda"):
        self.sizes = [int(v) for v in sizes]
        self.info, table, self.offsets = group_plan(self.sizes)
        self.device = torch.device(device)
        host = torch.frombuffer(bytearray(table), dtype=torch.uint8)
        self.d_table = host.to(self.device)
        self.total = int(self.info.total_elems)
        self.stream_bytes = int(self.info.stream_bytes)
        self.workspace_bytes = int(self.info.workspace_bytes)
        self.count = len(self.sizes)
        eo = [0]
        for v in self.sizes:
            eo.append(eo[-1] + v)
        self.elem_offsets = eo

    def workspace(self) -> torch.Tensor:
        return torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=self.device)

    def compress(self, x, err, s, *, out=None, out_lens=None, scales=None, workspace=None, status=None,
                 stream=None):
        """Returns (out, out_lens, scales, status)."""
        if x.numel() != self.total or err.numel() != self.total:
            raise ValueError("x and err must hold the whole group")
        dev = self.device
        out = out if out is not None else torch.empty(self.stream_bytes, dtype=torch.uint8, device=dev)
        out_lens = out_lens if out_lens is not None else torch.empty(self.count, dtype=torch.int64, device=dev)
        scales = scales if scales is not None else torch.zeros(self.count, dtype=torch.float32, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        self._need_out(out, out_lens, scales, status)
        workspace = workspace if workspace is not None else self.workspace()
        rc = lib().tlc_compress_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                      _ptr(x, torch.float32, "x"), _ptr(err, torch.float32, "err"), s,
                                      _ptr(out, torch.uint8, "out"), _ptr(out_lens, torch.int64, "out_lens"),
                                      _ptr(scales, torch.float32, "scales"),
                                      _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                      _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_compress_group")
        return out, out_lens, scales, status

    def server_compress(self, acc, workers, err, s, *, out=None, out_lens=None, scales=None, workspace=None,
                        status=None, stream=None):
        """Model-delta direction: per tensor, compress acc / workers with the
        server's error buffer err.  Returns (out, out_lens, scales, status)."""
        if acc.numel() != self.total or err.numel() != self.total:
            raise ValueError("acc and err must hold the whole group")
        dev = self.device
        out = out if out is not None else torch.empty(self.stream_bytes, dtype=torch.uint8, device=dev)
        out_lens = out_lens if out_lens is not None else torch.empty(self.count, dtype=torch.int64, device=dev)
        scales = scales if scales is not None else torch.zeros(self.count, dtype=torch.float32, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        self._need_out(out, out_lens, scales, status)
        workspace = workspace if workspace is not None else self.workspace()
        rc = lib().tlc_server_compress_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                             _ptr(acc, torch.float32, "acc"), workers,
                                             _ptr(err, torch.float32, "err"), s, _ptr(out, torch.uint8, "out"),
                                             _ptr(out_lens, torch.int64, "out_lens"),
                                             _ptr(scales, torch.float32, "scales"),
                                             _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                             _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_server_compress_group")
        return out, out_lens, scales, status

    def _fixed_layout(self, encoding: int):
        offs, at = [], 0
        for n in self.sizes:
            offs.append(at)
            nb = fixed_len(n, encoding)
            if nb == 0:
                raise ValueError("bad size or encoding")
            at += -(-nb // 16) * 16
        return offs, at

    def fixed_offsets(self, encoding: int):
        """(host offsets, device uint64 offsets, total bytes) of a fixed-length
        encoding: tensors back to back, 16-byte aligned."""
        offs, at = self._fixed_layout(encoding)
        d = torch.tensor(offs, dtype=torch.int64, device=self.device)
        return offs, d, at

    def _need_out(self, out, out_lens, scales, status):
        _need(out, self.stream_bytes, "out")
        _need(out_lens, self.count, "out_lens")
        _need(scales, self.count, "scales")
        _need(status, 1, "status")

    def _need_in(self, inp, in_lens, scales, dst, name, status):
        _need(inp, self.stream_bytes, "in")
        _need(in_lens, self.count, "in_lens")
        _need(scales, self.count, "scales")
        _need(dst, self.total, name)
        _need(status, 1, "status")

    def compress_fixed(self, x, err, s, encoding, out, d_offsets, *, scales=None, workspace=None, status=None,
                       stream=None):
        """Codes of every tensor in a fixed-length encoding at out[d_offsets[t]]
        (d_offsets as fixed_offsets returns them).  Returns (scales, status)."""
        if x.numel() != self.total or err.numel() != self.total:
            raise ValueError("x and err must hold the whole group")
        dev = self.device
        scales = scales if scales is not None else torch.zeros(self.count, dtype=torch.float32, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        _need(out, self._fixed_layout(encoding)[1], "out")
        _need(d_offsets, self.count, "offsets")
        _need(scales, self.count, "scales")
        _need(status, 1, "status")
        workspace = workspace if workspace is not None else self.workspace()
        rc = lib().tlc_compress_fixed_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                            encoding, _ptr(x, torch.float32, "x"), _ptr(err, torch.float32, "err"),
                                            s, _ptr(out, torch.uint8, "out"), _ptr(d_offsets, torch.int64, "offsets"),
                                            _ptr(scales, torch.float32, "scales"),
                                            _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                            _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_compress_fixed_group")
        return scales, status

    def decompress_fixed(self, inp, d_offsets, scales, s, encoding, *, y=None, status=None, stream=None):
        """Returns (y, status)."""
        dev = self.device
        y = y if y is not None else torch.empty(self.total, dtype=torch.float32, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        _need(inp, self._fixed_layout(encoding)[1], "in")
        _need(d_offsets, self.count, "offsets")
        _need(scales, self.count, "scales")
        _need(y, self.total, "y")
        _need(status, 1, "status")
        rc = lib().tlc_decompress_fixed_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                              encoding, _ptr(inp, torch.uint8, "in"),
                                              _ptr(d_offsets, torch.int64, "offsets"),
                                              _ptr(scales, torch.float32, "scales"), s, _ptr(y, torch.float32, "y"),
                                              _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_decompress_fixed_group")
        return y, status

    def decompress(self, inp, in_lens, scales, s, *, y=None, workspace=None, status=None, path_hint=None,
                   stream=None):
        """Returns (y, status).  path_hint as for decompress()."""
        dev = self.device
        y = y if y is not None else torch.empty(self.total, dtype=torch.float32, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        self._need_in(inp, in_lens, scales, y, "y", status)
        workspace = workspace if workspace is not None else self.workspace()
        rc = lib().tlc_decompress_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                        _ptr(inp, torch.uint8, "in"), _ptr(in_lens, torch.int64, "in_lens"),
                                        _ptr(scales, torch.float32, "scales"), s, _ptr(y, torch.float32, "y"),
                                        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                        _ptr(status, torch.int32, "status"), _hint_ptr(path_hint),
                                        _stream(stream))
        _check(rc, "tlc_decompress_group")
        return y, status

    def decompress_accumulate(self, inp, in_lens, scales, s, acc, *, workspace=None, status=None, stream=None):
        """acc is updated in place.  Returns (acc, status)."""
        dev = self.device
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        self._need_in(inp, in_lens, scales, acc, "acc", status)
        workspace = workspace if workspace is not None else self.workspace()
        rc = lib().tlc_decompress_accumulate_group(
            ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"), _ptr(inp, torch.uint8, "in"),
            _ptr(in_lens, torch.int64, "in_lens"), _ptr(scales, torch.float32, "scales"), s,
            _ptr(acc, torch.float32, "acc"), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
            _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_decompress_accumulate_group")
        return acc, status

    def wire_bound(self) -> int:
        """Most bytes a wire message of this group can need."""
        return int(lib().tlc_wire_bound(ctypes.byref(self.info)))

    def wire_workspace(self) -> torch.Tensor:
        nb = int(lib().tlc_wire_workspace_size(ctypes.byref(self.info)))
        return torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)

    def wire_pack(self, inp, in_lens, scales, *, wire=None, wire_len=None, workspace=None, status=None,
                  stream=None):
        """tlc_wire_pack_group: the payload (inp, in_lens, scales) as one
        contiguous message.  Returns (wire, wire_len, status); the message is
        wire[:wire_len]."""
        dev = self.device
        wire = wire if wire is not None else torch.empty(self.wire_bound(), dtype=torch.uint8, device=dev)
        wire_len = wire_len if wire_len is not None else torch.empty(1, dtype=torch.int64, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        _need(inp, self.stream_bytes, "in")
        _need(in_lens, self.count, "in_lens")
        _need(scales, self.count, "scales")
        _need(wire, self.wire_bound(), "wire")
        _need(wire_len, 1, "wire_len")
        _need(status, 1, "status")
        workspace = workspace if workspace is not None else self.wire_workspace()
        rc = lib().tlc_wire_pack_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                       _ptr(inp, torch.uint8, "in"), _ptr(in_lens, torch.int64, "in_lens"),
                                       _ptr(scales, torch.float32, "scales"), _ptr(wire, torch.uint8, "wire"),
                                       wire.numel(), _ptr(wire_len, torch.int64, "wire_len"),
                                       _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                       _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_wire_pack_group")
        return wire, wire_len, status

    def wire_pack_ranges(self, inp, in_lens, scales, cuts, *, wire=None, wire_lens=None, workspace=None,
                         status=None, stream=None):
        """tlc_wire_pack_ranges_group: one message per consecutive range of
        tensors (range k: tensors cuts[k] .. cuts[k+1]-1), back to back.
        Returns (wire, wire_lens, status); message k is
        wire[sum(wire_lens[:k]) : sum(wire_lens[:k+1])]."""
        dev = self.device
        c_cuts, n = self._cuts(cuts)
        wire = wire if wire is not None else torch.empty(self.wire_bound(), dtype=torch.uint8, device=dev)
        wire_lens = wire_lens if wire_lens is not None else torch.empty(n, dtype=torch.int64, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        _need(inp, self.stream_bytes, "in")
        _need(in_lens, self.count, "in_lens")
        _need(scales, self.count, "scales")
        _need(wire, self.wire_bound(), "wire")
        _need(wire_lens, n, "wire_lens")
        _need(status, 1, "status")
        workspace = workspace if workspace is not None else self.wire_workspace()
        rc = lib().tlc_wire_pack_ranges_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                              c_cuts, n, _ptr(inp, torch.uint8, "in"),
                                              _ptr(in_lens, torch.int64, "in_lens"),
                                              _ptr(scales, torch.float32, "scales"), _ptr(wire, torch.uint8, "wire"),
                                              wire.numel(), _ptr(wire_lens, torch.int64, "wire_lens"),
                                              _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                              _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_wire_pack_ranges_group")
        return wire, wire_lens, status

    def _cuts(self, cuts):
        cuts = [int(c) for c in cuts]
        n = len(cuts) - 1
        if n < 1 or n > 64 or cuts[0] != 0 or cuts[-1] != self.count or any(a >= b for a, b in zip(cuts, cuts[1:])):
            raise ValueError("cuts must rise from 0 to the tensor count, 1 to 64 ranges")
        return (ctypes.c_uint32 * (n + 1))(*cuts), n

    def wire_unpack_ranges(self, wire, cuts, *, wire_bytes=None, out=None, out_lens=None, scales=None,
                           workspace=None, status=None, stream=None):
        """tlc_wire_unpack_ranges_group: the messages of the ranges cuts[k] ..
        cuts[k+1]-1, back to back in wire, into one payload of the group.
        Returns (out, out_lens, scales, status)."""
        dev = self.device
        c_cuts, n = self._cuts(cuts)
        out = out if out is not None else torch.empty(self.stream_bytes, dtype=torch.uint8, device=dev)
        out_lens = out_lens if out_lens is not None else torch.empty(self.count, dtype=torch.int64, device=dev)
        scales = scales if scales is not None else torch.empty(self.count, dtype=torch.float32, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        nb = wire.numel() if wire_bytes is None else int(wire_bytes)
        if nb > wire.numel():
            raise ValueError("wire_bytes exceeds the wire tensor")
        self._need_out(out, out_lens, scales, status)
        workspace = workspace if workspace is not None else self.wire_workspace()
        rc = lib().tlc_wire_unpack_ranges_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                                c_cuts, n, _ptr(wire, torch.uint8, "wire"), nb,
                                                _ptr(out, torch.uint8, "out"), _ptr(out_lens, torch.int64, "out_lens"),
                                                _ptr(scales, torch.float32, "scales"),
                                                _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                                _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_wire_unpack_ranges_group")
        return out, out_lens, scales, status

    def wire_unpack(self, wire, *, wire_bytes=None, out=None, out_lens=None, scales=None, workspace=None,
                    status=None, stream=None):
        """tlc_wire_unpack_group: a message back into a payload.  wire_bytes:
        how many bytes of `wire` may be read (default all of it).  Returns
        (out, out_lens, scales, status)."""
        dev = self.device
        out = out if out is not None else torch.empty(self.stream_bytes, dtype=torch.uint8, device=dev)
        out_lens = out_lens if out_lens is not None else torch.empty(self.count, dtype=torch.int64, device=dev)
        scales = scales if scales is not None else torch.empty(self.count, dtype=torch.float32, device=dev)
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        nb = wire.numel() if wire_bytes is None else int(wire_bytes)
        if nb > wire.numel():
            raise ValueError("wire_bytes exceeds the wire tensor")
        self._need_out(out, out_lens, scales, status)
        workspace = workspace if workspace is not None else self.wire_workspace()
        rc = lib().tlc_wire_unpack_group(ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"),
                                         _ptr(wire, torch.uint8, "wire"), nb, _ptr(out, torch.uint8, "out"),
                                         _ptr(out_lens, torch.int64, "out_lens"),
                                         _ptr(scales, torch.float32, "scales"),
                                         _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                         _ptr(status, torch.int32, "status"), _stream(stream))
        _check(rc, "tlc_wire_unpack_group")
        return out, out_lens, scales, status

    def accumulate_many_workspace_size(self, payloads: int) -> int:
        nb = int(lib().tlc_accumulate_many_workspace_size(ctypes.byref(self.info), int(payloads)))
        if nb == 0:
            raise ValueError(f"payloads must be 1..64 (and payloads x tensors below 2^31), got {payloads}")
        return nb

    def decompress_accumulate_many(self, inp, in_lens, scales, s, acc, *, payloads=None, workspace=None,
                                   status=None, path_hint=None, stream=None):
        """tlc_decompress_accumulate_many_group: payload p's streams in
        inp[p] (a uint8 tensor of shape (payloads, stream_bytes) or a flat
        one of payloads * stream_bytes), its lengths and scales in row p of
        in_lens / scales (payloads x count); acc += every payload's values in
        payload order.  path_hint: None (the dense sequence) or a word from
        path_hint() holding 0 (sparse) or 1 (dense), rewritten by the device
        with the payloads' density class.  Returns (acc, status)."""
        dev = self.device
        P = int(payloads if payloads is not None else (inp.shape[0] if inp.dim() == 2 else 1))
        stride = int(inp.shape[1]) if inp.dim() == 2 else self.stream_bytes
        if P < 1 or P > 64:
            raise ValueError(f"payloads must be 1..64, got {P}")
        if P > 1 and (stride < self.stream_bytes or stride % 16):
            raise ValueError("each payload's stream buffer needs stream_bytes bytes at a 16-byte multiple stride")
        status = status if status is not None else torch.empty(1, dtype=torch.int32, device=dev)
        _need(inp, (P - 1) * stride + self.stream_bytes, "in")
        _need(in_lens, P * self.count, "in_lens")
        _need(scales, P * self.count, "scales")
        _need(acc, self.total, "acc")
        _need(status, 1, "status")
        wsb = self.accumulate_many_workspace_size(P)
        workspace = workspace if workspace is not None else torch.empty(wsb, dtype=torch.uint8, device=dev)
        rc = lib().tlc_decompress_accumulate_many_group(
            ctypes.byref(self.info), _ptr(self.d_table, torch.uint8, "table"), P, _ptr(inp, torch.uint8, "in"),
            stride, _ptr(in_lens, torch.int64, "in_lens"), _ptr(scales, torch.float32, "scales"), s,
            _ptr(acc, torch.float32, "acc"), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
            _ptr(status, torch.int32, "status"), _hint_ptr(path_hint), _stream(stream))
        _check(rc, "tlc_decompress_accumulate_many_group")
        return acc, status


def planes_gather(src: torch.Tensor, src_off: torch.Tensor, dst: torch.Tensor, dst_off: torch.Tensor,
                  n: torch.Tensor, max_n: int, stream=None):
    """tlc_planes_gather: each tensor's values into the five-plane order
    (offsets and sizes are device int64 tensors, one entry per tensor)."""
    _need(src_off, n.numel(), "src_off")
    _need(dst_off, n.numel(), "dst_off")
    _check(lib().tlc_planes_gather(_ptr(src, torch.float32, "src"), _ptr(src_off, torch.int64, "src_off"),
                                   _ptr(dst, torch.float32, "dst"), _ptr(dst_off, torch.int64, "dst_off"),
                                   _ptr(n, torch.int64, "n"), n.numel(), int(max_n), _stream(stream)),
           "tlc_planes_gather")


def planes_scatter(src: torch.Tensor, src_off: torch.Tensor, dst: torch.Tensor, dst_off: torch.Tensor,
                   n: torch.Tensor, max_n: int, stream=None):
    """tlc_planes_scatter: each tensor's values back from the five-plane order."""
    _need(src_off, n.numel(), "src_off")
    _need(dst_off, n.numel(), "dst_off")
    _check(lib().tlc_planes_scatter(_ptr(src, torch.float32, "src"), _ptr(src_off, torch.int64, "src_off"),
                                    _ptr(dst, torch.float32, "dst"), _ptr(dst_off, torch.int64, "dst_off"),
                                    _ptr(n, torch.int64, "n"), n.numel(), int(max_n), _stream(stream)),
           "tlc_planes_scatter")


def gather_probe(src: torch.Tensor, idx: torch.Tensor, dst: torch.Tensor, stream=None):
    """dst[i] = src[idx[i]] (tlc_gather_probe).  idx: int32 indices into src,
    checked here."""
    n = idx.numel()
    _need(dst, n, "dst")
    if n == 0 or int(idx.min().item()) < 0 or int(idx.max().item()) >= src.numel():
        raise ValueError("idx must hold indices into src")
    _check(lib().tlc_gather_probe(_ptr(src, torch.float32, "src"), _ptr(idx, torch.int32, "idx"), n,
                                  _ptr(dst, torch.float32, "dst"), _stream(stream)), "tlc_gather_probe")


def copy_probe(src: torch.Tensor, dst: torch.Tensor, nbytes: int, stream=None):
    for t, name in ((src, "src"), (dst, "dst")):
        if t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, fewer than {nbytes}")
    _check(lib().tlc_copy_probe(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "tlc_copy_probe")


def profile_enable(on: bool = True):
    _check(lib().tlc_profile_enable(1 if on else 0), "tlc_profile_enable")


def profile_only(kernel_name: str | None):
    _check(lib().tlc_profile_only(kernel_name.encode() if kernel_name else None), "tlc_profile_only")


def profile_read(capacity: int = 32) -> dict[str, tuple[int, float]]:
    """{kernel name: (launches, total ms)} since the last read (synchronises)."""
    buf = (KernelTime * capacity)()
    cnt = ctypes.c_int()
    _check(lib().tlc_profile_read(buf, capacity, ctypes.byref(cnt)), "tlc_profile_read")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(cnt.value)}
