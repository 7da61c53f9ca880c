"""The C-ABI library loads, exports every function include/tlc.h declares,
and its host-only logic (bounds, workspace sizes, group plans, argument
checks that fail before any launch) behaves as documented.  No GPU needed."""
import ctypes
import os
import re

import numpy as np
import pytest

from gradient_compression_distributed_lc_amd import tlc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tlc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tlc_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = tlc.lib()
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), f"{name} declared in tlc.h but not exported"
    # and the binding covers every declaration
    assert set(names) == set(tlc._SIGS)


def test_status_strings():
    for code in range(8):
        assert tlc.status_string(code)
    assert tlc.status_string(99) == "unknown status"


@pytest.mark.parametrize("n", [1, 4, 5, 6, 1_048_576, 16_777_216, 2 ** 32 - 1])
def test_compress_bound_is_ceil_n_over_5(n):
    assert tlc.compress_bound(n) == -(-n // 5)


def test_workspace_size():
    assert tlc.workspace_size(0) == 0
    assert tlc.workspace_size(2 ** 32) == 0
    small, big = tlc.workspace_size(1), tlc.workspace_size(335_000_000)
    assert 0 < small <= 8192 and small % 256 == 0
    # staging for the zero-run bytes of tiles with nonzero codes (ceil(n/5)); per 512-element flat
    # tile a partial max and a candidate list (count + 64 x (u32 index, f32 value)); a carry
    # word, a max and a 32-byte job per 5120-element encode tile; small per-call state
    n = 335_000_000
    assert big < n // 5 + (4 + 2 + 64 * 8) * (n // 512) + 48 * (n // 5120) + 1_000_000
    assert big % 256 == 0


def test_group_plan_layout():
    sizes = [10, 5120, 5121, 1, 33_000, 4 * 5120 * 5, 1023, 1025]
    info, table, offs = tlc.group_plan(sizes)
    N = sum(sizes)
    assert info.count == len(sizes)
    assert info.total_elems == N
    etiles = sum(-(-n // 5120) for n in sizes)
    spans = sum(-(-(-(-n // 5120)) // 256) for n in sizes)
    chunks = sum(max(1, -(-(-(-n // 5)) // 4096)) for n in sizes)
    ftiles = -(-N // 512)
    assert info.tiles == etiles and info.chunks == chunks and info.spans == spans
    assert len(table) == info.table_bytes
    # stream slots: 16-byte aligned, in order, each ceil(n/5) long, inside the buffer
    prev_end = 0
    for n, o in zip(sizes, offs):
        assert o % 16 == 0 and o >= prev_end
        prev_end = o + -(-n // 5)
    assert prev_end <= info.stream_bytes
    # table: header, per-tensor records, flat-tile info, span owners
    hdr = np.frombuffer(table[:64], dtype=np.uint64)
    assert hdr[1] == len(sizes) and hdr[2] == ftiles and hdr[3] == etiles and hdr[4] == spans
    assert hdr[5] == chunks and hdr[6] == N
    rec_t = np.dtype([("elem_off", "<u8"), ("n", "<u4"), ("etile0", "<u4"), ("stream_off", "<u8"),
                      ("span0", "<u4"), ("chunk0", "<u4")])
    rec = np.frombuffer(table[64:64 + 32 * len(sizes)], dtype=rec_t)
    assert rec["n"].tolist() == sizes
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    assert rec["elem_off"].tolist() == starts.tolist()
    assert rec["stream_off"].tolist() == offs
    assert rec["etile0"].tolist() == np.concatenate([[0], np.cumsum([-(-n // 5120) for n in sizes])[:-1]]).tolist()
    # flat tile t: tensor of its first element, high bit if it also holds a later tensor
    fi_at = -(-(64 + 32 * len(sizes)) // 16) * 16
    info_arr = np.frombuffer(table[fi_at:fi_at + 4 * ftiles], dtype=np.uint32)
    seg_of = np.searchsorted(np.cumsum(sizes), np.arange(N), side="right")
    for t in range(ftiles):
        first, last = t * 512, min(N, (t + 1) * 512) - 1
        want = int(seg_of[first]) | (0x80000000 if seg_of[last] != seg_of[first] else 0)
        assert int(info_arr[t]) == want, t
    # then the span owners and the encode-tile owners, and nothing after them
    up = lambda v: -(-v // 16) * 16
    span_at = up(fi_at + 4 * ftiles)
    et_at = up(span_at + 4 * spans)
    assert info.table_bytes == up(et_at + 4 * etiles)
    et = np.frombuffer(table[et_at:et_at + 4 * etiles], dtype=np.uint32)
    assert et.tolist() == [t for t, n in enumerate(sizes) for _ in range(-(-n // 5120))]


def test_group_plan_rejects_bad_sizes():
    info = tlc.GroupInfo()
    arr = (ctypes.c_uint64 * 2)(5, 0)
    assert tlc.lib().tlc_group_plan(arr, 2, ctypes.byref(info), None, 0, None) == tlc.ERR_INVALID_ARG
    arr = (ctypes.c_uint64 * 1)(2 ** 32)
    assert tlc.lib().tlc_group_plan(arr, 1, ctypes.byref(info), None, 0, None) == tlc.ERR_INVALID_ARG
    assert tlc.lib().tlc_group_plan(arr, 0, ctypes.byref(info), None, 0, None) == tlc.ERR_INVALID_ARG
    arr = (ctypes.c_uint64 * 1)(100)
    small = ctypes.create_string_buffer(8)
    assert tlc.lib().tlc_group_plan(arr, 1, ctypes.byref(info), small, 8, None) == tlc.ERR_CAPACITY


def test_planes_argument_errors_return_before_any_launch():
    L = tlc.lib()
    V = ctypes.c_void_p
    f = V(0x10000)  # never dereferenced: every case below fails validation first
    for fn in (L.tlc_planes_gather, L.tlc_planes_scatter):
        assert fn(None, f, f, f, f, 3, 100, None) == tlc.ERR_INVALID_ARG
        assert fn(f, f, f, f, None, 3, 100, None) == tlc.ERR_INVALID_ARG
        assert fn(f, f, f, f, f, 0, 100, None) == tlc.ERR_INVALID_ARG
        assert fn(f, f, f, f, f, 65536, 100, None) == tlc.ERR_INVALID_ARG
        assert fn(f, f, f, f, f, 3, 0, None) == tlc.ERR_INVALID_ARG
        assert fn(f, f, f, f, f, 3, 1 << 32, None) == tlc.ERR_INVALID_ARG


def test_argument_errors_return_before_any_launch():
    L = tlc.lib()
    V = ctypes.c_void_p
    fake = V(0x10000)          # never dereferenced: every case below fails validation first
    odd = V(0x10004)
    ws = V(0x20000)
    # n == 0, s out of range, capacity too small, null pointers, misaligned fp32, bad workspace
    assert L.tlc_compress(fake, fake, 0, 1.5, fake, 10, fake, fake, ws, 4096, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress(fake, fake, 10, 2.0, fake, 10, fake, fake, ws, 4096, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress(fake, fake, 10, 0.5, fake, 10, fake, fake, ws, 4096, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress(fake, fake, 10, float("nan"), fake, 10, fake, fake, ws, 4096, fake,
                          None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress(fake, fake, 11, 1.5, fake, 2, fake, fake, ws, 4096, fake, None) == tlc.ERR_CAPACITY
    assert L.tlc_compress(None, fake, 10, 1.5, fake, 10, fake, fake, ws, 4096, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress(odd, fake, 10, 1.5, fake, 10, fake, fake, ws, 4096, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress(fake, fake, 10, 1.5, fake, 10, fake, fake, None, 4096, fake, None) == tlc.ERR_WORKSPACE
    assert L.tlc_compress(fake, fake, 10, 1.5, fake, 10, fake, fake, ws, 16, fake, None) == tlc.ERR_WORKSPACE
    assert L.tlc_compress(fake, fake, 10, 1.5, fake, 10, fake, fake, V(0x20010), 4096, fake,
                          None) == tlc.ERR_WORKSPACE
    assert L.tlc_compress(fake, fake, 10, 1.5, fake, 10, fake, fake, ws, 4096, None, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress(fake, fake, fake, 0, 1.5, fake, ws, 4096, fake, None, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress(fake, fake, fake, 10, 1.5, odd, ws, 4096, fake, None, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress(fake, None, fake, 10, 1.5, fake, ws, 4096, fake, None, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress_accumulate(fake, fake, fake, 10, 1.99, fake, ws, 1, fake, None) == tlc.ERR_WORKSPACE
    assert L.tlc_copy_probe(fake, fake, 17, None) == tlc.ERR_INVALID_ARG
    # fixed-length encodings: lengths, unknown encodings, capacity
    assert tlc.fixed_len(10, tlc.ENC_QUARTIC) == 2 and tlc.fixed_len(10, tlc.ENC_TWOBIT) == 3
    assert tlc.fixed_len(10, 3) == 0 and tlc.fixed_len(0, tlc.ENC_TWOBIT) == 0
    assert tlc.fixed_len(2 ** 32 - 1, tlc.ENC_TWOBIT) == 2 ** 30 and tlc.fixed_len(2 ** 32, tlc.ENC_QUARTIC) == 0
    assert L.tlc_compress_fixed(fake, fake, 10, 1.5, 3, fake, 10, fake, ws, 4096, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress_fixed(fake, fake, 10, 1.5, tlc.ENC_TWOBIT, fake, 2, fake, ws, 4096, fake,
                                None) == tlc.ERR_CAPACITY
    assert L.tlc_decompress_fixed(fake, fake, 10, 1.5, 0, fake, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress_fixed(fake, fake, 10, 2.5, tlc.ENC_QUARTIC, fake, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress_fixed(fake, fake, 10, 1.5, tlc.ENC_QUARTIC, odd, fake, None) == tlc.ERR_INVALID_ARG
    # server compress: no workers, no elements, capacity, s out of range
    assert L.tlc_server_compress(fake, 0, fake, 10, 1.5, fake, 10, fake, fake, ws, 4096, fake,
                                 None) == tlc.ERR_INVALID_ARG
    assert L.tlc_server_compress(fake, 8, fake, 0, 1.5, fake, 10, fake, fake, ws, 4096, fake,
                                 None) == tlc.ERR_INVALID_ARG
    assert L.tlc_server_compress(fake, 8, fake, 11, 1.5, fake, 2, fake, fake, ws, 4096, fake,
                                 None) == tlc.ERR_CAPACITY
    assert L.tlc_server_compress(fake, 8, fake, 10, 2.0, fake, 10, fake, fake, ws, 4096, fake,
                                 None) == tlc.ERR_INVALID_ARG
    # grouped calls: the info/table pair must be consistent
    info, _, _ = tlc.group_plan([100, 200])
    bad = tlc.GroupInfo.from_buffer_copy(info)
    bad.table_bytes += 16
    assert L.tlc_compress_group(ctypes.byref(bad), fake, fake, fake, 1.5, fake, fake, fake, ws, 1 << 20, fake,
                                None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress_group(ctypes.byref(info), None, fake, fake, 1.5, fake, fake, fake, ws, 1 << 20, fake,
                                None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress_group(ctypes.byref(info), fake, fake, fake, fake, 1.5, fake, ws, 16, fake, None,
                                  None) == tlc.ERR_WORKSPACE
    assert L.tlc_server_compress_group(ctypes.byref(info), fake, fake, 0, fake, 1.5, fake, fake, fake, ws,
                                       1 << 20, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress_fixed_group(ctypes.byref(info), fake, tlc.ENC_QUARTIC, fake, fake, 1.5, fake, None,
                                      fake, ws, 1 << 20, fake, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress_fixed_group(ctypes.byref(info), fake, 7, fake, fake, fake, 1.5, fake, fake,
                                        None) == tlc.ERR_INVALID_ARG
    assert L.tlc_decompress_fixed_group(ctypes.byref(info), fake, tlc.ENC_TWOBIT, fake, fake, fake, 1.5, odd, fake,
                                        None) == tlc.ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tlc, "_lib", None)
    monkeypatch.setattr(tlc, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        tlc.lib()


def test_accumulate_many_host_checks():
    # workspace size and argument errors of the many-payload accumulate, all
    # decided before any launch
    L = tlc.lib()
    V = ctypes.c_void_p
    fake, ws = V(0x10000), V(0x20000)
    sizes = [100, 200, 5121]
    info, _, _ = tlc.group_plan(sizes)
    N, C = int(info.total_elems), len(sizes)
    one = L.tlc_accumulate_many_workspace_size(ctypes.byref(info), 1)
    eight = L.tlc_accumulate_many_workspace_size(ctypes.byref(info), 8)
    assert one > 0 and eight > 0 and one % 256 == 0 and eight % 256 == 0
    # per payload: a start record (8 bytes) and a literal flag (4 bytes) per encode tile, plus the
    # decoder's state; nothing the size of the streams (checked on a larger group)
    big, _, _ = tlc.group_plan(sizes + [3_000_000])
    T, K = int(big.tiles), int(big.chunks)
    b1 = L.tlc_accumulate_many_workspace_size(ctypes.byref(big), 1)
    b8 = L.tlc_accumulate_many_workspace_size(ctypes.byref(big), 8)
    assert b8 >= 8 * 12 * T and b8 - b1 >= 7 * 12 * T
    assert b8 < 8 * (12 * T + 16 * K + 8 * len(sizes) + 8) + 8 * 256 and b8 < int(big.stream_bytes)
    assert L.tlc_accumulate_many_workspace_size(ctypes.byref(info), 0) == 0
    assert L.tlc_accumulate_many_workspace_size(ctypes.byref(info), 65) == 0
    # payloads x tensors must stay below 2^31 (the decoder's unit ids), and the payloads' chunks below 2^32
    huge = tlc.GroupInfo.from_buffer_copy(info)
    huge.count, huge.chunks = 1 << 26, 1 << 26
    assert L.tlc_accumulate_many_workspace_size(ctypes.byref(huge), 31) > 0
    assert L.tlc_accumulate_many_workspace_size(ctypes.byref(huge), 32) == 0
    huge.count, huge.chunks = 3, (1 << 27) + 1
    assert L.tlc_accumulate_many_workspace_size(ctypes.byref(huge), 31) > 0
    assert L.tlc_accumulate_many_workspace_size(ctypes.byref(huge), 32) == 0
    SB = int(info.stream_bytes)

    def call(P, stride, ws_bytes, s=1.5, acc=fake):
        return L.tlc_decompress_accumulate_many_group(ctypes.byref(info), fake, P, fake, stride, fake, fake, s,
                                                      acc, ws, ws_bytes, fake, None, None)
    assert call(0, SB, eight) == tlc.ERR_INVALID_ARG
    assert call(65, SB, 1 << 40) == tlc.ERR_INVALID_ARG
    assert call(8, SB - 16, eight) == tlc.ERR_INVALID_ARG    # payload buffers would overlap
    assert call(8, SB + 8, eight) == tlc.ERR_INVALID_ARG     # stride not a multiple of 16
    assert call(8, SB, eight - 256) == tlc.ERR_WORKSPACE
    assert call(8, SB, eight, s=2.0) == tlc.ERR_INVALID_ARG
    assert call(8, SB, eight, acc=V(0x10004)) == tlc.ERR_INVALID_ARG
    # the binding's own checks
    import torch
    g = tlc.Group(sizes, device="cpu")
    with pytest.raises(ValueError, match="stream buffer needs"):
        g.decompress_accumulate_many(torch.zeros((8, SB - 16), dtype=torch.uint8), torch.zeros(8 * C, dtype=torch.int64),
                                     torch.zeros(8 * C), 1.5, torch.zeros(N))
    with pytest.raises(ValueError, match="in holds"):
        g.decompress_accumulate_many(torch.zeros(8 * SB - 1, dtype=torch.uint8), torch.zeros(8 * C, dtype=torch.int64),
                                     torch.zeros(8 * C), 1.5, torch.zeros(N), payloads=8)
    with pytest.raises(ValueError, match="in_lens holds"):
        g.decompress_accumulate_many(torch.zeros((8, SB), dtype=torch.uint8), torch.zeros(8 * C - 1, dtype=torch.int64),
                                     torch.zeros(8 * C), 1.5, torch.zeros(N))
    with pytest.raises(ValueError, match="acc holds"):
        g.decompress_accumulate_many(torch.zeros((2, SB), dtype=torch.uint8), torch.zeros(2 * C, dtype=torch.int64),
                                     torch.zeros(2 * C), 1.5, torch.zeros(N - 1))
    with pytest.raises(ValueError, match="payloads"):
        g.decompress_accumulate_many(torch.zeros((65, SB), dtype=torch.uint8), torch.zeros(65 * C, dtype=torch.int64),
                                     torch.zeros(65 * C), 1.5, torch.zeros(N))


def test_static_compress_rejects_n_above_its_maximum():
    # checked before any HIP call, so it runs without a GPU
    L = tlc.lib()
    assert L.tlc_compress_static_max_n() == 1 << 24
    assert L.tlc_compress_static(None, None, (1 << 24) + 1, 1.5, None, 1 << 30, None, None, None, None) \
        == tlc.ERR_TOO_LARGE
    assert L.tlc_compress_static(None, None, 0, 1.5, None, 1 << 30, None, None, None, None) == tlc.ERR_INVALID_ARG
    assert L.tlc_compress_static(None, None, 100, 1.5, None, 10, None, None, None, None) == tlc.ERR_CAPACITY


# The binding checks every buffer it is given against the sizes the call
# needs before any pointer reaches the library: an undersized tensor raises
# ValueError and nothing is launched.  CPU tensors stand in for device ones
# (the size checks run before the device check).

def _t(n, dtype):
    import torch
    return torch.zeros(max(n, 0), dtype=dtype)


def test_binding_rejects_undersized_single_tensor_buffers():
    import torch
    n, s = 1000, 1.5
    B = tlc.compress_bound(n)
    u8, i64, f32, i32 = torch.uint8, torch.int64, torch.float32, torch.int32
    ok = dict(inp=_t(B, u8), in_len=_t(1, i64), scale=_t(1, f32))
    with pytest.raises(ValueError, match="y holds"):
        tlc.decompress(ok["inp"], ok["in_len"], ok["scale"], n, s, y=_t(n - 1, f32))
    with pytest.raises(ValueError, match="in holds"):
        tlc.decompress(_t(B - 1, u8), ok["in_len"], ok["scale"], n, s, y=_t(n, f32))
    with pytest.raises(ValueError, match="in_len holds"):
        tlc.decompress(ok["inp"], _t(0, i64), ok["scale"], n, s, y=_t(n, f32))
    with pytest.raises(ValueError, match="scale holds"):
        tlc.decompress(ok["inp"], ok["in_len"], _t(0, f32), n, s, y=_t(n, f32))
    with pytest.raises(ValueError, match="acc holds"):
        tlc.decompress_accumulate(ok["inp"], ok["in_len"], ok["scale"], n, s, _t(n - 4, f32))
    with pytest.raises(ValueError, match="status holds"):
        tlc.decompress_accumulate(ok["inp"], ok["in_len"], ok["scale"], n, s, _t(n, f32), status=_t(0, i32))
    with pytest.raises(ValueError, match="scale holds"):
        tlc.compress(_t(n, f32), _t(n, f32), s, scale=_t(0, f32))
    with pytest.raises(ValueError, match="out_len holds"):
        tlc.compress_static(_t(n, f32), _t(n, f32), s, out_len=_t(0, i64))
    with pytest.raises(ValueError, match="y holds"):
        tlc.decompress_fixed(_t(tlc.fixed_len(n, tlc.ENC_QUARTIC), u8), ok["scale"], n, s, tlc.ENC_QUARTIC,
                             y=_t(n - 1, f32))
    with pytest.raises(ValueError, match="in holds"):
        tlc.decompress_fixed(_t(tlc.fixed_len(n, tlc.ENC_TWOBIT) - 1, u8), ok["scale"], n, s, tlc.ENC_TWOBIT,
                             y=_t(n, f32))
    with pytest.raises(ValueError, match="dst holds"):
        tlc.copy_probe(_t(64, u8), _t(32, u8), 64)


def test_binding_rejects_undersized_group_buffers():
    import torch
    sizes = [10, 5121, 3, 40_000]
    g = tlc.Group(sizes, device="cpu")
    N, C, SB = g.total, g.count, g.stream_bytes
    u8, i64, f32 = torch.uint8, torch.int64, torch.float32
    x, e = _t(N, f32), _t(N, f32)
    with pytest.raises(ValueError, match="out holds"):
        g.compress(x, e, 1.5, out=_t(SB - 1, u8))
    with pytest.raises(ValueError, match="out_lens holds"):
        g.compress(x, e, 1.5, out_lens=_t(C - 1, i64))
    with pytest.raises(ValueError, match="scales holds"):
        g.compress(x, e, 1.5, scales=_t(C - 1, f32))
    with pytest.raises(ValueError, match="out holds"):
        g.server_compress(x, 8, e, 1.5, out=_t(SB - 16, u8))
    args = (_t(SB, u8), _t(C, i64), _t(C, f32), 1.5)
    with pytest.raises(ValueError, match="y holds"):
        g.decompress(*args, y=_t(N - 1, f32))
    with pytest.raises(ValueError, match="in holds"):
        g.decompress(_t(SB - 1, u8), *args[1:], y=_t(N, f32))
    with pytest.raises(ValueError, match="in_lens holds"):
        g.decompress(args[0], _t(C - 1, i64), *args[2:], y=_t(N, f32))
    with pytest.raises(ValueError, match="scales holds"):
        g.decompress(args[0], args[1], _t(C - 1, f32), 1.5, y=_t(N, f32))
    with pytest.raises(ValueError, match="acc holds"):
        g.decompress_accumulate(*args, _t(N - 1, f32))
    total_q = g._fixed_layout(tlc.ENC_QUARTIC)[1]
    with pytest.raises(ValueError, match="out holds"):
        g.compress_fixed(x, e, 1.5, tlc.ENC_QUARTIC, _t(total_q - 1, u8), _t(C, i64))
    with pytest.raises(ValueError, match="offsets holds"):
        g.decompress_fixed(_t(total_q, u8), _t(C - 1, i64), _t(C, f32), 1.5, tlc.ENC_QUARTIC, y=_t(N, f32))
    with pytest.raises(ValueError, match="y holds"):
        g.decompress_fixed(_t(total_q, u8), _t(C, i64), _t(C, f32), 1.5, tlc.ENC_QUARTIC, y=_t(N - 1, f32))


def test_wire_host_checks():
    # bound, workspace size and argument errors of the wire pack and unpack,
    # all decided before any launch
    L = tlc.lib()
    V = ctypes.c_void_p
    fake = V(0x10000)
    odd = V(0x10008)
    ws = V(0x20000)
    info, _, offsets = tlc.group_plan([100, 7, 5121])
    bound = 8 * 3 + info.stream_bytes
    assert L.tlc_wire_bound(ctypes.byref(info)) == bound
    assert L.tlc_wire_bound(None) == 0
    wsz = L.tlc_wire_workspace_size(ctypes.byref(info))
    assert wsz > 0 and wsz % 256 == 0 and L.tlc_wire_workspace_size(None) == 0
    bi = ctypes.byref(info)
    ok_pack = lambda *a: L.tlc_wire_pack_group(bi, fake, *a)
    assert ok_pack(fake, fake, fake, fake, bound - 1, fake, ws, wsz, fake, None) == tlc.ERR_CAPACITY
    assert ok_pack(None, fake, fake, fake, bound, fake, ws, wsz, fake, None) == tlc.ERR_INVALID_ARG
    assert ok_pack(fake, fake, fake, odd, bound, fake, ws, wsz, fake, None) == tlc.ERR_INVALID_ARG
    assert ok_pack(fake, fake, fake, fake, bound, None, ws, wsz, fake, None) == tlc.ERR_INVALID_ARG
    assert ok_pack(fake, fake, fake, fake, bound, fake, ws, wsz, None, None) == tlc.ERR_INVALID_ARG
    assert ok_pack(fake, fake, fake, fake, bound, fake, ws, wsz - 1, fake, None) == tlc.ERR_WORKSPACE
    assert ok_pack(fake, fake, fake, fake, bound, fake, V(0x20010), wsz, fake, None) == tlc.ERR_WORKSPACE
    ok_unpack = lambda *a: L.tlc_wire_unpack_group(bi, fake, *a)
    assert ok_unpack(fake, 23, fake, fake, fake, ws, wsz, fake, None) == tlc.ERR_CAPACITY  # below 8 * count
    assert ok_unpack(odd, 24, fake, fake, fake, ws, wsz, fake, None) == tlc.ERR_INVALID_ARG
    assert ok_unpack(fake, 24, None, fake, fake, ws, wsz, fake, None) == tlc.ERR_INVALID_ARG
    assert ok_unpack(fake, 24, fake, fake, fake, None, wsz, fake, None) == tlc.ERR_WORKSPACE
    bad = tlc.GroupInfo.from_buffer_copy(info)
    bad.table_bytes += 16
    assert L.tlc_wire_pack_group(ctypes.byref(bad), fake, fake, fake, fake, fake, bound, fake, ws, wsz, fake,
                                 None) == tlc.ERR_INVALID_ARG
    # ranges: cuts must rise from 0 to the tensor count, 1 to 64 ranges
    C = ctypes.c_uint32
    pr = lambda cuts, n: L.tlc_wire_pack_ranges_group(bi, fake, cuts, n, fake, fake, fake, fake, bound, fake, ws, wsz,
                                                      fake, None)
    assert pr(None, 1) == tlc.ERR_INVALID_ARG
    assert pr((C * 3)(0, 3, 3), 2) == tlc.ERR_INVALID_ARG   # an empty range
    assert pr((C * 3)(1, 2, 3), 2) == tlc.ERR_INVALID_ARG   # not from 0
    assert pr((C * 3)(0, 1, 2), 2) == tlc.ERR_INVALID_ARG   # not to the count
    assert pr((C * 2)(0, 3), 0) == tlc.ERR_INVALID_ARG
    assert L.tlc_wire_pack_ranges_group(bi, fake, (C * 3)(0, 1, 3), 2, fake, fake, fake, fake, bound - 1, fake, ws,
                                        wsz, fake, None) == tlc.ERR_CAPACITY
    ur = lambda cuts, n, nb=24: L.tlc_wire_unpack_ranges_group(bi, fake, cuts, n, fake, nb, fake, fake, fake, ws, wsz,
                                                               fake, None)
    assert ur(None, 1) == tlc.ERR_INVALID_ARG
    assert ur((C * 3)(0, 3, 3), 2) == tlc.ERR_INVALID_ARG
    assert ur((C * 3)(0, 2, 4), 2) == tlc.ERR_INVALID_ARG
    assert ur((C * 66)(*range(66)), 65) == tlc.ERR_INVALID_ARG   # more than 64 ranges
    assert ur((C * 3)(0, 1, 3), 2, 23) == tlc.ERR_CAPACITY      # below 8 * count
    assert L.tlc_wire_unpack_ranges_group(bi, fake, (C * 3)(0, 1, 3), 2, odd, 24, fake, fake, fake, ws, wsz, fake,
                                          None) == tlc.ERR_INVALID_ARG
    assert L.tlc_wire_unpack_ranges_group(bi, fake, (C * 3)(0, 1, 3), 2, fake, 24, fake, fake, fake, ws, wsz - 1,
                                          fake, None) == tlc.ERR_WORKSPACE


def test_path_hint_word_is_checked_on_the_host():
    """The decompress and many-payload accumulate take the caller's hint word
    only as one pinned int32 on the host; anything else is refused before the
    library is called (no device is needed to check this)."""
    import torch
    assert tlc._hint_ptr(None) is None
    with pytest.raises(ValueError, match="pinned host tensor"):
        tlc._hint_ptr(torch.zeros(1, dtype=torch.int32))  # pageable host memory
    # the C ABI refuses a word the device cannot reach (here: no device at all,
    # or an address that is not pinned memory) with TLC_ERR_INVALID_ARG
    L = tlc.lib()
    info, _, _ = tlc.group_plan([1000, 2000])
    V = ctypes.c_void_p
    word = ctypes.c_uint32(0)
    rc = L.tlc_decompress_group(ctypes.byref(info), V(0x10000), V(0x10000), V(0x10000), V(0x10000), 1.5,
                                V(0x10000), V(0x20000), 1 << 30, V(0x10000), ctypes.byref(word), None)
    assert rc == tlc.ERR_INVALID_ARG
    rc = L.tlc_decompress_accumulate_many_group(ctypes.byref(info), V(0x10000), 2, V(0x10000),
                                                int(info.stream_bytes), V(0x10000), V(0x10000), 1.5, V(0x10000),
                                                V(0x20000), 1 << 30, V(0x10000), ctypes.byref(word), None)
    assert rc == tlc.ERR_INVALID_ARG
