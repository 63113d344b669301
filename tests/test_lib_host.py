"""CPU-side checks of the HIP library: it loads, exports every entry point the
header declares, the host packer round-trips bit-exactly, and invalid arguments
are rejected before anything is launched. No kernel runs here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

q = pytest.importorskip("quantized_mixture_experts_bit_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20, names
    lib = q.lib()
    for n in names:
        assert hasattr(lib, n), "libqmoe.so does not export %s" % n


def test_binding_has_the_same_names():
    for n in declared_functions():
        assert callable(getattr(q, n)), n


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    found = {}
    for name, val in re.findall(r"#define\s+(MOE_\w+)\s+(0x[0-9A-Fa-f]+|\d+)u?\b", text):
        found[name] = int(val, 0)
    for name, val in re.findall(r"\b(MOE_\w+)\s*=\s*(-?\d+)", text):
        found[name] = int(val)
    assert {"MOE_OK", "MOE_ERR_DEVICE_CHECK", "MOE_BF16", "MOE_DEVERR_SYNC_TIMEOUT", "MOE_SLOT_SKIP"} <= set(found)
    for name, val in found.items():
        assert getattr(q, name) == val, name


def test_sizes_match_the_format():
    s = q.MoeShape(2816, 704, 2112)
    # 4.5 bits per weight: codes + one (s, b) bf16 pair per 64 weights
    assert q.moe_matrix4_bytes(704, 2816) == 704 * 2816 // 2 + 704 * 44 * 4
    assert q.moe_expert_blob_bytes(s) == 3 * (704 * 2816 // 2 + 704 * 44 * 4) == 3345408
    assert q.moe_shared_blob_bytes(s) == 10036224
    assert q.moe_router_blob_bytes(s) == 128 * 2816 + 128 * 44 * 4 == 382976
    assert q.moe_matrix4_bytes(100, 64) == 0
    assert q.moe_workspace_bytes(s, 1) > 0
    assert q.moe_workspace_bytes(s, 256) >= q.moe_workspace_bytes(s, 1)


@pytest.mark.parametrize("bits,rows,cols", [(4, 64, 64), (4, 128, 512), (4, 704, 2816), (8, 128, 2816),
                                            (8, 64, 192)])
def test_packer_round_trip_bit_exact(bits, rows, cols):
    rng = np.random.default_rng(rows + cols + bits)
    m = synth.draw_qmat(rng, rows, cols, bits)
    if bits == 4:
        buf = np.empty(q.moe_matrix4_bytes(rows, cols), dtype=np.uint8)
        q.moe_pack_matrix4(m.q, m.s, m.b, buf)
        q2, s2, b2 = np.empty_like(m.q), np.empty_like(m.s), np.empty_like(m.b)
        q.moe_unpack_matrix4(buf, rows, cols, q2, s2, b2)
    else:
        buf = np.empty(q.moe_matrix8_bytes(rows, cols), dtype=np.uint8)
        q.moe_pack_matrix8(m.q, m.s, m.b, buf)
        q2, s2, b2 = np.empty_like(m.q), np.empty_like(m.s), np.empty_like(m.b)
        q.moe_unpack_matrix8(buf, rows, cols, q2, s2, b2)
    np.testing.assert_array_equal(q2, m.q)
    np.testing.assert_array_equal(s2, m.s)
    np.testing.assert_array_equal(b2, m.b)
    # the device format permutes the canonical codes (nibbles for 4-bit) and (s, b) pairs
    ncode = m.q.size
    if bits == 4:
        nib = lambda a: np.sort(np.concatenate([a.ravel() & 0xF, a.ravel() >> 4]))
        tiles = buf.reshape(-1, 2304)
        np.testing.assert_array_equal(nib(tiles[:, :2048]), nib(m.q))
        np.testing.assert_array_equal(np.sort(tiles[:, 2048:].ravel()),
                                      np.sort(np.stack([m.s, m.b], -1).view(np.uint8).ravel()))
    else:
        tiles = buf.reshape(-1, 4352)
        np.testing.assert_array_equal(np.sort(tiles[:, :4096].ravel()), np.sort(m.q.ravel()))
        assert tiles[:, :4096].size == ncode


def test_packed_nibble_positions():
    """Word j of half h of row r holds columns c0..c0+7 (c0 = h*32 + 8j) with column
    c0+2t in bits [4t, 4t+4) and c0+2t+1 in bits [16+4t, 16+4t+4)."""
    rows, cols = 64, 64
    codes = np.zeros((rows, cols), dtype=np.uint8)
    codes[5, :] = np.arange(64) % 16
    qb = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = np.zeros((rows, 1), np.uint16)
    b = np.zeros((rows, 1), np.uint16)
    buf = np.empty(q.moe_matrix4_bytes(rows, cols), dtype=np.uint8)
    q.moe_pack_matrix4(qb, s, b, buf)
    words = buf[:2048].view(np.uint32)
    for h in range(2):
        for j in range(4):
            w = int(words[(h * 1024 + 5 * 16 + j * 4) // 4])
            c0 = h * 32 + 8 * j
            for t in range(4):
                assert (w >> (4 * t)) & 0xF == (c0 + 2 * t) % 16
                assert (w >> (16 + 4 * t)) & 0xF == (c0 + 2 * t + 1) % 16


def _fake_layer():
    # aligned, never dereferenced: every call below fails validation first
    return q.moe_layer(0x10000, 3346432, 128, 0x20000, 0x30000, 0x40000)


def _call_router(shape, rows=1, ws_bytes=1 << 30, x=0x50000, dtype=q.MOE_BF16):
    lib = q.lib()
    return lib.moe_router_topk(C.byref(shape), C.byref(_fake_layer()), x, dtype, rows, None, 0x60000, 0x70000,
                               None, 0x80000, ws_bytes, None)


def test_invalid_arguments_are_rejected_before_launch():
    good = q.MoeShape(2816, 704, 2112)
    assert _call_router(q.MoeShape(2800, 704, 2112)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert _call_router(q.MoeShape(2816, 700, 2112)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert _call_router(q.MoeShape(2816, 704, 2112, n_experts=96)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    # a multiple of 64 that does not divide the rankers' 256 threads evenly
    assert _call_router(q.MoeShape(2816, 704, 2112, n_experts=192)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert _call_router(q.MoeShape(2816, 704, 2112, n_experts=320)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert _call_router(q.MoeShape(2816, 704, 2112, top_k=0)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert _call_router(q.MoeShape(2816, 704, 2112, top_k=17)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert _call_router(q.MoeShape(2816, 704, 2112, group=32)) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert _call_router(good, rows=-1) == q.MOE_ERR_INVALID_ARG
    assert _call_router(good, x=0x50004) == q.MOE_ERR_INVALID_ARG  # misaligned activations
    assert _call_router(good, dtype=7) == q.MOE_ERR_INVALID_ARG
    assert _call_router(good, ws_bytes=16) == q.MOE_ERR_WORKSPACE
    assert _call_router(good, rows=8192) == q.MOE_ERR_UNSUPPORTED_SHAPE  # rows*top_k >= 65536
    assert q.lib().moe_router_topk(None, None, 0, 1, 1, None, 0, 0, None, 0, 0, None) == q.MOE_ERR_INVALID_ARG
    # empty input: nothing to do, nothing launched
    assert _call_router(good, rows=0) == q.MOE_OK


def test_invalid_pool_is_rejected():
    lib = q.lib()
    s = q.MoeShape(2816, 704, 2112)
    bad_stride = q.moe_layer(0x10000, 4096, 128, 0x20000, 0x30000, 0x40000)
    st = lib.moe_expert_ffn_decode(C.byref(s), C.byref(bad_stride), 0x50000, q.MOE_BF16, 0x60000, 0x70000,
                                   0x80000, 1 << 30, None)
    assert st == q.MOE_ERR_INVALID_ARG
    no_pool = q.moe_layer(0, 3346432, 128, 0x20000, 0x30000, 0x40000)
    st = lib.moe_expert_ffn_decode(C.byref(s), C.byref(no_pool), 0x50000, q.MOE_BF16, 0x60000, 0x70000,
                                   0x80000, 1 << 30, None)
    assert st == q.MOE_ERR_INVALID_ARG


def test_misaligned_combine_buffers_are_rejected():
    # expert_out and y are read and written four floats at a time, the residual four bf16 at a time
    lib = q.lib()
    s = q.MoeShape(2816, 704, 2112)
    L = C.byref(_fake_layer())

    def combine(eo=0x60000, y=0x90000, res=None):
        return lib.moe_combine(C.byref(s), L, 0x50000, q.MOE_BF16, 4, eo, 0xA0000, 0x70000, y, res, 0x80000,
                               1 << 30, None)

    def prefill(eo=0x60000, y=0x90000, res=None):
        return lib.moe_layer_prefill(C.byref(s), L, 0x50000, q.MOE_BF16, 4, None, 0xB0000, 0x70000, 0xC0000,
                                     0xD0000, 0xE0000, 0xA0000, eo, y, res, 0x80000, 1 << 30, None)

    def combine_decode(eo=0x60000, y=0x90000, res=None):
        return lib.moe_combine_decode(C.byref(s), eo, 0x70000, y, res, 0x80000, 1 << 30, None)

    for call in (combine, prefill, combine_decode):
        assert call(eo=0x60004) == q.MOE_ERR_INVALID_ARG
        assert call(y=0x90008) == q.MOE_ERR_INVALID_ARG
        assert call(res=0x50002) == q.MOE_ERR_INVALID_ARG


def test_split_combine_arguments_are_rejected():
    lib = q.lib()
    s = q.MoeShape(2816, 704, 2112)
    assert lib.moe_combine_decode(C.byref(s), None, 0x70000, 0x90000, None, 0x80000, 1 << 30, None) == \
        q.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_decode(C.byref(s), 0x60000, 0x70000, 0x90000, None, 0x80010, 1 << 30, None) == \
        q.MOE_ERR_INVALID_ARG  # workspace not 256-byte aligned
    assert lib.moe_combine_decode(C.byref(s), 0x60000, 0x70000, 0x90000, None, 0x80000, 16, None) == \
        q.MOE_ERR_WORKSPACE
    assert lib.moe_combine_decode(C.byref(q.MoeShape(2816, 704, 2112, top_k=0)), 0x60000, 0x70000, 0x90000, None,
                                  0x80000, 1 << 30, None) == q.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.moe_shared_expert_decode(C.byref(s), None, 0x50000, q.MOE_BF16, 0x80000, 1 << 30, None) == \
        q.MOE_ERR_INVALID_ARG
    no_shared = q.moe_layer(0x10000, 3346432, 128, 0x20000, 0x30000, 0)
    assert lib.moe_shared_expert_decode(C.byref(s), C.byref(no_shared), 0x50000, q.MOE_BF16, 0x80000, 1 << 30,
                                        None) == q.MOE_ERR_INVALID_ARG
    assert lib.moe_shared_expert_decode(C.byref(s), C.byref(_fake_layer()), 0x50004, q.MOE_BF16, 0x80000, 1 << 30,
                                        None) == q.MOE_ERR_INVALID_ARG


def test_status_strings():
    for st in (q.MOE_OK, q.MOE_ERR_INVALID_ARG, q.MOE_ERR_UNSUPPORTED_SHAPE, q.MOE_ERR_WORKSPACE, q.MOE_ERR_HIP,
               q.MOE_ERR_DEVICE_CHECK):
        assert q.moe_status_string(st) and q.moe_status_string(st) != "unknown status"
