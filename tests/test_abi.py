"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, agrees with the header's constants, and rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import pytest

import gemv_shot_all_amd as gsa
from gemv_shot_all_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsa.h")


def header_text():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(gsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    L = ctypes.CDLL(_lib.LIBRARY)
    for n in names:
        assert hasattr(L, n), f"{n} declared in gsa.h but not exported"
    assert sorted(_lib.EXPORTS) == names


def test_constants_match_header():
    text = header_text()
    for name in ["GSA_OK", "GSA_EINVAL", "GSA_ENOMEM", "GSA_EHIP", "GSA_ETIMEOUT",
                 "GSA_ESTATE", "GSA_ESPLIT", "GSA_FLAG_TILE_ROWS", "GSA_FLAG_GROUP_TILES",
                 "GSA_FLAG_GROUP_WORDS",
                 "GSA_MOE_TILE_ROWS",
                 "GSA_PAD_HEADER_WORDS",
                 "GSA_MAX_W", "GSA_MAX_B", "GSA_MOE_MAX_TOKENS", "GSA_MOE_MAX_F"]:
        m = re.search(rf"#define\s+{name}\s+\(?\s*(-?\d+)\s*\)?", text)
        assert m, name
        assert int(m.group(1)) == getattr(_lib, name), name
    m = re.search(r"#define\s+GSA_FLAG_PUBLISHED\s+(0x[0-9A-Fa-f]+)u", text)
    assert int(m.group(1), 16) == _lib.GSA_FLAG_PUBLISHED
    m = re.search(r"#define\s+GSA_MAX_X_LDS_BYTES\s+\((\d+)\s*\*\s*(\d+)\)", text)
    assert int(m.group(1)) * int(m.group(2)) == _lib.GSA_MAX_X_LDS_BYTES


def test_strerror_covers_codes():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert gsa.gsa_strerror(code) != "unknown error"
    assert gsa.gsa_strerror(7) == "unknown error"


def test_row_stride():
    assert gsa.gsa_signal_pad_row_stride(0) == -1
    # one flag per 4 rows, groups of 4 flags 32 words apart, rounded up to 64 words
    assert gsa.gsa_signal_pad_row_stride(1) == 64
    assert gsa.gsa_signal_pad_row_stride(32) == 64
    assert gsa.gsa_signal_pad_row_stride(33) == 128
    assert gsa.gsa_signal_pad_row_stride(8192) == 16384
    # flag tile t at word (t // 4) * 32 + t % 4 of a rank's row
    assert [int(gsa.flag_word(t)) for t in range(10)] == [0, 1, 2, 3, 32, 33, 34, 35, 64, 65]


P = 0x10000  # a 16-byte-aligned fake address: never dereferenced, rejected first


@pytest.mark.parametrize("args", [
    # (A, x, slots, pad, out, W, rank, N, K, B)
    (P, P, P, P, P, 0, 0, 16, 64, 1),       # W < 1
    (P, P, P, P, P, 9, 0, 16, 72, 1),       # W > 8
    (P, P, P, P, P, 2, 2, 16, 64, 1),       # rank >= W
    (P, P, P, P, P, 2, -1, 16, 64, 1),      # rank < 0
    (P, P, P, P, P, 2, 0, 0, 64, 1),        # N < 1
    (P, P, P, P, P, 3, 0, 16, 64, 1),       # K % W != 0
    (P, P, P, P, P, 2, 0, 16, 36, 1),       # Ks % 8 != 0
    (P, P, P, P, P, 2, 0, 16, 64, 0),       # B < 1
    (P, P, P, P, P, 2, 0, 16, 64, 17),      # B > 16
    (0, P, P, P, P, 2, 0, 16, 64, 1),       # null A
    (P, P, P, P, 0, 2, 0, 16, 64, 1),       # null out
    (P + 4, P, P, P, P, 2, 0, 16, 64, 1),   # misaligned A
    (P, P + 8, P, P, P, 2, 0, 16, 64, 1),   # misaligned x
    (P, P, P, P, P, 1, 0, 16, 8 * 8193, 8),   # B <= 8: x staging beyond the LDS bound
    (P, P, P, P, P, 2, 0, 16, 64, 1),       # slots not from gsa_symm_alloc
])
def test_gemv_allreduce_rejects_bad_arguments(args):
    rc = _lib.lib().gsa_gemv_allreduce(*args, None)
    assert rc == gsa.GSA_EINVAL


def test_rmsnorm_entry_point_rejects_bad_arguments():
    L = _lib.lib()
    good = (P, P, P, P, P, 2, 0, 16, 64, 1)

    def ep(**kw):
        e = _lib.gsa_epilogue(None, None, 1e-5, gsa.GSA_DTYPE_F32, P, None)
        for k, v in kw.items():
            setattr(e, k, v)
        return ctypes.byref(e)

    assert L.gsa_gemv_allreduce_rmsnorm(*good, None, None) == gsa.GSA_EINVAL  # no epilogue
    for bad in [dict(y=None), dict(y_dtype=2), dict(y_dtype=-1), dict(eps=-1.0),
                dict(eps=float("nan")), dict(eps=float("inf")), dict(y=P + 2),
                dict(bias=P + 2), dict(rms_weight=P + 1), dict(inv_rms=P + 3)]:
        assert L.gsa_gemv_allreduce_rmsnorm(*good, ep(**bad), None) == gsa.GSA_EINVAL, bad
    # a bf16 y only needs 2-byte alignment; everything valid but the fake
    # slots still fails the buffer registry check
    assert L.gsa_gemv_allreduce_rmsnorm(*good, ep(y=P + 2, y_dtype=gsa.GSA_DTYPE_BF16),
                                        None) == gsa.GSA_EINVAL
    # N > 2^24 with the epilogue
    big = (P, P, P, P, P, 1, 0, (1 << 24) + 1, 8, 1)
    assert L.gsa_gemv_allreduce_rmsnorm(*big, ep(), None) == gsa.GSA_EINVAL


def test_unfused_rmsnorm_rejects_bad_arguments():
    """gsa_bias_rmsnorm validates every argument before any HIP call."""
    L = _lib.lib()

    def ep(**kw):
        e = _lib.gsa_epilogue(None, None, 1e-5, gsa.GSA_DTYPE_F32, P, None)
        for k, v in kw.items():
            setattr(e, k, v)
        return ctypes.byref(e)

    assert L.gsa_bias_rmsnorm(P, 16, 1, None, None) == gsa.GSA_EINVAL  # no epilogue
    assert L.gsa_bias_rmsnorm(None, 16, 1, ep(), None) == gsa.GSA_EINVAL
    for N, B in [(0, 1), (-1, 1), ((1 << 24) + 1, 1), (16, 0), (16, gsa.GSA_MAX_B + 1)]:
        assert L.gsa_bias_rmsnorm(P, N, B, ep(), None) == gsa.GSA_EINVAL, (N, B)
    assert L.gsa_bias_rmsnorm(P + 2, 16, 1, ep(), None) == gsa.GSA_EINVAL  # misaligned out
    for bad in [dict(y=None), dict(y_dtype=2), dict(eps=-1.0), dict(eps=float("nan")),
                dict(y=P + 2), dict(bias=P + 2), dict(rms_weight=P + 1), dict(inv_rms=P + 3)]:
        assert L.gsa_bias_rmsnorm(P, 16, 1, ep(**bad), None) == gsa.GSA_EINVAL, bad


def test_two_shot_entry_point_rejects_bad_arguments():
    L = _lib.lib()
    A, x, slots, pad, out = P, P, P, P, P
    good = (2, 0, 16, 64, 1)
    # no gathered buffer, a misaligned one, one that is not the buffer's own
    assert L.gsa_gemv_allreduce_two_shot(A, x, slots, pad, None, out, *good, None) == (
        gsa.GSA_EINVAL)
    assert L.gsa_gemv_allreduce_two_shot(A, x, slots, pad, P + 4, out, *good, None) == (
        gsa.GSA_EINVAL)
    assert L.gsa_gemv_allreduce_two_shot(A, x, slots, pad, P, out, *good, None) == (
        gsa.GSA_EINVAL)
    # the plain call's argument checks apply too
    for bad in [(2, 2, 16, 64, 1), (3, 0, 16, 64, 1), (2, 0, 16, 64, 17), (2, 0, 0, 64, 1)]:
        assert L.gsa_gemv_allreduce_two_shot(A, x, slots, pad, P, out, *bad, None) == (
            gsa.GSA_EINVAL), bad
    assert L.gsa_symm_gathered(ctypes.c_void_p(P)) is None


def test_moe_entry_points_reject_bad_arguments():
    L = _lib.lib()
    assert L.gsa_a2a_pad_words(0, 1, 16) == -1
    assert L.gsa_a2a_pad_words(2, 0, 16) == -1
    assert L.gsa_a2a_pad_words(2, 1, 0) == -1
    assert L.gsa_a2a_pad_words(2, 3, 100) == gsa.GSA_PAD_HEADER_WORDS + 2 * 3 * 64
    h = ctypes.c_void_p()
    assert L.gsa_a2a_alloc(0, 1, 16, 4, ctypes.byref(h)) == gsa.GSA_EINVAL
    assert L.gsa_a2a_alloc(2, 257, 16, 4, ctypes.byref(h)) == gsa.GSA_EINVAL
    assert L.gsa_a2a_alloc(2, 1, 16, 0, ctypes.byref(h)) == gsa.GSA_EINVAL
    assert L.gsa_a2a_alloc(2, 1, 16, 4, None) == gsa.GSA_EINVAL
    assert L.gsa_a2a_free(ctypes.c_void_p(P)) == gsa.GSA_EINVAL
    assert L.gsa_a2a_buffers(ctypes.c_void_p(P)) is None
    assert L.gsa_a2a_signal_pads(ctypes.c_void_p(P)) is None
    assert L.gsa_a2a_reset(P, 2, 1, 16, 0, None) == gsa.GSA_EINVAL  # unknown pads
    c, t, p = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
    assert L.gsa_a2a_status(P, 0, None, ctypes.byref(c), ctypes.byref(t),
                            ctypes.byref(p)) == gsa.GSA_EINVAL
    # (X, Wd, splits, dst_off, bufs, pads, W, rank, ne, H, F, rows_in, rows_out)
    good = [P, P, P, P, P, P, 2, 0, 2, 64, 128, 8, 8]
    bad_cases = [
        (6, 0), (6, 9), (7, 2), (7, -1), (8, 0), (8, 257),   # W, rank, ne
        (9, 0), (10, 0), (10, 12), (10, 4096), (11, 0), (12, 0),  # H, F, rows_in, rows_out
        (0, 0), (1, 0), (2, 0), (3, 0), (4, 0), (5, 0),      # null pointers
        (0, P + 8), (1, P + 4), (4, P + 4), (5, P + 8), (2, P + 2), (3, P + 1),  # alignment
    ]
    for i, v in bad_cases:
        args = list(good)
        args[i] = v
        assert L.gsa_moe_gemm_all_to_all(*args, None) == gsa.GSA_EINVAL, (i, v)
    big = list(good)
    big[9], big[10] = 1 << 20, 1024  # H * F * 2 = 2^31: one expert past a buffer resource
    assert L.gsa_moe_gemm_all_to_all(*big, None) == gsa.GSA_EINVAL
    # every argument valid but the pads are not from gsa_a2a_alloc
    assert L.gsa_moe_gemm_all_to_all(*good, None) == gsa.GSA_EINVAL


def test_other_entry_points_reject_bad_arguments():
    L = _lib.lib()
    h = ctypes.c_void_p()
    assert L.gsa_symm_alloc(0, 16, 1, ctypes.byref(h)) == gsa.GSA_EINVAL
    assert L.gsa_symm_alloc(2, 0, 1, ctypes.byref(h)) == gsa.GSA_EINVAL
    assert L.gsa_symm_alloc(2, 16, 17, ctypes.byref(h)) == gsa.GSA_EINVAL
    assert L.gsa_symm_alloc(2, 16, 1, None) == gsa.GSA_EINVAL
    assert L.gsa_signal_pad_reset(P, 2, 16, 0, None) == gsa.GSA_EINVAL  # unknown pad
    assert L.gsa_signal_pad_reset(P, 2, 16, 0b100, None) == gsa.GSA_EINVAL  # mask > W bits
    c, t, p = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
    assert L.gsa_signal_pad_status(P, None, ctypes.byref(c), ctypes.byref(t),
                                   ctypes.byref(p)) == gsa.GSA_EINVAL
    assert L.gsa_set_wait_timeout_us(0) == gsa.GSA_EINVAL
    assert L.gsa_symm_free(ctypes.c_void_p(P)) == gsa.GSA_EINVAL
    assert L.gsa_symm_slots(ctypes.c_void_p(P)) is None
    assert L.gsa_symm_free(None) == gsa.GSA_OK
