"""The C ABI on the host (no GPU): the library loads, exports every function
include/w4.h declares, and rejects bad arguments before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("w4_gemv", "w4_gemm_smallM", "w4_moe_gemv_ids", "w4_embed_gather",
              "w4_rms_renorm", "w4_gemv_chain", "w4_probe_stream", "w4_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import bit_weight_only_02_amd as w4
    for n in declared_functions():
        assert hasattr(w4.lib, n), n
        assert getattr(w4, n, None) is not None or n in ("w4_strerror", "w4_last_error_detail"), n


def test_strerror_texts():
    import bit_weight_only_02_amd as w4
    assert w4.lib.w4_strerror(0) == b"ok"
    for s in range(-6, 0):
        assert w4.lib.w4_strerror(s) not in (b"ok", b"unknown status")
    assert w4.lib.w4_strerror(-99) == b"unknown status"


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,expect", [
    # codes, steps, N, K, x, xdt, y
    ((FAKE, FAKE, 4, 33, FAKE, 0, FAKE), -1),          # K % 32
    ((FAKE, FAKE, -1, 32, FAKE, 0, FAKE), -1),         # negative N
    ((FAKE, FAKE, 4, 32768, FAKE, 0, FAKE), -4),       # K beyond the limit
    ((None, FAKE, 4, 32, FAKE, 0, FAKE), -1),          # null codes
    ((FAKE, FAKE, 4, 32, None, 0, FAKE), -1),          # null x
    ((FAKE, FAKE, 4, 32, FAKE, 0, None), -1),          # null y
    ((FAKE + 4, FAKE, 4, 32, FAKE, 0, FAKE), -2),      # codes not 16-B aligned
    ((FAKE, FAKE + 1, 4, 32, FAKE, 0, FAKE), -2),      # steps misaligned
    ((FAKE, FAKE, 4, 32, FAKE, 7, FAKE), -3),          # dtype
])
def test_gemv_argument_errors(args, expect):
    import bit_weight_only_02_amd as w4
    assert w4.lib.w4_gemv(*args, None) == expect
    assert w4.lib.w4_last_error_detail() != b""


def test_empty_gemv_is_a_no_op():
    import bit_weight_only_02_amd as w4
    assert w4.lib.w4_gemv(None, None, 0, 64, None, 0, None, None) == 0


def test_gather_and_renorm_argument_errors():
    import bit_weight_only_02_amd as w4
    L = w4.lib
    assert L.w4_embed_gather(FAKE, FAKE, 10, 48, FAKE, 4, FAKE, None, None) == -1   # K % 32
    assert L.w4_embed_gather(FAKE, FAKE, 10, 64, FAKE, 4, FAKE + 2, None, None) == -2
    assert L.w4_embed_gather(FAKE, FAKE, 10, 64, None, 4, FAKE, None, None) == -1
    assert L.w4_embed_gather(FAKE, FAKE, 10, 64, FAKE, 0, FAKE, None, None) == 0    # empty
    assert L.w4_rms_renorm(FAKE, 64, FAKE, 5, None) == -3
    assert L.w4_rms_renorm(None, 64, FAKE, 0, None) == -1
    assert L.w4_probe_stream(FAKE, 17, FAKE, None) == -1


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")
def test_valid_call_without_device_reports_an_error():
    import bit_weight_only_02_amd as w4
    rc = w4.lib.w4_gemv(FAKE, FAKE, 4, 32, FAKE, 0, FAKE, None)
    assert rc in (-5, -6)
