"""Host-only checks of the C ABI: the library loads, exports every function
that include/csa.h declares, and rejects bad arguments before enqueueing
anything.  No kernel runs here (these tests run without a GPU)."""
import ctypes
import os
import re

import pytest

import long_context_attention_24_amd as csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
A = 0x10000   # a 16-byte aligned fake device address: never dereferenced on these paths


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:csa_status_t|int|size_t|const char\s*\*)\s*(\w+)\s*\(", src, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(csa.library_path()):
        pytest.fail("libcsa.so is not built; run python -m long_context_attention_24_amd.build")
    return csa.load_library()


def test_header_and_binding_agree():
    assert _declared() == set(csa.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.csa_abi_version() == 1


def test_status_strings(lib):
    assert lib.csa_status_string(0) == b"CSA_OK"
    assert lib.csa_status_string(1) == b"CSA_ERR_INVALID_ARGUMENT"
    assert lib.csa_status_string(2) == b"CSA_ERR_UNSUPPORTED"
    assert lib.csa_status_string(3) == b"CSA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.csa_status_string(4) == b"CSA_ERR_HIP"


def test_compress_validation(lib):
    f = lib.csa_compress
    assert f(None, 0, 0, A, 0, A, 0, 0, 1, 1, 8, 64, 4, None) == INVALID
    assert f(A, 512, 64, A, 8, A, 128, 64, 1, 1, 8, 64, 0, None) == INVALID        # m = 0
    assert f(A, 512, 64, A, 8, A, 128, 64, 1, 0, 8, 64, 4, None) == INVALID        # B = 0
    assert f(A, 512, 64, A, 8, A, 128, 64, 2, 1, 8, 64, 4, None) == UNSUPPORTED    # FP4 data
    assert f(A, 512, 64, A, 8, A, 128, 64, 1, 1, 8, 60, 4, None) == UNSUPPORTED    # 120 B rows
    assert f(A + 2, 512, 64, A, 8, A, 128, 64, 1, 1, 8, 64, 4, None) == INVALID    # misaligned
    assert f(A, 512, 64, A, 8, A, 128, 64, 1, 1, 8, 64, 5000, None) == UNSUPPORTED
    assert b"m=5000" in lib.csa_last_error()


def test_quantize_mx4_validation(lib):
    f = lib.csa_quantize_mx4
    args = [A, 128, 1, 4, 128, A, 64, A, 4, None]          # bf16 [4, 128] -> codes, scales
    bad = list(args); bad[0] = None
    assert f(*bad) == INVALID
    bad = list(args); bad[4] = 96 + 8                      # D not a multiple of 32
    assert f(*bad) == INVALID
    bad = list(args); bad[2] = 2                           # FP4 input
    assert f(*bad) == UNSUPPORTED
    bad = list(args); bad[6] = 56                          # code rows not 16-byte multiples
    assert f(*bad) == INVALID
    bad = list(args); bad[8] = 3                           # scale rows shorter than D/32
    assert f(*bad) == INVALID
    bad = list(args); bad[5] = A + 8                       # misaligned codes
    assert f(*bad) == INVALID
    bad = list(args); bad[3] = 0                           # no rows
    assert f(*bad) == INVALID


def test_index_score_validation(lib):
    f = lib.csa_index_score
    args = [A, None, A, A, None, 32768 * 128, 128, 0, 0, 1, A, A, 2, 1, 32768, 64, 128, 4, A, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == INVALID
    bad = list(args); bad[16] = 96                       # D_I = 96
    assert f(*bad) == UNSUPPORTED
    bad = list(args); bad[15] = 65                       # H_I = 65
    assert f(*bad) == UNSUPPORTED
    bad = list(args); bad[6] = 100                       # row stride not 16-byte multiple
    assert f(*bad) == INVALID
    bad = list(args); bad[9] = 2                         # FP4 without scales
    assert f(*bad) == INVALID
    bad = list(args); bad[18] = None                     # no output
    assert f(*bad) == INVALID


def test_topk_validation_and_workspace(lib):
    sz = ctypes.c_size_t(123)
    assert lib.csa_topk_workspace(16, 1, 32768, 1024, ctypes.byref(sz)) == OK
    assert sz.value == 0                                  # one segment: no workspace
    assert lib.csa_topk_workspace(4, 1, 262144, 1024, ctypes.byref(sz)) == OK
    assert sz.value == 4 * 8 * 1024 * 8                   # 8 segments of candidates
    assert lib.csa_topk_workspace(1, 1, 32768, 0, ctypes.byref(sz)) == INVALID
    assert lib.csa_topk_workspace(1, 1, 32768, 4096, ctypes.byref(sz)) == UNSUPPORTED
    assert lib.csa_topk_workspace(1, 1, 1 << 22, 1024, ctypes.byref(sz)) == UNSUPPORTED
    f = lib.csa_topk
    # workspace too small for a multi-segment row; nothing is launched
    assert f(A, 262144, A, A, 4, 1, 262144, 4, 1024, A, None, A, 16, None) == WS_SMALL
    assert f(A, 30, A, A, 1, 1, 30, 4, 8, A, None, None, 0, None) == INVALID   # s_rs % 4
    assert f(None, 32, A, A, 1, 1, 32, 4, 8, A, None, None, 0, None) == INVALID


def test_index_topk_workspace(lib):
    sz = ctypes.c_size_t(0)
    assert lib.csa_index_topk_workspace(16, 1, 32768, 1024, ctypes.byref(sz)) == OK
    assert sz.value >= 16 * 32768 * 4
    f = lib.csa_index_topk
    args = [A, None, A, A, None, 32768 * 128, 128, 0, 0, 1, A, A, 16, 1, 32768, 64, 128, 4,
            1024, A, None, A, 1024, None]
    assert f(*args) == WS_SMALL


def test_index_topk_bf16_workspace_and_validation(lib):
    sz, sz32 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.csa_index_topk_bf16_workspace(16, 1, 32768, 1024, ctypes.byref(sz)) == OK
    assert lib.csa_index_topk_workspace(16, 1, 32768, 1024, ctypes.byref(sz32)) == OK
    assert 16 * 32768 * 2 <= sz.value < sz32.value     # 2-byte score rows
    assert lib.csa_index_topk_bf16_workspace(1, 1, 262145, 1024, ctypes.byref(sz)) == UNSUPPORTED
    assert lib.csa_index_topk_bf16_workspace(1, 1, 32768, 4096, ctypes.byref(sz)) == UNSUPPORTED
    assert lib.csa_index_topk_bf16_workspace(0, 1, 32768, 1024, ctypes.byref(sz)) == INVALID
    f = lib.csa_index_topk_bf16
    args = [A, A, A, 32768 * 128, 128, A, A, 16, 1, 32768, 4, 1024, A, None, A, 1024, None]
    assert f(*args) == WS_SMALL
    bad = list(args)
    bad[4] = 100                                        # key row stride below 128
    assert f(*bad) == INVALID
    assert f(*(args[:11] + [0] + args[12:])) == INVALID   # k = 0


def test_attend_validation(lib):
    sz = ctypes.c_size_t(0)
    assert lib.csa_attend_workspace(1, 16, 1, 64, 128, 1024, ctypes.byref(sz)) == OK
    assert sz.value > 0
    assert lib.csa_attend_workspace(0, 1, 256, 4, 64, 16, ctypes.byref(sz)) == OK
    assert sz.value == 0                                  # fp32 generic path: none
    f = lib.csa_attend
    good = [A, A, A, 32768 * 128, 128, A, A, 1, 16, 1, 64, 128, 32768, 1024, 0.088, A, None, A,
            1 << 30, None]
    bad = list(good); bad[5] = None
    assert f(*bad) == INVALID
    bad = list(good); bad[11] = 96
    assert f(*bad) == UNSUPPORTED
    bad = list(good); bad[10] = 128                       # H = 128
    assert f(*bad) == UNSUPPORTED
    bad = list(good); bad[18] = 16                        # workspace too small
    assert f(*bad) == WS_SMALL
    bad = list(good); bad[7] = 2                          # FP4 core attention
    assert f(*bad) == UNSUPPORTED
    g = lib.hca_attend
    good = [A, A, A, 8192 * 128, 128, A, A, 1, 32, 1, 64, 128, 8192, 128, 0.088, A, None, A,
            1 << 30, None]
    bad = list(good); bad[13] = 0                         # m = 0
    assert g(*bad) == INVALID
    bad = list(good); bad[4] = 120                        # row stride < D
    assert g(*bad) == INVALID


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(csa, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(csa, "_lib", None)
    with pytest.raises(ImportError):
        csa.load_library()
