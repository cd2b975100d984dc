"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects invalid arguments before touching the GPU (no compute
call is made here, so this runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "keops_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(keops_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from geometric_map_reduce_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    return binding.lib()


def test_header_declares_the_reductions():
    names = declared_functions()
    for n in ("keops_gauss_sum", "keops_gauss_lse", "keops_gauss_grad_x", "keops_gauss_grad_y",
              "keops_gauss_grad_b", "keops_gauss_cg", "keops_gauss_max", "keops_gauss_min", "keops_laplace_sum",
              "keops_kmin"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    from geometric_map_reduce_amd import binding
    assert binding.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert binding.status_string(s) not in ("ok", "unknown status")
    assert binding.status_string(-99) == "unknown status"


FAKE = ctypes.c_void_p(0x10000)     # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000000)


@pytest.mark.parametrize("args,rc", [
    ((None, None, None, -1, 0, 3, 1, 1.0, None, None), -1),        # M < 0
    ((None, None, None, 0, -1, 3, 1, 1.0, None, None), -1),        # N < 0
    ((None, None, None, 0, 0, 0, 1, 1.0, None, None), -1),         # D < 1
    ((None, None, None, 0, 0, 3, 0, 1.0, None, None), -1),         # E < 1
    ((None, None, None, 0, 0, 3, 1, 0.0, None, None), -1),         # sigma = 0
    ((None, None, None, 0, 0, 3, 1, -1.0, None, None), -1),        # sigma < 0
    ((None, None, None, 0, 0, 3, 1, float("nan"), None, None), -1),
    ((None, None, None, 0, 0, 3, 1, float("inf"), None, None), -1),
    ((None, FAKE, FAKE, 5, 7, 3, 1, 1.0, FAKE2, None), -1),        # x null with M > 0
    ((FAKE, None, FAKE, 5, 7, 3, 1, 1.0, FAKE2, None), -1),        # y null with N > 0
    ((FAKE, FAKE, FAKE, 5, 7, 3, 1, 1.0, None, None), -1),         # out null
    ((FAKE, FAKE2, FAKE2, 5, 7, 3, 1, 1.0, FAKE, None), -1),       # out overlaps x
    ((ctypes.c_void_p(0x10002), FAKE2, FAKE2, 5, 7, 3, 1, 1.0, ctypes.c_void_p(0x900000), None), -1),  # misaligned
    ((None, None, None, 0, 0, 9, 1, 1.0, None, None), -2),         # D not compiled
    ((None, None, None, 0, 0, 3, 5, 1.0, None, None), -2),         # E not compiled
    ((None, None, None, 0, 0, 3, 1, 1.0, None, None), 0),          # M = 0: no-op
])
def test_gauss_sum_validation(L, args, rc):
    assert L.keops_gauss_sum(*args) == rc
    assert L.keops_gauss_lse(*args) == rc


def test_grad_needs_g(L):
    assert L.keops_gauss_grad_x(FAKE, FAKE2, FAKE2, None, 5, 7, 3, 1, 1.0, ctypes.c_void_p(0x900000), None) == -1
    assert L.keops_gauss_grad_x(None, None, None, None, 0, 0, 3, 1, 1.0, None, None) == 0


def test_transposed_gradients_validation(L):
    out = ctypes.c_void_p(0x900000)
    # grad_y needs b (the cotangent side of the exchanged roles) and g when M > 0
    assert L.keops_gauss_grad_y(FAKE, FAKE2, None, FAKE, 5, 7, 3, 1, 1.0, out, None) == -1
    assert L.keops_gauss_grad_y(FAKE, FAKE2, FAKE2, None, 5, 7, 3, 1, 1.0, out, None) == -1
    assert L.keops_gauss_grad_b(FAKE, FAKE2, None, 5, 7, 3, 1, 1.0, out, None) == -1
    assert L.keops_gauss_grad_b(FAKE, FAKE2, FAKE, 5, 7, 3, 1, -1.0, out, None) == -1
    assert L.keops_gauss_grad_b(FAKE, FAKE2, FAKE, 5, 7, 99, 1, 1.0, out, None) == -2
    # N = 0: nothing to write
    assert L.keops_gauss_grad_y(None, None, None, None, 0, 0, 3, 1, 1.0, None, None) == 0
    assert L.keops_gauss_grad_b(None, None, None, 0, 0, 3, 1, 1.0, None, None) == 0


@pytest.mark.parametrize("args,rc", [
    ((None, None, None, 0, 5, 3, 0, 1.0, None, None, None), -1),       # K < 1
    ((None, None, None, 0, 5, 3, 6, 1.0, None, None, None), -1),       # K > N
    ((None, FAKE, None, 0, 5, 0, 1, 1.0, None, None, None), -1),       # D < 1
    ((None, FAKE, None, 0, 100, 3, 17, 1.0, None, None, None), -2),    # K not compiled
    ((None, FAKE, None, 0, 5, 9, 2, 1.0, None, None, None), -2),       # D not compiled
    ((None, FAKE, None, 0, 1 << 31, 3, 2, 1.0, None, None, None), -2),  # N >= 2^31
    ((None, FAKE, None, 0, 5, 3, 5, 1.0, None, None, None), 0),        # M = 0: no-op
    ((None, FAKE, FAKE2, 0, 5, 3, 5, float("nan"), None, None, None), 0),   # b, sigma never read
    ((FAKE, FAKE2, None, 4, 5, 3, 2, 1.0, None, ctypes.c_void_p(0x900000), None), -1),   # out_d null
    ((FAKE, FAKE2, None, 4, 5, 3, 2, 1.0, ctypes.c_void_p(0x900000), ctypes.c_void_p(0x900004), None), -1),  # idx misaligned
])
def test_kmin_validation(L, args, rc):
    assert L.keops_kmin(*args) == rc


def test_options(L):
    assert L.keops_set_option(99, 1) == -1
    assert L.keops_set_option(1, -1) == -1
    assert L.keops_set_option(2, 2) == -1
    assert L.keops_set_option(3, 4) == -1
    assert L.keops_set_option(5, -1) == -1
    assert L.keops_set_option(5, 4097) == -1
    assert L.keops_set_option(5, 16) == 0
    assert L.keops_set_option(6, 3) == -1
    assert L.keops_set_option(6, 2) == 0
    assert L.keops_set_option(6, 1) == 0
    assert L.keops_set_option(7, 3) == -1         # workspace cache: 0 automatic, 1 on, 2 off
    assert L.keops_set_option(7, 1) == 0
    assert L.keops_set_option(8, 2) == -1         # forced allocation failure: 0 / 1
    assert L.keops_set_option(8, 1) == 0
    for opt in (1, 2, 3, 5, 6, 7, 8):
        assert L.keops_set_option(opt, 0) == 0
    assert L.keops_version() >= 100


def test_cg_validation(L):
    out = ctypes.c_void_p(0x900000)
    it = ctypes.c_int32(7)
    res = (ctypes.c_float * 4)()
    for args in [(FAKE, FAKE2, 10, 3, 1, 0.0, 1.0, 1e-5, 10),      # sigma = 0
                 (FAKE, FAKE2, 10, 3, 1, 1.0, -1.0, 1e-5, 10),     # lambda < 0
                 (FAKE, FAKE2, 10, 3, 1, 1.0, 1.0, -1e-5, 10),     # rtol < 0
                 (FAKE, FAKE2, 10, 3, 1, 1.0, 1.0, 1e-5, -1),      # max_iter < 0
                 (None, FAKE2, 10, 3, 1, 1.0, 1.0, 1e-5, 10)]:     # missing x
        assert L.keops_gauss_cg(*args, out, ctypes.byref(it), res, None) == -1
    assert L.keops_gauss_cg(FAKE, FAKE2, 10, 3, 5, 1.0, 1.0, 1e-5, 10, out, None, None, None) == -2   # E > 4
    assert L.keops_gauss_cg(FAKE, FAKE2, 10, 99, 1, 1.0, 1.0, 1e-5, 10, out, None, None, None) == -2  # D
    assert L.keops_gauss_cg(None, None, 0, 3, 2, 1.0, 0.0, 1e-5, 10, None, ctypes.byref(it), res, None) == 0
    assert it.value == 0 and res[0] == 0.0 and res[1] == 0.0


def test_max_validation(L):
    out = ctypes.c_void_p(0x900000)
    idx = ctypes.c_void_p(0xA00000)
    assert L.keops_gauss_max(FAKE, FAKE2, FAKE2, 5, 7, 3, 1, 1.0, out, None, None) == -1          # no indices
    assert L.keops_gauss_max(FAKE, FAKE2, FAKE2, 5, 7, 3, 1, 1.0, out, ctypes.c_void_p(0xA00004), None) == -1
    assert L.keops_gauss_min(FAKE, FAKE2, FAKE2, 5, 7, 3, 1, 0.0, out, idx, None) == -1            # sigma
    assert L.keops_gauss_min(FAKE, FAKE2, FAKE2, 5, 7, 99, 1, 1.0, out, idx, None) == -2           # D
    assert L.keops_gauss_max(None, None, None, 0, 0, 3, 1, 1.0, None, None, None) == 0



def test_noalloc_validation(L):
    out = ctypes.c_void_p(0x900000)
    # the same argument rules as keops_gauss_sum
    assert L.keops_gauss_sum_noalloc(FAKE, FAKE2, FAKE2, 5, 7, 3, 1, 0.0, out, None) == -1
    assert L.keops_gauss_sum_noalloc(None, None, None, 0, 0, 9, 1, 1.0, None, None) == -2
    assert L.keops_gauss_sum_noalloc(None, None, None, 0, 0, 3, 1, 1.0, None, None) == 0
    # D >= 32 with more rows than the scratch has form flags for: rejected before any HIP call
    M = 1 << 36
    x, y, o = ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 48), ctypes.c_void_p(1 << 52)
    assert L.keops_gauss_sum_noalloc(x, y, y, M, 10, 50, 1, 1.0, o, None) == -5
    from geometric_map_reduce_amd import binding
    assert "scratch" in binding.status_string(-5)
