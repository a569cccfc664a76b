"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching any device.

Only argument combinations that the library refuses during host-side
validation are passed with fake pointers; nothing here can reach a kernel."""

import ctypes
import os
import re

import pytest
import torch

import fp8_precision_numerics_amd as fm
from fp8_precision_numerics_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mi.h")

OK, ENULL, ESHAPE, EALIGN, EFMT, EDTYPE, ELAUNCH, EDEV, EACCUM = 0, -1, -2, -3, -4, -5, -6, -7, -8
A16 = ctypes.c_void_p(0x10000)        # 16-B aligned fake address (never dereferenced)
A8 = ctypes.c_void_p(0x10008)         # misaligned fake address


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^FP8MI_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.MULTILINE)))


@pytest.fixture(scope="module")
def lib():
    return fm.load_library()


def test_header_declares_the_bound_symbols():
    assert declared_symbols() == sorted(_binding.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert fm.version() == 800
    for code in (OK, ENULL, ESHAPE, EALIGN, EFMT, EDTYPE, ELAUNCH, EDEV, EACCUM):
        assert fm.status_string(code) and fm.status_string(code) != "unknown status"
    assert fm.status_string(12345) == "unknown status"


def test_quantize_argument_errors(lib):
    q = lib.fp8_quantize
    assert q(A16, 7, 4, 16, 0, A16, A16, None, None, None, None, 0, None) == EDTYPE
    assert q(A16, 0, 4, 16, 9, A16, A16, None, None, None, None, 0, None) == EFMT
    assert q(A16, 0, -1, 16, 0, A16, A16, None, None, None, None, 0, None) == ESHAPE
    assert q(A16, 0, 1 << 40, 1 << 40, 0, A16, A16, None, None, None, None, 0, None) == ESHAPE
    assert q(A16, 0, 4, 16, 0, A16, None, None, None, None, None, 0, None) == ENULL      # no output at all
    assert q(A16, 0, 4, 16, 0, None, A16, None, None, None, None, 0, None) == ENULL      # cast without a scale
    assert q(None, 0, 4, 16, 0, A16, A16, None, None, None, None, 0, None) == ENULL
    assert q(A8, 0, 4, 16, 0, A16, A16, None, None, None, None, 0, None) == EALIGN
    assert q(A16, 0, 4, 16, 0, A16, A8, None, None, None, None, 0, None) == EALIGN
    assert q(A16, 0, 4, 24, 0, A16, None, A16, None, None, None, 0, None) == EALIGN      # transpose needs 16 | cols
    assert q(A16, 0, 20, 16, 0, A16, None, A16, None, None, None, 0, None) == EALIGN     # ... and 16 | rows
    assert q(None, 0, 0, 16, 0, A16, A16, None, None, None, None, 0, None) == OK         # empty, no reductions
    assert q(A16, 0, 4, 16, 0, A16, A16, None, A16, None, A8, 64, None) == EALIGN       # workspace alignment
    assert q(A16, 0, 4, 16, 0, A16, A16, None, A16, None, A16, 8, None) == EALIGN       # workspace < 16 B


def test_gemm_requant_argument_errors(lib):
    g = lib.fp8_gemm_requant
    #      A    fa  B    fb  M   N   K   sa   sb  ofmt out_s Cq  amax sat accum stream
    assert g(A16, 0, A16, 0, 16, 16, 16, A16, A16, 7, A16, A16, None, None, 0, None) == EFMT     # out format
    assert g(A16, 2, A16, 0, 16, 16, 16, A16, A16, 0, A16, A16, None, None, 0, None) == EFMT
    assert g(A16, 0, A16, 0, 16, 16, 16, A16, A16, 0, A16, A16, None, None, 5, None) == EACCUM
    assert g(A16, 0, A16, 0, 16, 16, 24, A16, A16, 0, A16, A16, None, None, 0, None) == EALIGN   # 16 | K
    assert g(A16, 0, A16, 0, -1, 16, 16, A16, A16, 0, A16, A16, None, None, 0, None) == ESHAPE
    assert g(A16, 0, A16, 0, 16, 16, 1 << 24, A16, A16, 0, A16, A16, None, None, 0, None) == ESHAPE
    assert g(A16, 0, A16, 0, 16, 16, 16, A16, A16, 0, None, A16, None, None, 0, None) == ENULL    # no out scale
    assert g(A16, 0, A16, 0, 16, 16, 16, A16, A16, 0, A16, None, None, None, 0, None) == ENULL    # no output
    assert g(A16, 0, A16, 0, 16, 16, 16, A16, A16, 0, A16, A8, None, None, 0, None) == EALIGN
    assert g(None, 0, None, 0, 0, 16, 16, None, None, 0, None, None, None, None, 0, None) == OK  # empty, no stats


def test_allreduce_parts_argument_errors(lib):
    sc, ds = lib.fp8_shared_scale, lib.fp8_dequant_sum
    assert sc(A16, 4, 3, A16, A16, None) == EFMT
    assert sc(A16, 0, 1, A16, A16, None) == ESHAPE
    assert sc(A16, 65537, 1, A16, A16, None) == ESHAPE
    assert sc(None, 4, 1, A16, A16, None) == ENULL
    assert sc(A16, 4, 1, A16, None, None) == ENULL
    #        q    R  n    stride fmt sinv out otype stream
    assert ds(A16, 2, 64, 64, 7, A16, A16, 0, None) == EFMT
    assert ds(A16, 2, 64, 64, 1, A16, A16, 9, None) == EDTYPE
    assert ds(A16, 0, 64, 64, 1, A16, A16, 0, None) == ESHAPE
    assert ds(A16, 2, 64, 32, 1, A16, A16, 0, None) == ESHAPE       # stride < n
    assert ds(A16, 2, 64, 72, 1, A16, A16, 0, None) == EALIGN       # stride not a multiple of 16
    assert ds(A8, 2, 64, 64, 1, A16, A16, 0, None) == EALIGN
    assert ds(A16, 2, 64, 64, 1, A16, A8, 0, None) == EALIGN
    assert ds(A16, 2, 64, 64, 1, None, A16, 0, None) == ENULL
    assert ds(None, 2, 0, 0, 1, None, None, 0, None) == OK          # empty


def test_mx_argument_errors(lib):
    qm, gm = lib.fp8_quantize_mx, lib.fp8_gemm_mx
    assert qm(A16, 7, 4, 64, 0, A16, A16, None) == EDTYPE
    assert qm(A16, 0, 4, 64, 9, A16, A16, None) == EFMT
    assert qm(A16, 0, 4, 48, 0, A16, A16, None) == EALIGN        # 32 | cols
    assert qm(A16, 0, -1, 64, 0, A16, A16, None) == ESHAPE
    assert qm(A16, 0, 4, 64, 0, A16, None, None) == ENULL
    assert qm(A8, 0, 4, 64, 0, A16, A16, None) == EALIGN
    assert qm(None, 0, 0, 64, 0, None, None, None) == OK           # empty
    #        A    fa  sa   B    fb  sb   M   N   K    C   ct acc stream
    assert gm(A16, 0, A16, A16, 3, A16, 16, 16, 128, A16, 0, 0, None) == EFMT
    assert gm(A16, 0, A16, A16, 0, A16, 16, 16, 128, A16, 4, 0, None) == EDTYPE
    assert gm(A16, 0, A16, A16, 0, A16, 16, 16, 128, A16, 0, 5, None) == EACCUM
    assert gm(A16, 0, A16, A16, 0, A16, 16, 16, 96, A16, 0, 0, None) == EALIGN   # 128 | K
    assert gm(A16, 0, None, A16, 0, A16, 16, 16, 128, A16, 0, 0, None) == ENULL
    assert gm(A16, 0, ctypes.c_void_p(0x10002), A16, 0, A16, 16, 16, 128, A16, 0, 0, None) == EALIGN
    assert gm(A16, 0, A16, A16, 0, A16, 16, 16, 1 << 24, A16, 0, 0, None) == ESHAPE
    # the A scale matrix (K/32 x 2^20 bytes = 4 GiB) would not fit a 32-bit load offset
    assert gm(A16, 0, A16, A16, 0, A16, 1 << 20, 16, 1 << 17, A16, 0, 0, None) == ESHAPE


def test_quantize_update_argument_errors(lib):
    u = lib.fp8_quantize_update
    #        x   xt rows cols fmt q    qt    amax sat  ws   wsb hist  len head scale sinv status used stream
    assert u(A16, 7, 4, 16, 0, A16, None, A16, None, None, 0, A16, 16, A16, A16, A16, None, None, None) == EDTYPE
    assert u(A16, 0, 4, 16, 9, A16, None, A16, None, None, 0, A16, 16, A16, A16, A16, None, None, None) == EFMT
    assert u(A16, 0, 4, 16, 0, A16, None, A16, None, None, 0, A16, 0, A16, A16, A16, None, None, None) == ESHAPE
    assert u(A16, 0, 4, 16, 0, A16, None, None, None, None, 0, A16, 16, A16, A16, A16, None, None, None) == ENULL
    assert u(A16, 0, 4, 16, 0, A16, None, A16, None, None, 0, None, 16, A16, A16, A16, None, None, None) == ENULL
    assert u(A16, 0, 4, 16, 0, A16, None, A16, None, None, 0, A16, 16, A16, None, A16, None, None, None) == ENULL
    assert u(A8, 0, 4, 16, 0, A16, None, A16, None, None, 0, A16, 16, A16, A16, A16, None, None, None) == EALIGN
    assert u(A16, 0, 4, 24, 0, None, A16, A16, None, None, 0, A16, 16, A16, A16, A16, None, None, None) == EALIGN


def test_amax_update_argument_errors(lib):
    u = lib.fp8_amax_update
    #        hist len  head amax fmt scale sinv status stream
    assert u(A16, 16, A16, A16, 5, A16, A16, None, None) == EFMT
    assert u(None, 16, A16, A16, 0, A16, A16, None, None) == ENULL
    assert u(A16, 16, A16, A16, 0, None, A16, None, None) == ENULL
    assert u(A16, 0, A16, A16, 0, A16, A16, None, None) == ESHAPE
    assert u(A16, 4097, A16, A16, 0, A16, A16, None, None) == ESHAPE


def test_gemm_argument_errors(lib):
    g = lib.fp8_gemm
    #        A   fa  B   fb bt  M   N   K   sa   sb   C   ct acc stream
    assert g(A16, 3, A16, 0, 0, 16, 16, 16, A16, A16, A16, 0, 0, None) == EFMT
    assert g(A16, 0, A16, 0, 0, 16, 16, 16, A16, A16, A16, 4, 0, None) == EDTYPE
    assert g(A16, 0, A16, 0, 0, 16, 16, 16, A16, A16, A16, 0, 7, None) == EACCUM
    assert g(A16, 0, A16, 0, 0, 16, 16, 0, A16, A16, A16, 0, 0, None) == ESHAPE
    assert g(A16, 0, A16, 0, 0, -1, 16, 16, A16, A16, A16, 0, 0, None) == ESHAPE
    assert g(A16, 0, A16, 0, 0, 1 << 31, 16, 16, A16, A16, A16, 0, 0, None) == ESHAPE
    assert g(A16, 0, A16, 0, 0, 16, 16, (1 << 23) + 16, A16, A16, A16, 0, 0, None) == ESHAPE   # K limit
    assert g(A16, 0, A16, 0, 0, 16, 16, 24, A16, A16, A16, 0, 0, None) == EALIGN     # K % 16
    assert g(None, 0, A16, 0, 0, 16, 16, 16, A16, A16, A16, 0, 0, None) == ENULL
    assert g(A16, 0, A16, 0, 0, 16, 16, 16, None, A16, A16, 0, 0, None) == ENULL
    assert g(A8, 0, A16, 0, 0, 16, 16, 16, A16, A16, A16, 0, 0, None) == EALIGN
    assert g(A16, 0, A16, 0, 0, 16, 16, 16, A16, A16, A8, 0, 0, None) == EALIGN
    assert g(None, 0, None, 0, 0, 0, 16, 16, None, None, None, 0, 0, None) == OK      # M == 0 is a no-op
    # B stored [K x N]: N a multiple of 16, K * N < 2^31
    assert g(A16, 0, A16, 0, 1, 16, 24, 16, A16, A16, A16, 0, 0, None) == EALIGN
    assert g(A16, 0, A16, 0, 1, 16, 1 << 20, 1 << 11, A16, A16, A16, 0, 0, None) == ESHAPE


def test_blockwise_and_grouped_argument_errors(lib):
    b = lib.fp8_quantize_blockwise
    assert b(A16, 0, 4, 128, 2, 0, A16, A16, None) == ESHAPE
    assert b(A16, 0, 4, 120, 1, 0, A16, A16, None) == EALIGN
    assert b(A16, 0, 4, 128, 1, 0, None, A16, None) == ENULL
    assert b(A8, 0, 4, 128, 1, 0, A16, A16, None) == EALIGN
    gg = lib.fp8_grouped_gemm
    assert gg(A16, A16, A16, A16, A16, 0, 16, 16, 128, A16, 0, 0, None) == ESHAPE
    assert gg(A16, A16, A16, A16, A16, 2000, 16, 16, 128, A16, 0, 0, None) == ESHAPE
    assert gg(A16, A16, A16, A16, A16, 2, 16, 16, 120, A16, 0, 0, None) == EALIGN
    assert gg(A16, A16, A16, A16, None, 2, 16, 16, 128, A16, 0, 0, None) == ENULL
    assert gg(A16, A16, A16, A16, A16, 2, 16, 16, 128, A16, 9, 0, None) == EDTYPE
    assert gg(A16, A16, A16, A16, A16, 2, 16, 16, 128, A16, 0, 2, None) == EACCUM
    assert gg(A16, A16, A16, A16, A16, 2, 16, 16, (1 << 22) + 16, A16, 0, 0, None) == ESHAPE   # K limit


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path")
def test_valid_arguments_without_a_device_report_device_error(lib):
    assert lib.fp8_gemm(A16, 0, A16, 0, 0, 16, 16, 16, A16, A16, A16, 0, 0, None) == EDEV
    assert lib.fp8_amax_update(A16, 16, A16, A16, 0, A16, A16, None, None) == EDEV


def test_python_binding_rejects_host_tensors():
    x = torch.zeros(4, 16)
    with pytest.raises(ValueError):
        fm.fp8_quantize(x, "e4m3", amax=torch.zeros(1))
    with pytest.raises(ValueError):
        fm.fp8_quantize(x, "e9m9", amax=torch.zeros(1))


def test_recipe_defaults_follow_the_pages():
    r = fm.Recipe()
    assert (r.fmt_fwd, r.fmt_bwd, r.history_len, r.algo) == ("e4m3", "e5m2", 16, "max")
    with pytest.raises(ValueError):
        fm.Recipe(algo="most_recent")
