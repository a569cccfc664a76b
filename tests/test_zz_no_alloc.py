"""GPU: fp8_quantize_update_noalloc (the library's own per-GPU scratch) against
fp8_quantize_update with a caller workspace, through the C ABI.

Two delayed-scaling states start identical; each call goes to one of them
through each entry point, and every output (codes, transposed codes, amax,
saturation count, history ring, head, scale, inverse scale, status, the
inverse scale the cast used) must agree bit for bit.  Calls follow each other
with smaller inputs, so the shared scratch holds more slots from the previous
call than the next grid writes: those leftovers must not leak into a result."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device

pytestmark = pytest.mark.gpu


class State:
    def __init__(self, fmt, length, dev):
        self.fmt = fmt
        self.history = torch.zeros(length, dtype=torch.float32, device=dev)
        self.head = torch.zeros(1, dtype=torch.int32, device=dev)
        self.scale = torch.ones(1, dtype=torch.float32, device=dev)
        self.scale_inv = torch.ones(1, dtype=torch.float32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.amax = torch.full((1,), -7.0, dtype=torch.float32, device=dev)
        self.sat = torch.full((1,), 99, dtype=torch.int64, device=dev)
        self.used = torch.full((1,), -3.0, dtype=torch.float32, device=dev)

    def snapshot(self):
        return [t.detach().cpu().numpy().copy() for t in
                (self.history, self.head, self.scale, self.scale_inv, self.status, self.amax, self.sat, self.used)]


def run_pair(x, fmt, with_q, with_qt, a, b, dev):
    n = x.numel()
    rows, cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, n)
    outs = []
    for st, noalloc in ((a, False), (b, True)):
        q = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device=dev) if with_q else None
        qt = torch.full((cols, rows), 0x5A, dtype=torch.uint8, device=dev) if with_qt else None
        if noalloc:
            fm.fp8_quantize_update_noalloc(x, fmt, st.history, st.head, st.scale, st.scale_inv, st.amax, q=q,
                                           q_t=qt, sat=st.sat, status=st.status, scale_inv_used=st.used)
        else:
            ws = torch.empty(fm.QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
            fm.fp8_quantize_update(x, fmt, st.history, st.head, st.scale, st.scale_inv, st.amax, q=q, q_t=qt,
                                   sat=st.sat, status=st.status, workspace=ws, scale_inv_used=st.used)
        torch.cuda.synchronize()
        outs.append((None if q is None else q.cpu().numpy(), None if qt is None else qt.cpu().numpy()))
    for i in range(2):
        if outs[0][i] is None:
            assert outs[1][i] is None
        else:
            assert np.array_equal(outs[0][i], outs[1][i])
    for u, v in zip(a.snapshot(), b.snapshot()):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_noalloc_matches_workspace_entry_point_over_shrinking_calls(fmt):
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(123)
    a, b = State(fmt, 16, dev), State(fmt, 16, dev)
    cases = [
        # (shape, dtype, q, q_t, sigma): the first fills the most scratch slots
        ((4096, 8192), torch.bfloat16, True, True, 3.0),     # cast-transpose grid (up to 8 groups per CU)
        ((2048, 4096), torch.float32, True, False, 0.02),   # flat cast, fewer groups
        ((48, 160), torch.bfloat16, False, True, 50.0),     # a handful of tiles, mostly saturating
        ((3, 1000), torch.float32, True, False, 1.0),       # one workgroup
        ((0, 64), torch.float32, True, False, 1.0),         # empty: amax 0 pushed into the ring
        ((1000, 4096), torch.bfloat16, True, False, 1e-3),  # larger again after the empty one
        ((64, 4096), torch.float32, True, True, 1e4),       # an Inf: the scale is held, status set
    ]
    for shape, dtype, with_q, with_qt, sigma in cases:
        announce(f"noalloc {fmt} {shape} {dtype} q={with_q} q_t={with_qt}")
        x = (torch.randn(shape, generator=g) * sigma).to(dtype).to(dev)
        if sigma == 1e4:
            x.view(-1)[7] = float("inf")
        run_pair(x, fmt, with_q, with_qt, a, b, dev)
    assert a.head.item() == len(cases) % 16
    assert a.status.item() & 1                    # the Inf amax held the scale


def test_noalloc_argument_errors_match():
    """Host-side validation is that of fp8_quantize_update (nothing launched)."""
    lib = fm.load_library()
    import ctypes
    A16 = ctypes.c_void_p(0x10000)
    u = lib.fp8_quantize_update_noalloc
    #        x   xt rows cols fmt q    qt    amax sat  hist len head scale sinv status used stream
    assert u(A16, 7, 4, 16, 0, A16, None, A16, None, A16, 16, A16, A16, A16, None, None, None) == -5
    assert u(A16, 0, 4, 16, 9, A16, None, A16, None, A16, 16, A16, A16, A16, None, None, None) == -4
    assert u(A16, 0, 4, 16, 0, A16, None, A16, None, A16, 0, A16, A16, A16, None, None, None) == -2
    assert u(A16, 0, 4, 16, 0, A16, None, None, None, A16, 16, A16, A16, A16, None, None, None) == -1
    assert u(A16, 0, 4, 24, 0, None, A16, A16, None, A16, 16, A16, A16, A16, None, None, None) == -3
