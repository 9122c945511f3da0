"""The measurement-only probe library: it loads, exports its entry point, and
rejects bad arguments before touching the device.  It is not part of the
forward path's library."""
import ctypes

import pytest

UNSUP, SHAPE, NULL, WS = 4, 2, 1, 6


@pytest.fixture(scope="module")
def P():
    import measure
    return measure.lib()


def test_probe_validation(P):
    flop = ctypes.c_double(0.0)
    sink = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails validation first
    assert P.dsa_probe_mfma(2, 1, 10, 0, sink, 1 << 16, None, 0, ctypes.byref(flop), None) == UNSUP
    assert P.dsa_probe_mfma(0, 3, 10, 0, sink, 1 << 16, None, 0, ctypes.byref(flop), None) == UNSUP
    assert P.dsa_probe_mfma(1, 1, 0, 1, sink, 1 << 16, None, 0, ctypes.byref(flop), None) == SHAPE
    assert P.dsa_probe_mfma(1, 1, 10, 0, sink, 1 << 16, None, 0, None, None) == NULL
    assert P.dsa_probe_mfma(1, 1, 10, 0, None, 1 << 16, None, 0, ctypes.byref(flop), None) == NULL
    assert b"dsa_probe_mfma" in P.dsa_probe_last_error()
