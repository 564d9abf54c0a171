"""libmhc_mover.so (the access-pattern ceilings bench.py reports): it loads,
exports mhc_mover_run, and refuses arguments outside its shapes before it
touches memory or the device."""
import ctypes
import os

import pytest

from mhc_hyper_connection_boundary_amd import build


@pytest.fixture(scope="module")
def mover():
    if not os.path.exists(build.MOVER_LIB):
        pytest.skip("libmhc_mover.so not built (run __graft_entry__.build())")
    L = ctypes.CDLL(build.MOVER_LIB)
    L.mhc_mover_run.restype = ctypes.c_int
    L.mhc_mover_run.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    return L


@pytest.mark.parametrize("tokens,hidden,mode", [
    (0, 7168, 0), (100, 7168, 0), (64, 100, 0), (64, 7168, 4), (64, 7168, -1),
    (64, 256, 3), (64, 7168 + 256, 3), (64, 32768, 0),
])
def test_mover_refuses_bad_shapes(mover, tokens, hidden, mode):
    p = ctypes.c_void_p(256)  # never dereferenced: the checks come first
    assert mover.mhc_mover_run(tokens, hidden, p, p, p, p, mode, None) == 1


def test_mover_refuses_null_pointers(mover):
    p = ctypes.c_void_p(256)
    assert mover.mhc_mover_run(64, 7168, None, p, p, p, 0, None) == 1
