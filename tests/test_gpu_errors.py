"""Error reporting of the C ABI on the GPU ([P1] s4: a missed fusion or a refused call may cost
time, never correctness): a HIP error the caller left pending is not reported as the library's
(the library takes each launch's status from hipLaunchKernel and never reads the thread's
pending error), and the call's results are correct."""
import ctypes

import numpy as np
import pytest

import synth
from _gpu import check_row_exact, ensure_built, poisoned, up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
ensure_built()
from int8_quantized_projections_amd import q8lib  # noqa: E402


def test_pending_hip_error_is_the_callers():
    L = q8lib.lib()
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already loaded by torch and the library
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipGetLastError.restype = ctypes.c_int
    x = synth.normal((3, 256), stream=9900)
    xd = up(x)
    nq, ns = q8lib.act_bytes(3, 256, q8lib.LAYOUT_ROW)
    qs, sd = poisoned(nq, torch.int8), poisoned(ns // 4, torch.int32)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    assert hip.hipGetLastError() == 0
    stale = hip.hipSetDevice(1 << 20)  # no such device: the call fails and leaves its error pending
    assert stale != 0
    rc = L.q8_quantize(xd.data_ptr(), 3, 256, q8lib.LAYOUT_ROW, qs.data_ptr(), sd.data_ptr(), stream)
    assert rc == 0, f"the library reported the caller's pending error as its own ({rc})"
    # whether the runtime still holds the caller's error after the library's successful launch
    # is the runtime's rule, not the library's; reported for the record
    print(f"pending error {stale} -> after the call: {hip.hipGetLastError()}")
    torch.cuda.synchronize()
    check_row_exact(qs, sd, x, "q8_quantize after a pending error")
    assert np.all(np.isfinite(x))
