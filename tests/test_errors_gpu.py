"""Error state of the HIP runtime around the library's calls: a call reports
the status of its own launches and leaves an error the caller left pending
(here from hipSetDevice with an invalid device index, a harmless argument
error) for the caller to read."""
import ctypes

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _hip_runtime():
    """The HIP runtime library that torch (and the library) loaded."""
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    assert paths, "HIP runtime not loaded"
    rt = ctypes.CDLL(sorted(paths)[0])
    rt.hipGetLastError.restype = ctypes.c_int
    rt.hipSetDevice.restype = ctypes.c_int
    rt.hipSetDevice.argtypes = [ctypes.c_int]
    return rt


def test_pending_caller_error_is_left_pending(itk):
    case = synth.gen_ragged(4, 4096, 64, seed=1)
    x = torch.from_numpy(case.scores).cuda()
    rl = torch.from_numpy(case.row_len).cuda()
    out = torch.empty((4, 64), dtype=torch.int32, device="cuda")
    ws = torch.empty(itk.topk_ragged_workspace_size(4, 4096, 64), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    rt = _hip_runtime()
    assert rt.hipGetLastError() == 0
    bad = rt.hipSetDevice(12345)
    assert bad != 0
    st = itk.lib().topk_ragged(ctypes.c_void_p(x.data_ptr()), 4096, ctypes.c_void_p(rl.data_ptr()), 4, 64,
                               ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    assert rt.hipGetLastError() == bad  # still pending for the caller
    assert rt.hipGetLastError() == 0
    torch.cuda.synchronize()
