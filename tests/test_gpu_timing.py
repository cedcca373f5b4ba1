"""The measurement hook pkv_time_next_kernel: the next kernel launched
through the library records the caller's events at its own dispatch start
and end, and each setting is consumed by one launch."""

import ctypes

import pytest
import torch

from paged_kv_cache_39_amd import binding
from paged_kv_cache_39_amd import workloads as wl
from tests.gpu_util import DeviceCase

pytestmark = pytest.mark.gpu


def _hip():
    torch.cuda.init()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("HIP runtime not loaded")


def _event(hip):
    e = ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(e)) == 0
    return e.value


def _elapsed_ms(hip, a, b):
    out = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
    return out.value


def test_kernel_events_bracket_the_armed_kernel():
    print("timing hook: decode on the LLaMA-7B-shaped batch", flush=True)
    hip = _hip()
    dc = DeviceCase(wl.workload(2, values=True))
    dc.decode()
    torch.cuda.synchronize()
    evs = [_event(hip) for _ in range(10)]
    # the first armed launch of a process carries one-time set-up: not timed
    binding.time_next_kernel(evs[8], evs[9])
    dc.decode()
    # one kernel between each pair (a, b); the median of three is "one"
    for i in range(3):
        binding.time_next_kernel(evs[2 * i], evs[2 * i + 1])
        dc.decode()
    c, d = evs[6], evs[7]
    # start of the first of two calls, end of the second: each call consumes
    # its own setting
    binding.time_next_kernel(c, None)
    dc.decode()
    binding.time_next_kernel(None, d)
    dc.decode()
    torch.cuda.synchronize()
    ones = sorted(_elapsed_ms(hip, evs[2 * i], evs[2 * i + 1]) for i in range(3))
    one = ones[1]
    two = _elapsed_ms(hip, c, d)
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    print(f"one kernel {[round(x * 1e3, 1) for x in ones]} us, two calls {two * 1e3:.1f} us",
          flush=True)
    assert 5e-3 < one < 5.0
    assert two > 1.5 * one
