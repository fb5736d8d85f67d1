"""Stage timing and cache eviction for measurements (no part of the forward).

StageEvents holds hipEvent_t handles for the profiled entry points
(kda_fwd_profiled, kda_bwd_profiled), which record them around each stage on
the stream the kernels run on.  evict_caches() writes a scratch buffer larger
than the MI355X's last-level cache (256 MB of memory-side cache plus the
XCDs' L2) so that the next timed call reads its inputs from HBM.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import kda

EVICT_BYTES = 1 << 30   # 1 GiB: four times the 256 MB last-level cache


def hip_runtime():
    """The HIP runtime torch already loaded (same soname as libkda.so's)."""
    try:
        return ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
    except OSError:
        return ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))


class StageEvents:
    """2*nstages hipEvents per step, read back after the timed region."""

    def __init__(self, steps, nstages=None):
        self.nstages = kda.NUM_STAGES if nstages is None else nstages
        self.hip = hip_runtime()
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        n = 2 * self.nstages
        self.arrays = []
        for _ in range(steps):
            arr = (ctypes.c_void_p * n)()
            for i in range(n):
                ev = ctypes.c_void_p()
                rc = self.hip.hipEventCreate(ctypes.byref(ev))
                if rc != 0:
                    raise RuntimeError("hipEventCreate failed (%d)" % rc)
                arr[i] = ev.value
            self.arrays.append(arr)

    def _elapsed(self, a, b):
        ms = ctypes.c_float(0.0)
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def per_step_stage_ms(self):
        """[steps, nstages] durations (ms) of each stage of each step."""
        return np.array([[self._elapsed(arr[2 * s], arr[2 * s + 1]) for s in range(self.nstages)]
                         for arr in self.arrays])

    def per_step_ms(self):
        """Duration (ms) of each step, first stage start to last stage end."""
        return np.array([self._elapsed(arr[0], arr[2 * self.nstages - 1]) for arr in self.arrays])

    def stage_ms(self):
        """Average duration (ms) of each stage over the recorded steps."""
        return self.per_step_stage_ms().mean(axis=0)

    def close(self):
        for arr in self.arrays:
            for ev in arr:
                self.hip.hipEventDestroy(ev)


_scratch = {}


def evict_caches(device=None):
    """Overwrite EVICT_BYTES of device memory (on the current stream)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    buf = _scratch.get(dev)
    if buf is None:
        buf = _scratch[dev] = torch.empty(EVICT_BYTES // 4, dtype=torch.float32, device=dev)
    buf.fill_(1.0)
