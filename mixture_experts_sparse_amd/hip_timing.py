"""HIP events for per-stage timing of moe_layer_forward_traced.

The event functions are looked up through libmoe.so's handle, i.e. in the
HIP runtime the library (and torch) are bound to, so no second runtime is
loaded. Events are recorded by the library on the stream it launches on.
"""

from __future__ import annotations

import ctypes

from . import binding as B


def _hip():
    L = B.lib()
    for name, args in (("hipEventCreate", [ctypes.POINTER(ctypes.c_void_p)]),
                       ("hipEventDestroy", [ctypes.c_void_p]),
                       ("hipEventSynchronize", [ctypes.c_void_p]),
                       ("hipEventRecord", [ctypes.c_void_p, ctypes.c_void_p]),
                       ("hipEventElapsedTime", [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p])):
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    return L


class StageEvents:
    """steps x (MOE_NUM_STAGES + 1) events; row i is passed to the traced
    layer call of step i."""

    def __init__(self, steps: int, stages: int = None):
        self.hip = _hip()
        self.n = (B.MOE_NUM_STAGES if stages is None else stages) + 1
        self.rows = []
        for _ in range(steps):
            arr = (ctypes.c_void_p * self.n)()
            for j in range(self.n):
                ev = ctypes.c_void_p()
                st = self.hip.hipEventCreate(ctypes.byref(ev))
                if st != 0:
                    raise RuntimeError(f"hipEventCreate failed ({st})")
                arr[j] = ev.value
            self.rows.append(arr)

    def row(self, i: int):
        return self.rows[i]

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def stage_ms(self):
        """Per-stage durations [steps][stages] in ms."""
        self.hip.hipEventSynchronize(self.rows[-1][self.n - 1])
        return [[self.elapsed_ms(r[s], r[s + 1]) for s in range(self.n - 1)] for r in self.rows]

    def span_ms(self):
        """First event of the first step to the last event of the last step."""
        self.hip.hipEventSynchronize(self.rows[-1][self.n - 1])
        return self.elapsed_ms(self.rows[0][0], self.rows[-1][self.n - 1])

    def destroy(self):
        for r in self.rows:
            for j in range(self.n):
                self.hip.hipEventDestroy(r[j])
        self.rows = []
