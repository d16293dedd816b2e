"""Binding of libneox_stream_probe.so (include/neox_stream_probe.h): attainable-bandwidth
probes used by the benchmark to put the step's throughput next to a measured ceiling."""
import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libneox_stream_probe.so")
EXPORTS = ("neox_probe_copy", "neox_probe_update_pattern", "neox_probe_last_error")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build the package first")
        L = C.CDLL(LIB_PATH)
        L.neox_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_void_p]
        L.neox_probe_copy.restype = C.c_int
        L.neox_probe_update_pattern.argtypes = [C.c_void_p] * 5 + [C.c_uint64, C.c_int32, C.c_int32,
                                                                   C.c_int32, C.c_int32, C.c_void_p]
        L.neox_probe_update_pattern.restype = C.c_int
        L.neox_probe_last_error.argtypes = []
        L.neox_probe_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise RuntimeError(f"stream probe error {rc}: {lib().neox_probe_last_error().decode()}")


def neox_probe_copy(src_ptr, dst_ptr, nbytes, nt_stores=0, stream_ptr=0):
    _check(lib().neox_probe_copy(src_ptr, dst_ptr, nbytes, int(nt_stores), stream_ptr))


def neox_probe_update_pattern(grad, half, master, exp_avg, exp_avg_sq, n, threads=256, vectors=2,
                              blocks_per_cu=0, nt_stores=0, stream_ptr=0):
    _check(lib().neox_probe_update_pattern(grad, half, master, exp_avg, exp_avg_sq, n, threads,
                                           vectors, blocks_per_cu, int(nt_stores), stream_ptr))
