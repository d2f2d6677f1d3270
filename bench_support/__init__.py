"""Read-bandwidth reference probes used by bench.py (not part of the C128 library)."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stream_probe.hip")
LIB = os.path.join(HERE, "libstream_probe.so")


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        from paged_kv_cache_fp32_amd.build import HIPCC_FLAGS, hipcc
        tmp = LIB + ".tmp"
        subprocess.check_call([hipcc(), *HIPCC_FLAGS, SRC, "-o", tmp])
        os.replace(tmp, LIB)
    return LIB


class IdxProbe(ctypes.Structure):
    """The probe_indexer_window_read / probe_c4_window_read arguments (struct IdxProbe in
    stream_probe.hip)."""
    _fields_ = [("pool", ctypes.c_void_p), ("s0", ctypes.c_int64), ("s1", ctypes.c_int64),
                ("positions", ctypes.c_void_p), ("slot", ctypes.c_void_p),
                ("req", ctypes.c_void_p), ("bt", ctypes.c_void_p), ("bt_stride", ctypes.c_int64),
                ("bt_rows", ctypes.c_int32), ("bt_cols", ctypes.c_int32),
                ("n_blocks", ctypes.c_int32), ("offs", ctypes.c_void_p),
                ("cs", ctypes.c_void_p), ("cs_stride", ctypes.c_int64),
                ("cs_rows", ctypes.c_int32), ("T", ctypes.c_int32), ("kpw", ctypes.c_int32),
                ("nb_mask", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.probe_stream_read.argtypes = [vp, i64, vp, ci, ci, ci, vp]
        L.probe_stream_read.restype = ci
        L.probe_stream_chunks.argtypes = [vp, i64, vp, ci, ci, ci, ci, vp]
        L.probe_stream_chunks.restype = ci
        L.probe_window_read_split.argtypes = [vp, i64, vp, ci, ci, ci, ci, vp, vp]
        L.probe_window_read_split.restype = ci
        L.probe_window_read_persistent.argtypes = [vp, i64, vp, ci, ci, ci, ci, vp, vp]
        L.probe_window_read_persistent.restype = ci
        L.probe_block_gather_read.argtypes = [vp, i64, vp, ci, vp, ci, vp]
        L.probe_block_gather_read.restype = ci
        L.probe_indexer_window_read.argtypes = [ctypes.POINTER(IdxProbe), ci, vp, vp]
        L.probe_indexer_window_read.restype = ci
        L.probe_c4_window_read.argtypes = [ctypes.POINTER(IdxProbe), ci, vp, vp]
        L.probe_c4_window_read.restype = ci
        _lib = L
    return _lib
