"""CPU oracle of the compress-store paths: the sparse-attention compressors C128 and C4 and the
indexer's compressor with its FP8 and MXFP4 caches (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never links or calls
it; the two share no code.  See ``c128_oracle.c`` for what it computes and
which passages of the DeepSeek-V4 compressor pages each step follows.

Parity pins (tests/test_oracle_pins.py) tie every step to something other
than the oracle itself: library routines, closed forms, invariants and
brute force.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "c128_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

HEAD = 512
INDEXER_HEAD = 128
NOPE = 448
ROPE = 64
RECORD = 576
SCALE_DIM = 8

STATUS_INACTIVE, STATUS_WRITTEN, STATUS_NO_SLOT, STATUS_BAD_INDEX = 0, 1, 2, -1
FMT_SPARSE, FMT_INDEXER_FP8, FMT_INDEXER_MXFP4 = 0, 1, 2   # cache formats


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (host code, fp64, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fno-fast-math", "-ffp-contract=off",
             "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The loaded oracle library.  ``DSV4_ORACLE_LIB`` names another build of the same source
    (the mutation tests load deliberately broken copies through it)."""
    global _lib
    if _lib is None:
        path = os.environ.get("DSV4_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(path)
        i64, vp, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_c128_compress_store.argtypes = [
            vp, i64, i64, i64, i64,          # state, n blocks, state bs, s0, s1
            vp, i64, i64, i64,               # block table, rows, cols, stride
            vp, vp, vp, i64,                 # token_to_req, positions, slot_mapping, T
            vp, dbl, vp, i64, i64,           # rms_w, eps, cos_sin, rows, stride
            vp, i64, i64, i64, vp,           # k_cache, kv bs, stride0 (bytes), blocks, kv slots
            vp, vp, vp, vp,                  # diagnostics
            i64, i64, ctypes.c_int]          # token range, threads
        L.oracle_c128_compress_store.restype = ctypes.c_int
        L.oracle_compress_store.argtypes = [i64, i64, i64] + L.oracle_c128_compress_store.argtypes
        L.oracle_compress_store.restype = ctypes.c_int
        L.oracle_compress_store_fmt.argtypes = [i64, ctypes.c_int, i64, i64, i64] + \
            L.oracle_c128_compress_store.argtypes
        L.oracle_compress_store_fmt.restype = ctypes.c_int
        L.oracle_bf16_bits.argtypes = [dbl]
        L.oracle_bf16_bits.restype = ctypes.c_uint16
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = dbl
        L.oracle_e4m3_code.argtypes = [dbl]
        L.oracle_e4m3_code.restype = ctypes.c_uint8
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = dbl
        L.oracle_ceil_log2.argtypes = [dbl]
        L.oracle_ceil_log2.restype = ctypes.c_int
        L.oracle_ue8m0_exponent.argtypes = [dbl]
        L.oracle_ue8m0_exponent.restype = ctypes.c_int
        L.oracle_e2m1_code.argtypes = [dbl]
        L.oracle_e2m1_code.restype = ctypes.c_uint8
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_value.restype = dbl
        L.oracle_mxfp4_exponent.argtypes = [dbl]
        L.oracle_mxfp4_exponent.restype = ctypes.c_int
        for name in ("oracle_bf16_bits_array", "oracle_e4m3_code_array",
                     "oracle_ue8m0_exponent_array", "oracle_e2m1_code_array",
                     "oracle_mxfp4_exponent_array"):
            getattr(L, name).argtypes = [vp, vp, i64]
            getattr(L, name).restype = None
        _lib = L
    return _lib


def bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_bits_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def e4m3_codes(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_code_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def ue8m0_exponents(absmax) -> np.ndarray:
    x = np.ascontiguousarray(absmax, dtype=np.float64)
    out = np.empty(x.shape, np.int32)
    lib().oracle_ue8m0_exponent_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def e2m1_codes(x) -> np.ndarray:
    """E2M1 codes (low nibble; 0x8 = sign) of the values ``x``."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e2m1_code_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def mxfp4_exponents(absmax) -> np.ndarray:
    x = np.ascontiguousarray(absmax, dtype=np.float64)
    out = np.empty(x.shape, np.int32)
    lib().oracle_mxfp4_exponent_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


class OracleResult:
    """k_cache after the oracle ran, plus per-token fp64 diagnostics."""

    def __init__(self, k_cache_base, k_cache, compressed, absnorm, normed, status):
        self.k_cache_base = k_cache_base
        self.k_cache = k_cache
        self.compressed = compressed
        self.absnorm = absnorm
        self.normed = normed
        self.status = status


def run(wl, nthreads: int = 1, tokens=None, diagnostics: bool = True,
        state_block_size: int | None = None) -> OracleResult:
    """Run the oracle on a ``synth.Workload`` (host arrays).

    ``tokens``: ``(lo, hi)`` range, default all.  The workload's k_cache is
    copied first, so the workload stays untouched.  Diagnostics rows of
    tokens outside the range or that fail the gate are NaN.  Compress ratio
    and overlap come from the workload (C128 when absent); an indexer workload
    (``wl.indexer``) has head 128 and the indexer's FP8 cache format, or its MXFP4
    format when ``wl.indexer_fp4`` is set, and its ``normed`` rows hold the
    rotated values that were quantised (before their bf16 round trip).
    """
    T = wl.num_tokens
    lo, hi = (0, T) if tokens is None else tokens
    state = wl.state
    s0, s1, s2 = (s // 4 for s in state.strides)
    assert s2 == 1 and state.dtype == np.float32
    sbs = state.shape[1] if state_block_size is None else state_block_size
    bt = wl.block_table
    assert bt.dtype == np.int32 and bt.strides[1] == 4
    kc_src = wl.k_cache
    assert kc_src.dtype == np.uint8
    stride0 = kc_src.strides[0]
    n_kv_blocks, kv_bs = kc_src.shape[0], kc_src.shape[1]
    if wl.k_cache_base is not None:
        kc_base = wl.k_cache_base.copy()
        assert kc_src.ctypes.data == wl.k_cache_base.ctypes.data
        kc = np.lib.stride_tricks.as_strided(kc_base, shape=kc_src.shape, strides=kc_src.strides)
    else:
        kc = np.ascontiguousarray(kc_src).copy()
        kc_base = kc.reshape(-1)
        stride0 = kc.strides[0]
    cs = wl.cos_sin
    assert cs.dtype == np.float32 and cs.strides[1] == 4
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in
            (wl.token_to_req, wl.positions, wl.slot_mapping, wl.kv_slot_mapping)]
    rms_w = np.ascontiguousarray(wl.rms_w, dtype=np.float32)
    indexer = bool(getattr(wl, "indexer", False))
    head = INDEXER_HEAD if indexer else HEAD
    fmt = (FMT_INDEXER_MXFP4 if getattr(wl, "indexer_fp4", False) else FMT_INDEXER_FP8) \
        if indexer else FMT_SPARSE
    comp = absn = normd = None
    if diagnostics:
        comp = np.full((T, head), np.nan)
        absn = np.full((T, head), np.nan)
        normd = np.full((T, head), np.nan)
    status = np.full(T, -99, np.int32)
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    cr = int(getattr(wl, "compress_ratio", 128))
    overlap = int(getattr(wl, "overlap", 0))
    rc = lib().oracle_compress_store_fmt(
        head, fmt, cr, overlap, (1 + overlap) * head, state.ctypes.data, state.shape[0], sbs, s0, s1,
        bt.ctypes.data, bt.shape[0], bt.shape[1], bt.strides[0] // 4,
        arrs[0].ctypes.data, arrs[1].ctypes.data, arrs[2].ctypes.data, T,
        rms_w.ctypes.data, float(wl.eps), cs.ctypes.data, cs.shape[0], cs.strides[0] // 4,
        kc.ctypes.data, kv_bs, stride0, n_kv_blocks, arrs[3].ctypes.data,
        ptr(comp), ptr(absn), ptr(normd), status.ctypes.data, lo, hi, nthreads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return OracleResult(kc_base, kc, comp, absn, normd, status)
