"""MI355X (gfx950) compress-store for the DeepSeek-V4 compressors: C128 (single pass, staged
schedule from 2048 tokens, small-batch fan-out, compacted varlen schedule), C4 and the
indexer's compressor with its FP8 and MXFP4 caches.

Thin ctypes binding of ``libdsv4_c128.so`` (C ABI in ``include/dsv4_c128.h``).
The binding only marshals torch tensors into descriptors and passes torch's
current HIP stream; every step of the computation runs in the HIP kernels.
Loading fails loudly when the library is missing -- there is no fallback.

    import paged_kv_cache_fp32_amd as c128
    c128.compress_store(state_cache, block_table, token_to_req, positions,
                        slot_mapping, rms_w, eps, cos_sin, k_cache, kv_slot_mapping)
    c128.compress_store_varlen(...)       # long prefill batches
    c128.c4_compress_store(...)           # ratio 4, overlapping window
    c128.indexer_compress_store(...)      # head 128, fp8 + fp32 scale
"""

from __future__ import annotations

import ctypes
import os
import struct

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libdsv4_c128.so")

DSV4_F32, DSV4_I32, DSV4_U8 = 1, 2, 3
DSV4_OK = 0
ERRORS = {
    -1: "DSV4_ERR_NULL",
    -2: "DSV4_ERR_DTYPE",
    -3: "DSV4_ERR_RANK",
    -4: "DSV4_ERR_SHAPE",
    -5: "DSV4_ERR_STRIDE",
    -6: "DSV4_ERR_ALIGN",
    -7: "DSV4_ERR_LAUNCH",
    -8: "DSV4_ERR_ARG",
}
_DTYPES = {torch.float32: DSV4_F32, torch.int32: DSV4_I32, torch.uint8: DSV4_U8}


class Dsv4Error(RuntimeError):
    """A call into the library returned a negative status."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


class Tensor(ctypes.Structure):
    """dsv4_tensor: pointer, dtype code, rank, shape and strides in elements."""

    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


# dsv4_tensor of rank nd, field by field: pointer, dtype, rank, the nd shape entries, zeros to
# 4, the nd strides, zeros to 4 (80 bytes, no padding between fields).
_DESC = [struct.Struct(f"<Qii{nd}q{8 * (4 - nd)}x{nd}q{8 * (4 - nd)}x") for nd in range(5)]
_DESC_BYTES = _DESC[0].size


def _pack(t: torch.Tensor) -> bytes:
    shape = t.shape
    nd = len(shape)
    if nd > 4:
        raise ValueError("at most 4 dimensions")
    return _DESC[nd].pack(0 if 0 in shape else t.data_ptr(), _DTYPES.get(t.dtype, 0), nd, *shape,
                          *t.stride())


def describe(t: torch.Tensor) -> Tensor:
    """Descriptor of a torch tensor (any device; the library never reads host data)."""
    return Tensor.from_buffer_copy(_pack(t))


_lib = None


def library():
    """The loaded ``libdsv4_c128.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY_PATH):
            raise ImportError(
                f"{LIBRARY_PATH} is missing: build it with "
                "`python -m paged_kv_cache_fp32_amd.build` (there is no fallback path)")
        lib = ctypes.CDLL(LIBRARY_PATH)
        P = ctypes.c_void_p  # const dsv4_tensor*
        args10 = [P, P, P, P, P, P, ctypes.c_float, P, P, P]
        lib.dsv4_c128_compress_store.argtypes = args10 + [ctypes.c_void_p]
        lib.dsv4_c128_compress_store.restype = ctypes.c_int
        lib.dsv4_c128_compress_store_debug.argtypes = args10 + [ctypes.c_void_p, ctypes.c_void_p]
        lib.dsv4_c128_compress_store_debug.restype = ctypes.c_int
        lib.dsv4_c128_compress_store_ex.argtypes = args10 + [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
        lib.dsv4_c128_compress_store_ex.restype = ctypes.c_int
        lib.dsv4_c128_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int]
        lib.dsv4_c128_workspace_bytes.restype = ctypes.c_size_t
        lib.dsv4_c128_compress_store_varlen.argtypes = args10 + [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.dsv4_c128_compress_store_varlen.restype = ctypes.c_int
        lib.dsv4_c128_compress_store_varlen_noalloc.argtypes = args10 + [ctypes.c_void_p,
                                                                        ctypes.c_void_p]
        lib.dsv4_c128_compress_store_varlen_noalloc.restype = ctypes.c_int
        lib.dsv4_c128_varlen_workspace_bytes.argtypes = [ctypes.c_int64]
        lib.dsv4_c128_varlen_workspace_bytes.restype = ctypes.c_size_t
        lib.dsv4_c4_compress_store.argtypes = args10 + [ctypes.c_void_p]
        lib.dsv4_c4_compress_store.restype = ctypes.c_int
        lib.dsv4_c4_compress_store_debug.argtypes = args10 + [ctypes.c_void_p, ctypes.c_void_p]
        lib.dsv4_c4_compress_store_debug.restype = ctypes.c_int
        lib.dsv4_indexer_compress_store.argtypes = args10 + [ctypes.c_void_p]
        lib.dsv4_indexer_compress_store.restype = ctypes.c_int
        lib.dsv4_indexer_compress_store_debug.argtypes = args10 + [ctypes.c_void_p,
                                                                  ctypes.c_void_p]
        lib.dsv4_indexer_compress_store_debug.restype = ctypes.c_int
        lib.dsv4_indexer_validate.argtypes = args10
        lib.dsv4_indexer_validate.restype = ctypes.c_int
        lib.dsv4_indexer_mxfp4_compress_store.argtypes = args10 + [ctypes.c_void_p]
        lib.dsv4_indexer_mxfp4_compress_store.restype = ctypes.c_int
        lib.dsv4_indexer_mxfp4_compress_store_debug.argtypes = args10 + [ctypes.c_void_p,
                                                                        ctypes.c_void_p]
        lib.dsv4_indexer_mxfp4_compress_store_debug.restype = ctypes.c_int
        lib.dsv4_indexer_mxfp4_validate.argtypes = args10
        lib.dsv4_indexer_mxfp4_validate.restype = ctypes.c_int
        lib.dsv4_e2m1_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p]
        lib.dsv4_e2m1_encode.restype = ctypes.c_int
        lib.dsv4_c4_validate.argtypes = args10
        lib.dsv4_c4_validate.restype = ctypes.c_int
        lib.dsv4_c128_validate.argtypes = args10
        lib.dsv4_c128_validate.restype = ctypes.c_int
        lib.dsv4_e4m3_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p]
        lib.dsv4_e4m3_encode.restype = ctypes.c_int
        lib.dsv4_last_error.argtypes = []
        lib.dsv4_last_error.restype = ctypes.c_char_p
        lib.dsv4_abi_version.argtypes = []
        lib.dsv4_abi_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def last_error() -> str:
    return library().dsv4_last_error().decode()


def abi_version() -> int:
    return library().dsv4_abi_version()


def _check(rc: int):
    if rc != DSV4_OK:
        raise Dsv4Error(rc, last_error())


def _descriptors(tensors):
    """The descriptors of ``tensors`` packed in one buffer, and their addresses: one struct
    packing per tensor instead of a ctypes field write per shape and stride entry (about 40%
    less host time per call).  The caller keeps the buffer alive through the call."""
    buf = ctypes.create_string_buffer(b"".join([_pack(t) for t in tensors]))
    base = ctypes.addressof(buf)
    return buf, [base + _DESC_BYTES * i for i in range(len(tensors))]


def _require_cuda(tensors):
    dev = None
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("compress_store needs device tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


# torch's raw accessor of the current stream skips building a Stream object (about 2 us of host
# time per call); the public call serves where it is absent.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    if _raw_current_stream is not None and device.index is not None:
        return _raw_current_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def compress_store(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                   cos_sin, k_cache, kv_slot_mapping, stream: int | None = None) -> None:
    """Fused C128 compress -> RMSNorm -> FP8/UE8M0 quant -> RoPE -> paged insert (in place
    on ``k_cache``), enqueued on ``stream`` (default: torch's current stream).  One kernel
    launch: a workgroup per token below 2048 tokens; from 2048 on, the staged schedule (a
    workgroup per CU, each taking an equal share of the tokens that close a window)."""
    ts = (state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping)
    dev = _require_cuda(ts)
    keep, refs = _descriptors(ts)
    s = _stream(dev) if stream is None else stream
    _check(library().dsv4_c128_compress_store(*refs[:6], float(eps), *refs[6:], s))


def compress_store_debug(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                         eps, cos_sin, k_cache, kv_slot_mapping, compressed_out,
                         stream: int | None = None) -> None:
    """``compress_store`` that also writes the fp32 pooled vector of each token passing the
    gate into ``compressed_out`` ([T, 512] fp32, contiguous, on the device)."""
    ts = (state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping, compressed_out)
    dev = _require_cuda(ts)
    if compressed_out.dtype != torch.float32 or not compressed_out.is_contiguous() or \
            tuple(compressed_out.shape) != (positions.shape[0], 512):
        raise ValueError("compressed_out must be a contiguous float32 [T, 512] tensor")
    keep, refs = _descriptors(ts[:-1])
    s = _stream(dev) if stream is None else stream
    _check(library().dsv4_c128_compress_store_debug(*refs[:6], float(eps), *refs[6:],
                                                    compressed_out.data_ptr(), s))


def workspace_bytes(num_tokens: int, splits: int = 0) -> int:
    """Workspace bytes ``compress_store_ex`` needs for ``num_tokens`` tokens and ``splits``
    workgroups per token (0 = the library's choice); 0 when none is needed."""
    return int(library().dsv4_c128_workspace_bytes(int(num_tokens), int(splits)))


def fanout_workspace(num_tokens: int, splits: int = 0, device="cuda"):
    """A zero-filled workspace for ``compress_store_ex`` (``workspace_bytes(T, splits)`` bytes, at
    least 16).  Its arrival counters must start at zero; every call leaves them zero, so one
    workspace, allocated once, serves later calls with any T and split count that fit it."""
    return torch.zeros(max(workspace_bytes(num_tokens, splits), 16), dtype=torch.uint8,
                       device=device)


def compress_store_ex(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                      cos_sin, k_cache, kv_slot_mapping, compressed_out=None, workspace=None,
                      splits: int = 0, stream: int | None = None) -> None:
    """``compress_store`` with the small-batch fan-out: each token's window is split over
    ``splits`` workgroups (0 = automatic; 1 = single pass) whose partial states go to
    ``workspace`` and are merged by the last of them to finish.  ``workspace``: a device tensor
    of at least ``workspace_bytes(T, splits)`` bytes whose first 16384 bytes were zero-filled
    before its first use (``fanout_workspace`` makes one).  ``compressed_out`` as in
    ``compress_store_debug``."""
    ts = [state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping]
    extra = [t for t in (compressed_out, workspace) if t is not None]
    dev = _require_cuda(ts + extra)
    if compressed_out is not None and (
            compressed_out.dtype != torch.float32 or not compressed_out.is_contiguous() or
            tuple(compressed_out.shape) != (positions.shape[0], 512)):
        raise ValueError("compressed_out must be a contiguous float32 [T, 512] tensor")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    keep, refs = _descriptors(ts)
    s = _stream(dev) if stream is None else stream
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    out_ptr = compressed_out.data_ptr() if compressed_out is not None else None
    _check(library().dsv4_c128_compress_store_ex(*refs[:6], float(eps), *refs[6:], out_ptr,
                                                 ws_ptr, ws_len, int(splits), s))


def varlen_workspace_bytes(num_tokens: int) -> int:
    """Workspace bytes ``compress_store_varlen`` needs for ``num_tokens`` tokens."""
    return int(library().dsv4_c128_varlen_workspace_bytes(int(num_tokens)))


def compress_store_varlen(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                          eps, cos_sin, k_cache, kv_slot_mapping, compressed_out=None,
                          workspace=None, stream: int | None = None) -> None:
    """``compress_store`` on a compacted schedule for long varlen (prefill) batches: a gate scan
    lists the tokens that close a window, then a persistent grid processes only those.
    ``workspace``: a contiguous device tensor of at least ``varlen_workspace_bytes(T)`` bytes
    (allocated here when None).  ``compressed_out`` as in ``compress_store_debug``."""
    ts = [state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping]
    extra = [t for t in (compressed_out, workspace) if t is not None]
    dev = _require_cuda(ts + extra)
    if compressed_out is not None and (
            compressed_out.dtype != torch.float32 or not compressed_out.is_contiguous() or
            tuple(compressed_out.shape) != (positions.shape[0], 512)):
        raise ValueError("compressed_out must be a contiguous float32 [T, 512] tensor")
    s = _stream(dev) if stream is None else stream
    if workspace is None:
        # Allocated on the launch stream: torch's caching allocator then reuses this memory
        # only in that stream's order, after the two kernels that use it.
        nbytes = max(varlen_workspace_bytes(positions.shape[0]), 16)
        if stream is None or stream == _stream(dev):
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        else:
            with torch.cuda.stream(torch.cuda.ExternalStream(stream, device=dev)):
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    elif not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    keep, refs = _descriptors(ts)
    out_ptr = compressed_out.data_ptr() if compressed_out is not None else None
    _check(library().dsv4_c128_compress_store_varlen(
        *refs[:6], float(eps), *refs[6:], out_ptr, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), s))


VARLEN_NOALLOC_MAX_TOKENS = 1 << 20


def compress_store_varlen_noalloc(state_cache, block_table, token_to_req, positions,
                                  slot_mapping, rms_w, eps, cos_sin, k_cache, kv_slot_mapping,
                                  compressed_out=None, stream: int | None = None) -> None:
    """``compress_store_varlen`` with no workspace and no allocation: its scratch is a fixed
    array of the library on each device (at most ``VARLEN_NOALLOC_MAX_TOKENS`` tokens per call;
    calls that overlap on one device race).  ``compressed_out`` as in
    ``compress_store_debug``."""
    ts = [state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping]
    dev = _require_cuda(ts + ([compressed_out] if compressed_out is not None else []))
    if compressed_out is not None and (
            compressed_out.dtype != torch.float32 or not compressed_out.is_contiguous() or
            tuple(compressed_out.shape) != (positions.shape[0], 512)):
        raise ValueError("compressed_out must be a contiguous float32 [T, 512] tensor")
    keep, refs = _descriptors(ts)
    s = _stream(dev) if stream is None else stream
    out_ptr = compressed_out.data_ptr() if compressed_out is not None else None
    _check(library().dsv4_c128_compress_store_varlen_noalloc(*refs[:6], float(eps), *refs[6:],
                                                             out_ptr, s))


def c4_compress_store(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                      eps, cos_sin, k_cache, kv_slot_mapping, compressed_out=None,
                      stream: int | None = None) -> None:
    """The C4 compressor (ratio 4, overlapping 8-row window; state rows kv 2x512 | score 2x512,
    any state block size) into the same k_cache layout; ``compressed_out`` as in
    ``compress_store_debug`` (optional)."""
    ts = [state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping]
    dev = _require_cuda(ts + ([compressed_out] if compressed_out is not None else []))
    if compressed_out is not None and (
            compressed_out.dtype != torch.float32 or not compressed_out.is_contiguous() or
            tuple(compressed_out.shape) != (positions.shape[0], 512)):
        raise ValueError("compressed_out must be a contiguous float32 [T, 512] tensor")
    keep, refs = _descriptors(ts)
    s = _stream(dev) if stream is None else stream
    out_ptr = compressed_out.data_ptr() if compressed_out is not None else None
    _check(library().dsv4_c4_compress_store_debug(*refs[:6], float(eps), *refs[6:], out_ptr, s))


def c4_validate(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                cos_sin, k_cache, kv_slot_mapping) -> int:
    """Host-only validation of C4 descriptors; returns the status code."""
    ts = (state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping)
    keep, refs = _descriptors(ts)
    return library().dsv4_c4_validate(*refs[:6], float(eps), *refs[6:])


def indexer_compress_store(state_cache, block_table, token_to_req, positions, slot_mapping,
                           rms_w, eps, cos_sin, k_cache, kv_slot_mapping, compressed_out=None,
                           stream: int | None = None) -> None:
    """The indexer's FP8 compressor (head 128, ratio 4 with the overlapping window; state rows
    kv 2x128 | score 2x128, any state block size; k_cache u8 [B, bs, 132]).
    ``compressed_out``: optional contiguous float32 [T, 128] device tensor."""
    ts = [state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping]
    dev = _require_cuda(ts + ([compressed_out] if compressed_out is not None else []))
    if compressed_out is not None and (
            compressed_out.dtype != torch.float32 or not compressed_out.is_contiguous() or
            tuple(compressed_out.shape) != (positions.shape[0], 128)):
        raise ValueError("compressed_out must be a contiguous float32 [T, 128] tensor")
    keep, refs = _descriptors(ts)
    s = _stream(dev) if stream is None else stream
    out_ptr = compressed_out.data_ptr() if compressed_out is not None else None
    _check(library().dsv4_indexer_compress_store_debug(*refs[:6], float(eps), *refs[6:],
                                                       out_ptr, s))


def indexer_mxfp4_compress_store(state_cache, block_table, token_to_req, positions,
                                 slot_mapping, rms_w, eps, cos_sin, k_cache, kv_slot_mapping,
                                 compressed_out=None, stream: int | None = None) -> None:
    """The indexer's compressor with the MXFP4 cache (k_cache u8 [B, bs, 68]: bs records of 64
    bytes of E2M1 codes, two a byte, then bs x 4 UE8M0 bytes); inputs as for
    ``indexer_compress_store``."""
    ts = [state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping]
    dev = _require_cuda(ts + ([compressed_out] if compressed_out is not None else []))
    if compressed_out is not None and (
            compressed_out.dtype != torch.float32 or not compressed_out.is_contiguous() or
            tuple(compressed_out.shape) != (positions.shape[0], 128)):
        raise ValueError("compressed_out must be a contiguous float32 [T, 128] tensor")
    keep, refs = _descriptors(ts)
    s = _stream(dev) if stream is None else stream
    out_ptr = compressed_out.data_ptr() if compressed_out is not None else None
    _check(library().dsv4_indexer_mxfp4_compress_store_debug(*refs[:6], float(eps), *refs[6:],
                                                             out_ptr, s))


def indexer_mxfp4_validate(state_cache, block_table, token_to_req, positions, slot_mapping,
                           rms_w, eps, cos_sin, k_cache, kv_slot_mapping) -> int:
    """Host-only validation of MXFP4 indexer descriptors; returns the status code."""
    ts = (state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping)
    keep, refs = _descriptors(ts)
    return library().dsv4_indexer_mxfp4_validate(*refs[:6], float(eps), *refs[6:])


def indexer_validate(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                     cos_sin, k_cache, kv_slot_mapping) -> int:
    """Host-only validation of indexer descriptors; returns the status code."""
    ts = (state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping)
    keep, refs = _descriptors(ts)
    return library().dsv4_indexer_validate(*refs[:6], float(eps), *refs[6:])


def validate(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
             cos_sin, k_cache, kv_slot_mapping) -> int:
    """Host-only validation of the descriptors (no HIP call); returns the status code."""
    ts = (state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, cos_sin,
          k_cache, kv_slot_mapping)
    keep, refs = _descriptors(ts)
    return library().dsv4_c128_validate(*refs[:6], float(eps), *refs[6:])


def e4m3_encode(x: torch.Tensor, stream: int | None = None) -> torch.Tensor:
    """The kernel's E4M3FN encoder (clamp to +-448, round to nearest even) on a float32
    device tensor; returns the uint8 codes."""
    if x.dtype != torch.float32 or not x.is_cuda:
        raise ValueError("x must be a float32 device tensor")
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = _stream(x.device) if stream is None else stream
    _check(library().dsv4_e4m3_encode(x.data_ptr(), out.data_ptr(), x.numel(), s))
    return out


def e2m1_encode(x: torch.Tensor, stream: int | None = None) -> torch.Tensor:
    """The kernel's E2M1 encoder (nearest, ties to even, saturating at 6, sign in bit 3) on a
    float32 device tensor; returns one uint8 code per value."""
    if x.dtype != torch.float32 or not x.is_cuda:
        raise ValueError("x must be a float32 device tensor")
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = _stream(x.device) if stream is None else stream
    _check(library().dsv4_e2m1_encode(x.data_ptr(), out.data_ptr(), x.numel(), s))
    return out


__all__ = ["compress_store", "compress_store_debug", "compress_store_ex", "workspace_bytes",
           "fanout_workspace",
           "compress_store_varlen", "varlen_workspace_bytes", "compress_store_varlen_noalloc",
           "VARLEN_NOALLOC_MAX_TOKENS", "c4_compress_store", "c4_validate",
           "indexer_compress_store", "indexer_validate", "indexer_mxfp4_compress_store",
           "indexer_mxfp4_validate", "validate", "e4m3_encode", "e2m1_encode", "last_error",
           "abi_version", "library", "describe", "Tensor", "Dsv4Error", "LIBRARY_PATH"]
