"""Host-only tests of the C ABI: the library loads without a GPU, exports every function
the header declares, and its descriptor validation returns each documented error code
before any HIP call (validation reads descriptors only, never the data)."""

import ctypes
import os
import re

import pytest
import torch

import paged_kv_cache_fp32_amd as c128

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsv4_c128.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dsv4_\w+)\s*\(", text, re.M)))


def header_constant(name):
    m = re.search(rf"#define\s+{name}\s+(\d+)", open(HEADER).read())
    return int(m.group(1))


def test_library_exports_every_declared_function():
    lib = c128.library()
    names = declared_functions()
    assert {"dsv4_c128_compress_store", "dsv4_c128_compress_store_debug", "dsv4_c128_validate",
            "dsv4_e4m3_encode", "dsv4_last_error", "dsv4_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header():
    assert c128.abi_version() == header_constant("DSV4_ABI_VERSION")


def test_error_codes_match_header():
    text = open(HEADER).read()
    for code, name in c128.ERRORS.items():
        m = re.search(rf"{name}\s*=\s*(-?\d+)", text)
        assert m and int(m.group(1)) == code, name


def valid_args(T=4, S=32, bs=4):
    """CPU tensors with valid shapes/strides (validation never reads them)."""
    return dict(
        state_cache=torch.zeros(S, 8, 1024, dtype=torch.float32),
        block_table=torch.zeros(T, 64, dtype=torch.int32),
        token_to_req=torch.zeros(T, dtype=torch.int32),
        positions=torch.zeros(T, dtype=torch.int32),
        slot_mapping=torch.zeros(T, dtype=torch.int32),
        rms_w=torch.ones(512, dtype=torch.float32),
        eps=1e-6,
        cos_sin=torch.zeros(128, 64, dtype=torch.float32),
        k_cache=torch.zeros(2, bs, 584, dtype=torch.uint8),
        kv_slot_mapping=torch.zeros(T, dtype=torch.int32),
    )


def call_validate(a):
    return c128.validate(a["state_cache"], a["block_table"], a["token_to_req"], a["positions"],
                         a["slot_mapping"], a["rms_w"], a["eps"], a["cos_sin"], a["k_cache"],
                         a["kv_slot_mapping"])


def test_valid_layout_passes():
    assert call_validate(valid_args()) == 0
    assert c128.last_error() == ""


def padded(shape, dtype, pad_last=0, pad_dim0=0):
    big = torch.zeros(*[s + (pad_dim0 if i == 0 else 0) for i, s in enumerate(shape[:-1])],
                      shape[-1] + pad_last, dtype=dtype)
    return big[tuple(slice(0, s) for s in shape)]


def test_kv_block_size_one_passes():
    """bs = 1 gives a 584-byte block stride: 8-byte aligned, which is all the stores need."""
    a = valid_args(bs=1)
    assert call_validate(a) == 0, c128.last_error()


def test_padded_views_pass():
    a = valid_args()
    a["state_cache"] = torch.zeros(32, 8, 1024 + 64)[:, :, :1024]
    a["k_cache"] = torch.as_strided(torch.zeros(2 * (4 * 584 + 48), dtype=torch.uint8),
                                    (2, 4, 584), (4 * 584 + 48, 584, 1))
    a["cos_sin"] = torch.zeros(128, 96)[:, :64]
    a["block_table"] = torch.zeros(4, 80, dtype=torch.int32)[:, :64]
    assert call_validate(a) == 0, c128.last_error()


CASES = [
    # (name, mutation, expected code)
    ("state dtype", lambda a: a.update(state_cache=a["state_cache"].double()), -2),
    ("state rank", lambda a: a.update(state_cache=a["state_cache"].view(32, 8192)), -3),
    ("state block 16", lambda a: a.update(state_cache=torch.zeros(16, 16, 1024)), -4),
    ("state row 512", lambda a: a.update(state_cache=torch.zeros(32, 8, 512)), -4),
    ("state row 2048", lambda a: a.update(state_cache=torch.zeros(32, 8, 2048)), -4),
    ("state transposed", lambda a: a.update(
        state_cache=torch.zeros(1024, 8, 32).permute(2, 1, 0)), -5),
    ("state rows overlap", lambda a: a.update(
        state_cache=torch.as_strided(torch.zeros(40000), (32, 8, 1024), (1024, 512, 1))), -5),
    ("state misaligned", lambda a: a.update(
        state_cache=torch.zeros(32 * 8 * 1024 + 1)[1:].view(32, 8, 1024)), -6),
    ("state stride not x4", lambda a: a.update(
        state_cache=torch.zeros(32, 8, 1026)[:, :, :1024]), -6),
    ("block table rank", lambda a: a.update(block_table=torch.zeros(256, dtype=torch.int32)), -3),
    ("block table dtype", lambda a: a.update(block_table=torch.zeros(4, 64, dtype=torch.int64)), -2),
    ("block table narrow", lambda a: a.update(block_table=torch.zeros(4, 8, dtype=torch.int32)), -4),
    ("block table col-major", lambda a: a.update(
        block_table=torch.zeros(64, 4, dtype=torch.int32).t()), -5),
    ("T mismatch", lambda a: a.update(token_to_req=torch.zeros(5, dtype=torch.int32)), -4),
    ("slot T mismatch", lambda a: a.update(slot_mapping=torch.zeros(3, dtype=torch.int32)), -4),
    ("kv slot T mismatch", lambda a: a.update(kv_slot_mapping=torch.zeros(2, dtype=torch.int32)),
     -4),
    ("positions strided", lambda a: a.update(positions=torch.zeros(8, dtype=torch.int32)[::2]), -5),
    ("positions int64", lambda a: a.update(positions=torch.zeros(4, dtype=torch.int64)), -2),
    ("rms 448", lambda a: a.update(rms_w=torch.ones(448)), -4),
    ("rms strided", lambda a: a.update(rms_w=torch.ones(1024)[::2]), -5),
    ("rms misaligned", lambda a: a.update(rms_w=torch.ones(513)[1:]), -6),
    ("cos_sin narrow", lambda a: a.update(cos_sin=torch.zeros(128, 32)), -4),
    ("cos_sin col-major", lambda a: a.update(cos_sin=torch.zeros(64, 128).t()), -5),
    ("k_cache dtype", lambda a: a.update(k_cache=torch.zeros(2, 4, 584, dtype=torch.int32)), -2),
    ("k_cache row 576", lambda a: a.update(k_cache=torch.zeros(2, 4, 576, dtype=torch.uint8)), -4),
    ("k_cache rank", lambda a: a.update(k_cache=torch.zeros(2, 4 * 584, dtype=torch.uint8)), -3),
    ("k_cache stride0 small", lambda a: a.update(k_cache=torch.as_strided(
        torch.zeros(8 * 584, dtype=torch.uint8), (2, 4, 584), (3 * 584, 584, 1))), -5),
    ("k_cache stride0 unaligned", lambda a: a.update(k_cache=torch.as_strided(
        torch.zeros(2 * (4 * 584 + 4), dtype=torch.uint8), (2, 4, 584), (4 * 584 + 4, 584, 1))), -6),
    ("k_cache base unaligned", lambda a: a.update(k_cache=torch.zeros(
        2 * 4 * 584 + 4, dtype=torch.uint8)[4:].view(2, 4, 584)), -6),
    ("negative eps", lambda a: a.update(eps=-1.0), -4),
    ("nan eps", lambda a: a.update(eps=float("nan")), -4),
]


@pytest.mark.parametrize("name,mut,code", CASES, ids=[c[0] for c in CASES])
def test_validation_error_codes(name, mut, code):
    a = valid_args()
    mut(a)
    assert call_validate(a) == code, c128.last_error()
    assert c128.last_error() != ""


def test_null_descriptor():
    a = valid_args()
    lib = c128.library()
    d = [c128.describe(a[k]) for k in ("state_cache", "block_table", "token_to_req", "positions",
                                       "slot_mapping", "rms_w")]
    rest = [c128.describe(a[k]) for k in ("cos_sin", "k_cache", "kv_slot_mapping")]
    refs = [ctypes.byref(x) for x in d]
    rc = lib.dsv4_c128_validate(None, *refs[1:], 1e-6, *[ctypes.byref(x) for x in rest])
    assert rc == -1
    # a null data pointer on a non-empty tensor
    d[0].data = None
    rc = lib.dsv4_c128_validate(*[ctypes.byref(x) for x in d], 1e-6,
                                *[ctypes.byref(x) for x in rest])
    assert rc == -1


TOKEN_ARRAYS = ("token_to_req", "positions", "slot_mapping", "kv_slot_mapping")
ARG_ORDER = ("state_cache", "block_table", "token_to_req", "positions", "slot_mapping", "rms_w",
             "cos_sin", "k_cache", "kv_slot_mapping")


def descriptors_with_tokens(a, T):
    """Descriptors of ``a`` whose four token arrays claim T tokens (validation reads only the
    descriptors, so a small buffer stands behind them)."""
    ds = [c128.describe(a[k]) for k in ARG_ORDER]
    for k, d in zip(ARG_ORDER, ds):
        if k in TOKEN_ARRAYS:
            d.shape[0] = T
    refs = [ctypes.byref(d) for d in ds]
    return refs[:6], refs[6:]


@pytest.mark.parametrize("fn,args", [("dsv4_c128_validate", valid_args),
                                     ("dsv4_c4_validate", lambda: c4_args()),
                                     ("dsv4_indexer_validate", lambda: idx_args()),
                                     ("dsv4_indexer_mxfp4_validate", lambda: fp4_args())])
def test_token_count_limit(fn, args):
    """DSV4_MAX_TOKENS tokens pass validation; one more is DSV4_ERR_SHAPE with a message that
    names the limit, for every compressor."""
    limit = header_constant("DSV4_MAX_TOKENS")
    assert limit == 1 << 27
    lib = c128.library()
    a = args()
    head, tail = descriptors_with_tokens(a, limit)
    assert getattr(lib, fn)(*head, 1e-6, *tail) == 0, c128.last_error()
    head, tail = descriptors_with_tokens(a, limit + 1)
    assert getattr(lib, fn)(*head, 1e-6, *tail) == -4
    assert f"at most {limit}" in c128.last_error()


def test_compute_entry_point_rejects_too_many_tokens_before_launch():
    """The limit is checked before any HIP call (host pointers, no GPU)."""
    lib = c128.library()
    head, tail = descriptors_with_tokens(valid_args(), header_constant("DSV4_MAX_TOKENS") + 1)
    assert lib.dsv4_c128_compress_store(*head, 1e-6, *tail, None) == -4


def test_compute_entry_points_reject_before_any_hip_call():
    """The compute entry points validate first: with an invalid layout they return the error
    code without launching (safe with host pointers and no GPU)."""
    a = valid_args()
    a["state_cache"] = torch.zeros(32, 8, 512)
    lib = c128.library()
    ts = [a[k] for k in ("state_cache", "block_table", "token_to_req", "positions",
                         "slot_mapping", "rms_w")]
    rest = [a[k] for k in ("cos_sin", "k_cache", "kv_slot_mapping")]
    ds = [c128.describe(t) for t in ts]
    rs = [c128.describe(t) for t in rest]
    rc = lib.dsv4_c128_compress_store(*[ctypes.byref(x) for x in ds], 1e-6,
                                      *[ctypes.byref(x) for x in rs], None)
    assert rc == -4
    rc = lib.dsv4_c128_compress_store_debug(*[ctypes.byref(x) for x in ds], 1e-6,
                                            *[ctypes.byref(x) for x in rs], None, None)
    assert rc == -4


def test_empty_batch_returns_before_launch():
    """T == 0 is a no-op that returns before any HIP call."""
    a = valid_args(T=0)
    a["block_table"] = torch.zeros(1, 16, dtype=torch.int32)
    lib = c128.library()
    ts = [a[k] for k in ("state_cache", "block_table", "token_to_req", "positions",
                         "slot_mapping", "rms_w")]
    rest = [a[k] for k in ("cos_sin", "k_cache", "kv_slot_mapping")]
    rc = lib.dsv4_c128_compress_store(*[ctypes.byref(c128.describe(t)) for t in ts], 1e-6,
                                      *[ctypes.byref(c128.describe(t)) for t in rest], None)
    assert rc == 0
    assert lib.dsv4_e4m3_encode(None, None, 0, None) == 0
    assert lib.dsv4_e4m3_encode(None, None, -1, None) == -4


def test_python_binding_rejects_host_tensors():
    a = valid_args()
    with pytest.raises(ValueError):
        c128.compress_store(**a)


def test_workspace_bytes_rules():
    """Automatic splits: 8 up to 16 tokens, 4 up to 64, 2 up to 128, 1 (no workspace) above;
    explicit splits give the 16 KiB counter region plus T*splits*3*512 floats; invalid splits,
    or more than 4096 tokens with splits > 1, give 0."""
    wb = c128.workspace_bytes
    per = 3 * 512 * 4
    cnt = 16384
    assert wb(1, 0) == cnt + 1 * 8 * per
    assert wb(16, 0) == cnt + 16 * 8 * per
    assert wb(17, 0) == cnt + 17 * 4 * per
    assert wb(64, 0) == cnt + 64 * 4 * per
    assert wb(65, 0) == cnt + 65 * 2 * per and wb(128, 0) == cnt + 128 * 2 * per
    assert wb(129, 0) == 0 and wb(512, 0) == 0 and wb(16384, 0) == 0
    assert wb(10, 4) == cnt + 10 * 4 * per and wb(10, 1) == 0
    assert wb(100, 16) == cnt + 100 * 16 * per
    assert wb(4096, 2) == cnt + 4096 * 2 * per and wb(4097, 2) == 0
    assert wb(10, 3) == 0 and wb(10, 32) == 0 and wb(0, 4) == 0


def ex_call(a, splits, workspace=None, nbytes=0, out=None):
    lib = c128.library()
    ts = [a[k] for k in ("state_cache", "block_table", "token_to_req", "positions",
                         "slot_mapping", "rms_w")]
    rest = [a[k] for k in ("cos_sin", "k_cache", "kv_slot_mapping")]
    return lib.dsv4_c128_compress_store_ex(*[ctypes.byref(c128.describe(t)) for t in ts], 1e-6,
                                           *[ctypes.byref(c128.describe(t)) for t in rest], out,
                                           workspace, nbytes, splits, None)


def test_fanout_argument_errors_before_launch():
    """Invalid splits, or explicit splits > 1 without a big enough workspace, fail with
    DSV4_ERR_ARG before any HIP call; a bad layout still fails with its own code first."""
    a = valid_args()
    assert ex_call(a, 3) == -8 and "splits" in c128.last_error()
    assert ex_call(a, 32) == -8
    assert ex_call(a, 4) == -8 and "workspace" in c128.last_error()
    assert ex_call(a, 4, workspace=16, nbytes=16) == -8
    big = valid_args(T=4097)
    assert ex_call(big, 2, workspace=16, nbytes=1 << 40) == -8 and "4096" in c128.last_error()
    bad = valid_args()
    bad["state_cache"] = torch.zeros(32, 8, 512)
    assert ex_call(bad, 4) == -4


def test_fanout_empty_batch_is_a_noop_on_host():
    a = valid_args(T=0)
    a["block_table"] = torch.zeros(1, 16, dtype=torch.int32)
    assert ex_call(a, 16) == 0
    assert ex_call(a, 0) == 0


def varlen_call(a, workspace=None, nbytes=0, out=None):
    lib = c128.library()
    ts = [a[k] for k in ("state_cache", "block_table", "token_to_req", "positions",
                         "slot_mapping", "rms_w")]
    rest = [a[k] for k in ("cos_sin", "k_cache", "kv_slot_mapping")]
    return lib.dsv4_c128_compress_store_varlen(
        *[ctypes.byref(c128.describe(t)) for t in ts], 1e-6,
        *[ctypes.byref(c128.describe(t)) for t in rest], out, workspace, nbytes, None)


def test_varlen_workspace_bytes_rule():
    """Counts of up to 1024 scan blocks, then one list entry per token; 16-byte granules."""
    vb = c128.varlen_workspace_bytes
    assert vb(0) == 0 and vb(-3) == 0
    assert vb(1) == 4112 and vb(4) == 4112 and vb(5) == 4128
    assert vb(34323) == (4 * (1024 + 34323) + 15) // 16 * 16
    assert vb(2 ** 31 - 1) == (4 * (1024 + 2 ** 31 - 1) + 15) // 16 * 16


def test_varlen_argument_errors_before_launch():
    """No or too small a workspace is DSV4_ERR_ARG, a misaligned one DSV4_ERR_ALIGN, both
    before any HIP call; layout errors keep their own codes; T == 0 needs no workspace."""
    a = valid_args()
    assert varlen_call(a) == -8 and "workspace" in c128.last_error()
    assert varlen_call(a, workspace=16, nbytes=c128.varlen_workspace_bytes(4) - 16) == -8
    assert varlen_call(a, workspace=24, nbytes=c128.varlen_workspace_bytes(4)) == -6
    assert varlen_call(a, workspace=16, nbytes=8192, out=8) == -6
    bad = valid_args()
    bad["k_cache"] = torch.zeros(2, 4, 576, dtype=torch.uint8)
    assert varlen_call(bad) == -4
    e = valid_args(T=0)
    assert varlen_call(e) == 0


def test_varlen_noalloc_errors_before_launch():
    """The allocation-free compacted schedule validates like the others, then rejects more
    tokens than its fixed scratch holds (DSV4_ERR_ARG, naming the limit), all before any HIP
    call; T == 0 is a no-op."""
    lib = c128.library()
    limit = header_constant("DSV4_VARLEN_NOALLOC_MAX_TOKENS")
    assert limit == 1 << 20 == c128.VARLEN_NOALLOC_MAX_TOKENS
    head, tail = descriptors_with_tokens(valid_args(), limit + 1)
    assert lib.dsv4_c128_compress_store_varlen_noalloc(*head, 1e-6, *tail, None, None) == -8
    assert f"at most {limit}" in c128.last_error()
    bad = valid_args()
    bad["k_cache"] = torch.zeros(2, 4, 576, dtype=torch.uint8)
    head, tail = descriptors_with_tokens(bad, 4)
    assert lib.dsv4_c128_compress_store_varlen_noalloc(*head, 1e-6, *tail, None, None) == -4
    head, tail = descriptors_with_tokens(valid_args(), 4)
    assert lib.dsv4_c128_compress_store_varlen_noalloc(*head, 1e-6, *tail, 8, None) == -6
    head, tail = descriptors_with_tokens(valid_args(T=0), 0)
    assert lib.dsv4_c128_compress_store_varlen_noalloc(*head, 1e-6, *tail, None, None) == 0


def c4_args(T=4, S=16, sbs=8, bs=4):
    a = valid_args(T=T, S=S, bs=bs)
    a["state_cache"] = torch.zeros(S, sbs, 2048, dtype=torch.float32)
    a["block_table"] = torch.zeros(T, 4, dtype=torch.int32)
    return a


def c4_validate(a):
    return c128.c4_validate(a["state_cache"], a["block_table"], a["token_to_req"],
                            a["positions"], a["slot_mapping"], a["rms_w"], a["eps"],
                            a["cos_sin"], a["k_cache"], a["kv_slot_mapping"])


@pytest.mark.parametrize("sbs", [1, 2, 4, 8, 16, 64])
def test_c4_accepts_any_state_block_size(sbs):
    assert c4_validate(c4_args(sbs=sbs)) == 0, c128.last_error()


def test_c4_layout_errors():
    """The C4 state row is 2048 floats (kv 2x512 | score 2x512); the C128 row is rejected and
    the C4 row is rejected by the C128 entry point; strides and alignment as for C128."""
    a = c4_args()
    a["state_cache"] = torch.zeros(16, 8, 1024)
    assert c4_validate(a) == -4 and "2048" in c128.last_error()
    a = c4_args()
    assert call_validate(a) == -4
    a = c4_args()
    a["state_cache"] = torch.zeros(16, 8, 4096)[:, :, :2048]
    assert c4_validate(a) == 0
    a["state_cache"] = torch.zeros(16, 8, 2049)[:, :, :2048]
    assert c4_validate(a) == -6
    a = c4_args()
    a["state_cache"] = torch.zeros(8, 16, 2048).transpose(0, 1)
    assert c4_validate(a) == -5
    a = c4_args()
    a["block_table"] = torch.zeros(4, 0, dtype=torch.int32)
    assert c4_validate(a) == -4
    a = c4_args()
    a["block_table"] = torch.zeros(4, 1, dtype=torch.int32)
    assert c4_validate(a) == 0


def idx_args(T=4, S=16, sbs=8, bs=4):
    a = c4_args(T=T, S=S, sbs=sbs, bs=bs)
    a["state_cache"] = torch.zeros(S, sbs, 512, dtype=torch.float32)
    a["rms_w"] = torch.ones(128, dtype=torch.float32)
    a["k_cache"] = torch.zeros(2, bs, 132, dtype=torch.uint8)
    return a


def idx_validate(a):
    return c128.indexer_validate(a["state_cache"], a["block_table"], a["token_to_req"],
                                 a["positions"], a["slot_mapping"], a["rms_w"], a["eps"],
                                 a["cos_sin"], a["k_cache"], a["kv_slot_mapping"])


@pytest.mark.parametrize("sbs", [1, 4, 8, 64])
def test_indexer_accepts_layout(sbs):
    assert idx_validate(idx_args(sbs=sbs)) == 0, c128.last_error()


def test_indexer_layout_errors():
    """State row 512 floats, rms_w 128, k_cache [B, bs, 132] with 4-byte alignment; the sparse
    layouts are rejected and the indexer layout is rejected by the C4 entry point."""
    a = idx_args()
    a["state_cache"] = torch.zeros(16, 8, 2048)
    assert idx_validate(a) == -4
    a = idx_args()
    a["rms_w"] = torch.ones(512)
    assert idx_validate(a) == -4 and "128" in c128.last_error()
    a = idx_args()
    a["k_cache"] = torch.zeros(2, 4, 584, dtype=torch.uint8)
    assert idx_validate(a) == -4 and "132" in c128.last_error()
    a = idx_args()
    a["k_cache"] = torch.zeros(2 * 4 * 132 + 2, dtype=torch.uint8)[2:].view(2, 4, 132)
    assert idx_validate(a) == -6
    a = idx_args()
    a["k_cache"] = torch.as_strided(torch.zeros(2 * 530, dtype=torch.uint8), (2, 4, 132),
                                    (530, 132, 1))
    assert idx_validate(a) == -6
    a = idx_args()
    a["k_cache"] = torch.as_strided(torch.zeros(2 * 532, dtype=torch.uint8), (2, 4, 132),
                                    (532, 132, 1))
    assert idx_validate(a) == 0
    assert c4_validate(idx_args()) == -4


def fp4_args(T=4, S=16, sbs=8, bs=4):
    a = idx_args(T=T, S=S, sbs=sbs, bs=bs)
    a["k_cache"] = torch.zeros(2, bs, 68, dtype=torch.uint8)
    return a


def fp4_validate(a):
    return c128.indexer_mxfp4_validate(a["state_cache"], a["block_table"], a["token_to_req"],
                                       a["positions"], a["slot_mapping"], a["rms_w"], a["eps"],
                                       a["cos_sin"], a["k_cache"], a["kv_slot_mapping"])


@pytest.mark.parametrize("sbs", [1, 4, 8, 64])
def test_indexer_mxfp4_accepts_layout(sbs):
    assert fp4_validate(fp4_args(sbs=sbs)) == 0, c128.last_error()


def test_indexer_mxfp4_layout_errors():
    """k_cache [B, bs, 68] (64 code bytes + 4 scale bytes) with 4-byte alignment; the FP8
    indexer's 132-byte slots are rejected, and the MXFP4 cache by the FP8 entry point."""
    a = fp4_args()
    a["k_cache"] = torch.zeros(2, 4, 132, dtype=torch.uint8)
    assert fp4_validate(a) == -4 and "68" in c128.last_error()
    assert idx_validate(fp4_args()) == -4
    a = fp4_args()
    a["k_cache"] = torch.zeros(2 * 4 * 68 + 2, dtype=torch.uint8)[2:].view(2, 4, 68)
    assert fp4_validate(a) == -6
    a = fp4_args()
    a["k_cache"] = torch.as_strided(torch.zeros(2 * 274, dtype=torch.uint8), (2, 4, 68),
                                    (274, 68, 1))
    assert fp4_validate(a) == -6
    a = fp4_args()
    a["k_cache"] = torch.as_strided(torch.zeros(2 * 276, dtype=torch.uint8), (2, 4, 68),
                                    (276, 68, 1))
    assert fp4_validate(a) == 0
    a = fp4_args()
    a["k_cache"] = torch.as_strided(torch.zeros(2 * 272, dtype=torch.uint8), (2, 4, 68),
                                    (268, 68, 1))
    assert fp4_validate(a) == -5          # stride[0] below bs * 68
    a = fp4_args()
    a["rms_w"] = torch.ones(512)
    assert fp4_validate(a) == -4


def test_indexer_mxfp4_rejects_before_any_hip_call():
    lib = c128.library()
    a = fp4_args()
    a["k_cache"] = torch.zeros(2, 4, 132, dtype=torch.uint8)
    ds = [ctypes.byref(c128.describe(a[k])) for k in ARG_ORDER]
    assert lib.dsv4_indexer_mxfp4_compress_store(*ds[:6], 1e-6, *ds[6:], None) == -4
    assert lib.dsv4_e2m1_encode(None, None, 0, None) == 0
    assert lib.dsv4_e2m1_encode(None, None, -1, None) == -4
    assert lib.dsv4_e2m1_encode(None, None, 4, None) == -1


def test_negative_and_overflowing_strides_are_rejected():
    """A negative stride on a dimension longer than 1, or strides whose span passes 2^48 bytes,
    is DSV4_ERR_STRIDE before any launch (no index times stride can then overflow); the same
    strides on a dimension of length 1 are never multiplied by a nonzero index and pass."""
    lib = c128.library()
    for k, dim, stride in (("state_cache", 0, 1 << 50), ("state_cache", 0, -8192),
                           ("block_table", 0, 1 << 47), ("cos_sin", 0, -64),
                           ("k_cache", 0, 1 << 48)):
        ds = [c128.describe(valid_args()[n]) for n in ARG_ORDER]
        ds[ARG_ORDER.index(k)].stride[dim] = stride
        refs = [ctypes.byref(d) for d in ds]
        assert lib.dsv4_c128_validate(*refs[:6], 1e-6, *refs[6:]) == -5, (k, stride)
        assert "stride" in c128.last_error() or "span" in c128.last_error()
    a = valid_args()
    a["block_table"] = torch.zeros(1, 64, dtype=torch.int32)
    ds = [c128.describe(a[n]) for n in ARG_ORDER]
    ds[ARG_ORDER.index("block_table")].stride[0] = -(1 << 60)
    refs = [ctypes.byref(d) for d in ds]
    assert lib.dsv4_c128_validate(*refs[:6], 1e-6, *refs[6:]) == 0, c128.last_error()
    # the largest span that passes: 2^48 bytes of k_cache blocks
    ds = [c128.describe(valid_args()[n]) for n in ARG_ORDER]
    kc = ds[ARG_ORDER.index("k_cache")]
    kc.stride[0] = ((1 << 48) - 3 * 584 - 583) // (kc.shape[0] - 1) // 8 * 8
    refs = [ctypes.byref(d) for d in ds]
    assert lib.dsv4_c128_validate(*refs[:6], 1e-6, *refs[6:]) == 0, c128.last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises: there is no fallback path."""
    monkeypatch.setattr(c128, "LIBRARY_PATH", str(tmp_path / "libdsv4_c128.so"))
    monkeypatch.setattr(c128, "_lib", None)
    with pytest.raises(ImportError, match="no fallback"):
        c128.abi_version()
    a = valid_args()
    with pytest.raises(ImportError):
        call_validate(a)
