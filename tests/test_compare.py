"""Host tests of the parity checker (oracle/compare.py): it passes the oracle's own output
and flags each kind of planted mistake."""

import numpy as np
import pytest

import oracle
import synth
from oracle.compare import compare, record_offsets


@pytest.fixture(scope="module")
def case():
    wl = synth.decode_batch("cmp", 8, 12, 400, 6, 96, kv_bs=4, kv_blocks=8, cs_rows=768)
    return wl, oracle.run(wl, 2)


def test_identical_output_passes(case):
    wl, orc = case
    rep = compare(wl, orc.k_cache_base.copy(), orc, gpu_compressed=orc.compressed.astype(np.float32))
    assert rep.ok(), rep.summary()
    assert rep["written"] == 12


def planted(wl, orc, fn):
    body = orc.k_cache_base.copy()
    s = int(wl.kv_slot_mapping[5])
    rec, scl = record_offsets(s, wl.k_cache.shape[1], wl.k_cache.strides[0])
    fn(body, rec, scl)
    return compare(wl, body, orc)


def test_flags_code_off_by_two(case):
    wl, orc = case

    def f(b, rec, scl):
        c = int(b[rec + 10])
        b[rec + 10] = (c & 0x80) | ((c & 0x7F) - 2 if (c & 0x7F) >= 2 else (c & 0x7F) + 2)
    assert not planted(wl, orc, f).ok()


def test_flags_scale_byte(case):
    wl, orc = case
    assert not planted(wl, orc, lambda b, rec, scl: b.__setitem__(scl + 2, b[scl + 2] + 1)).ok()


def test_flags_pad_byte(case):
    wl, orc = case
    assert not planted(wl, orc, lambda b, rec, scl: b.__setitem__(scl + 7, 1)).ok()


def test_flags_rope_far_off(case):
    wl, orc = case

    def f(b, rec, scl):
        v = b[rec + 448:rec + 576].view("<u2")
        i = int(np.argmax(np.abs((v.astype(np.uint32) << 16).view(np.float32))))
        v[i] = v[i] + 3 if (v[i] & 0x7FFF) < 0x7F00 else v[i] - 3
    assert not planted(wl, orc, f).ok()


def test_flags_write_outside_records(case):
    wl, orc = case
    body = orc.k_cache_base.copy()
    written = np.zeros(body.size, bool)
    for s in wl.kv_slot_mapping:
        rec, scl = record_offsets(int(s), wl.k_cache.shape[1], wl.k_cache.strides[0])
        written[rec:rec + 576] = True
        written[scl:scl + 8] = True
    idx = int(np.nonzero(~written)[0][0])
    body[idx] ^= 0xFF
    assert not compare(wl, body, orc).ok()


def test_flags_compressed_error(case):
    wl, orc = case
    g = orc.compressed.astype(np.float32).copy()
    g[3, 100] += np.float32(1e-3)
    assert not compare(wl, orc.k_cache_base.copy(), orc, gpu_compressed=g).ok()


# ---------------------------------------------------------------- indexer cache

@pytest.fixture(scope="module")
def icase():
    wl = synth.indexer_decode_batch("icmp", 8, 12, 60, 8, 8, kv_bs=4, kv_blocks=8, cs_rows=64)
    return wl, oracle.run(wl, 2)


def iplanted(wl, orc, fn):
    from oracle.compare import indexer_offsets
    body = orc.k_cache_base.copy()
    rec, scl = indexer_offsets(int(wl.kv_slot_mapping[5]), wl.k_cache.shape[1],
                               wl.k_cache.strides[0])
    fn(body, rec, scl)
    return compare(wl, body, orc)


def test_indexer_identical_output_passes(icase):
    wl, orc = icase
    rep = compare(wl, orc.k_cache_base.copy(), orc,
                  gpu_compressed=orc.compressed.astype(np.float32))
    assert rep.ok(), rep.summary()
    assert rep["written"] == 12


def test_indexer_flags_code_scale_and_stray_bytes(icase):
    wl, orc = icase

    def code(b, rec, scl):
        c = int(b[rec + 3])
        b[rec + 3] = (c & 0x80) | ((c & 0x7F) - 2 if (c & 0x7F) >= 2 else (c & 0x7F) + 2)

    def scale(b, rec, scl):
        b[scl:scl + 4] = np.frombuffer(np.float32(b[scl:scl + 4].view("<f4")[0] * 2).tobytes(),
                                       np.uint8)

    assert not iplanted(wl, orc, code).ok()
    assert not iplanted(wl, orc, scale).ok()
    # a byte of a kv slot that no token writes
    from oracle.compare import indexer_offsets
    free = sorted(set(range(32)) - set(int(x) for x in wl.kv_slot_mapping))[0]
    rec, _ = indexer_offsets(free, wl.k_cache.shape[1], wl.k_cache.strides[0])
    body = orc.k_cache_base.copy()
    body[rec] ^= 0xFF
    rep = compare(wl, body, orc)
    assert not rep.ok() and rep["untouched_mismatch"] == 1


# ---------------------------------------------------------------- indexer MXFP4 cache

@pytest.fixture(scope="module")
def fcase():
    wl = synth.indexer_decode_batch("fcmp", 8, 12, 60, 8, 8, kv_bs=4, kv_blocks=8, cs_rows=64,
                                    fp4=True)
    return wl, oracle.run(wl, 2)


def fplanted(wl, orc, fn):
    from oracle.compare import fp4_offsets
    body = orc.k_cache_base.copy()
    rec, scl = fp4_offsets(int(wl.kv_slot_mapping[5]), wl.k_cache.shape[1],
                           wl.k_cache.strides[0])
    fn(body, rec, scl)
    return compare(wl, body, orc)


def test_mxfp4_identical_output_passes(fcase):
    wl, orc = fcase
    rep = compare(wl, orc.k_cache_base.copy(), orc,
                  gpu_compressed=orc.compressed.astype(np.float32))
    assert rep.ok(), rep.summary()
    assert rep["written"] == 12


def _nudge(c, by):
    """E2M1 code c moved by ``by`` steps in magnitude (within 0..7), sign kept."""
    mag = c & 7
    mag = mag - by if mag >= by else mag + by
    return (c & 8) | mag


def test_mxfp4_flags_codes_scales_and_stray_bytes(fcase):
    wl, orc = fcase

    def low_two(b, rec, scl):      # the even dim of byte 3 off by two steps
        b[rec + 3] = (b[rec + 3] & 0xF0) | _nudge(int(b[rec + 3]) & 0xF, 2)

    def high_two(b, rec, scl):     # the odd dim of byte 40 off by two steps
        b[rec + 40] = (b[rec + 40] & 0x0F) | (_nudge(int(b[rec + 40]) >> 4, 2) << 4)

    def one_step(b, rec, scl):     # one step on one dim: within the code tolerance
        b[rec + 7] = (b[rec + 7] & 0xF0) | _nudge(int(b[rec + 7]) & 0xF, 1)

    def scale(b, rec, scl):
        b[scl + 2] += 1

    assert not fplanted(wl, orc, low_two).ok()
    assert not fplanted(wl, orc, high_two).ok()
    rep = fplanted(wl, orc, one_step)
    assert rep.ok() and rep["code_diff1"] == 1, rep.summary()
    assert not fplanted(wl, orc, scale).ok()
    from oracle.compare import fp4_offsets
    free = sorted(set(range(32)) - set(int(x) for x in wl.kv_slot_mapping))[0]
    rec, scl = fp4_offsets(free, wl.k_cache.shape[1], wl.k_cache.strides[0])
    for off in (rec + 63, scl):
        body = orc.k_cache_base.copy()
        body[off] ^= 0xFF
        rep = compare(wl, body, orc)
        assert not rep.ok() and rep["untouched_mismatch"] == 1


def test_mxfp4_knife_edge_excuses_a_flipped_scale():
    """A block whose fp64 absmax sits on the bf16 midpoint 1.50390625 * 2^k may come out with
    either exponent; the checker excuses a flipped scale there when the dequantised values agree
    within one step, and flags it elsewhere."""
    from oracle.compare import knife_edge, KNIFE_FP4
    assert knife_edge(1.50390625 * 4, KNIFE_FP4) and knife_edge(1.50390625 * 2 ** -3, KNIFE_FP4)
    assert not knife_edge(1.5 * 4, KNIFE_FP4) and not knife_edge(1.507 * 4, KNIFE_FP4)
