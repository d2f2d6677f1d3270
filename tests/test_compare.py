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


# ---------------------------------------------------------------- C128 knife edge

def _fake_result(orc):
    """A copy of an oracle result whose arrays a test may edit."""
    return oracle.OracleResult(orc.k_cache_base.copy(), None, orc.compressed.copy(),
                               orc.absnorm.copy(), orc.normed.copy(), orc.status.copy())


def _bf16(x):
    """Round-to-nearest-even bf16 of fp64 values through fp32, as the quantiser's input."""
    b = oracle.bf16_bits(np.asarray(x, np.float64).astype(np.float32).astype(np.float64))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _encode_block(u, e):
    """E4M3FN codes of the bf16 values ``u`` under the block scale 2^e, and the scale byte."""
    return oracle.e4m3_codes(np.clip(u * 2.0 ** -e, -448.0, 448.0)), np.uint8(e + 127)


def _knife_case(case, rel_offset):
    """Token 5's quantisation block 2 scaled so that its fp64 absmax is the bf16 midpoint
    1.75390625 * 2^k times (1 + rel_offset).  Returns (fake oracle result with that block
    encoded as the oracle encodes it, GPU bytes with the block encoded as if fp32 rounding had
    put bf16(absmax) on the other side of the midpoint, offsets)."""
    wl, orc = case
    t, g = 5, 2
    res = _fake_result(orc)
    v = res.normed[t, 64 * g:64 * (g + 1)]
    amax = float(np.abs(v).max())
    k = np.floor(np.log2(amax / 1.75390625))
    v *= 1.75390625 * 2.0 ** k * (1.0 + rel_offset) / amax
    res.normed[t, 64 * g:64 * (g + 1)] = v
    rec, scl = record_offsets(int(wl.kv_slot_mapping[t]), wl.k_cache.shape[1],
                              wl.k_cache.strides[0])
    u = _bf16(v)
    e_orc = int(oracle.ue8m0_exponents(np.array([np.abs(u).max()]))[0])
    codes, byte = _encode_block(u, e_orc)
    res.k_cache_base[rec + 64 * g:rec + 64 * (g + 1)] = codes
    res.k_cache_base[scl + g] = byte
    # the GPU's bf16 absmax lands on the other neighbour of the midpoint
    i = int(np.argmax(np.abs(v)))
    ug = u.copy()
    up = 1.7578125 * 2.0 ** k
    ug[i] = np.sign(v[i]) * (up if abs(u[i]) < up else 1.75 * 2.0 ** k)
    e_gpu = int(oracle.ue8m0_exponents(np.array([np.abs(ug).max()]))[0])
    assert e_gpu != e_orc
    body = res.k_cache_base.copy()
    gcodes, gbyte = _encode_block(ug, e_gpu)
    body[rec + 64 * g:rec + 64 * (g + 1)] = gcodes
    body[scl + g] = gbyte
    return res, body, rec + 64 * g


def test_knife_edge_excuses_a_flipped_c128_scale(case):
    """At a true knife edge (absmax on the bf16 midpoint 1.75390625 * 2^k) a scale byte one
    step off is excused when every dequantised value lies within one code step of the coarser
    scale at its own binade."""
    wl, _ = case
    res, body, _ = _knife_case(case, 0.0)
    rep = compare(wl, body, res)
    assert rep.ok(), rep.summary()
    assert rep["excused_blocks"] == 1 and rep["scale_mismatch"] == 0


def test_knife_edge_flags_a_flip_outside_the_band(case):
    """The same flip with the absmax 2e-5 (relative) away from the midpoint is not excused."""
    wl, _ = case
    res, body, _ = _knife_case(case, 2e-5)
    rep = compare(wl, body, res)
    assert not rep.ok() and rep["scale_mismatch"] == 1 and rep["excused_blocks"] == 0


def test_knife_edge_flags_values_two_steps_off(case):
    """An excused block still fails when one of its elements is two code steps off at its own
    binade (a small element: the step there is far below the top binade's)."""
    wl, _ = case
    res, body, start = _knife_case(case, 0.0)
    codes = body[start:start + 64]
    mags = codes & 0x7F
    j = int(np.nonzero((mags > 8) & (mags < 0x40))[0][0])   # a small normal element
    body[start + j] = (codes[j] & 0x80) | (mags[j] + 2)
    rep = compare(wl, body, res)
    assert not rep.ok() and rep["excused_blocks"] == 1
    assert any("excused block values differ" in f for f in rep["failures"])


def test_knife_edge_band_limits():
    from oracle.compare import knife_edge
    for k in (-20, -3, 0, 5, 30):
        edge = 1.75390625 * 2.0 ** k
        assert knife_edge(edge) and knife_edge(edge * (1 + 9e-6)) and knife_edge(edge * (1 - 9e-6))
        assert not knife_edge(edge * (1 + 1.1e-5)) and not knife_edge(edge * (1 - 1.1e-5))
        assert not knife_edge(1.75 * 2.0 ** k) and not knife_edge(1.7578125 * 2.0 ** k)


# ---------------------------------------------------------------- RoPE band

def _rope_cancel_case(case):
    """Token 5 of the case with its pooled pair (448, 449) replaced so that the first rotated
    value cancels to about 1e-6 of its inputs.  Returns (fake oracle result encoding that
    token's RoPE exactly, the GPU's pooled rows (fp32) with element 448 moved by 3e-6 of its
    value, the GPU bytes with RoPE computed in fp64 from those rows, the byte offset of the
    token's RoPE values)."""
    from oracle.compare import bf16_ulp
    wl, orc = case
    t = 5
    res = _fake_result(orc)
    P = (int(wl.positions[t]) // 128) * 128
    C, S = (float(x) for x in wl.cos_sin[P, [0, 32]])
    w = wl.rms_w.astype(np.float64)
    c = res.compressed[t].copy()
    c[449] = c[448] * (w[448] / w[449]) * (C / S) * (1 + 1e-6)
    res.compressed[t] = c

    def rope(cv):
        n = cv / np.sqrt(np.mean(cv * cv) + float(wl.eps)) * w
        x, y = n[448::2], n[449::2]
        cs = wl.cos_sin[P].astype(np.float64)
        z = np.empty(64)
        z[0::2] = x * cs[:32] - y * cs[32:]
        z[1::2] = y * cs[:32] + x * cs[32:]
        return z

    res.normed[t] = c / np.sqrt(np.mean(c * c) + float(wl.eps)) * w
    rec, _ = record_offsets(int(wl.kv_slot_mapping[t]), wl.k_cache.shape[1], wl.k_cache.strides[0])
    z_orc = rope(c)
    res.k_cache_base[rec + 448:rec + 576] = oracle.bf16_bits(z_orc).view(np.uint8)
    gc = res.compressed.astype(np.float32)
    gc[t, 448] *= np.float32(1 + 3e-6)
    z_gpu = rope(gc[t].astype(np.float64))
    body = res.k_cache_base.copy()
    body[rec + 448:rec + 576] = oracle.bf16_bits(z_gpu).view(np.uint8)
    # the planted cancellation really moves the first value by many ulps
    assert abs(z_gpu[0] - z_orc[0]) > 4 * bf16_ulp(np.array([z_orc[0]]))[0]
    return res, gc, body, rec + 448


def test_rope_band_follows_the_gpu_pooled_vector(case):
    """Under cancellation a RoPE value far (in ulps) from the oracle's passes when it is the
    rotation of the GPU's own pooled vector, which is within the compressed tolerance; the
    report counts it and gives the band's use."""
    wl, _ = case
    res, gc, body, _ = _rope_cancel_case(case)
    rep = compare(wl, body, res, gpu_compressed=gc)
    assert rep.ok(), rep.summary()
    assert rep["rope_band"] >= 1 and rep["rope_max_ulp"] > 4
    assert rep["rope_band_basis"] == "gpu pooled vector"
    assert 0.0 <= rep["rope_band_max_use"] <= 1.0
    assert rep["compressed_max_ratio"] <= 1e-5


def test_rope_band_flags_a_value_off_its_own_rotation(case):
    """The same element moved three band widths away from the rotation of the GPU's pooled
    vector fails.  That band (the epilogue's fp32 error around the rotation) is several times
    narrower than the band the compressed tolerance alone would allow."""
    from oracle.compare import rope_band
    wl, _ = case
    res, gc, body, off = _rope_cancel_case(case)
    z, tol = rope_band(wl, res, 5, gc[5])
    _, tol_loose = rope_band(wl, res, 5)
    assert tol[0] < tol_loose[0] / 4
    v = body[off:off + 2].view("<u2")
    v[0] = oracle.bf16_bits(np.array([z[0] + 3 * tol[0]]))[0]
    rep = compare(wl, body, res, gpu_compressed=gc)
    assert not rep.ok()
    assert any("cancellation band" in f for f in rep["failures"])
