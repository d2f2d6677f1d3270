"""Pins of the CPU oracle's MXFP4 indexer cache (head 128).

The vLLM "fused_compress_quant_cache" API page's MXFP4 indexer kernel pools, normalises and
rotates a head of 128 as the FP8 indexer kernel does, rounds every rotated value through bf16,
and quantises four blocks of 32 consecutive dims: scale 2^ceil(log2(absmax / 6)) stored as a
UE8M0 byte, E2M1 codes packed two a byte, the even dim in the low nibble.  A cache block holds
bs records of 64 bytes, then bs x 4 scale bytes.  Each test ties one step to something other
than the oracle's own code: the OCP table of E2M1 values (golden fixture), a brute-force
nearest-code search, exact rational exponents, hand-derived records, dequantisation bounds
against torch's bf16 rounding, and two-fill byte offsets.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

H = 128
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fp4_small(T=16, seed=7, k_max=4, state_bs=8, score_std=1.0, kv_bs=4, **kw):
    return synth.indexer_decode_batch("mxfp4 small", seed, T, T * 4, k_max, 4 * k_max,
                                      kv_bs=kv_bs, kv_blocks=kw.pop("kv_blocks", -(-2 * T // kv_bs)),
                                      cs_rows=kw.pop("cs_rows", 4 * k_max + 4), state_bs=state_bs,
                                      score_std=score_std, fp4=True, **kw)


def record(wl, kc_base, t):
    """(128 codes unpacked low nibble first, 4 scale bytes) of token t's kv slot."""
    bs = wl.k_cache.shape[1]
    stride0 = wl.k_cache.strides[0]
    s = int(wl.kv_slot_mapping[t])
    blk, off = s // bs, s % bs
    b = kc_base[blk * stride0 + off * 64: blk * stride0 + off * 64 + 64]
    codes = np.empty(128, np.uint8)
    codes[0::2], codes[1::2] = b & 0xF, b >> 4
    scl = kc_base[blk * stride0 + bs * 64 + off * 4: blk * stride0 + bs * 64 + off * 4 + 4]
    return codes, scl.copy(), b.copy()


def ocp_table():
    """{code: value} from the golden fixture."""
    table = {}
    for line in open(os.path.join(GOLDEN, "e2m1_ocp_points.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        val, code = line.split()
        v = -0.0 if val == "-0" else float(Fraction(val))
        table[int(code, 16)] = v
    assert sorted(table) == list(range(16))
    return table


def all_bf16_finite():
    bits = np.arange(0x10000, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    ok = np.isfinite(vals)
    return bits[ok], vals[ok].astype(np.float64)


def test_e2m1_ocp_table():
    """Every one of the 16 codes decodes to the specification's value, and each value
    encodes back to its code (-0 to 0x8)."""
    for code, v in ocp_table().items():
        got = oracle.e2m1_value(code)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (code, got, v)
        assert int(oracle.e2m1_codes([v])[0]) == code, (v, code)


def test_e2m1_exhaustive_against_nearest_code_search():
    """Every value the quantiser can see (all bf16 values with |x| <= 16; a bf16 value times a
    power of two is again bf16; beyond 6 the nearest value is 6, the saturation) encodes to
    the nearest value of the OCP table, ties to the even code, sign kept (brute force)."""
    table = ocp_table()
    pcodes = np.array([c for c in range(8)])
    pvals = np.array([table[c] for c in range(8)])
    _, vals = all_bf16_finite()
    vals = vals[np.abs(vals) <= 16.0]
    # the E2M1 rounding midpoints themselves are bf16 values: ties are exercised
    assert all(np.any(vals == m) for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0))
    ours = oracle.e2m1_codes(vals)
    d = np.abs(np.abs(vals)[:, None] - pvals[None, :])  # exact: all values are dyadic
    dmin = d.min(axis=1, keepdims=True)
    tie_pick = np.where(d == dmin, (pcodes[None, :] & 1) * 100 + pcodes[None, :], 10 ** 6)
    want = pcodes[np.argmin(tie_pick, axis=1)].astype(np.uint8)
    want = want | np.where(np.signbit(vals), 0x8, 0).astype(np.uint8)
    assert np.array_equal(ours, want)


def test_mxfp4_exponent_exact_for_every_bf16_absmax():
    """For every positive finite bf16 absmax (and 0): the exponent from the fp32 product
    absmax * fl32(1/6) equals the exact smallest e with max(absmax, 6 * 2^-126) <= 6 * 2^e
    (exact rationals), so max(absmax, floor) / 2^e lies in (3, 6]: no E2M1 code saturates.
    A zero block gets e = -126 (scale byte 1)."""
    _, vals = all_bf16_finite()
    vals = np.concatenate([[0.0], vals[vals > 0]])
    got = oracle.mxfp4_exponents(vals)
    floor_ = Fraction(6) * Fraction(2) ** -126
    for A, e in zip(vals, got):
        a = max(Fraction(float(A)), floor_)
        k = math.floor(math.log2(a / 6)) - 2
        while a / 6 > Fraction(2) ** k:
            k += 1
        assert int(e) == k, (A, e, k)
        assert Fraction(3) < a / Fraction(2) ** k <= Fraction(6)
    assert int(oracle.mxfp4_exponents([0.0])[0]) == -126


def one_token(v, pos=3, seed=21):
    """One token whose pooled vector is exactly v: uniform scores over the window's rows and
    every existing row's kv equal to v (position 3: only the current window's 4 rows, table
    row 0, so RoPE is the identity: cos 0 = 1, sin 0 = 0 exactly)."""
    wl = fp4_small(T=1, seed=seed, k_max=2, cs_rows=16)
    wl.positions[:] = pos
    bs = wl.state.shape[1]
    for i in range(8):
        q = pos - 7 + i
        if q < 0:
            continue
        blk = int(wl.block_table[0, q // bs])
        h = H if i >= 4 else 0
        wl.state[blk, q % bs, 2 * H + h:2 * H + h + H] = 0.5
        wl.state[blk, q % bs, h:h + H] = np.asarray(v, np.float32)
    wl.rms_w[:] = 1.0
    wl.eps = 0.0
    return wl


@pytest.mark.parametrize("j0,sign", [(0, 1), (1, 1), (37, -1), (64, 1), (127, -1)])
def test_mxfp4_one_hot_record(j0, sign):
    """Pooled vector sign * e_j0, w = 1, eps = 0: n_j0 = sign * sqrt(128) = 11.3137..., whose
    bf16 value is 11.3125; its block's exponent is ceil(log2(11.3125 / 6)) = 1 (byte 128) and
    11.3125 / 2 = 5.65625 > 5 rounds to 6 (code 7).  Every other dim is 0: code 0, and the
    three other blocks are all-zero blocks (byte 1).  So byte j0 // 2 holds 7 (or 0xF when
    negative) in the low nibble for even j0, the high nibble for odd j0, and every other byte
    is 0."""
    v = np.zeros(H)
    v[j0] = sign
    wl = one_token(v)
    r = oracle.run(wl, 1)
    assert r.status[0] == oracle.STATUS_WRITTEN
    _, scl, raw = record(wl, r.k_cache_base, 0)
    want_scl = np.ones(4, np.uint8)
    want_scl[j0 // 32] = 128
    assert np.array_equal(scl, want_scl)
    want = np.zeros(64, np.uint8)
    code = 0x7 | (0x8 if sign < 0 else 0)
    want[j0 // 2] = code << (4 * (j0 & 1))
    assert np.array_equal(raw, want)


def test_mxfp4_zero_window_record():
    """An all-zero pooled vector (eps > 0): every code 0, every block an all-zero block whose
    exponent is -126 (byte 1)."""
    wl = one_token(np.zeros(H))
    wl.eps = 1e-6
    r = oracle.run(wl, 1)
    _, scl, raw = record(wl, r.k_cache_base, 0)
    assert np.array_equal(raw, np.zeros(64, np.uint8))
    assert np.array_equal(scl, np.ones(4, np.uint8))


def test_mxfp4_dequantised_within_half_a_step():
    """Random windows at positions with P > 0 (RoPE active): per block, the scale byte b gives
    2^(b-127), the block's largest bf16 rotated value over the scale lies in (3, 6], and every
    code decodes (OCP table) to within half an E2M1 step of bf16(x) / scale, x the rotated
    value held in fp32 and rounded to bf16 by torch.  The rotated values are the FP8 indexer's
    on the same inputs: only the cache format differs."""
    wl = fp4_small(T=16, seed=13, k_max=30, cs_rows=124)
    assert (wl.positions > 3).sum() >= 12
    r = oracle.run(wl, 2)
    table = ocp_table()
    lut = np.array([table[c] for c in range(16)])
    fp8 = synth.indexer_decode_batch("fp8 twin", 13, 16, 64, 30, 120, kv_bs=4, kv_blocks=8,
                                     cs_rows=124, state_bs=8, score_std=1.0)
    r8 = oracle.run(fp8, 2)
    np.testing.assert_array_equal(r.normed, r8.normed)
    for t in range(wl.num_tokens):
        codes, scl, _ = record(wl, r.k_cache_base, t)
        x32 = r.normed[t].astype(np.float32)
        u = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
        for g in range(4):
            sl = slice(32 * g, 32 * g + 32)
            scale = 2.0 ** (int(scl[g]) - 127)
            assert 3 < np.abs(u[sl]).max() / scale <= 6
            y = u[sl] / scale
            step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
            assert np.all(np.abs(lut[codes[sl]] - y) <= step / 2), (t, g)


@pytest.mark.parametrize("bs,pad", [(1, 0), (2, 20), (64, 0), (64, 12)])
def test_mxfp4_insert_byte_offsets(bs, pad):
    """Two runs with different prefill bytes: the bytes equal in both are exactly those written,
    at blk*stride0 + off*64 (64 bytes) and blk*stride0 + bs*64 + off*4 (4 bytes)."""
    outs = []
    for fill in (0xAB, 0x54):
        wl = fp4_small(T=5, kv_bs=bs, kv_blocks=-(-12 // bs) + 1, kc_block_pad=pad, seed=51)
        wl.k_cache_base[:] = fill
        outs.append(oracle.run(wl, 1).k_cache_base)
    written = outs[0] == outs[1]
    expect = np.zeros_like(written)
    stride0 = bs * 68 + pad
    for t in range(5):
        s = int(wl.kv_slot_mapping[t])
        blk, off = s // bs, s % bs
        expect[blk * stride0 + off * 64: blk * stride0 + off * 64 + 64] = True
        expect[blk * stride0 + bs * 64 + off * 4: blk * stride0 + bs * 64 + off * 4 + 4] = True
    assert np.array_equal(written, expect)
