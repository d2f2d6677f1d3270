"""Pins of the CPU oracle's indexer compressor (FP8 cache, head 128).

The vLLM "fused_compress_quant_cache" API page's indexer kernel pools a head of 128 over the
compressor's window (here the 8-row overlapping window of ratio 4), applies RMSNorm, rotates
dims 64..127 as GPT-J pairs by the table row (pos // 4) * 4, and only then quantises all 128
dims as one block: bf16 round trip, absmax with a 1e-4 floor, scale 2^ceil(log2(absmax/448))
stored as one fp32, E4M3 codes.  A block holds bs records of 128 bytes, then bs fp32 scales.
Each test checks one step against something other than the oracle's own loop: scipy's softmax,
closed forms, numpy's complex rotation, quantisation invariants, a case where rotating before
or after quantising gives different scales, brute force over the gate, two-fill byte offsets.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

H = 128


def idx_small(T=16, seed=7, k_max=4, state_bs=8, score_std=1.0, kv_bs=4, **kw):
    return synth.indexer_decode_batch("indexer small", seed, T, T * 4, k_max, 4 * k_max,
                                      kv_bs=kv_bs, kv_blocks=kw.pop("kv_blocks", -(-2 * T // kv_bs)),
                                      cs_rows=kw.pop("cs_rows", 4 * k_max + 4), state_bs=state_bs,
                                      score_std=score_std, **kw)


def window(wl, t):
    """(kv [n, 128], score [n, 128]) of token t's existing window rows, halves chosen by the
    row's place in the window (test-side gather)."""
    pos, req, bs = int(wl.positions[t]), int(wl.token_to_req[t]), wl.state.shape[1]
    kv, sc = [], []
    for i in range(8):
        q = pos - 7 + i
        if q < 0:
            continue
        row = wl.state[int(wl.block_table[req, q // bs]), q % bs].astype(np.float64)
        h = H if i >= 4 else 0
        kv.append(row[h:h + H])
        sc.append(row[2 * H + h:2 * H + h + H])
    return np.stack(kv), np.stack(sc)


def record(wl, kc_base, t):
    """(128 code bytes, fp32 scale) of token t's kv slot."""
    bs = wl.k_cache.shape[1]
    stride0 = wl.k_cache.strides[0]
    s = int(wl.kv_slot_mapping[t])
    blk, off = s // bs, s % bs
    codes = kc_base[blk * stride0 + off * 128: blk * stride0 + off * 128 + 128]
    scale = kc_base[blk * stride0 + bs * 128 + off * 4: blk * stride0 + bs * 128 + off * 4 + 4]
    return codes.copy(), float(scale.view("<f4")[0])


def e4m3_lut():
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v


def test_indexer_pool_matches_library_softmax():
    wl = idx_small(score_std=0.8)
    assert (wl.positions == 3).any()
    r = oracle.run(wl, 2)
    for t in range(wl.num_tokens):
        kv, sc = window(wl, t)
        p = scipy.special.softmax(sc, axis=0)
        np.testing.assert_allclose(r.compressed[t], (p * kv).sum(axis=0), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r.absnorm[t], (p * np.abs(kv)).sum(axis=0), rtol=1e-12)


def test_indexer_rmsnorm_closed_form_survives_rotation():
    """w = 1, eps = 0: mean(n^2) = 1 over the 128 dims.  RoPE keeps every pair's norm up to the
    fp32 rounding of the table (cos^2 + sin^2 = 1 within 2^-22), exactly at table row 0 (cos 1,
    sin 0, position 3), so the quantised values keep it too; the nope half is c scaled by one
    constant."""
    wl = idx_small(T=12, seed=9)
    wl.rms_w[:] = 1.0
    wl.eps = 0.0
    r = oracle.run(wl, 1)
    assert (wl.positions == 3).any() and (wl.positions > 3).any()
    for t in range(wl.num_tokens):
        tol = 1e-14 if wl.positions[t] == 3 else 2.0 ** -21
        assert abs(np.mean(r.normed[t] ** 2) - 1.0) < tol
        ratio = r.normed[t][:64] / r.compressed[t][:64]
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-14)


def test_indexer_rope_against_complex_multiply():
    """Dims 64..127 of the quantised values equal (x + iy) * exp(i P theta_m) of the normalised
    pairs, P = (pos // 4) * 4, theta_m = 10000^(-2m/64) from numpy's complex exp (not the
    table); dims 0..63 are the normalised values unchanged."""
    wl = idx_small(T=12, seed=11, k_max=60, cs_rows=4 * 60 + 4)
    r = oracle.run(wl, 2)
    theta = 10000.0 ** (-2.0 * np.arange(32) / 64)
    w = wl.rms_w.astype(np.float64)
    for t in range(wl.num_tokens):
        c = r.compressed[t]
        n = c / np.sqrt(np.mean(c * c) + wl.eps) * w
        P = (int(wl.positions[t]) // 4) * 4
        z = (n[64::2] + 1j * n[65::2]) * np.exp(1j * P * theta)
        got = r.normed[t]
        np.testing.assert_allclose(got[:64], n[:64], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(got[64::2], z.real, rtol=0, atol=1e-6 * np.abs(z).max())
        np.testing.assert_allclose(got[65::2], z.imag, rtol=0, atol=1e-6 * np.abs(z).max())


def test_indexer_quant_invariants():
    """The scale is an exact power of two 2^e (as fp32); absmax/scale in (224, 448] over the
    bf16-rounded rotated values; every code decodes to within half an E4M3 step of
    bf16(x)/scale (torch's float8_e4m3fn decoding of the bytes)."""
    wl = idx_small(T=16, seed=13, k_max=30, cs_rows=124)
    r = oracle.run(wl, 2)
    lut = e4m3_lut()
    for t in range(wl.num_tokens):
        codes, scale = record(wl, r.k_cache_base, t)
        m, e = math.frexp(scale)
        assert m == 0.5
        e -= 1
        x32 = r.normed[t].astype(np.float32)
        u = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
        A = max(np.abs(u).max(), float(np.float32(1e-4)))
        assert 224 < A / scale <= 448
        x = u / scale
        ex = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6)))
        assert np.all(np.abs(lut[codes] - x) <= np.exp2(ex - 3) / 2)


def test_indexer_rotates_before_quantising():
    """One-hot scores make the pooled vector a chosen kv row: dim 64 large, dim 65 zero, the
    rest small.  At P = 4 the pair rotates by 4 rad, so the largest magnitude shrinks from
    |n_64| to |n_64 sin 4| ~ 0.757 |n_64|.  With w_64 chosen so that |n_64| / 448 = 1.1, the
    scale from the rotated values is 2^0 = 1; quantising before rotating would give 2^1."""
    wl = idx_small(T=1, seed=17, k_max=2, cs_rows=16)
    wl.positions[:] = 7                       # window rows 0..7, P = 4
    t, bs = 0, wl.state.shape[1]
    for i in range(8):
        blk = int(wl.block_table[0, i // bs])
        h = H if i >= 4 else 0
        wl.state[blk, i % bs, 2 * H + h:2 * H + h + H] = 0.0 if i == 5 else -1000.0
    v = np.full(H, 0.01)
    v[64], v[65] = 1.0, 0.0
    blk = int(wl.block_table[0, 5 // bs])
    wl.state[blk, 5 % bs, H:2 * H] = v.astype(np.float32)
    wl.eps = 0.0
    vf = v.astype(np.float32).astype(np.float64)
    rms = math.sqrt(np.mean(vf * vf))
    wl.rms_w[:] = 1.0
    wl.rms_w[64] = np.float32(448 * 1.1 * rms)
    r = oracle.run(wl, 1)
    n64 = 1.0 / rms * float(wl.rms_w[64])
    assert abs(n64 / 448 - 1.1) < 1e-6
    # the table holds cos/sin rounded to fp32: relative error below 1e-7
    assert abs(abs(r.normed[t][64]) - abs(n64 * math.cos(4.0))) < 1e-6 * n64
    assert abs(abs(r.normed[t][65]) - abs(n64 * math.sin(4.0))) < 1e-6 * n64
    _, scale = record(wl, r.k_cache_base, t)
    assert scale == 1.0


def test_indexer_gate_brute_force():
    pos = np.tile(np.arange(128), 3).astype(np.int32)
    slot = np.repeat(np.array([-1, 0, 5], np.int32), 128)
    T = pos.size
    base, state = synth.alloc_state(16, row_width=synth.INDEXER_ROW)
    synth.fill_state(state, 5, 1.0, 1.0, width=2 * H)
    bt = synth.permutation(16, 5, 2).astype(np.int32).reshape(1, 16)
    kc_base, kc = synth.alloc_indexer_cache(T // 16, 16)
    wl = synth.Workload("indexer gate", state, bt, np.zeros(T, np.int32), pos, slot,
                        np.ones(H, np.float32), 1e-6, synth.rope_table(128), kc,
                        np.arange(T, dtype=np.int32), 5, base, kc_base, compress_ratio=4,
                        overlap=1, indexer=True)
    r = oracle.run(wl, 4)
    active = ((pos + 1) % 4 == 0) & (slot >= 0)
    assert active.sum() == 64
    assert np.array_equal(r.status == oracle.STATUS_WRITTEN, active)
    per_blk = r.k_cache_base.reshape(T // 16, 16 * 132)
    for t in range(T):
        b, o = t // 16, t % 16
        touched = (np.any(per_blk[b, o * 128:(o + 1) * 128] != 0xAB) or
                   np.any(per_blk[b, 16 * 128 + o * 4:16 * 128 + o * 4 + 4] != 0xAB))
        assert touched == active[t], t


@pytest.mark.parametrize("bs,pad", [(1, 0), (2, 20), (64, 0), (64, 12)])
def test_indexer_insert_byte_offsets(bs, pad):
    """Two runs with different prefill bytes: the bytes equal in both are exactly those written,
    at blk*stride0 + off*128 (128 bytes) and blk*stride0 + bs*128 + off*4 (4 bytes)."""
    outs = []
    for fill in (0xAB, 0x54):
        wl = idx_small(T=5, kv_bs=bs, kv_blocks=-(-12 // bs) + 1, kc_block_pad=pad, seed=51)
        wl.k_cache_base[:] = fill
        outs.append(oracle.run(wl, 1).k_cache_base)
    written = outs[0] == outs[1]
    expect = np.zeros_like(written)
    stride0 = bs * 132 + pad
    for t in range(5):
        s = int(wl.kv_slot_mapping[t])
        blk, off = s // bs, s % bs
        expect[blk * stride0 + off * 128: blk * stride0 + off * 128 + 128] = True
        expect[blk * stride0 + bs * 128 + off * 4: blk * stride0 + bs * 128 + off * 4 + 4] = True
    assert np.array_equal(written, expect)
