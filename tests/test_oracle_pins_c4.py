"""Pins of the CPU oracle's C4 compressor (compress ratio 4 with the overlapping window).

The vLLM "fused_compress_quant_cache" API page's sparse-attention fused kernel is generic in
its compress ratio and overlap: with ratio 4 and overlap 1 a boundary token (pos % 4 == 3)
pools the 8 rows pos-7 .. pos, rows before position 0 take no part, the first 4 window rows
read the first 512-column half of the state row's kv and score parts and the last 4 the
second half, and RoPE uses the table row (pos // 4) * 4.  Each test checks one of these facts
against something other than the oracle's own loop: scipy's softmax over a test-side gather,
a closed form that tells the halves apart, exact means, brute force over the gate, numpy's
complex rotation, and re-blocking the same rows.
"""

import math

import numpy as np
import scipy.special

import oracle
import synth

HALF = 512


def c4_small(T=16, seed=7, k_max=4, state_bs=8, score_std=1.0, kv_bs=4):
    return synth.c4_decode_batch("c4 small", seed, T, T * 4, k_max, 4 * k_max, kv_bs=kv_bs,
                                 kv_blocks=-(-2 * T // kv_bs), cs_rows=4 * k_max + 4,
                                 state_bs=state_bs, score_std=score_std)


def c4_window(wl, t):
    """(kv [n, 512], score [n, 512]) of token t's window rows that exist, in window order,
    each row's half chosen by its place in the window (test-side gather)."""
    pos = int(wl.positions[t])
    req = int(wl.token_to_req[t])
    bs = wl.state.shape[1]
    kv, sc = [], []
    for i in range(8):
        q = pos - 7 + i
        if q < 0:
            continue
        row = wl.state[int(wl.block_table[req, q // bs]), q % bs].astype(np.float64)
        h = HALF if i >= 4 else 0
        kv.append(row[h:h + HALF])
        sc.append(row[1024 + h:1024 + h + HALF])
    return np.stack(kv), np.stack(sc)


def decode_record(kc, slot):
    bs = kc.shape[1]
    blk, off = slot // bs, slot % bs
    flat = np.lib.stride_tricks.as_strided(kc[blk], shape=(kc.strides[0],), strides=(1,))
    return flat[off * 576: off * 576 + 576].copy()


def test_c4_generator_has_first_windows():
    """The small workloads below include tokens at position 3, whose previous window does not
    exist, and tokens at positions >= 7 with both halves."""
    wl = c4_small()
    assert (wl.positions == 3).any() and (wl.positions >= 7).any()


def test_c4_pool_matches_library_softmax():
    wl = c4_small(score_std=0.8)
    r = oracle.run(wl, 2)
    for t in range(wl.num_tokens):
        kv, sc = c4_window(wl, t)
        assert kv.shape[0] == (4 if wl.positions[t] == 3 else 8)
        p = scipy.special.softmax(sc, axis=0)
        np.testing.assert_allclose(r.compressed[t], (p * kv).sum(axis=0), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r.absnorm[t], (p * np.abs(kv)).sum(axis=0), rtol=1e-12)


def test_c4_halves_closed_form():
    """kv = 1 in every first half and 3 in every second half, score 0 in first halves and 1 in
    second halves.  A full window gives (4*1*1 + 4*e*3) / (4 + 4e) = (1 + 3e) / (1 + e); a
    window at position 3 (current rows only) gives 3.  Swapping the kv halves or the score
    halves would give (3 + e) / (1 + e) instead."""
    wl = c4_small(T=12, seed=9)
    st = wl.state
    st[:, :, 0:512] = 1.0
    st[:, :, 512:1024] = 3.0
    st[:, :, 1024:1536] = 0.0
    st[:, :, 1536:2048] = 1.0
    r = oracle.run(wl, 2)
    e = math.e
    for t in range(wl.num_tokens):
        want = 3.0 if wl.positions[t] == 3 else (1 + 3 * e) / (1 + e)
        np.testing.assert_allclose(r.compressed[t], want, rtol=1e-14)


def test_c4_one_hot_selects_each_row_and_half():
    """One window row's score 0 and the others' -1000: the output equals exactly the kv half
    that row contributes, for every row of the window (rows 4..7 only at position 3)."""
    wl = c4_small(T=32, seed=11, k_max=6)
    bs = wl.state.shape[1]
    pick = {}
    for t in range(wl.num_tokens):
        pos = int(wl.positions[t])
        rows = range(4, 8) if pos == 3 else range(8)
        sel = list(rows)[t % len(rows)]
        pick[t] = sel
        for i in rows:
            q = pos - 7 + i
            h = HALF if i >= 4 else 0
            blk = int(wl.block_table[t, q // bs])
            wl.state[blk, q % bs, 1024 + h:1024 + h + HALF] = 0.0 if i == sel else -1000.0
    r = oracle.run(wl, 2)
    for t in range(wl.num_tokens):
        pos, i = int(wl.positions[t]), pick[t]
        q = pos - 7 + i
        h = HALF if i >= 4 else 0
        want = wl.state[int(wl.block_table[t, q // bs]), q % bs, h:h + HALF].astype(np.float64)
        assert np.array_equal(r.compressed[t], want), (t, i)


def test_c4_uniform_scores_give_the_mean():
    wl = c4_small(T=10, seed=13)
    # equal scores down each output column: the same value in both halves
    wl.state[:, :, 1024:2048] = np.float32(0.25) * ((np.arange(1024) % 512) % 5)[None, None, :]
    r = oracle.run(wl, 1)
    for t in range(wl.num_tokens):
        kv, _ = c4_window(wl, t)
        want = np.array([math.fsum(kv[:, j]) / kv.shape[0] for j in range(HALF)])
        np.testing.assert_allclose(r.compressed[t], want, rtol=1e-15, atol=1e-16)


def test_c4_gate_brute_force():
    """Positions 0..255 x state slot in {-1, 0, 5}: exactly the tokens with (pos + 1) % 4 == 0
    and slot >= 0 write their kv slot; every other byte stays 0xAB."""
    pos = np.tile(np.arange(256), 3).astype(np.int32)
    slot = np.repeat(np.array([-1, 0, 5], np.int32), 256)
    T = pos.size
    base, state = synth.alloc_state(32, row_width=synth.C4_ROW)
    synth.fill_state(state, 5, 1.0, 1.0, width=1024)
    bt = synth.permutation(32, 5, 2).astype(np.int32).reshape(1, 32)
    kc_base, kc = synth.alloc_k_cache(T // 16, 16)
    wl = synth.Workload("c4 gate", state, bt, np.zeros(T, np.int32), pos, slot,
                        np.ones(512, np.float32), 1e-6, synth.rope_table(256), kc,
                        np.arange(T, dtype=np.int32), 5, base, kc_base, compress_ratio=4,
                        overlap=1)
    r = oracle.run(wl, 4)
    active = ((pos + 1) % 4 == 0) & (slot >= 0)
    assert active.sum() == 128
    assert np.array_equal(r.status == oracle.STATUS_WRITTEN, active)
    assert np.array_equal(r.status == oracle.STATUS_INACTIVE, ~active)
    per_slot = r.k_cache_base.reshape(T // 16, 16 * 584)
    for t in range(T):
        b, o = t // 16, t % 16
        touched = (np.any(per_slot[b, o * 576:(o + 1) * 576] != 0xAB) or
                   np.any(per_slot[b, 16 * 576 + o * 8:16 * 576 + o * 8 + 8] != 0xAB))
        assert touched == active[t], t


def test_c4_rope_row_and_rotation():
    """(x' + i y') = (x + i y) * exp(i P theta_m) with P = (pos // 4) * 4, theta_m =
    10000^(-2m/64), from numpy's complex exp (not the table), within one bf16 step; at
    position 3 (P = 0) the rotation is the identity."""
    wl = c4_small(T=16, seed=17, k_max=40)
    wl.cos_sin = synth.rope_table(4 * 40 + 4)
    r = oracle.run(wl, 2)
    theta = 10000.0 ** (-2.0 * np.arange(32) / 64)
    step = lambda v: np.exp2(np.floor(np.log2(np.abs(v) + 1e-300)) - 7)  # noqa: E731
    for t in range(wl.num_tokens):
        P = (int(wl.positions[t]) // 4) * 4
        n = r.normed[t]
        z = (n[448::2] + 1j * n[449::2]) * np.exp(1j * P * theta)
        rec = decode_record(r.k_cache, int(wl.kv_slot_mapping[t]))
        got = ((rec[448:576].view("<u2").astype(np.uint32) << 16).view(np.float32)
               .astype(np.float64))
        if P == 0:
            assert np.array_equal(rec[448:576].view("<u2"), oracle.bf16_bits(n[448:512]))
        assert np.all(np.abs(got[0::2] - z.real) <= step(z.real) + 1e-6 * np.abs(z))
        assert np.all(np.abs(got[1::2] - z.imag) <= step(z.imag) + 1e-6 * np.abs(z))


def test_c4_state_block_size_relayout_invariance():
    """The same logical rows in 4-row blocks (each 8-row block cut in two, table doubled) and in
    16-row blocks (pairs glued, table halved) give identical k_cache bytes."""
    wl = c4_small(T=12, seed=19, k_max=8)
    r0 = oracle.run(wl, 1)
    T, cols = wl.block_table.shape
    # 4-row blocks
    st4 = np.zeros((wl.state.shape[0] * 2, 4, synth.C4_ROW), np.float32)
    st4[0::2] = wl.state[:, :4]
    st4[1::2] = wl.state[:, 4:]
    bt4 = np.zeros((T, cols * 2), np.int32)
    bt4[:, 0::2] = 2 * wl.block_table
    bt4[:, 1::2] = 2 * wl.block_table + 1
    # 16-row blocks
    st16 = np.zeros((T * cols // 2, 16, synth.C4_ROW), np.float32)
    bt16 = np.zeros((T, cols // 2), np.int32)
    nb = 0
    for r_ in range(T):
        for m in range(cols // 2):
            st16[nb, :8] = wl.state[wl.block_table[r_, 2 * m]]
            st16[nb, 8:] = wl.state[wl.block_table[r_, 2 * m + 1]]
            bt16[r_, m] = nb
            nb += 1
    for st, bt in ((st4, bt4), (st16, bt16)):
        wl2 = c4_small(T=12, seed=19, k_max=8)
        wl2.state, wl2.block_table = st, bt
        r1 = oracle.run(wl2, 1)
        assert np.array_equal(r0.k_cache_base, r1.k_cache_base)
