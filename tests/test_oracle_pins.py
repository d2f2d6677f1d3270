"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks one oracle step against something other than the oracle's
own formula: a library routine (torch's bf16 cast, scipy's softmax), exact
rational arithmetic (fractions / decimal), a brute-force search, a closed
form, an invariant, or a hand-derived golden record.  A plausible slip in the
oracle (a dropped term, a wrong sign or index, a transposed operand) fails at
least one of them.
"""

import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def small_decode(T=4, n_blocks=None, k_max=4, kv_bs=4, seed=77, score_std=1.0, **kw):
    n_blocks = n_blocks or 16 * T
    kv_blocks = kw.pop("kv_blocks", -(-2 * T // kv_bs))
    return synth.decode_batch("small", seed, T, n_blocks, k_max, 16 * k_max, kv_bs=kv_bs,
                              kv_blocks=kv_blocks, cs_rows=128 * k_max, score_std=score_std, **kw)


def window_rows(wl, t):
    """[128, W] fp32 rows of token t's window, in window order (test-side gather)."""
    pos = int(wl.positions[t])
    req = int(wl.token_to_req[t])
    rows = []
    for q in range(pos - 127, pos + 1):
        blk = int(wl.block_table[req, q // 8])
        rows.append(wl.state[blk, q % 8])
    return np.stack(rows)


def decode_record(kc, slot):
    """(codes[448], scale bytes[8], rope bf16 bits[64]) of kv slot `slot`."""
    bs = kc.shape[1]
    blk, off = slot // bs, slot % bs
    flat = np.lib.stride_tricks.as_strided(kc[blk], shape=(kc.strides[0],), strides=(1,))
    rec = flat[off * 576: off * 576 + 576]
    sc = flat[bs * 576 + off * 8: bs * 576 + off * 8 + 8]
    codes = rec[:448].copy()
    rope = rec[448:576].copy().view("<u2")
    return codes, sc.copy(), rope


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def all_bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return b[np.isfinite(f)].astype(np.uint16), f[np.isfinite(f)].astype(np.float64)


# ---------------------------------------------------------------- number formats

def test_bf16_matches_torch_cast_on_structured_fp32():
    """fp32 -> bf16 RNE equals torch's CPU cast (library routine) on every high half-word
    combined with tie, near-tie and random low half-words."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    rnd = synth.bits(1 << 16, 5, 1).astype(np.uint32) & 0xFFFF
    pats = np.concatenate([(hi[:, None] | lows[None, :]).ravel(), hi | rnd])
    f = pats.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]  # keep the rounding inside the finite range
    ours = oracle.bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_of_double_is_single_rounding_by_exact_arithmetic():
    """A double is rounded once to bf16: brute force over the two bracketing bf16 values with
    exact rational distances, ties to the even pattern."""
    rng_vals = synth.normal(4000, 9, 1).astype(np.float64) * np.exp2(
        synth.randint(4000, -30, 30, 9, 2).astype(np.float64))
    perturb = synth.uniform(4000, 9, 3) * 2 ** -20
    xs = list(rng_vals * (1 + perturb))
    # exact ties and near ties in double precision
    for b in (0x3F80, 0x3F81, 0x4123, 0xC0FF, 0x0081, 0x0001):
        lo = float(bf16_to_f64([b])[0])
        nxt = float(bf16_to_f64([b + 1])[0])
        mid = (lo + nxt) / 2
        xs += [mid, math.nextafter(mid, math.inf), math.nextafter(mid, -math.inf)]
    xs = np.array(xs)
    ours = oracle.bf16_bits(xs)
    _, grid = all_bf16_finite()
    pos = np.sort(np.unique(np.abs(grid)))
    for x, got in zip(xs, ours):
        a = Fraction(abs(float(x)))
        i = np.searchsorted(pos, abs(x))
        cands = [pos[max(i - 1, 0)], pos[min(i, len(pos) - 1)]]
        best = None
        for c in cands:
            d = abs(Fraction(float(c)) - a)
            bits = int(np.float32(c).view(np.uint32) >> 16)
            key = (d, bits & 1)
            if best is None or key < best[0]:
                best = (key, bits)
        want = best[1] | (0x8000 if x < 0 else 0)
        assert int(got) == want, (x, hex(int(got)), hex(want))


def _e4m3_table():
    """Values of the 254 finite E4M3FN codes from the format definition (OCP OFP8:
    bias 7, subnormals m*2^-9, S.1111.111 is NaN)."""
    codes = np.arange(256, dtype=np.int64)
    s = codes >> 7
    e = (codes >> 3) & 15
    m = codes & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -val, val)
    finite = (codes & 0x7F) != 0x7F
    return codes[finite], val[finite]


def test_e4m3_exhaustive_against_nearest_code_search():
    """Every value the quantiser can see (all bf16 values with |x| <= 448: a bf16 value times
    a power of two is again bf16) encodes to the nearest finite E4M3FN code, ties to the even
    code, sign kept (brute force over all codes)."""
    _, vals = all_bf16_finite()
    vals = vals[np.abs(vals) <= 448.0]
    ours = oracle.e4m3_codes(vals)
    codes, table = _e4m3_table()
    pos = table >= 0
    pcodes, ptable = codes[pos & (codes < 128)], table[pos & (codes < 128)]
    a = np.abs(vals)
    d = np.abs(a[:, None] - ptable[None, :])  # exact: all values are dyadic
    dmin = d.min(axis=1, keepdims=True)
    tie_pick = np.where(d == dmin, (pcodes[None, :] & 1) * 1000 + pcodes[None, :], 10 ** 9)
    want = pcodes[np.argmin(tie_pick, axis=1)].astype(np.uint8)
    want = want | np.where(np.signbit(vals), 0x80, 0).astype(np.uint8)
    assert np.array_equal(ours, want)


def test_e4m3_ocp_reference_points():
    """Encodings fixed by the OCP 8-bit floating point specification (golden fixture)."""
    path = os.path.join(GOLDEN, "e4m3_ocp_points.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        val, code = line.split()
        x = float(Fraction(val))
        assert int(oracle.e4m3_codes([x])[0]) == int(code, 16), line
        assert oracle.e4m3_value(int(code, 16)) == x, line
        n += 1
    assert n >= 10


def test_ue8m0_exponent_exact_for_every_bf16_absmax():
    """For every positive finite bf16 absmax (and 0): the exponent from the fp32 product
    absmax*fl32(1/448) equals the exact smallest e with max(absmax, 1e-4) <= 448*2^e
    (exact rationals), and max(absmax, floor)/2^e lies in (224, 448]."""
    _, vals = all_bf16_finite()
    vals = np.concatenate([[0.0], vals[vals > 0]])
    got = oracle.ue8m0_exponents(vals)
    floor_ = Fraction(float(np.float32(1e-4)))
    for A, e in zip(vals, got):
        a = max(Fraction(float(A)), floor_)
        # smallest integer e with a/448 <= 2^e
        k = math.floor(math.log2(a / 448)) - 2
        while a / 448 > Fraction(2) ** k:
            k += 1
        assert int(e) == k, (A, e, k)
        q = a / Fraction(2) ** k
        assert Fraction(224) < q <= Fraction(448)
    assert int(oracle.ue8m0_exponents([0.0])[0]) == -22  # zero block: byte 105


# ---------------------------------------------------------------- pooling

def test_pool_matches_library_softmax_on_tiny_window():
    """compressed_j = sum_i softmax_i(score_ij) kv_ij with scipy's softmax and a numpy
    weighted sum (library routines), on a small-range window."""
    wl = small_decode(T=3, score_std=0.7)
    r = oracle.run(wl, 1)
    for t in range(3):
        rows = window_rows(wl, t).astype(np.float64)
        p = scipy.special.softmax(rows[:, 512:1024], axis=0)
        want = (p * rows[:, :512]).sum(axis=0)
        np.testing.assert_allclose(r.compressed[t], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r.absnorm[t], (p * np.abs(rows[:, :512])).sum(axis=0),
                                   rtol=1e-12)


def test_pool_against_high_precision_decimal():
    """Three columns recomputed with 40-digit decimal arithmetic (exact result to far below
    fp64): the oracle agrees to 1e-14 relative in the convex-combination norm."""
    wl = small_decode(T=1, score_std=3.0)
    r = oracle.run(wl, 1)
    rows = window_rows(wl, 0)
    getcontext().prec = 40
    for j in (0, 257, 511):
        s = [Decimal(float(v)) for v in rows[:, 512 + j]]
        kv = [Decimal(float(v)) for v in rows[:, j]]
        w = [x.exp() for x in s]
        num = sum(wi * ki for wi, ki in zip(w, kv))
        den = sum(w)
        want = float(num / den)
        scale = float(sum(wi * abs(ki) for wi, ki in zip(w, kv)) / den)
        assert abs(r.compressed[0, j] - want) <= 1e-14 * scale


def test_pool_uniform_scores_give_the_mean():
    """Equal scores in a column: softmax is 1/128, the output is the plain mean of kv."""
    wl = small_decode(T=2)
    for b in range(wl.state.shape[0]):
        wl.state[b, :, 512:1024] = np.float32(0.375) * (np.arange(512) % 7)[None, :]
    r = oracle.run(wl, 1)
    for t in range(2):
        rows = window_rows(wl, t).astype(np.float64)
        want = np.array([math.fsum(rows[:, j]) / 128 for j in range(512)])
        np.testing.assert_allclose(r.compressed[t], want, rtol=1e-15, atol=1e-16)


@pytest.mark.parametrize("seed", [3, 4])
def test_one_hot_scores_select_each_window_row(seed):
    """One row's score 0 and all others -1000 (their weight underflows to exactly 0): the
    output equals kv of logical window row i, for every i < 128, whatever physical block
    the block table puts it in."""
    T = 128
    wl = small_decode(T=T, n_blocks=16 * T, k_max=3, kv_bs=16, seed=seed)
    # token t selects window row t
    for t in range(T):
        pos = int(wl.positions[t])
        for i in range(128):
            q = pos - 127 + i
            blk = int(wl.block_table[t, q // 8])
            wl.state[blk, q % 8, 512:1024] = 0.0 if i == t else -1000.0
    r = oracle.run(wl, 4)
    for t in range(T):
        pos = int(wl.positions[t])
        q = pos - 127 + t
        want = wl.state[int(wl.block_table[t, q // 8]), q % 8, :512].astype(np.float64)
        assert np.array_equal(r.compressed[t], want), t


def test_shift_invariance_of_the_pool():
    """Adding a per-column integer to every score of that column leaves the output unchanged
    (scores on a 2^-10 grid so the shifted fp32 inputs are exact)."""
    wl = small_decode(T=2)
    st = wl.state
    st[:, :, 512:1024] = np.round(st[:, :, 512:1024] * 1024) / 1024
    r0 = oracle.run(wl, 1)
    shift = (synth.randint(512, -20, 20, 5, 7)).astype(np.float32)
    st[:, :, 512:1024] += shift[None, None, :]
    r1 = oracle.run(wl, 1)
    np.testing.assert_allclose(r1.compressed, r0.compressed, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- addressing

def test_pool_is_a_convex_combination_of_the_window():
    """Every pooled value lies between the smallest and the largest kv value of its column over
    the window's 128 rows (the softmax weights are positive and sum to one), with score spreads
    from near-uniform (std 0.01) to near one-hot (std 100)."""
    for seed, std in ((31, 0.01), (32, 1.0), (33, 100.0)):
        wl = small_decode(T=3, seed=seed, score_std=std)
        r = oracle.run(wl, 1)
        for t in range(wl.num_tokens):
            assert r.status[t] == 1
            kv = window_rows(wl, t)[:, :512].astype(np.float64)
            lo, hi = kv.min(0), kv.max(0)
            slack = 1e-12 * np.maximum(np.abs(lo), np.abs(hi))
            c = r.compressed[t]
            assert np.all(c >= lo - slack) and np.all(c <= hi + slack)
            assert np.any(c > lo + 1e-6) and np.any(c < hi - 1e-6)  # not a corner row


def test_record_invariant_under_power_of_two_kv_scaling():
    """With eps = 0, multiplying every kv value by 2^k multiplies the pooled values by exactly
    2^k, and RMSNorm divides it out again (every step is exact under power-of-two scaling): the
    records are byte-identical for k from -20 to 20."""
    def run(k):
        wl = small_decode(T=4, seed=41)
        wl.eps = 0.0
        wl.state[:, :, :512] *= np.float32(2.0 ** k)
        return oracle.run(wl, 1)
    base = run(0)
    assert (base.status == 1).all()
    for k in (-20, -3, 1, 7, 20):
        assert np.array_equal(run(k).k_cache_base, base.k_cache_base), k


def test_pool_invariant_under_permuting_window_rows():
    """Moving whole state rows (kv with its score) to other places inside a token's own window
    blocks leaves every record unchanged: the pooling is a sum over the window's rows, in any
    order (fp64 sums in another order differ in the last bits, far below any rounding of the
    record)."""
    wl = small_decode(T=3, seed=51)
    r0 = oracle.run(wl, 1)
    for t in range(wl.num_tokens):
        pos, req = int(wl.positions[t]), int(wl.token_to_req[t])
        slots = [(int(wl.block_table[req, q // 8]), q % 8) for q in range(pos - 127, pos + 1)]
        rows = np.stack([wl.state[b, i].copy() for b, i in slots])
        perm = synth.permutation(128, 52, t)
        for (b, i), src in zip(slots, perm):
            wl.state[b, i] = rows[src]
    r1 = oracle.run(wl, 1)
    assert np.array_equal(r1.k_cache_base, r0.k_cache_base)
    np.testing.assert_allclose(r1.compressed, r0.compressed, rtol=0, atol=1e-13)  # |kv| <= ~5


def test_physical_relocation_invariance():
    """Permuting the pool's physical blocks and remapping the block table gives identical
    k_cache bytes."""
    wl = small_decode(T=6, n_blocks=200, seed=11)
    r0 = oracle.run(wl, 2)
    perm = synth.permutation(200, 12, 1)  # new position of old block b is perm[b]
    moved = np.empty_like(wl.state)
    moved[perm] = wl.state
    wl2 = small_decode(T=6, n_blocks=200, seed=11)
    wl2.state[:] = moved
    wl2.block_table[:] = perm[wl.block_table]
    wl2.slot_mapping[:] = wl.slot_mapping  # only its sign is used
    r1 = oracle.run(wl2, 2)
    assert np.array_equal(r0.k_cache_base, r1.k_cache_base)
    assert np.array_equal(r0.compressed, r1.compressed)


def test_state_block_size_relayout_invariance():
    """The same logical rows laid out in 16-row blocks (pairs of 8-row blocks glued together,
    table halved) give identical output: the gather's q // bs and q % bs are right."""
    wl = small_decode(T=5, n_blocks=80, seed=21)
    r0 = oracle.run(wl, 1)
    T, cols = wl.block_table.shape
    big = np.zeros((T * cols // 2, 16, 1024), np.float32)
    bt16 = np.zeros((T, cols // 2), np.int32)
    nb = 0
    for r in range(T):
        for m in range(cols // 2):
            big[nb, :8] = wl.state[wl.block_table[r, 2 * m]]
            big[nb, 8:] = wl.state[wl.block_table[r, 2 * m + 1]]
            bt16[r, m] = nb
            nb += 1
    wl.state, wl.block_table = big, bt16
    r1 = oracle.run(wl, 1, state_block_size=16)
    assert np.array_equal(r0.k_cache_base, r1.k_cache_base)


# ---------------------------------------------------------------- norm

def test_rmsnorm_closed_form():
    """w = 1, eps = 0: mean(n^2) = 1 exactly in fp64 up to rounding; n/c is one constant."""
    wl = small_decode(T=3)
    wl.rms_w[:] = 1.0
    wl.eps = 0.0
    r = oracle.run(wl, 1)
    for t in range(3):
        assert abs(np.mean(r.normed[t] ** 2) - 1.0) < 1e-14
        ratio = r.normed[t] / r.compressed[t]
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-14)


def test_rmsnorm_weight_and_eps():
    """n_j = c_j * w_j / sqrt(mean c^2 + eps), checked column by column with math.fsum."""
    wl = small_decode(T=2)
    wl.eps = 0.25
    r = oracle.run(wl, 1)
    for t in range(2):
        c = r.compressed[t]
        rr = 1.0 / math.sqrt(math.fsum(c * c) / 512 + 0.25)
        np.testing.assert_allclose(r.normed[t], c * rr * wl.rms_w.astype(np.float64), rtol=1e-14)


# ---------------------------------------------------------------- quant + rope + insert

def test_zero_window_record():
    """All-zero window: c = 0, n = 0; every block's absmax hits the 1e-4 floor, so each
    scale byte is 105 (e = -22), codes are 0x00, the pad byte 0 and the rope bf16 zeros
    (+0 or -0: a zero pair rotated by a negative cosine gives -0 in IEEE arithmetic)."""
    wl = small_decode(T=1, kv_bs=2)
    wl.state[:, :, :512] = 0.0
    r = oracle.run(wl, 1)
    codes, sc, rope = decode_record(r.k_cache, int(wl.kv_slot_mapping[0]))
    assert np.all(codes == 0) and list(sc) == [105] * 7 + [0] and np.all((rope & 0x7FFF) == 0)


def test_quant_invariants_on_random_windows():
    """Scale = 2^(byte-127); absmax/scale in (224, 448]; every code decodes to within half an
    e4m3 step of bf16(n)/scale; the pad byte is 0."""
    wl = small_decode(T=8, k_max=6, seed=31)
    r = oracle.run(wl, 2)
    codes_all, vals = _e4m3_table()
    lut = np.zeros(256)
    lut[codes_all] = vals
    for t in range(8):
        codes, sc, _ = decode_record(r.k_cache, int(wl.kv_slot_mapping[t]))
        assert sc[7] == 0
        n32 = r.normed[t][:448].astype(np.float32)
        u = torch.from_numpy(n32).to(torch.bfloat16).to(torch.float64).numpy()
        for g in range(7):
            e = int(sc[g]) - 127
            blk = u[64 * g: 64 * (g + 1)]
            A = max(np.abs(blk).max(), float(np.float32(1e-4)))
            assert 224 < A / 2.0 ** e <= 448
            x = blk / 2.0 ** e
            deq = lut[codes[64 * g: 64 * (g + 1)]]
            # e4m3 spacing at |x|: 2^(floor(log2|x|)-3), 2^-9 in the subnormal range
            ex = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6)))
            half_step = np.exp2(ex - 3) / 2
            assert np.all(np.abs(deq - x) <= half_step)


def test_rope_identity_at_position_zero():
    """Config 0 (position 127 -> angle row 0, cos 1, sin 0): the rope bf16 equal bf16(n)."""
    wl = synth.config0()
    r = oracle.run(wl, 1)
    _, _, rope = decode_record(r.k_cache, 3)
    want = oracle.bf16_bits(r.normed[0][448:512])
    assert np.array_equal(rope, want)


def test_rope_rotation_against_complex_multiply():
    """For windows at positions > 127: (x' + i y') = (x + i y) * exp(i P theta_m),
    theta_m = 10000^(-2m/64), P = the window's first position.  numpy's complex exp in fp64
    (not the table) agrees within one bf16 step; pair norms are kept."""
    wl = small_decode(T=6, k_max=40, seed=41)
    wl.cos_sin = synth.rope_table(128 * 40)
    r = oracle.run(wl, 2)
    m = np.arange(32)
    theta = 10000.0 ** (-2.0 * m / 64)
    for t in range(6):
        P = (int(wl.positions[t]) // 128) * 128
        n = r.normed[t]
        z = (n[448::2] + 1j * n[449::2]) * np.exp(1j * P * theta)
        _, _, rope = decode_record(r.k_cache, int(wl.kv_slot_mapping[t]))
        got = bf16_to_f64(rope)
        gx, gy = got[0::2], got[1::2]
        step = lambda v: np.exp2(np.floor(np.log2(np.abs(v) + 1e-300)) - 7)  # noqa: E731
        assert np.all(np.abs(gx - z.real) <= step(z.real) + 1e-6 * np.abs(z))
        assert np.all(np.abs(gy - z.imag) <= step(z.imag) + 1e-6 * np.abs(z))
        np.testing.assert_allclose(gx ** 2 + gy ** 2, np.abs(z) ** 2, rtol=2 ** -6)


def test_rope_table_matches_fp64_trig():
    """The RoPE input table: every entry within 1 fp32 ulp of fp64 cos/sin."""
    cs = synth.rope_table(8192).astype(np.float64)
    i = np.arange(32)
    ang = np.arange(8192)[:, None] * 10000.0 ** (-2.0 * i / 64)[None, :]
    ulp = np.spacing(np.float32(1.0)) * np.maximum(np.abs(cs), 2 ** -126)
    assert np.all(np.abs(cs[:, :32] - np.cos(ang)) <= ulp[:, :32])
    assert np.all(np.abs(cs[:, 32:] - np.sin(ang)) <= ulp[:, 32:])


def test_gate_brute_force():
    """Positions 0..1023 x state slot in {-1, 0, 5}: exactly the tokens with (pos+1) % 128 == 0
    and slot >= 0 write their kv slot; every other byte stays 0xAB."""
    pos = np.tile(np.arange(1024), 3).astype(np.int32)
    slot = np.repeat(np.array([-1, 0, 5], np.int32), 1024)
    T = pos.size
    n_blocks = 128
    base, state = synth.alloc_state(n_blocks)
    synth.fill_state(state, 5, 1.0, 1.0)
    bt = synth.permutation(n_blocks, 5, 2).astype(np.int32).reshape(1, 128)
    kc_base, kc = synth.alloc_k_cache(T // 16, 16)
    wl = synth.Workload("gate", state, bt, np.zeros(T, np.int32), pos, slot,
                        np.ones(512, np.float32), 1e-6, synth.rope_table(1024), kc,
                        np.arange(T, dtype=np.int32), 5, base, kc_base)
    r = oracle.run(wl, 4)
    active = ((pos + 1) % 128 == 0) & (slot >= 0)
    assert active.sum() == 16
    assert np.array_equal(r.status == oracle.STATUS_WRITTEN, active)
    assert np.array_equal(r.status == oracle.STATUS_INACTIVE, ~active)
    per_slot = r.k_cache_base.reshape(T // 16, 16 * 584)
    for t in range(T):
        b, o = t // 16, t % 16
        rec = per_slot[b, o * 576:(o + 1) * 576]
        scl = per_slot[b, 16 * 576 + o * 8: 16 * 576 + o * 8 + 8]
        touched = np.any(rec != 0xAB) or np.any(scl != 0xAB)
        assert touched == active[t], t


@pytest.mark.parametrize("bs,pad", [(1, 0), (2, 48), (64, 0), (64, 16)])
def test_insert_byte_offsets(bs, pad):
    """Run with two different prefill bytes: the bytes that come out equal in both runs are
    exactly those written, and they sit at blk*stride0 + off*576 (576 bytes) and
    blk*stride0 + bs*576 + off*8 (8 bytes) -- the hand-computed layout."""
    outs = []
    for fill in (0xAB, 0x54):
        wl = small_decode(T=5, kv_bs=bs, kv_blocks=-(-12 // bs) + 1, kc_block_pad=pad, seed=51)
        wl.k_cache_base[:] = fill
        outs.append(oracle.run(wl, 1).k_cache_base)
    written = outs[0] == outs[1]
    expect = np.zeros_like(written)
    stride0 = bs * 584 + pad
    for t in range(5):
        s = int(wl.kv_slot_mapping[t])
        blk, off = s // bs, s % bs
        expect[blk * stride0 + off * 576: blk * stride0 + off * 576 + 576] = True
        expect[blk * stride0 + bs * 576 + off * 8: blk * stride0 + bs * 576 + off * 8 + 8] = True
    assert np.array_equal(written, expect)


def test_negative_kv_slot_writes_nothing():
    wl = small_decode(T=3, seed=61)
    wl.kv_slot_mapping[1] = -1
    r = oracle.run(wl, 1)
    assert list(r.status) == [1, 2, 1]
    assert np.isfinite(r.compressed[1]).all()
    ref = small_decode(T=3, seed=61)
    # the other two records are the same as in a run where token 1 also writes
    r2 = oracle.run(ref, 1)
    s1 = int(ref.kv_slot_mapping[1])
    c, s, ro = decode_record(r.k_cache, s1)
    assert np.all(c == 0xAB) and np.all(s == 0xAB) and np.all(ro == 0xABAB)
    for t in (0, 2):
        a = decode_record(r.k_cache, int(wl.kv_slot_mapping[t]))
        b = decode_record(r2.k_cache, int(wl.kv_slot_mapping[t]))
        assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_quant_rounds_through_bf16_first():
    """The quantiser takes the bf16 value of each normalised fp32 value before the block's
    absmax and codes (the API page, FP8 UE8M0 quant block).  On the input of
    tests/golden/handworked.py's build_double_rounding the first block's values are exactly
    +-(1 + 2^-4 + 2^-10): through bf16 they code to 256 * sign (0x78 / 0xF8, the even neighbour
    of the midpoint 272), with scale byte 127 - 8.  The other blocks (w = 1) give the same codes
    and exponent."""
    from tests.golden.handworked import build_double_rounding
    wl = build_double_rounding()
    r = oracle.run(wl, 1)
    codes, sc, _ = decode_record(r.k_cache, int(wl.kv_slot_mapping[0]))
    sign = np.arange(448) % 3 == 0
    assert np.array_equal(codes, np.where(sign, 0x78, 0xF8).astype(np.uint8))
    assert list(sc[:7]) == [119] * 7


def test_handworked_golden_record():
    """Hand-derived record (tests/golden/c128_handworked.txt): kv = +-1 per column, w a power of
    two per quant block, eps = 0, position 127."""
    from tests.golden.handworked import build_handworked, expected_record
    wl = build_handworked()
    r = oracle.run(wl, 1)
    codes, sc, rope = decode_record(r.k_cache, int(wl.kv_slot_mapping[0]))
    want_codes, want_scales, want_rope = expected_record()
    assert np.array_equal(codes, want_codes)
    assert np.array_equal(sc, want_scales)
    assert np.array_equal(rope, want_rope)
