"""Parity check of a k_cache produced by the HIP path against the oracle.

Test infrastructure (see ``oracle/__init__.py``).  Pass criteria:

* every byte outside the records of written tokens is unchanged (bit-exact);
* UE8M0 scale bytes bit-exact, the pad byte 0 -- except a quantisation block
  whose fp64 absmax lies within rel 1e-5 of a bf16 rounding midpoint
  1.75390625 * 2^k ("knife edge"): there fp32 rounding may legitimately move
  bf16(absmax) across the power-of-two boundary of absmax/448, so the block is
  excused, counted, and compared by dequantised value instead;
* E4M3 codes within 1 code step (ordinal distance, +0 == -0), on at most 0.1%
  of the compared nope elements;
* RoPE bf16 within 1 ulp (ordinal distance, +0 == -0).  Under cancellation --
  a rotated value x*C - y*S much smaller than its inputs -- the fp32 error that
  the pooled vector carries is worth more than one ulp of the small result.
  Such an element is counted ("rope_band") and passes if it lies within the
  band of ``rope_band``: with the GPU's own pooled vector (debug export), 1 ulp
  plus an fp32 error bound of the epilogue (RMSNorm and rotation) around the
  rotation of that vector, which is itself checked against the oracle below;
  without it, 1 ulp plus the compressed tolerance carried through the norm and
  the rotation.  ``rope_band_max_use`` is the largest error / band ratio;
* debug fp32 compressed vector: |gpu - oracle| <= 1e-5 * sum_i p_ij |kv_ij|.

An excused knife-edge block is compared by dequantised value: each element within one code
step of the coarser of the two scales, at that element's own binade.

The indexer cache (records of 128 E4M3 codes and one fp32 scale 2^e, quantised after RoPE)
is checked by ``compare_indexer`` with the same rules: untouched bytes bit-exact; the scale
bit-exact unless the block's absmax sits on a knife edge (then excused and compared by
dequantised value); codes within 1 step on at most 0.1% of the elements; the debug pooled
vector within the compressed tolerance.

The indexer's MXFP4 cache (64 bytes of E2M1 codes, two a byte with the even dim in the low
nibble, then four UE8M0 bytes, one per 32-dim block) is checked by ``compare_indexer_mxfp4``
with the same rules.  Its knife edge is the bf16 midpoint 1.50390625 * 2^k above 1.5 * 2^k,
where absmax / 6 crosses a power of two.
"""

from __future__ import annotations

import numpy as np

RECORD = 576
SCALE = 8
SLOT = 584
KNIFE = 1.75390625
KNIFE_REL = 1e-5
CODE_FRAC_MAX = 1e-3
COMPRESSED_REL = 1e-5


def record_offsets(slot: int, bs: int, stride0: int):
    blk, off = slot // bs, slot % bs
    rec = blk * stride0 + off * RECORD
    scl = blk * stride0 + bs * RECORD + off * SCALE
    return rec, scl


def written_byte_mask(total: int, slots, bs: int, stride0: int) -> np.ndarray:
    m = np.zeros(total, dtype=bool)
    for s in slots:
        rec, scl = record_offsets(int(s), bs, stride0)
        m[rec:rec + RECORD] = True
        m[scl:scl + SCALE] = True
    return m


def e4m3_ord(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def e4m3_val(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(c & 0x80, -v, v)


def bf16_ord(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_val(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


# Relative error bound of the kernel's fp32 epilogue from its own pooled vector c to the
# normalised value n = c * rrms * w.  The sum of squares adds 512 non-negative terms in at most
# 11 rounding steps (4 per lane, 6 shuffle levels, the two column halves): <= 11u; the 1/512
# scale is exact; + eps: u; sqrt and the reciprocal: <= 2 ulp each (4u relative each); so rrms
# is within (12u)/2 + 8u = 14u; the two products c * rrms * w add 2u.  24u leaves margin.
U32 = 2.0 ** -24
EPILOGUE_REL = 24 * U32


def _rotation(n, C, S):
    """The 64 rotated values of the pairs (448+2m, 449+2m) of n, and |x*C| + |y*S| per value."""
    x, y = n[448::2], n[449::2]
    z = np.empty(64)
    mag = np.empty(64)
    z[0::2], z[1::2] = x * C - y * S, y * C + x * S
    mag[0::2], mag[1::2] = np.abs(x * C) + np.abs(y * S), np.abs(y * C) + np.abs(x * S)
    return z, mag


def rope_band(wl, orc, t: int, gpu_compressed_row=None) -> tuple[np.ndarray, np.ndarray]:
    """(centre, allowed |gpu - centre|) for the 64 RoPE dims of token t.

    With ``gpu_compressed_row`` (the GPU's fp32 pooled vector of the token): the centre is the
    rotation, in fp64, of that vector normalised in fp64; the band is 1 bf16 ulp plus the
    epilogue's fp32 error (EPILOGUE_REL on the normalised pair, 2u for the products and the
    difference of the rotation).  The pooled vector itself is checked against the oracle
    separately, so the band is as wide as the error the kernel actually carries into RoPE.

    Without it: the centre is the oracle's exact rotation and the band is 1 ulp plus the
    compressed tolerance (1e-5 of sum p|kv|) carried through RMSNorm and the rotation, plus the
    fp32 rounding of the rotation."""
    cr = int(getattr(wl, "compress_ratio", 128))
    P = (int(wl.positions[t]) // cr) * cr
    cs = wl.cos_sin[P].astype(np.float64)
    C, S = cs[:32], cs[32:64]
    w = wl.rms_w.astype(np.float64)
    if gpu_compressed_row is not None:
        g = np.asarray(gpu_compressed_row, dtype=np.float64)
        n = g / np.sqrt(np.mean(g * g) + float(wl.eps)) * w
        z, mag = _rotation(n, C, S)
        return z, bf16_ulp(z) + (EPILOGUE_REL + 2 * U32) * mag
    c = orc.compressed[t]
    n = orc.normed[t]
    A = orc.absnorm[t]
    r = 1.0 / np.sqrt(np.mean(c * c) + float(wl.eps))
    dn = r * np.abs(w) * COMPRESSED_REL * A + COMPRESSED_REL * np.abs(n)
    z, mag = _rotation(n, C, S)
    dx, dy = dn[448::2], dn[449::2]
    prop = np.empty(64)
    prop[0::2] = np.abs(C) * dx + np.abs(S) * dy
    prop[1::2] = np.abs(C) * dy + np.abs(S) * dx
    return z, bf16_ulp(z) + prop + 4 * U32 * mag


def e4m3_step(v_abs: np.ndarray, scale: float) -> np.ndarray:
    """Spacing of the E4M3FN values around |v| when a block is scaled by ``scale`` (a power of
    two): 2^(floor(log2 |v|/scale) - 3) * scale in the normal range, 2^-9 * scale below 2^-6."""
    q = np.maximum(np.asarray(v_abs, dtype=np.float64) / scale, 2.0 ** -12)
    return scale * np.exp2(np.maximum(np.floor(np.log2(q)), -6.0) - 3.0)


def e2m1_step(v_abs: np.ndarray, scale: float) -> np.ndarray:
    """Spacing of the E2M1 values around |v| under the block scale: 0.5 below 2, 1 in [2, 4),
    2 from 4 on (times the scale)."""
    q = np.asarray(v_abs, dtype=np.float64) / scale
    return scale * np.where(q < 2.0, 0.5, np.where(q < 4.0, 1.0, 2.0))


def knife_edge(absmax: float, knife: float = KNIFE) -> bool:
    if absmax <= 0:
        return False
    k = np.floor(np.log2(absmax / knife))
    for kk in (k - 1, k, k + 1):
        edge = knife * 2.0 ** kk
        if abs(absmax - edge) <= KNIFE_REL * edge:
            return True
    return False


class Report(dict):
    def ok(self) -> bool:
        return not self["failures"]

    def summary(self) -> str:
        keys = ["tokens", "written", "untouched_mismatch", "scale_mismatch", "excused_blocks",
                "code_diff1", "code_diff1_frac", "code_fail", "rope_max_ulp", "rope_band",
                "rope_band_max_use", "rope_band_basis", "compressed_max_ratio",
                "compressed_max_rel"]
        return ", ".join(f"{k}={self.get(k)}" for k in keys) + (
            "" if self.ok() else f"; FAIL: {self['failures'][:5]}")


def compare(wl, gpu_kc_base: np.ndarray, orc, tokens=None, gpu_compressed=None,
            initial_kc_base: np.ndarray | None = None) -> Report:
    """Compare the GPU k_cache bytes (the whole underlying buffer of the workload's
    k_cache view) with the oracle's, on ``tokens`` (indices; default all) and check
    that every byte outside the written records equals the initial buffer."""
    if getattr(wl, "indexer_fp4", False):
        return compare_indexer_mxfp4(wl, gpu_kc_base, orc, tokens, gpu_compressed,
                                     initial_kc_base)
    if getattr(wl, "indexer", False):
        return compare_indexer(wl, gpu_kc_base, orc, tokens, gpu_compressed, initial_kc_base)
    kc = wl.k_cache
    bs = kc.shape[1]
    stride0 = kc.strides[0]
    init = wl.k_cache_base if initial_kc_base is None else initial_kc_base
    assert gpu_kc_base.shape == init.shape
    T = wl.num_tokens
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    written = wl.written_mask()
    rep = Report(tokens=int(len(toks)), failures=[])

    # 1. untouched bytes (all tokens, from the workload alone)
    wmask = written_byte_mask(init.size, wl.kv_slot_mapping[written], bs, stride0)
    diff = (gpu_kc_base != init) & ~wmask
    rep["untouched_mismatch"] = int(diff.sum())
    if rep["untouched_mismatch"]:
        rep["failures"].append(f"{rep['untouched_mismatch']} bytes outside written records changed")

    # 2-4. records of the compared written tokens
    n_code = n_diff1 = n_scale_bad = n_excused = n_band = 0
    rope_max = 0
    band_use = 0.0
    band_basis = set()
    for t in toks:
        t = int(t)
        if not written[t]:
            continue
        rec, scl = record_offsets(int(wl.kv_slot_mapping[t]), bs, stride0)
        g_codes = gpu_kc_base[rec:rec + 448]
        o_codes = orc.k_cache_base[rec:rec + 448]
        g_rope = gpu_kc_base[rec + 448:rec + RECORD].view("<u2")
        o_rope = orc.k_cache_base[rec + 448:rec + RECORD].view("<u2")
        g_sc = gpu_kc_base[scl:scl + SCALE]
        o_sc = orc.k_cache_base[scl:scl + SCALE]
        if g_sc[7] != 0 or o_sc[7] != 0:
            rep["failures"].append(f"token {t}: pad byte not zero")
        n64 = orc.normed[t] if orc.normed is not None else None
        for g in range(7):
            gc, oc = g_codes[64 * g:64 * (g + 1)], o_codes[64 * g:64 * (g + 1)]
            n_code += 64
            if g_sc[g] != o_sc[g]:
                amax = float(np.abs(n64[64 * g:64 * (g + 1)]).max()) if n64 is not None else 0.0
                if knife_edge(amax):
                    n_excused += 1
                    gv = e4m3_val(gc) * 2.0 ** (int(g_sc[g]) - 127)
                    ov = e4m3_val(oc) * 2.0 ** (int(o_sc[g]) - 127)
                    coarse = 2.0 ** (max(int(g_sc[g]), int(o_sc[g])) - 127)
                    step = e4m3_step(np.maximum(np.abs(gv), np.abs(ov)), coarse)
                    if np.any(np.abs(gv - ov) > step):
                        rep["failures"].append(f"token {t} block {g}: excused block values differ")
                    continue
                n_scale_bad += 1
                rep["failures"].append(
                    f"token {t} block {g}: scale byte {int(g_sc[g])} != {int(o_sc[g])}")
                continue
            d = np.abs(e4m3_ord(gc) - e4m3_ord(oc))
            n_diff1 += int((d == 1).sum())
            if np.any(d > 1):
                rep["failures"].append(f"token {t} block {g}: code differs by {int(d.max())}")
        rd = np.abs(bf16_ord(g_rope) - bf16_ord(o_rope))
        rope_max = max(rope_max, int(rd.max()))
        far = rd > 1
        if far.any():
            grow = None
            if gpu_compressed is not None and np.isfinite(gpu_compressed[t]).all():
                grow = gpu_compressed[t]
            if grow is None and (orc.compressed is None or
                                 not np.isfinite(orc.compressed[t]).all()):
                rep["failures"].append(f"token {t}: rope differs by {int(rd.max())} ulp")
            else:
                z, tol = rope_band(wl, orc, t, grow)
                err = np.abs(bf16_val(g_rope) - z)
                n_band += int(far.sum())
                use = float((err[far] / tol[far]).max())
                band_use = max(band_use, use)
                band_basis.add("gpu pooled vector" if grow is not None else "tolerance")
                if use > 1.0:
                    rep["failures"].append(
                        f"token {t}: rope beyond 1 ulp + cancellation band "
                        f"({use:.2f} of the band)")
    rep["written"] = int(written[toks].sum())
    rep["scale_mismatch"] = n_scale_bad
    rep["excused_blocks"] = n_excused
    rep["code_diff1"] = n_diff1
    rep["code_diff1_frac"] = (n_diff1 / n_code) if n_code else 0.0
    rep["code_fail"] = rep["code_diff1_frac"] > CODE_FRAC_MAX
    if rep["code_fail"]:
        rep["failures"].append(f"code diff-1 fraction {rep['code_diff1_frac']:.2e} > 1e-3")
    rep["rope_max_ulp"] = rope_max
    rep["rope_band"] = n_band
    rep["rope_band_max_use"] = round(band_use, 4)
    rep["rope_band_basis"] = "+".join(sorted(band_basis)) if band_basis else None

    # 5. compressed fp32 (debug export)
    if gpu_compressed is not None and orc.compressed is not None:
        act = wl.active_mask()
        worst = 0.0
        worst_rel = 0.0
        for t in toks:
            t = int(t)
            if not act[t] or not np.isfinite(orc.compressed[t]).all():
                continue
            g = gpu_compressed[t].astype(np.float64)
            o = orc.compressed[t]
            ratio = np.abs(g - o) / np.maximum(orc.absnorm[t], 1e-300)
            worst = max(worst, float(ratio.max()))
            big = np.abs(o) > 1e-3 * np.abs(o).max()
            if big.any():
                worst_rel = max(worst_rel, float((np.abs(g - o)[big] / np.abs(o[big])).max()))
        rep["compressed_max_ratio"] = worst
        rep["compressed_max_rel"] = worst_rel
        if worst > COMPRESSED_REL:
            rep["failures"].append(f"compressed error {worst:.3e} > 1e-5 of sum p|kv|")
    return rep


IDX_RECORD = 128
IDX_SCALE = 4


def indexer_offsets(slot: int, bs: int, stride0: int):
    blk, off = slot // bs, slot % bs
    return blk * stride0 + off * IDX_RECORD, blk * stride0 + bs * IDX_RECORD + off * IDX_SCALE


def _compressed_check(wl, orc, toks, gpu_compressed, rep):
    act = wl.active_mask()
    worst = 0.0
    for t in toks:
        t = int(t)
        if not act[t] or not np.isfinite(orc.compressed[t]).all():
            continue
        g = gpu_compressed[t].astype(np.float64)
        ratio = np.abs(g - orc.compressed[t]) / np.maximum(orc.absnorm[t], 1e-300)
        worst = max(worst, float(ratio.max()))
    rep["compressed_max_ratio"] = worst
    if worst > COMPRESSED_REL:
        rep["failures"].append(f"compressed error {worst:.3e} > 1e-5 of sum p|kv|")


def compare_indexer(wl, gpu_kc_base: np.ndarray, orc, tokens=None, gpu_compressed=None,
                    initial_kc_base: np.ndarray | None = None) -> Report:
    """``compare`` for the indexer's FP8 cache ([bs*128 codes][bs*4 fp32 scales] blocks)."""
    kc = wl.k_cache
    bs = kc.shape[1]
    stride0 = kc.strides[0]
    init = wl.k_cache_base if initial_kc_base is None else initial_kc_base
    assert gpu_kc_base.shape == init.shape
    T = wl.num_tokens
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    written = wl.written_mask()
    rep = Report(tokens=int(len(toks)), failures=[])

    wmask = np.zeros(init.size, dtype=bool)
    for s_ in wl.kv_slot_mapping[written]:
        rec, scl = indexer_offsets(int(s_), bs, stride0)
        wmask[rec:rec + IDX_RECORD] = True
        wmask[scl:scl + IDX_SCALE] = True
    diff = (gpu_kc_base != init) & ~wmask
    rep["untouched_mismatch"] = int(diff.sum())
    if rep["untouched_mismatch"]:
        rep["failures"].append(f"{rep['untouched_mismatch']} bytes outside written records changed")

    n_code = n_diff1 = n_scale_bad = n_excused = 0
    for t in toks:
        t = int(t)
        if not written[t]:
            continue
        rec, scl = indexer_offsets(int(wl.kv_slot_mapping[t]), bs, stride0)
        gc, oc = gpu_kc_base[rec:rec + IDX_RECORD], orc.k_cache_base[rec:rec + IDX_RECORD]
        gs = float(gpu_kc_base[scl:scl + IDX_SCALE].view("<f4")[0])
        os_ = float(orc.k_cache_base[scl:scl + IDX_SCALE].view("<f4")[0])
        n_code += IDX_RECORD
        if gs != os_:
            # the block's fp64 absmax (orc.normed holds the quantised values, after RoPE)
            amax = float(np.abs(orc.normed[t]).max()) if orc.normed is not None else 0.0
            if knife_edge(amax):
                n_excused += 1
                gv, ov = e4m3_val(gc) * gs, e4m3_val(oc) * os_
                step = e4m3_step(np.maximum(np.abs(gv), np.abs(ov)), max(gs, os_))
                if np.any(np.abs(gv - ov) > step):
                    rep["failures"].append(f"token {t}: excused block values differ")
                continue
            n_scale_bad += 1
            rep["failures"].append(f"token {t}: scale {gs} != {os_}")
            continue
        d = np.abs(e4m3_ord(gc) - e4m3_ord(oc))
        n_diff1 += int((d == 1).sum())
        if np.any(d > 1):
            rep["failures"].append(f"token {t}: code differs by {int(d.max())}")
    rep["written"] = int(written[toks].sum())
    rep["scale_mismatch"] = n_scale_bad
    rep["excused_blocks"] = n_excused
    rep["code_diff1"] = n_diff1
    rep["code_diff1_frac"] = (n_diff1 / n_code) if n_code else 0.0
    rep["code_fail"] = rep["code_diff1_frac"] > CODE_FRAC_MAX
    if rep["code_fail"]:
        rep["failures"].append(f"code diff-1 fraction {rep['code_diff1_frac']:.2e} > 1e-3")
    if gpu_compressed is not None and orc.compressed is not None:
        _compressed_check(wl, orc, toks, gpu_compressed, rep)
    return rep


FP4_RECORD = 64
FP4_SCALES = 4
FP4_BLOCK = 32
KNIFE_FP4 = 1.50390625


def fp4_offsets(slot: int, bs: int, stride0: int):
    blk, off = slot // bs, slot % bs
    return blk * stride0 + off * FP4_RECORD, blk * stride0 + bs * FP4_RECORD + off * FP4_SCALES


def e2m1_unpack(b: np.ndarray) -> np.ndarray:
    """128 codes from 64 bytes: dim 2p in the low nibble of byte p, dim 2p+1 in the high."""
    out = np.empty(2 * b.size, np.uint8)
    out[0::2] = b & 0xF
    out[1::2] = b >> 4
    return out


def e2m1_ord(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int32)
    mag = c & 7
    return np.where(c & 8, -mag, mag)


def e2m1_val(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    e, m = (c >> 1) & 3, c & 1
    v = np.where(e == 0, 0.5 * m, (1 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(c & 8, -v, v)


def compare_indexer_mxfp4(wl, gpu_kc_base: np.ndarray, orc, tokens=None, gpu_compressed=None,
                          initial_kc_base: np.ndarray | None = None) -> Report:
    """``compare`` for the indexer's MXFP4 cache ([bs*64 packed codes][bs*4 UE8M0] blocks)."""
    kc = wl.k_cache
    bs = kc.shape[1]
    stride0 = kc.strides[0]
    init = wl.k_cache_base if initial_kc_base is None else initial_kc_base
    assert gpu_kc_base.shape == init.shape
    T = wl.num_tokens
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    written = wl.written_mask()
    rep = Report(tokens=int(len(toks)), failures=[])

    wmask = np.zeros(init.size, dtype=bool)
    for s_ in wl.kv_slot_mapping[written]:
        rec, scl = fp4_offsets(int(s_), bs, stride0)
        wmask[rec:rec + FP4_RECORD] = True
        wmask[scl:scl + FP4_SCALES] = True
    diff = (gpu_kc_base != init) & ~wmask
    rep["untouched_mismatch"] = int(diff.sum())
    if rep["untouched_mismatch"]:
        rep["failures"].append(f"{rep['untouched_mismatch']} bytes outside written records changed")

    n_code = n_diff1 = n_scale_bad = n_excused = 0
    for t in toks:
        t = int(t)
        if not written[t]:
            continue
        rec, scl = fp4_offsets(int(wl.kv_slot_mapping[t]), bs, stride0)
        g_codes = e2m1_unpack(gpu_kc_base[rec:rec + FP4_RECORD])
        o_codes = e2m1_unpack(orc.k_cache_base[rec:rec + FP4_RECORD])
        g_sc = gpu_kc_base[scl:scl + FP4_SCALES]
        o_sc = orc.k_cache_base[scl:scl + FP4_SCALES]
        for g in range(FP4_SCALES):
            sl = slice(FP4_BLOCK * g, FP4_BLOCK * (g + 1))
            gc, oc = g_codes[sl], o_codes[sl]
            n_code += FP4_BLOCK
            if g_sc[g] != o_sc[g]:
                # the block's fp64 absmax (orc.normed holds the rotated values)
                amax = float(np.abs(orc.normed[t][sl]).max()) if orc.normed is not None else 0.0
                if knife_edge(amax, KNIFE_FP4):
                    n_excused += 1
                    gv = e2m1_val(gc) * 2.0 ** (int(g_sc[g]) - 127)
                    ov = e2m1_val(oc) * 2.0 ** (int(o_sc[g]) - 127)
                    coarse = 2.0 ** (max(int(g_sc[g]), int(o_sc[g])) - 127)
                    step = e2m1_step(np.maximum(np.abs(gv), np.abs(ov)), coarse)
                    if np.any(np.abs(gv - ov) > step):
                        rep["failures"].append(f"token {t} block {g}: excused block values differ")
                    continue
                n_scale_bad += 1
                rep["failures"].append(
                    f"token {t} block {g}: scale byte {int(g_sc[g])} != {int(o_sc[g])}")
                continue
            d = np.abs(e2m1_ord(gc) - e2m1_ord(oc))
            n_diff1 += int((d == 1).sum())
            if np.any(d > 1):
                rep["failures"].append(f"token {t} block {g}: code differs by {int(d.max())}")
    rep["written"] = int(written[toks].sum())
    rep["scale_mismatch"] = n_scale_bad
    rep["excused_blocks"] = n_excused
    rep["code_diff1"] = n_diff1
    rep["code_diff1_frac"] = (n_diff1 / n_code) if n_code else 0.0
    rep["code_fail"] = rep["code_diff1_frac"] > CODE_FRAC_MAX
    if rep["code_fail"]:
        rep["failures"].append(f"code diff-1 fraction {rep['code_diff1_frac']:.2e} > 1e-3")
    if gpu_compressed is not None and orc.compressed is not None:
        _compressed_check(wl, orc, toks, gpu_compressed, rep)
    return rep
