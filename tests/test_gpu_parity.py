"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Pass criteria (oracle/compare.py): untouched bytes and UE8M0 scale bytes
bit-exact (knife-edge blocks excused and counted), E4M3 codes within one step
on <= 0.1% of elements, RoPE bf16 within 1 ulp, fp32 compressed within 1e-5
of sum_i p_ij |kv_ij|.  Every test prints its case before touching the GPU.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.compare import compare
from synth.device import DeviceWorkload, relocated_pool, run_gpu

pytestmark = pytest.mark.gpu

THREADS = synth.default_threads()


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def check(wl, debug=True, tokens=None, nthreads=THREADS, label=None):
    announce(label or wl.name)
    body, comp, guards_ok = run_gpu(wl, debug=debug)
    assert guards_ok, "k_cache guard bands were written"
    orc = oracle.run(wl, nthreads)
    rep = compare(wl, body, orc, tokens=tokens, gpu_compressed=comp)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    return rep, body, comp, orc


# ---------------------------------------------------------------- conversion

def test_e4m3_encoder_exhaustive():
    """The kernel's E4M3FN encoder on every bf16 value (the quantiser's domain after the
    power-of-two scale), values beyond +-448 (clamped), fp32 subnormals and signed zeros,
    against the oracle's encoder (itself pinned by brute force)."""
    announce("e4m3 encoder exhaustive")
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    f = f[np.isfinite(f)]
    extra = np.array([0.0, -0.0, 1e-40, -1e-40, 2.0 ** -149, 449.0, -449.0, 464.0, 1e30, -1e30,
                      2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -10 * 1.0000001], np.float32)
    x = np.concatenate([f, extra]).astype(np.float32)
    got = c128_encode(x)
    want = oracle.e4m3_codes(np.clip(x.astype(np.float64), -448.0, 448.0))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def c128_encode(x):
    import paged_kv_cache_fp32_amd as c128
    out = c128.e4m3_encode(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---------------------------------------------------------------- workloads

def test_config0_single_token():
    rep, _, comp, orc = check(synth.config0())
    assert rep["written"] == 1


def test_handworked_golden_bit_exact():
    """The hand-derived record (tests/golden/c128_handworked.txt) comes out bit-exact, and the
    non-boundary token at position 126 leaves its slot at 0xAB."""
    from tests.golden.handworked import build_handworked, expected_record
    wl = build_handworked()
    announce("handworked golden")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    codes = body[0:448]
    rope = body[448:576].view("<u2")
    scales = body[2 * 576:2 * 576 + 8]
    want_codes, want_scales, want_rope = expected_record()
    assert np.array_equal(codes, want_codes)
    assert np.array_equal(scales, want_scales)
    assert np.array_equal(rope, want_rope)
    assert np.all(body[576:2 * 576] == 0xAB) and np.all(body[2 * 576 + 8:] == 0xAB)
    sign = np.where(np.arange(512) % 3 == 0, 1.0, -1.0)
    assert np.array_equal(comp[0], sign.astype(np.float32))


def test_config1_decode_batch():
    rep, *_ = check(synth.config1())
    assert rep["written"] == 128


def test_config2_varlen_prefill():
    wl = synth.config2()
    rep, *_ = check(wl)
    assert rep["written"] == int(wl.written_mask().sum()) > 100


@pytest.fixture(scope="module")
def sweep_pool():
    return synth.config3_pool()


@pytest.mark.parametrize("T", [1, 2, 8, 64, 256, 1024, 4096])
def test_config3_decode_sweep(sweep_pool, T):
    wl = synth.config3(T, state=sweep_pool[1])
    rep, *_ = check(wl)
    assert rep["written"] == T


def test_config3_rotated_window_sets(sweep_pool):
    """The bench rotates over disjoint window sets of the same pool; each set is correct."""
    for s in (1, 3):
        wl = synth.config3(512, state=sweep_pool[1], window_set=s)
        check(wl, label=f"cfg3 T=512 window set {s}")


def test_config4_full_size():
    """16384 boundary tokens over the 8.59 GB pool, in the bench's launch configuration (the
    staged schedule): every record and, through the debug entry point, every fp32 pooled vector
    compared against the oracle (half the windows have near-constant scores).  The debug call
    writes the same k_cache bytes as the plain call."""
    wl = synth.config4()
    announce(f"{wl.name} (debug entry point, then the plain one)")
    d = DeviceWorkload(wl)
    comp = d.run(debug=True).cpu().numpy()
    body_debug, ok_debug = d.k_cache_bytes()
    d.kc_buf[d.guard:d.guard + wl.k_cache_base.size].copy_(torch.from_numpy(wl.k_cache_base))
    d.run(debug=False)
    body, ok = d.k_cache_bytes()
    del d
    torch.cuda.empty_cache()
    assert ok and ok_debug, "k_cache guard bands were written"
    assert np.array_equal(body, body_debug)
    rep = compare(wl, body, oracle.run(wl, THREADS), gpu_compressed=comp)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == 16384
    assert rep["compressed_max_ratio"] is not None and rep["compressed_max_ratio"] <= 1e-5


# ---------------------------------------------------------------- edge cases

def small(T=8, seed=5, **kw):
    kv_bs = kw.pop("kv_bs", 4)
    return synth.decode_batch("edge", seed, T, kw.pop("n_blocks", 16 * T + 16), kw.pop("k_max", 8),
                              kw.pop("table_cols", 128), kv_bs=kv_bs,
                              kv_blocks=kw.pop("kv_blocks", -(-2 * T // kv_bs)),
                              cs_rows=kw.pop("cs_rows", 1024), **kw)


def test_non_boundary_and_negative_slots():
    """Positions 126, 128, 255 (boundary), 254, 383 (boundary); slot -1 on a boundary; kv slot -1
    on a boundary: only real boundary tokens with both slots >= 0 write."""
    wl = small(T=6, seed=7)
    wl.positions[:] = np.array([126, 128, 255, 254, 383, 511], np.int32)
    wl.slot_mapping[:] = np.array([3, 3, 3, 3, -1, 9], np.int32)
    wl.kv_slot_mapping[5] = -1
    rep, body, comp, orc = check(wl, label="non-boundary / negative slots")
    assert list(np.nonzero(wl.written_mask())[0]) == [2]
    assert np.isfinite(comp[5]).all() and np.isnan(comp[4]).all() and np.isnan(comp[0]).all()


@pytest.mark.parametrize("mode", ["single", "fanout", "varlen"])
def test_kv_slot_edges_without_pooled_output(mode):
    """Without the pooled-vector output the single pass drops a token with a negative kv slot
    at its gate: kv slots -1, -7 and one past the last slot (each on a boundary token) write
    nothing and every other boundary token is inserted, on the plain entry point, the fan-out
    and the compacted schedule alike."""
    wl = small(T=10, seed=29)
    n_slots = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    wl.kv_slot_mapping[[1, 4, 8]] = np.array([-1, -7, n_slots], np.int32)
    announce(f"kv slot edges, no pooled output ({mode})")
    kw = {"splits": 4} if mode == "fanout" else ({"varlen": True} if mode == "varlen" else {})
    body, _, guards_ok = run_gpu(wl, debug=False, **kw)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [1, 2, 1, 1, 2, 1, 1, 1, -1, 1]
    wl.kv_slot_mapping[8] = -1
    rep = compare(wl, body, orc)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == 7


def test_all_zero_window():
    wl = small(T=2, seed=9)
    wl.state[:, :, :512] = 0.0
    rep, body, *_ = check(wl, label="all-zero window")


@pytest.mark.parametrize("kv_bs", [1, 2, 64])
def test_kv_block_sizes(kv_bs):
    check(small(T=16, seed=11, kv_bs=kv_bs, kv_blocks=-(-40 // kv_bs)), label=f"kv bs {kv_bs}")


def test_padded_strides():
    """Padded state rows and blocks and a padded k_cache block stride."""
    wl = small(T=12, seed=13, row_pad=32, block_pad=64, kc_block_pad=48)
    check(wl, label="padded strides")


def test_peaky_and_near_constant_scores():
    wl = small(T=16, seed=17, score_std=8.0)
    check(wl, label="peaky scores std 8")
    wl = small(T=16, seed=18, score_std=1.0, score_mix=True)
    check(wl, label="near-constant windows")


@pytest.mark.parametrize("score_std", [1e2, 1e4, 1e6])
def test_extreme_scores(score_std):
    """Scores spread so far (std 1e2 to 1e6) that each column's softmax is one-hot or nearly so:
    the max-subtracted exponentials must neither overflow nor produce NaN, and near ties stay
    within the compressed tolerance, on the single pass, the fan-out and the compacted schedule
    (16 tokens) and the staged schedule (2048 tokens)."""
    wl = small(T=16, seed=19, score_std=score_std)
    check(wl, label=f"scores std {score_std:g}, single pass")
    for label, kw in (("fan-out", {"splits": 8}), ("compacted", {"varlen": True})):
        announce(f"scores std {score_std:g}, {label}")
        body, comp, guards_ok = run_gpu(wl, debug=True, **kw)
        assert guards_ok
        rep = compare(wl, body, oracle.run(wl, THREADS), gpu_compressed=comp)
        assert rep.ok(), rep.summary()
    big = synth.shared_pool_batch(f"scores std {score_std:g}", 5300, 2048, 2048, 8, 64, 34,
                                  1024, score_std=score_std)
    rep, *_ = check(big, label=f"scores std {score_std:g}, staged")
    assert rep["written"] == 2048


@pytest.mark.parametrize("scale", [1e-4, 1e4])
def test_kv_magnitudes(scale):
    """kv scaled by 1e-4 (mean(c^2) far below eps = 1e-6, so eps sets the norm and the codes
    shrink towards the scale floor) and by 1e4 (sums of squares near 1e10): the single pass and
    the staged schedule agree with the oracle."""
    wl = small(T=16, seed=23)
    wl.state[:, :, :512] *= np.float32(scale)
    check(wl, label=f"kv x {scale:g}, single pass")
    big = synth.shared_pool_batch(f"kv x {scale:g}", 5400, 2048, 2048, 8, 64, 34, 1024)
    big.state[:, :, :512] *= np.float32(scale)
    rep, *_ = check(big, label=f"kv x {scale:g}, staged")
    assert rep["written"] == 2048


def test_out_of_range_device_indices_write_nothing():
    """Indices that live in device memory and are out of range (request, block id, kv slot,
    RoPE row) make the kernel skip the token: nothing is written, no fault."""
    wl = small(T=6, seed=19, cs_rows=1024)
    wl.positions[:] = 127                               # window 0, RoPE row 0 ...
    wl.positions[4] = 1023                              # ... except token 4: RoPE row 896
    wl.token_to_req[0] = wl.block_table.shape[0]        # request out of range
    wl.block_table[1, 15] = wl.state.shape[0] + 5       # a window block id out of range
    wl.kv_slot_mapping[2] = wl.k_cache.shape[0] * wl.k_cache.shape[1]  # kv slot out of range
    wl.cos_sin = wl.cos_sin[:128].copy()                # RoPE rows 0..127 only
    announce("out-of-range device indices")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [-1, -1, -1, 1, -1, 1]
    # the oracle's k_cache has exactly the two valid tokens' records; so must the GPU's
    keep = np.array([False, False, False, True, False, True])
    wl.kv_slot_mapping[~keep] = -1                      # compare as if only they write
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    # tokens rejected on the state side produce no pooled vector; an out-of-range kv slot
    # behaves like a negative one (pooled, nothing stored)
    assert np.isnan(comp[:2]).all() and np.isnan(comp[4]).all() and np.isfinite(comp[2]).all()


def test_empty_batch_is_a_noop():
    import paged_kv_cache_fp32_amd as c128
    announce("T = 0")
    d = DeviceWorkload(small(T=1, seed=23))
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    before = d.kc_buf.clone()
    c128.compress_store(d.state, d.block_table, e, e, e, d.rms_w, 1e-6, d.cos_sin, d.k_cache, e)
    torch.cuda.synchronize()
    assert torch.equal(before, d.kc_buf)


def test_repeatable_and_debug_matches_plain():
    """Two runs give identical bytes; the debug entry point writes the same k_cache bytes."""
    wl = small(T=32, seed=29)
    announce("determinism")
    a, _, ga = run_gpu(wl, debug=False)
    b, _, gb = run_gpu(wl, debug=False)
    c, _, gc = run_gpu(wl, debug=True)
    assert ga and gb and gc
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_stream_argument_is_used():
    """Launch on a side stream; the result is there after that stream synchronises."""
    import paged_kv_cache_fp32_amd as c128
    wl = small(T=8, seed=31)
    announce("side stream")
    d = DeviceWorkload(wl)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c128.compress_store(*d.args())
    s.synchronize()
    body, ok = d.k_cache_bytes()
    orc = oracle.run(wl, 2)
    rep = compare(wl, body, orc)
    assert ok and rep.ok(), rep.summary()


def test_varlen_on_a_side_stream_without_workspace():
    """The compacted schedule launched on an explicit side stream with the workspace left to the
    binding (allocated on that stream), while the current stream allocates and fills other
    memory: the result is there after the side stream synchronises."""
    import paged_kv_cache_fp32_amd as c128
    wl = small(T=40, seed=33, kv_bs=16, kv_blocks=6)
    announce("compacted schedule on a side stream, binding-allocated workspace")
    d = DeviceWorkload(wl)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    c128.compress_store_varlen(*d.args(), stream=side.cuda_stream)
    junk = [torch.full((1 << 16,), 7, dtype=torch.int32, device="cuda") for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    body, ok = d.k_cache_bytes()
    rep = compare(wl, body, oracle.run(wl, 2))
    assert ok and rep.ok(), rep.summary()


# ---------------------------------------------------------------- small-batch fan-out

def check_ex(wl, splits, label, debug=True):
    announce(f"{label} (fan-out splits={splits})")
    body, comp, guards_ok = run_gpu(wl, debug=debug, splits=splits)
    assert guards_ok, "k_cache guard bands were written"
    orc = oracle.run(wl, THREADS)
    rep = compare(wl, body, orc, gpu_compressed=comp)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    return rep, body, comp


@pytest.mark.parametrize("splits", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("T", [1, 7, 64, 130])
def test_fanout_parity(T, splits):
    """Every split count on small decode batches (one token, a ragged 7, 64, 130)."""
    wl = small(T=T, seed=100 + T, kv_bs=16, kv_blocks=-(-2 * T // 16))
    rep, *_ = check_ex(wl, splits, f"decode T={T}")
    assert rep["written"] == T


def test_fanout_automatic_on_workloads():
    """Automatic split choice on the single-token workload (8 splits), a 40-token batch (4),
    the T=128 workload and a 600-token batch (single pass, no workspace needed)."""
    check_ex(synth.config0(), 0, "cfg0")
    check_ex(small(T=40, seed=41, kv_bs=16, kv_blocks=5), 0, "decode T=40")
    check_ex(synth.config1(), 0, "cfg1")
    check_ex(small(T=600, seed=77, kv_bs=64, kv_blocks=20), 0, "decode T=600")


def test_fanout_workspace_reuse():
    """One workspace, zero-filled once, serves a sequence of calls with different batch sizes,
    split counts and windows (the same token indices get new windows in every call).  Between
    calls the partial-state region is filled with NaN, so a read of anything but this call's
    partials would show; after every call the 16 KiB counter region is zero again, and every
    call's bytes agree with the oracle."""
    import paged_kv_cache_fp32_amd as c128
    ws = c128.fanout_workspace(130, 16)
    counters, partials = ws[:16384], ws[16384:].view(torch.float32)
    for i, (T, splits) in enumerate([(130, 16), (7, 8), (64, 2), (1, 4), (130, 2), (40, 0),
                                     (16, 16), (100, 0)]):
        wl = small(T=T, seed=900 + i, kv_bs=16, kv_blocks=-(-2 * T // 16) + 1)
        d = DeviceWorkload(wl)
        partials.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"fan-out workspace reuse: call {i}, T={T}, splits={splits}")
        c128.compress_store_ex(*d.args(), workspace=ws, splits=splits)
        torch.cuda.synchronize()
        assert int(counters.count_nonzero()) == 0, f"call {i}: counters not back at zero"
        body, ok = d.k_cache_bytes()
        rep = compare(wl, body, oracle.run(wl, THREADS))
        assert ok and rep.ok(), f"call {i}: {rep.summary()}"
        assert rep["written"] == T


def test_fanout_many_calls_one_workspace():
    """24 calls in a row on one workspace, nothing cleared in between: random batch sizes (1 to
    64 tokens) and split counts, new windows for the same token indices every call, so a read of
    a previous call's partial state (a valid-looking value) would show against the oracle."""
    import paged_kv_cache_fp32_amd as c128
    ws = c128.fanout_workspace(64, 16)
    rng = np.random.default_rng(7700)
    for i in range(24):
        T = int(rng.integers(1, 65))
        splits = int(rng.choice([2, 4, 8, 16]))
        wl = small(T=T, seed=7700 + i, kv_bs=16, kv_blocks=-(-2 * T // 16) + 1)
        d = DeviceWorkload(wl)
        announce(f"fan-out call {i}: T={T}, splits={splits}")
        c128.compress_store_ex(*d.args(), workspace=ws, splits=splits)
        body, ok = d.k_cache_bytes()
        rep = compare(wl, body, oracle.run(wl, THREADS))
        assert ok and rep.ok(), f"call {i}: {rep.summary()}"
    assert int(ws[:16384].count_nonzero()) == 0


@pytest.fixture(scope="module")
def batch_4096():
    T = 4096
    return synth.decode_batch(f"fan-out T={T}", 4100, T, 16 * T + 16, 64, 1024, kv_bs=64,
                              kv_blocks=T // 64 + 1, cs_rows=8192)


@pytest.mark.parametrize("splits", [2, 16])
def test_fanout_largest_batch(batch_4096, splits):
    """4096 tokens, the most the fan-out takes: the last arrival counter of the workspace's
    counter region is used, and every token agrees with the oracle."""
    rep, *_ = check_ex(batch_4096, splits, "decode T=4096")
    assert rep["written"] == 4096


def test_fanout_gate_and_bad_indices():
    """Non-boundary tokens, negative slots and out-of-range device indices take the same
    decision in every workgroup of the token: nothing is written for them, and the token's
    arrival counter is never touched."""
    wl = small(T=6, seed=7)
    wl.positions[:] = np.array([126, 128, 255, 254, 383, 511], np.int32)
    wl.slot_mapping[:] = np.array([3, 3, 3, 3, -1, 9], np.int32)
    wl.kv_slot_mapping[5] = -1
    rep, body, comp = check_ex(wl, 8, "fan-out gate")
    assert list(np.nonzero(wl.written_mask())[0]) == [2]
    assert np.isfinite(comp[5]).all() and np.isnan(comp[4]).all()

    wl = small(T=6, seed=19, cs_rows=1024)
    wl.positions[:] = 127
    wl.positions[4] = 1023
    wl.token_to_req[0] = wl.block_table.shape[0]
    wl.block_table[1, 15] = wl.state.shape[0] + 5
    wl.kv_slot_mapping[2] = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    wl.cos_sin = wl.cos_sin[:128].copy()
    announce("fan-out out-of-range indices (splits=16)")
    body, comp, guards_ok = run_gpu(wl, debug=True, splits=16)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [-1, -1, -1, 1, -1, 1]
    wl.kv_slot_mapping[[0, 1, 2, 4]] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[:2]).all() and np.isnan(comp[4]).all() and np.isfinite(comp[2]).all()


def test_quant_rounds_through_bf16_first():
    """The kernel codes the bf16 value of each normalised value, as the oracle does: on
    build_double_rounding's input (tests/golden/handworked.py) the first quantisation block's
    values are exactly +-(1 + 2^-4 + 2^-10), whose bf16 value lands on an E4M3 midpoint after the
    block's scale; the codes are the even neighbour, 0x78 / 0xF8."""
    from tests.golden.handworked import build_double_rounding
    wl = build_double_rounding()
    announce("bf16 before the E4M3 codes")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    rep = compare(wl, body, oracle.run(wl, 1), gpu_compressed=comp)
    assert rep.ok(), rep.summary()
    rec = body[:448]  # kv slot 0 of the first block
    assert np.array_equal(rec, np.where(np.arange(448) % 3 == 0, 0x78, 0xF8).astype(np.uint8))


# ---------------------------------------------------------------- staged schedule (large batches)

def shared(T, seed):
    """T boundary tokens whose windows draw from a 2048-block pool (64 MiB), one request each."""
    return synth.shared_pool_batch(f"shared pool T={T}", seed, T, 2048, 8, 64, T // 64 + 2, 1024)


@pytest.mark.parametrize("T", [2047, 2048, 8192, 20000])
def test_staged_threshold_and_stages(T):
    """2047 tokens take the single pass and 2048 the staged schedule (8 tokens per workgroup of
    256, one stage); 8192 give 32 tokens each, and 20000 give 78 or 79 each, in two stages.
    Every record and every pooled vector of the debug entry point agrees with the oracle."""
    rep, *_ = check(shared(T, 5000 + T), label=f"shared pool T={T}")
    assert rep["written"] == T


def test_staged_near_constant_score_windows():
    """The staged schedule on the large batch's score mix at 3000 tokens (a ragged share per
    workgroup): half the windows score N(0,1), half near-constant (c_w + 1e-3 N(0,1)), so many
    columns pool with almost uniform weights.  Records and pooled vectors agree with the
    oracle."""
    wl = synth.decode_batch("staged score mix T=3000", 5500, 3000, 48000, 64, 1024, kv_bs=64,
                            kv_blocks=48, cs_rows=8192, score_std=1.0, score_mix=True)
    rep, *_ = check(wl, label="staged score mix T=3000")
    assert rep["written"] == 3000


def test_staged_padded_strides_and_largest_position():
    """The staged schedule on padded state rows and blocks and padded k_cache blocks (8192
    tokens); then a token at position 2^31 - 1 (a boundary of ratio 128) is skipped without
    overflow and the others still agree with the oracle."""
    wl = synth.shared_pool_batch("staged padded", 5200, 8192, 2048, 8, 64, 130, 1024,
                                 row_pad=16, block_pad=32, kc_block_pad=24)
    rep, *_ = check(wl, label="staged padded strides T=8192")
    assert rep["written"] == 8192
    wl.positions[4321] = 2 ** 31 - 1
    announce("staged largest position")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, THREADS)
    assert orc.status[4321] == -1 and (np.delete(orc.status, 4321) == 1).all()
    wl.kv_slot_mapping[4321] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[4321]).all()


def test_staged_gates_and_bad_indices():
    """A 12,000-token staged batch with non-boundary positions, negative state and kv slots, and
    out-of-range requests, block ids and kv slots scattered through it: the tokens the oracle
    skips write nothing, every other record matches."""
    T = 12000
    wl = shared(T, 5100)
    rng = np.random.default_rng(5100)
    off = rng.random(T) < 0.1
    wl.positions[off] -= rng.integers(1, 127, int(off.sum())).astype(np.int32)
    wl.slot_mapping[rng.random(T) < 0.05] = -1
    wl.kv_slot_mapping[rng.random(T) < 0.05] = -1
    bad = rng.choice(np.nonzero(~off)[0], 30, replace=False)
    wl.token_to_req[bad[:10]] = wl.block_table.shape[0] + 1
    wl.kv_slot_mapping[bad[10:20]] = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    for t in bad[20:30]:
        wl.block_table[t, (wl.positions[t] // 128) * 16 + int(rng.integers(0, 16))] = \
            wl.state.shape[0] + 7
    announce("staged gates and bad indices T=12000")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, THREADS)
    assert (orc.status[bad[:10]] == -1).all() and (orc.status[bad[20:30]] == -1).all()
    wl.kv_slot_mapping[orc.status == -1] = -1  # out-of-range tokens: nothing may be written
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[bad[:10]]).all() and np.isnan(comp[bad[20:30]]).all()


def test_staged_gate_density_regions():
    """160,000 tokens in four regions of gate density, with a fifth of the state slots negative
    throughout: one position in 128 closes a window (a chunked prefill), then one in eight, then
    every position (10,000 tokens), then one in 128 again.  The staged schedule's workgroups
    start their count pass at different chunks and keep all 625 chunks' gate masks; every
    workgroup must derive the same ranks from them, so each passing token is written once, by
    one workgroup: every record agrees with the oracle and nothing else is written."""
    T = 160000
    wl = synth.shared_pool_batch("gate density regions", 5700, T, 2048, 8, 64, T // 64 + 1, 1024)
    rng = np.random.default_rng(5700)
    t = np.arange(T)
    u = rng.random(T)
    keep = np.where(t < 40000, u < 1 / 128, np.where(t < 120000, u < 1 / 8,
                                                     np.where(t < 130000, True, u < 1 / 128)))
    wl.positions[~keep] -= rng.integers(1, 128, int((~keep).sum())).astype(np.int32)
    wl.slot_mapping[rng.random(T) < 0.2] = -1
    rep, *_ = check(wl, label="staged gate density regions T=160000")
    assert rep["written"] == int(wl.written_mask().sum()) > 10000


# ---------------------------------------------------------------- compacted schedule (varlen)

def check_varlen(wl, label, debug=True):
    announce(f"{label} (compacted schedule)")
    body, comp, guards_ok = run_gpu(wl, debug=debug, varlen=True)
    assert guards_ok, "k_cache guard bands were written"
    orc = oracle.run(wl, THREADS)
    rep = compare(wl, body, orc, gpu_compressed=comp)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    return rep, body, comp


def test_varlen_config2_and_plain_entry_point():
    """The varlen prefill workload on the compacted schedule and on the plain entry point (which
    takes the staged schedule at this size, 34,323 tokens): both agree with the oracle.  Their
    bytes may differ in the last place of a code: the staged schedule merges 8 row groups, the
    compacted one 4, so the fp32 summation orders differ."""
    wl = synth.config2()
    rep, body, _ = check_varlen(wl, "cfg2 varlen prefill")
    assert rep["written"] == int(wl.written_mask().sum()) > 100
    announce("cfg2 varlen prefill (plain entry point)")
    plain, comp, ok = run_gpu(wl, debug=True)
    rep2 = compare(wl, plain, oracle.run(wl, THREADS), gpu_compressed=comp)
    assert ok and rep2.ok(), rep2.summary()


def test_varlen_decode_batches():
    """Every token active: a ragged 37 and the T=128 workload; bytes equal the single pass."""
    for wl in (small(T=37, seed=43, kv_bs=16, kv_blocks=5), synth.config1()):
        rep, body, _ = check_varlen(wl, wl.name + f" T={wl.num_tokens}")
        assert rep["written"] == wl.num_tokens
        plain, _, ok = run_gpu(wl, debug=False)
        assert ok and np.array_equal(body, plain)


def test_varlen_many_scan_blocks():
    """262,400 tokens at random positions, about 1,850 of them written: 513 scan blocks of 512
    tokens, so the prefix over scan blocks spans many lanes and the persistent grid of 512
    workgroups takes several tokens each.  Only tokens that close a window write, so the oracle
    runs on that sub-batch (its diagnostics for all 262,400 rows would take 3 GB): it fixes
    every record written and every byte that must stay untouched."""
    import dataclasses
    wl = synth.scattered_batch("scattered", 61, 262400, 8, 64, 1024, kv_bs=64, kv_blocks=64,
                               cs_rows=8192)
    announce("scattered T=262400 (compacted schedule)")
    body, _, guards_ok = run_gpu(wl, debug=False, varlen=True)
    assert guards_ok
    act = np.nonzero(wl.active_mask())[0]
    sub = dataclasses.replace(wl, token_to_req=wl.token_to_req[act], positions=wl.positions[act],
                              slot_mapping=wl.slot_mapping[act],
                              kv_slot_mapping=wl.kv_slot_mapping[act])
    rep = compare(sub, body, oracle.run(sub, THREADS))
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == int(wl.written_mask().sum()) > 1500


def test_plain_entry_point_on_the_scattered_batch():
    """The scattered 262,400-token batch (1,025 chunks of 256 tokens: the staged schedule keeps
    every chunk's gate masks in LDS) through the plain entry point; the oracle runs on the
    tokens that close a window."""
    import dataclasses
    wl = synth.scattered_batch("scattered", 61, 262400, 8, 64, 1024, kv_bs=64, kv_blocks=64,
                               cs_rows=8192)
    announce("scattered T=262400 (plain entry point)")
    body, _, guards_ok = run_gpu(wl, debug=False)
    assert guards_ok
    act = np.nonzero(wl.active_mask())[0]
    sub = dataclasses.replace(wl, token_to_req=wl.token_to_req[act], positions=wl.positions[act],
                              slot_mapping=wl.slot_mapping[act],
                              kv_slot_mapping=wl.kv_slot_mapping[act])
    rep = compare(sub, body, oracle.run(sub, THREADS))
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == int(wl.written_mask().sum()) > 1500


def test_large_chunked_prefill_both_schedules():
    """A 32-request chunked prefill of 246,933 tokens, 1,730 of them closing a window, with
    distinct windows in a 4.3 GB pool: the plain entry point (the staged schedule, 965 chunks of
    gate masks) and the compacted schedule write the same records, and the oracle, run on the
    tokens that close a window, fixes every record and every byte that must stay untouched."""
    import dataclasses
    wl = synth.large_prefill()
    announce("large chunked prefill T=246933 (plain entry point)")
    plain, _, ok_plain = run_gpu(wl, debug=False)
    announce("large chunked prefill T=246933 (compacted schedule)")
    body, _, ok_varlen = run_gpu(wl, debug=False, varlen=True)
    assert ok_plain and ok_varlen
    act = np.nonzero(wl.active_mask())[0]
    sub = dataclasses.replace(wl, token_to_req=wl.token_to_req[act], positions=wl.positions[act],
                              slot_mapping=wl.slot_mapping[act],
                              kv_slot_mapping=wl.kv_slot_mapping[act])
    orc = oracle.run(sub, THREADS)
    for got in (plain, body):
        rep = compare(sub, got, orc)
        print(rep.summary(), flush=True)
        assert rep.ok(), rep.summary()
        assert rep["written"] == int(wl.written_mask().sum()) > 1500


def compare_token_range(wl, body, lo, hi):
    """Parity of the records of tokens lo .. hi - 1, and of every byte outside all written
    records, without the oracle's diagnostics for the whole batch: the oracle runs on the
    sub-batch, and the records of the other written tokens are taken from the GPU bytes into
    the initial image (so only bytes outside every record are held to it)."""
    import dataclasses
    from oracle.compare import written_byte_mask
    sl = slice(lo, hi)
    sub = dataclasses.replace(wl, token_to_req=wl.token_to_req[sl], positions=wl.positions[sl],
                              slot_mapping=wl.slot_mapping[sl],
                              kv_slot_mapping=wl.kv_slot_mapping[sl])
    others = wl.written_mask().copy()
    others[sl] = False
    init = wl.k_cache_base.copy()
    m = written_byte_mask(init.size, wl.kv_slot_mapping[others], wl.k_cache.shape[1],
                          wl.k_cache.strides[0])
    init[m] = body[m]
    return compare(sub, body, oracle.run(sub, THREADS), initial_kc_base=init)


@pytest.mark.parametrize("T", [327680, 330017])
def test_staged_beyond_the_gate_masks(T):
    """Batches at and beyond the largest one whose gate masks fit in LDS (1280 chunks of 256
    tokens): at 330,017 tokens the staged schedule counts per block and reads the gates of the
    blocks that hold a stage's tokens again.  Every token is active, so each workgroup runs
    about 1,290 tokens in stages of 64 (windows share the blocks of a 2048-block pool).  The
    oracle checks token ranges spread over several workgroups and stages, and every byte
    outside the written records."""
    wl = synth.shared_pool_batch(f"shared pool T={T}", 5600, T, 2048, 4, 64, -(-T // 64), 512)
    announce(f"staged schedule, every token active, T={T}")
    body, _, guards_ok = run_gpu(wl, debug=False)
    assert guards_ok
    for lo, hi in ((0, 1500), (T // 2 - 700, T // 2 + 800), (T - 1500, T)):
        rep = compare_token_range(wl, body, lo, hi)
        print(rep.summary(), flush=True)
        assert rep.ok(), rep.summary()
        assert rep["written"] == hi - lo


def test_staged_sparse_beyond_the_gate_masks():
    """A 400,000-token scattered batch (about 2,900 tokens close a window) through the plain
    entry point: beyond the gate masks, with count blocks of 256 tokens, the stages locate their
    tokens by reading gates again."""
    import dataclasses
    wl = synth.scattered_batch("scattered 400k", 71, 400000, 8, 64, 1024, kv_bs=64,
                               kv_blocks=64, cs_rows=8192)
    announce("scattered T=400000 (plain entry point)")
    body, _, guards_ok = run_gpu(wl, debug=False)
    assert guards_ok
    act = np.nonzero(wl.active_mask())[0]
    sub = dataclasses.replace(wl, token_to_req=wl.token_to_req[act], positions=wl.positions[act],
                              slot_mapping=wl.slot_mapping[act],
                              kv_slot_mapping=wl.kv_slot_mapping[act])
    rep = compare(sub, body, oracle.run(sub, THREADS))
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == int(wl.written_mask().sum()) > 2500


def test_varlen_nothing_active():
    """3,000 tokens none of which closes a window, and one lone non-boundary token: nothing is
    written and the compacted list is empty."""
    wl = synth.scattered_batch("scattered", 67, 3000, 4, 32, 256, kv_bs=16, kv_blocks=4,
                               cs_rows=2048)
    wl.positions[wl.active_mask()] -= 1
    rep, *_ = check_varlen(wl, "no active token")
    assert rep["written"] == 0
    wl = small(T=1, seed=3)
    wl.positions[:] = 126
    rep, *_ = check_varlen(wl, "one inactive token")
    assert rep["written"] == 0


def test_varlen_gate_and_bad_indices():
    """Gate decisions and out-of-range device indices on the compacted schedule: the gate scan
    lists boundary tokens with slot >= 0, and the main kernel still range-checks each one."""
    wl = small(T=6, seed=7)
    wl.positions[:] = np.array([126, 128, 255, 254, 383, 511], np.int32)
    wl.slot_mapping[:] = np.array([3, 3, 3, 3, -1, 9], np.int32)
    wl.kv_slot_mapping[5] = -1
    rep, body, comp = check_varlen(wl, "varlen gate")
    assert list(np.nonzero(wl.written_mask())[0]) == [2]
    assert np.isfinite(comp[5]).all() and np.isnan(comp[4]).all()

    wl = small(T=6, seed=19, cs_rows=1024)
    wl.positions[:] = 127
    wl.positions[4] = 1023
    wl.token_to_req[0] = wl.block_table.shape[0]
    wl.block_table[1, 15] = wl.state.shape[0] + 5
    wl.kv_slot_mapping[2] = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    wl.cos_sin = wl.cos_sin[:128].copy()
    announce("varlen out-of-range indices")
    body, comp, guards_ok = run_gpu(wl, debug=True, varlen=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [-1, -1, -1, 1, -1, 1]
    wl.kv_slot_mapping[[0, 1, 2, 4]] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[:2]).all() and np.isnan(comp[4]).all() and np.isfinite(comp[2]).all()


# ---------------------------------------------------------------- layouts and extremes on
# every schedule

@pytest.mark.parametrize("mode", ["fanout", "varlen"])
def test_padded_strides_other_schedules(mode):
    """Padded state rows and blocks and a padded k_cache block stride through the fan-out
    (8 splits) and the compacted schedule."""
    wl = small(T=12, seed=17, row_pad=32, block_pad=64, kc_block_pad=48)
    label = f"padded strides ({mode})"
    if mode == "fanout":
        check_ex(wl, 8, label)
    else:
        check_varlen(wl, label)


@pytest.mark.parametrize("mode", ["single", "fanout2", "fanout8", "fanout16", "varlen", "staged"])
def test_cos_sin_rows_67_floats_apart(mode):
    """A cos/sin table whose rows are 67 floats apart (so most rows are only 4-byte aligned),
    NaN in the 3 padding floats: every schedule reads its token's row at rope_row * stride and
    only its first 64 columns (a stray read shows up as NaN codes).  The fan-out fetches the
    row into LDS with one 4-byte load per lane."""
    if mode == "staged":
        wl = synth.shared_pool_batch("cos/sin stride 67 (staged)", 5700, 2048, 2048, 8, 64, 34,
                                     1024)
    else:
        wl = small(T=12, seed=23)
    announce(f"cos/sin row stride 67 ({mode})")
    d = DeviceWorkload(wl)
    rows = d.cos_sin.shape[0]
    padded = torch.full((rows, 67), float("nan"), dtype=torch.float32, device=d.state.device)
    padded[:, :64] = d.cos_sin
    d.cos_sin = padded[:, :64]
    assert d.cos_sin.stride() == (67, 1)
    if mode.startswith("fanout"):
        comp = d.run(debug=True, splits=int(mode[6:]))
    else:
        comp = d.run(debug=True, varlen=(mode == "varlen"))
    body, guards_ok = d.k_cache_bytes()
    assert guards_ok, "k_cache guard bands were written"
    orc = oracle.run(wl, THREADS)
    rep = compare(wl, body, orc, gpu_compressed=comp.cpu().numpy())
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == wl.num_tokens


@pytest.mark.parametrize("mode", ["single", "fanout", "varlen"])
def test_largest_position_is_skipped(mode):
    """A boundary token at position 2^31 - 1 needs block-table column 2^28 - 1: no table is that
    wide, so the token is skipped (nothing written, no overflow); the others are unaffected."""
    wl = small(T=5, seed=19)
    wl.positions[2] = 2 ** 31 - 1
    announce(f"largest position ({mode})")
    kw = {"splits": 4} if mode == "fanout" else ({"varlen": True} if mode == "varlen" else {})
    body, comp, guards_ok = run_gpu(wl, debug=True, **kw)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [1, 1, -1, 1, 1]
    wl.kv_slot_mapping[2] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[2]).all()


# ---------------------------------------------------------------- pool beyond 2^31 floats

def test_state_pool_beyond_2_31_floats():
    """A 17.2 GB state pool of 2^19 + 64 blocks (more than 2^32 floats).  A 2048-token batch's
    2048 distinct blocks are placed at random ids across the whole pool, the last block among
    them, so row addresses pass 2^31 and 2^32 floats.  The plain entry point (staged at 2048
    tokens), a 40-token single pass, the fan-out and the compacted schedule each agree with
    the oracle run on the compact pool: moving blocks and renumbering the table changes no
    result (a pinned property of the oracle)."""
    n_big = (1 << 19) + 64
    wl = synth.shared_pool_batch("pool beyond 2^31 floats", 7300, 2048, 2048, 8, 64, 34, 1024)
    n_small = wl.state.shape[0]
    assert wl.block_table.min() >= 0 and wl.block_table.max() < n_small
    rng = np.random.default_rng(7301)
    ids = rng.choice(n_big - 1, size=n_small - 1, replace=False)
    ids = rng.permutation(np.append(ids, n_big - 1)).astype(np.int64)
    cols = (wl.positions // 8)[:, None] - np.arange(16)[None, :]     # each token's window
    top = int(ids[wl.block_table[np.arange(wl.num_tokens)[:, None], cols]].max())
    assert top == n_big - 1 and top * 8 * 1024 > (1 << 32)
    announce(f"pool beyond 2^31 floats: allocating {n_big} blocks ({n_big * 32 / 2**20:.1f} GiB)")
    pool, big_table = relocated_pool(wl, n_big, ids)
    sub = dataclasses.replace(wl, name="pool beyond 2^31 floats, 40 tokens",
                              token_to_req=wl.token_to_req[:40], positions=wl.positions[:40],
                              slot_mapping=wl.slot_mapping[:40],
                              kv_slot_mapping=wl.kv_slot_mapping[:40])
    try:
        for w, kw, label in ((wl, {}, "plain entry point (staged), 2048 tokens"),
                             (sub, {}, "plain entry point (single pass), 40 tokens"),
                             (sub, {"splits": 4}, "fan-out splits=4, 40 tokens"),
                             (wl, {"varlen": True}, "compacted schedule, 2048 tokens")):
            announce(f"pool beyond 2^31 floats: {label}")
            d = DeviceWorkload(w, state=(pool, pool))
            d.block_table = big_table
            comp = d.run(debug=True, **kw)
            body, guards_ok = d.k_cache_bytes()
            assert guards_ok, "k_cache guard bands were written"
            rep = compare(w, body, oracle.run(w, THREADS), gpu_compressed=comp.cpu().numpy())
            print(rep.summary(), flush=True)
            assert rep.ok(), rep.summary()
            assert rep["written"] == w.num_tokens
    finally:
        del pool
        torch.cuda.empty_cache()


# ---------------------------------------------------------------- error attribution

def loaded_hip_runtime():
    """The HIP runtime library already mapped into this process (the one the library uses)."""
    import ctypes
    paths = sorted({line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line})
    assert len(paths) == 1, paths
    return ctypes.CDLL(paths[0])


def test_earlier_hip_error_is_not_reported_as_a_launch_failure():
    """A failed HIP call before the compress call (hipSetDevice on a device that does not exist)
    leaves an error in the thread's last-error slot.  Every entry point reports only the status
    of its own launches, so the call succeeds, writes the same bytes, and the earlier error is
    still there for whoever made it."""
    import paged_kv_cache_fp32_amd as c128
    hip = loaded_hip_runtime()
    wl = small(T=9, seed=77)
    d = DeviceWorkload(wl)
    ws = c128.fanout_workspace(wl.num_tokens, 4)
    vws = torch.empty(c128.varlen_workspace_bytes(wl.num_tokens), dtype=torch.uint8,
                      device="cuda")
    torch.cuda.synchronize()
    announce("earlier HIP error, then the entry points")
    for label, call in (("plain", lambda: c128.compress_store(*d.args())),
                        ("fan-out", lambda: c128.compress_store_ex(*d.args(), workspace=ws,
                                                                   splits=4)),
                        ("compacted", lambda: c128.compress_store_varlen(*d.args(),
                                                                         workspace=vws))):
        planted = hip.hipSetDevice(12345)
        assert planted != 0
        call()                                   # raises if the call reported an error
        assert hip.hipGetLastError() == planted, label   # read (and clear) the planted error
        torch.cuda.synchronize()
    body, guards_ok = d.k_cache_bytes()
    assert guards_ok
    rep = compare(wl, body, oracle.run(wl, THREADS))
    assert rep.ok(), rep.summary()
