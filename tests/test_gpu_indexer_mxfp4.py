"""GPU parity of the indexer's MXFP4 cache (dsv4_indexer_mxfp4_compress_store) against the CPU
oracle: the kernel's E2M1 encoder over its whole domain, decode batches over several state and
cache block sizes (windows at position 3 included), gate decisions and out-of-range device
indices, all-zero windows, padded strides, and the 16384-token batch the bench times."""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fp32_amd as c128
import synth
from oracle.compare import compare
from synth.device import DeviceWorkload, run_gpu

pytestmark = pytest.mark.gpu

THREADS = synth.default_threads()


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def check(wl, label, debug=True):
    announce(label)
    body, comp, guards_ok = run_gpu(wl, debug=debug)
    assert guards_ok, "k_cache guard bands were written"
    orc = oracle.run(wl, THREADS)
    rep = compare(wl, body, orc, gpu_compressed=comp)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    return rep, body, comp


def fp4_batch(T, seed, state_bs=8, k_max=16, kv_bs=16, score_std=2 ** 0.5, kc_block_pad=0):
    return synth.indexer_decode_batch(f"mxfp4 T={T} bs={state_bs}", seed, T,
                                      T * (-(-8 // state_bs) + 1) + 8, k_max,
                                      -(-4 * k_max // state_bs) + 1, kv_bs=kv_bs,
                                      kv_blocks=-(-2 * T // kv_bs), cs_rows=4 * k_max + 4,
                                      state_bs=state_bs, score_std=score_std,
                                      kc_block_pad=kc_block_pad, fp4=True)


def test_e2m1_encoder_exhaustive():
    """The kernel's E2M1 encoder on every bf16 value with |x| <= 16 (the quantiser's domain
    after the power-of-two scale, and saturation), the fp32 neighbours of every rounding
    midpoint, signed zeros, fp32 subnormals and large magnitudes, against the oracle's encoder
    (pinned by brute force over the OCP table)."""
    bits = np.arange(0x10000, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 16.0)]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9))])
    extra = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-39, 3e38, -3e38, 6.5, 7.0, 100.0], np.float32)
    x = np.concatenate([vals, near, -near, extra]).astype(np.float32)
    announce(f"e2m1 encoder: {x.size} values")
    got = c128.e2m1_encode(torch.from_numpy(x).cuda()).cpu().numpy()
    want = oracle.e2m1_codes(x.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("state_bs", [8, 4, 1])
@pytest.mark.parametrize("T", [1, 5, 300, 2500])
def test_mxfp4_decode_parity(T, state_bs):
    wl = fp4_batch(T, 700 + T + state_bs, state_bs=state_bs, k_max=3 if T == 1 else 40)
    rep, *_ = check(wl, f"mxfp4 decode T={T} state bs={state_bs}")
    assert rep["written"] == T


@pytest.mark.parametrize("kv_bs,pad", [(1, 0), (3, 4), (64, 8)])
def test_mxfp4_cache_block_sizes(kv_bs, pad):
    wl = fp4_batch(40, 771, kv_bs=kv_bs, kc_block_pad=pad)
    check(wl, f"mxfp4 cache bs={kv_bs} pad={pad}")


def test_mxfp4_first_windows_and_peaky_scores():
    wl = fp4_batch(64, 773, k_max=2, score_std=4.0)
    assert set(wl.positions.tolist()) == {3, 7}
    check(wl, "mxfp4 positions 3 and 7, score std 4")


def test_mxfp4_gate_and_bad_indices():
    wl = fp4_batch(8, 779, k_max=8)
    wl.positions[:] = np.array([2, 4, 7, 6, 11, 15, 19, 23], np.int32)
    wl.slot_mapping[:] = np.array([1, 1, 1, 1, -1, 1, 1, 1], np.int32)
    wl.kv_slot_mapping[5] = -1
    wl.token_to_req[6] = wl.block_table.shape[0]
    wl.kv_slot_mapping[7] = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    announce("mxfp4 gate / bad indices")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [0, 0, 1, 0, 0, 2, -1, -1]
    wl.kv_slot_mapping[[6, 7]] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert rep["written"] == 1
    assert np.isnan(comp[[0, 1, 3, 4, 6]]).all() and np.isfinite(comp[[2, 5, 7]]).all()


def test_mxfp4_large_batch():
    wl = synth.indexer_decode_batch("mxfp4 decode T=16384", 1106, 16384, 16384 * 2, 1024, 512,
                                    kv_bs=64, kv_blocks=256, cs_rows=4096, fp4=True)
    rep, *_ = check(wl, "mxfp4 decode T=16384")
    assert rep["written"] == 16384


def test_mxfp4_empty_batch_and_zero_window():
    """T = 0 is a no-op; an all-zero window gives zero magnitudes in every code and the scale
    byte 1 in every block (the 6 * 2^-126 floor: exponent -126)."""
    announce("mxfp4 T = 0")
    d = DeviceWorkload(fp4_batch(1, 801))
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    before = d.kc_buf.clone()
    c128.indexer_mxfp4_compress_store(d.state, d.block_table, e, e, e, d.rms_w, 1e-6,
                                      d.cos_sin, d.k_cache, e)
    torch.cuda.synchronize()
    assert torch.equal(before, d.kc_buf)
    wl = fp4_batch(4, 803)
    wl.state[:, :, :256] = 0.0
    rep, body, comp = check(wl, "mxfp4 all-zero windows")
    assert np.all(comp == 0.0)
    kc = wl.k_cache
    for t in range(4):
        s = int(wl.kv_slot_mapping[t])
        blk, off = s // kc.shape[1], s % kc.shape[1]
        base = blk * kc.strides[0]
        assert np.all(body[base + off * 64: base + off * 64 + 64] & 0x77 == 0)
        sc = body[base + kc.shape[1] * 64 + off * 4: base + kc.shape[1] * 64 + off * 4 + 4]
        assert np.all(sc == 1)


def test_mxfp4_padded_strides_and_largest_position():
    wl = synth.indexer_decode_batch("mxfp4 padded", 809, 24, 24 * 2 + 8, 16, 9, kv_bs=16,
                                    kv_blocks=3, cs_rows=68, row_pad=16, block_pad=32,
                                    kc_block_pad=12, fp4=True)
    check(wl, "mxfp4 padded strides")
    wl.positions[5] = 2 ** 31 - 1
    announce("mxfp4 largest position")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert orc.status[5] == -1 and (np.delete(orc.status, 5) == 1).all()
    wl.kv_slot_mapping[5] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[5]).all()


@pytest.mark.parametrize("T", [12290])
def test_mxfp4_pipelined_mixed_batch(T):
    """Beyond 8192 tokens a wave takes several tokens and keeps the next token's loads in flight
    while it reduces the current one.  Every kind of token in one batch there: a seeded 30% with
    state slot -1, 10% moved off the window boundary, windows at position 3, 5% with no kv slot
    and five request ids out of range; T leaves a ragged last wave."""
    wl = fp4_batch(T, 1400 + T, k_max=40)
    rng = np.random.default_rng(1400 + T)
    wl.slot_mapping[rng.random(T) < 0.3] = -1
    wl.positions[rng.random(T) < 0.1] -= 1
    wl.kv_slot_mapping[rng.random(T) < 0.05] = -1
    bad = rng.choice(T, 5, replace=False)
    wl.token_to_req[bad] = wl.block_table.shape[0]
    assert (wl.positions == 3).any()
    announce(f"mxfp4 pipelined mixed batch T={T}")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok, "k_cache guard bands were written"
    orc = oracle.run(wl, THREADS)
    gate = (wl.slot_mapping >= 0) & (wl.positions % 4 == 3)
    assert (orc.status[~gate] == 0).all() and (orc.status[bad[gate[bad]]] == -1).all()
    computed = gate & (wl.token_to_req < wl.block_table.shape[0])
    assert np.isfinite(comp[computed]).all() and np.isnan(comp[~computed]).all()
    wl.kv_slot_mapping[orc.status == -1] = -1
    rep = compare(wl, body, orc, gpu_compressed=comp)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == int((orc.status == 1).sum()) > T // 2


@pytest.mark.parametrize("nreq,seed,max_start", [(64, 1402, 4096), (210, 1413, 512)])
def test_mxfp4_chunked_prefill(nreq, seed, max_start):
    """Chunked prefills of 33,908 and 107,030 tokens: contiguous positions per request, about one
    token in four closing a window, 10% of the state slots dropped, a distinct kv slot each."""
    wl = synth.indexer_varlen_prefill(f"indexer mxfp4 prefill {nreq} req", seed, nreq, 1024,
                                      max_start, kv_bs=64, cs_rows=8192, fp4=True)
    rep, *_ = check(wl, f"indexer mxfp4 prefill T={wl.num_tokens}")
    assert rep["written"] == int(wl.written_mask().sum()) > 7000
