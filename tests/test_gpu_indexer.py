"""GPU parity of the indexer's FP8 compressor kernel (dsv4_indexer_compress_store) against the
CPU oracle: decode batches over several state and cache block sizes (including windows at
position 3), gate decisions and out-of-range device indices, and the 16384-token batch the
bench times."""

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


def check(wl, label, debug=True):
    announce(label)
    body, comp, guards_ok = run_gpu(wl, debug=debug)
    assert guards_ok, "k_cache guard bands were written"
    orc = oracle.run(wl, THREADS)
    rep = compare(wl, body, orc, gpu_compressed=comp)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    return rep, body, comp


def idx_batch(T, seed, state_bs=8, k_max=16, kv_bs=16, score_std=2 ** 0.5, kc_block_pad=0):
    return synth.indexer_decode_batch(f"indexer T={T} bs={state_bs}", seed, T,
                                      T * (-(-8 // state_bs) + 1) + 8, k_max,
                                      -(-4 * k_max // state_bs) + 1, kv_bs=kv_bs,
                                      kv_blocks=-(-2 * T // kv_bs), cs_rows=4 * k_max + 4,
                                      state_bs=state_bs, score_std=score_std,
                                      kc_block_pad=kc_block_pad)


@pytest.mark.parametrize("state_bs", [8, 4, 1])
@pytest.mark.parametrize("T", [1, 5, 300, 2500])
def test_indexer_decode_parity(T, state_bs):
    wl = idx_batch(T, 500 + T + state_bs, state_bs=state_bs, k_max=3 if T == 1 else 40)
    rep, *_ = check(wl, f"indexer decode T={T} state bs={state_bs}")
    assert rep["written"] == T


@pytest.mark.parametrize("kv_bs,pad", [(1, 0), (3, 4), (64, 8)])
def test_indexer_cache_block_sizes(kv_bs, pad):
    wl = idx_batch(40, 71, kv_bs=kv_bs, kc_block_pad=pad)
    check(wl, f"indexer cache bs={kv_bs} pad={pad}")


def test_indexer_first_windows_and_peaky_scores():
    wl = idx_batch(64, 73, k_max=2, score_std=4.0)
    assert set(wl.positions.tolist()) == {3, 7}
    check(wl, "indexer positions 3 and 7, score std 4")


def test_indexer_gate_and_bad_indices():
    wl = idx_batch(8, 79, k_max=8)
    wl.positions[:] = np.array([2, 4, 7, 6, 11, 15, 19, 23], np.int32)
    wl.slot_mapping[:] = np.array([1, 1, 1, 1, -1, 1, 1, 1], np.int32)
    wl.kv_slot_mapping[5] = -1
    wl.token_to_req[6] = wl.block_table.shape[0]
    wl.kv_slot_mapping[7] = wl.k_cache.shape[0] * wl.k_cache.shape[1]
    announce("indexer gate / bad indices")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [0, 0, 1, 0, 0, 2, -1, -1]
    wl.kv_slot_mapping[[6, 7]] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert rep["written"] == 1
    assert np.isnan(comp[[0, 1, 3, 4, 6]]).all() and np.isfinite(comp[[2, 5, 7]]).all()


def test_indexer_large_batch():
    wl = synth.indexer_decode_batch("indexer decode T=16384", 1006, 16384, 16384 * 2, 1024, 512,
                                    kv_bs=64, kv_blocks=256, cs_rows=4096)
    rep, *_ = check(wl, "indexer decode T=16384")
    assert rep["written"] == 16384


def test_indexer_empty_batch_and_zero_window():
    """T = 0 is a no-op; an all-zero window gives zero codes and the scale 2^-22 (the 1e-4
    floor: ceil(log2(1e-4 / 448)) = -22)."""
    import torch

    import paged_kv_cache_fp32_amd as c128
    from synth.device import DeviceWorkload
    announce("indexer T = 0")
    d = DeviceWorkload(idx_batch(1, 101))
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    before = d.kc_buf.clone()
    c128.indexer_compress_store(d.state, d.block_table, e, e, e, d.rms_w, 1e-6, d.cos_sin,
                                d.k_cache, e)
    torch.cuda.synchronize()
    assert torch.equal(before, d.kc_buf)
    wl = idx_batch(4, 103)
    wl.state[:, :, :256] = 0.0
    rep, body, comp = check(wl, "indexer all-zero windows")
    assert np.all(comp == 0.0)
    kc = wl.k_cache
    for t in range(4):
        s = int(wl.kv_slot_mapping[t])
        blk, off = s // kc.shape[1], s % kc.shape[1]
        base = blk * kc.strides[0]
        assert np.all(body[base + off * 128: base + off * 128 + 128] & 0x7F == 0)
        sc = body[base + kc.shape[1] * 128 + off * 4: base + kc.shape[1] * 128 + off * 4 + 4]
        assert float(sc.view("<f4")[0]) == 2.0 ** -22


def test_indexer_padded_strides_and_largest_position():
    wl = synth.indexer_decode_batch("indexer padded", 109, 24, 24 * 2 + 8, 16, 9, kv_bs=16,
                                    kv_blocks=3, cs_rows=68, row_pad=16, block_pad=32,
                                    kc_block_pad=12)
    check(wl, "indexer padded strides")
    wl.positions[5] = 2 ** 31 - 1
    announce("indexer largest position")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert orc.status[5] == -1 and (np.delete(orc.status, 5) == 1).all()
    wl.kv_slot_mapping[5] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[5]).all()


def test_indexer_state_pool_beyond_2_31_floats():
    """A 17.2 GB indexer state pool (more than 2^32 floats: rows of 512 floats, blocks of 8 rows).
    A 2500-token batch's blocks are placed at random ids across it, one window block at the last
    id, and the kernel agrees with the oracle run on the compact pool (relocating blocks and
    renumbering the table changes no result)."""
    wl = idx_batch(2500, 7400 + 512, state_bs=8)
    n_small, sbs = wl.state.shape[0], wl.state.shape[1]
    n_big = (1 << 32) // (sbs * 512) + 64
    rng = np.random.default_rng(7401)
    ids = rng.choice(n_big - 1, size=n_small, replace=False).astype(np.int64)
    pos = wl.positions.astype(np.int64)
    first = int(wl.block_table[0, pos[0] // sbs])          # a block that token 0's window reads
    ids[first] = n_big - 1
    assert (n_big - 1) * sbs * 512 > (1 << 32)
    announce(f"indexer pool beyond 2^31 floats: {n_big} blocks")
    pool, table = relocated_pool(wl, n_big, ids)
    try:
        d = DeviceWorkload(wl, state=(pool, pool))
        d.block_table = table
        comp = d.run(debug=True)
        body, guards_ok = d.k_cache_bytes()
        assert guards_ok, "k_cache guard bands were written"
        rep = compare(wl, body, oracle.run(wl, THREADS), gpu_compressed=comp.cpu().numpy())
        print(rep.summary(), flush=True)
        assert rep.ok(), rep.summary()
        assert rep["written"] == wl.num_tokens
    finally:
        del pool
        torch.cuda.empty_cache()


@pytest.mark.parametrize("score_std", [1e2, 1e4])
def test_indexer_extreme_scores(score_std):
    """Scores spread so far that each column's softmax is one-hot or nearly so: no overflow, no
    NaN, and near ties within the compressed tolerance."""
    wl = idx_batch(300, 950 + int(score_std), score_std=score_std)
    rep, *_ = check(wl, f"indexer scores std {score_std:g}")
    assert rep["written"] == 300


@pytest.mark.parametrize("T", [8193, 20001])
def test_indexer_pipelined_mixed_batch(T):
    """Beyond 8192 tokens a wave takes several tokens and keeps the next token's loads in flight
    while it reduces the current one.  Every kind of token in one batch there: a seeded 30% with
    state slot -1, 10% moved off the window boundary, windows at position 3, 5% with no kv slot
    and five request ids out of range; T leaves a ragged last wave."""
    wl = idx_batch(T, 1300 + T, k_max=40)
    rng = np.random.default_rng(1300 + T)
    wl.slot_mapping[rng.random(T) < 0.3] = -1
    wl.positions[rng.random(T) < 0.1] -= 1
    wl.kv_slot_mapping[rng.random(T) < 0.05] = -1
    bad = rng.choice(T, 5, replace=False)
    wl.token_to_req[bad] = wl.block_table.shape[0]
    assert (wl.positions == 3).any()
    announce(f"indexer pipelined mixed batch T={T}")
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
def test_indexer_chunked_prefill(nreq, seed, max_start):
    """Chunked prefills of 33,908 and 107,030 tokens: contiguous positions per request, about one
    token in four closing a window, 10% of the state slots dropped, a distinct kv slot each."""
    wl = synth.indexer_varlen_prefill(f"indexer prefill {nreq} req", seed, nreq, 1024,
                                      max_start, kv_bs=64, cs_rows=8192, fp4=False)
    rep, *_ = check(wl, f"indexer prefill T={wl.num_tokens}")
    assert rep["written"] == int(wl.written_mask().sum()) > 7000
