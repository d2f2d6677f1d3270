"""GPU parity of the C4 compressor kernel (dsv4_c4_compress_store) against the CPU oracle:
decode batches over several state block sizes (including windows at position 3, whose
previous window does not exist), a chunked-prefill batch where every fourth token is active,
gate decisions and out-of-range device indices, and the 16384-token batch the bench times."""

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


def c4_batch(T, seed, state_bs=8, k_max=16, kv_bs=16, score_std=2 ** 0.5):
    return synth.c4_decode_batch(f"c4 decode T={T} bs={state_bs}", seed, T,
                                 T * (-(-8 // state_bs) + 1) + 8, k_max,
                                 -(-4 * k_max // state_bs) + 1, kv_bs=kv_bs,
                                 kv_blocks=-(-2 * T // kv_bs), cs_rows=4 * k_max + 4,
                                 state_bs=state_bs, score_std=score_std)


@pytest.mark.parametrize("state_bs", [8, 4, 16, 1])
@pytest.mark.parametrize("T", [1, 5, 64, 1000])
def test_c4_decode_parity(T, state_bs):
    wl = c4_batch(T, 300 + T + state_bs, state_bs=state_bs, k_max=3 if T == 1 else 16)
    rep, *_ = check(wl, f"c4 decode T={T} state bs={state_bs}")
    assert rep["written"] == T


def test_c4_first_windows():
    """Every token at position 3 (only the current window exists) or 7 (first full overlap)."""
    wl = c4_batch(40, 41, k_max=2)
    assert set(wl.positions.tolist()) == {3, 7}
    rep, *_ = check(wl, "c4 positions 3 and 7")
    assert rep["written"] == 40


def test_c4_varlen_prefill():
    wl = synth.c4_varlen_prefill("c4 varlen prefill", 1202, 16, 512, 1024, kv_bs=64,
                                 cs_rows=1600)
    rep, *_ = check(wl, "c4 varlen prefill")
    assert rep["written"] == int(wl.written_mask().sum()) > 300


def test_c4_peaky_scores():
    wl = c4_batch(256, 53, score_std=4.0)
    check(wl, "c4 peaky scores (std 4)")


def test_c4_gate_and_bad_indices():
    wl = c4_batch(8, 61, k_max=8)
    wl.positions[:] = np.array([2, 4, 7, 6, 11, 15, 19, 23], np.int32)
    wl.slot_mapping[:] = np.array([1, 1, 1, 1, -1, 1, 1, 1], np.int32)
    wl.kv_slot_mapping[5] = -1
    wl.token_to_req[6] = wl.block_table.shape[0]          # request out of range
    wl.kv_slot_mapping[7] = wl.k_cache.shape[0] * wl.k_cache.shape[1]  # kv slot out of range
    announce("c4 gate / bad indices")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [0, 0, 1, 0, 0, 2, -1, -1]
    wl.kv_slot_mapping[[6, 7]] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert rep["written"] == 1
    assert np.isfinite(comp[2]).all() and np.isfinite(comp[5]).all() and np.isfinite(comp[7]).all()
    assert np.isnan(comp[[0, 1, 3, 4, 6]]).all()


def test_c4_bad_block_id_and_rope_row():
    wl = c4_batch(4, 67, k_max=8)
    wl.positions[:] = 31
    bs = wl.state.shape[1]
    wl.block_table[1, 31 // bs] = wl.state.shape[0] + 3   # block id out of range
    wl.cos_sin = wl.cos_sin[:28].copy()                    # rope row 28 missing for pos 31
    wl.positions[3] = 23                                    # rope row 20: present
    announce("c4 bad block id / rope row")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert list(orc.status) == [-1, -1, -1, 1]
    wl.kv_slot_mapping[[0, 1, 2]] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()


def test_c4_large_batch():
    """The 16384-token C4 decode batch of the bench, every token against the oracle."""
    wl = synth.c4_decode_batch("c4 decode T=16384", 1005, 16384, 16384 * 2, 1024, 512,
                               kv_bs=64, kv_blocks=256, cs_rows=4096)
    rep, *_ = check(wl, "c4 decode T=16384")
    assert rep["written"] == 16384


def test_c4_empty_batch_and_zero_window():
    """T = 0 is a no-op; an all-zero window gives zero codes, scale bytes 105 (e = -22 from the
    1e-4 floor) and a zero pad byte."""
    import torch

    import paged_kv_cache_fp32_amd as c128
    from synth.device import DeviceWorkload
    announce("c4 T = 0")
    d = DeviceWorkload(c4_batch(1, 83))
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    before = d.kc_buf.clone()
    c128.c4_compress_store(d.state, d.block_table, e, e, e, d.rms_w, 1e-6, d.cos_sin, d.k_cache,
                           e)
    torch.cuda.synchronize()
    assert torch.equal(before, d.kc_buf)
    wl = c4_batch(4, 89)
    wl.state[:, :, :1024] = 0.0
    rep, body, comp = check(wl, "c4 all-zero windows")
    assert np.all(comp == 0.0)
    kc = wl.k_cache
    for t in range(4):
        s = int(wl.kv_slot_mapping[t])
        blk, off = s // kc.shape[1], s % kc.shape[1]
        base = blk * kc.strides[0]
        assert np.all(body[base + off * 576: base + off * 576 + 448] & 0x7F == 0)
        scl = body[base + kc.shape[1] * 576 + off * 8: base + kc.shape[1] * 576 + off * 8 + 8]
        assert list(scl) == [105] * 7 + [0]


def test_c4_side_stream():
    import torch

    import paged_kv_cache_fp32_amd as c128
    from synth.device import DeviceWorkload
    wl = c4_batch(16, 97)
    announce("c4 side stream")
    d = DeviceWorkload(wl)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c128.c4_compress_store(*d.args())
    s.synchronize()
    body, ok = d.k_cache_bytes()
    rep = compare(wl, body, oracle.run(wl, 2))
    assert ok and rep.ok(), rep.summary()


def test_c4_padded_strides_and_largest_position():
    """Padded state rows/blocks and k_cache blocks; a token at position 2^31 - 1 (a boundary of
    ratio 4) is skipped without overflow."""
    wl = synth.c4_decode_batch("c4 padded", 107, 24, 24 * 2 + 8, 16, 9, kv_bs=16, kv_blocks=3,
                               cs_rows=68, row_pad=16, block_pad=32, kc_block_pad=24)
    check(wl, "c4 padded strides")
    wl.positions[5] = 2 ** 31 - 1
    announce("c4 largest position")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok
    orc = oracle.run(wl, 2)
    assert orc.status[5] == -1 and (np.delete(orc.status, 5) == 1).all()
    wl.kv_slot_mapping[5] = -1
    rep = compare(wl, body, orc)
    assert rep.ok(), rep.summary()
    assert np.isnan(comp[5]).all()


def test_c4_state_pool_beyond_2_31_floats():
    """A 17.2 GB C4 state pool (more than 2^32 floats: rows of 2048 floats, blocks of 8 rows).
    A 1000-token batch's blocks are placed at random ids across it, one window block at the last
    id, and the kernel agrees with the oracle run on the compact pool (relocating blocks and
    renumbering the table changes no result)."""
    wl = c4_batch(1000, 7400 + 2048, state_bs=8)
    n_small, sbs = wl.state.shape[0], wl.state.shape[1]
    n_big = (1 << 32) // (sbs * 2048) + 64
    rng = np.random.default_rng(7401)
    ids = rng.choice(n_big - 1, size=n_small, replace=False).astype(np.int64)
    pos = wl.positions.astype(np.int64)
    first = int(wl.block_table[0, pos[0] // sbs])          # a block that token 0's window reads
    ids[first] = n_big - 1
    assert (n_big - 1) * sbs * 2048 > (1 << 32)
    announce(f"C4 pool beyond 2^31 floats: {n_big} blocks")
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
def test_c4_extreme_scores(score_std):
    """Scores spread so far that each column's softmax is one-hot or nearly so: no overflow, no
    NaN, and near ties within the compressed tolerance."""
    wl = c4_batch(300, 900 + int(score_std), score_std=score_std)
    rep, *_ = check(wl, f"c4 scores std {score_std:g}")
    assert rep["written"] == 300


@pytest.mark.parametrize("T", [8192, 13001, 30001])
def test_c4_wide_workgroups_mixed_batch(T):
    """From 8192 tokens, while one round of 12-wave workgroups (one per CU) covers the batch, a
    workgroup gates all of its tokens first and deals the passing ones out to its waves (up to 16
    tokens a wave, resolved 8 at a time: 30001 tokens take 10).  Every kind of token in one such
    batch: a seeded 30% with state slot -1, 10% moved off the window boundary, windows at
    position 3, 5% with no kv slot and five request ids out of range; T leaves a ragged last
    workgroup."""
    wl = c4_batch(T, 1500 + T, k_max=40)
    rng = np.random.default_rng(1500 + T)
    wl.slot_mapping[rng.random(T) < 0.3] = -1
    wl.positions[rng.random(T) < 0.1] -= 1
    wl.kv_slot_mapping[rng.random(T) < 0.05] = -1
    bad = rng.choice(T, 5, replace=False)
    wl.token_to_req[bad] = wl.block_table.shape[0]
    assert (wl.positions == 3).any()
    announce(f"c4 wide workgroups, mixed batch T={T}")
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


def test_c4_wide_rounds_on_dense_workgroups():
    """A 60,000-token batch: 20,000 decode tokens that all write, then 40,000 that do not close a
    window.  One round of wide workgroups holds it at 20 tokens a wave, so every workgroup over
    the dense part deals 20 writing tokens to each wave, more than its 16-record stage: it
    inserts twice (16 records a wave, then 4); the workgroups over the rest insert nothing."""
    wl = c4_batch(20000, 1530, k_max=40)
    extra = 40000
    rng = np.random.default_rng(1531)
    wl.positions = np.concatenate(
        [wl.positions, (4 * rng.integers(1, 40, extra) + 1).astype(np.int32)])
    wl.slot_mapping = np.concatenate([wl.slot_mapping, np.zeros(extra, np.int32)])
    wl.token_to_req = np.concatenate([wl.token_to_req, np.zeros(extra, np.int32)])
    wl.kv_slot_mapping = np.concatenate([wl.kv_slot_mapping, np.full(extra, -1, np.int32)])
    assert wl.num_tokens == 60000
    rep, *_ = check(wl, "c4 dense workgroups in two rounds, T=60000")
    assert rep["written"] == 20000


@pytest.mark.parametrize("nreq,seed", [(160, 1210), (210, 1213)])
def test_c4_prefill_beyond_one_wide_round(nreq, seed):
    """Chunked prefills of 87,880 and 109,751 tokens (about a fifth of them writing), beyond the
    49,152 tokens that 16 tokens a wave cover: wide waves gate 29 and 36 tokens each and deal the
    writing ones, about 7 and 8 a wave, into their stages."""
    announce(f"c4 prefill beyond one wide round: generating {nreq} requests")
    wl = synth.c4_varlen_prefill(f"c4 varlen prefill {nreq} req", seed, nreq, 1024, 512,
                                 kv_bs=64, cs_rows=2048)
    assert wl.num_tokens > 49152
    rep, *_ = check(wl, f"c4 prefill beyond one wide round T={wl.num_tokens}")
    assert rep["written"] == int(wl.written_mask().sum()) > 15000


@pytest.mark.parametrize("nreq,seed", [(32, 1203), (64, 1202)])
def test_c4_wide_workgroups_sparse_prefill(nreq, seed):
    """Chunked prefills of about 14k and 32k tokens (one wide round, one or two batches a wave;
    about a quarter of the tokens close a window, and 10% of the slots are dropped)."""
    wl = synth.c4_varlen_prefill(f"c4 varlen prefill {nreq} req", seed, nreq, 1024, 4096,
                                 kv_bs=64, cs_rows=8192)
    assert 8192 <= wl.num_tokens <= 49152
    rep, *_ = check(wl, f"c4 sparse prefill T={wl.num_tokens}")
    assert rep["written"] == int(wl.written_mask().sum()) > 2000
