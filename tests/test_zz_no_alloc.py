"""The allocation-free compacted schedule (dsv4_c128_compress_store_varlen_noalloc) against the
compacted schedule with a caller workspace (dsv4_c128_compress_store_varlen), through the C ABI:
identical k_cache bytes and pooled vectors on two calls in a row, the second on a smaller
batch, both also within the oracle's pass criteria.  Nothing of the first call's scratch
contents may leak into the second."""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.compare import compare
from synth.device import DeviceWorkload

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_both(wl, debug=True):
    """(bytes, pooled vectors or None) of the workspace entry point, then of the allocation-free
    one, each on a fresh copy of the workload's k_cache."""
    import paged_kv_cache_fp32_amd as c128
    out = []
    for noalloc in (False, True):
        d = DeviceWorkload(wl)
        comp = torch.full((wl.num_tokens, 512), float("nan"), dtype=torch.float32,
                          device="cuda") if debug else None
        torch.cuda.synchronize()
        if noalloc:
            before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
            c128.compress_store_varlen_noalloc(*d.args(), compressed_out=comp)
            after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
            assert after == before, "the binding allocated device memory"
        else:
            ws = torch.empty(c128.varlen_workspace_bytes(wl.num_tokens), dtype=torch.uint8,
                             device="cuda")
            c128.compress_store_varlen(*d.args(), compressed_out=comp, workspace=ws)
        torch.cuda.synchronize()
        body, ok = d.k_cache_bytes()
        assert ok, "k_cache guard bands were written"
        out.append((body, comp.cpu().numpy() if debug else None))
        del d
    return out


def test_noalloc_matches_the_workspace_entry_point():
    big = synth.config2()
    smaller = synth.varlen_prefill("varlen prefill, 16 requests", 1203, 16, 700, 2048, 8192,
                                   kv_bs=16, cs_rows=4096)
    assert smaller.num_tokens < big.num_tokens
    for wl in (big, smaller):
        announce(f"no-alloc vs workspace: {wl.name} T={wl.num_tokens}")
        (ref, ref_c), (got, got_c) = run_both(wl)
        assert np.array_equal(got, ref)
        assert np.array_equal(np.isnan(got_c), np.isnan(ref_c))
        assert np.array_equal(np.nan_to_num(got_c), np.nan_to_num(ref_c))
        rep = compare(wl, got, oracle.run(wl, synth.default_threads()), gpu_compressed=got_c)
        print(rep.summary(), flush=True)
        assert rep.ok(), rep.summary()
        assert rep["written"] == int(wl.written_mask().sum()) > 20


def test_noalloc_at_its_token_limit():
    """2^20 tokens, the most the allocation-free schedule's scratch holds (scattered positions,
    about one in 128 closing a window): the same bytes as the workspace entry point, and every
    record and untouched byte as the oracle fixes them on the sub-batch of the tokens that close
    a window (the same bytes: the others write nothing)."""
    import dataclasses

    import paged_kv_cache_fp32_amd as c128
    T = c128.VARLEN_NOALLOC_MAX_TOKENS
    wl = synth.scattered_batch("no-alloc limit", 67, T, 8, 64, 1024, kv_bs=64, kv_blocks=256,
                               cs_rows=8192)
    announce(f"no-alloc vs workspace at the token limit T={T}")
    (ref, _), (got, _) = run_both(wl, debug=False)
    assert np.array_equal(got, ref)
    act = np.nonzero(wl.active_mask())[0]
    sub = dataclasses.replace(wl, token_to_req=wl.token_to_req[act], positions=wl.positions[act],
                              slot_mapping=wl.slot_mapping[act],
                              kv_slot_mapping=wl.kv_slot_mapping[act])
    rep = compare(sub, got, oracle.run(sub, synth.default_threads()))
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep["written"] == int(wl.written_mask().sum()) > 7000


def test_noalloc_rejects_more_tokens_than_its_scratch_holds():
    import paged_kv_cache_fp32_amd as c128
    announce("no-alloc token limit")
    wl = synth.decode_batch("limit", 5, 1, 32, 1, 16, kv_bs=4, kv_blocks=1, cs_rows=256)
    d = DeviceWorkload(wl)
    n = c128.VARLEN_NOALLOC_MAX_TOKENS + 1
    big = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    args = list(d.args())
    for i in (2, 3, 4, 9):   # token_to_req, positions, slot_mapping, kv_slot_mapping
        args[i] = big
    before = d.kc_buf.clone()
    with pytest.raises(c128.Dsv4Error) as e:
        c128.compress_store_varlen_noalloc(*args)
    assert e.value.code == -8 and "at most 1048576" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(before, d.kc_buf)


def test_noalloc_under_graph_capture():
    """The allocation-free call captured into a HIP graph: each replay, with an eager call on
    another batch run between replays (it rewrites the shared scratch with other counts and
    another token list), gives the bytes of the eager call.  The scratch address is looked up
    by an eager call before capture, as the header asks."""
    import paged_kv_cache_fp32_amd as c128
    a = DeviceWorkload(synth.varlen_prefill("no-alloc graph", 1208, 8, 600, 1024, 8 * 208,
                                            kv_bs=64, cs_rows=2048))
    b_wl = synth.varlen_prefill("no-alloc graph, other batch", 1209, 16, 700, 2048, 8192,
                                kv_bs=16, cs_rows=4096)
    b = DeviceWorkload(b_wl)
    b_initial = b.kc_buf.clone()
    c128.compress_store_varlen_noalloc(*b.args())
    torch.cuda.synchronize()
    b_eager = b.kc_buf.clone()
    announce("no-alloc under graph capture")

    a_initial = a.kc_buf.clone()
    c128.compress_store_varlen_noalloc(*a.args())
    torch.cuda.synchronize()
    a_eager = a.kc_buf.clone()
    assert not torch.equal(a_eager, a_initial)
    a.kc_buf.copy_(a_initial)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c128.compress_store_varlen_noalloc(*a.args())  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c128.compress_store_varlen_noalloc(*a.args())
    for i in range(3):
        b.kc_buf.copy_(b_initial)
        c128.compress_store_varlen_noalloc(*b.args())
        torch.cuda.synchronize()
        assert torch.equal(b.kc_buf, b_eager), f"eager call {i} on the other batch differs"
        a.kc_buf.copy_(a_initial)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a.kc_buf, a_eager), f"replay {i} differs from the eager call"
