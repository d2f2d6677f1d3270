"""Every entry point is stream-ordered with no host synchronisation, no allocation in the
library and no memset, so it can be captured into a HIP graph.  Each test captures one call,
then replays the graph several times; before each replay the k_cache is restored by eager work
on the host side of the program, and after it the bytes must equal those of an eager call."""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_fp32_amd as c128
import synth
from synth.device import DeviceWorkload

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def capture_and_replay(d, call, replays=3):
    initial = d.kc_buf.clone()
    call()
    torch.cuda.synchronize()
    eager = d.kc_buf.clone()
    assert not torch.equal(eager, initial)
    d.kc_buf.copy_(initial)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream, as torch's capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(replays):
        d.kc_buf.copy_(initial)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.kc_buf, eager), f"replay {i} differs from the eager call"
    d.kc_buf.copy_(initial)  # leave the cache as found, for the next capture on it
    torch.cuda.synchronize()


def test_graph_single_pass_and_fanout():
    wl = synth.decode_batch("graph", 1301, 40, 40 * 16 + 16, 8, 128, kv_bs=16, kv_blocks=5,
                            cs_rows=1024)
    d = DeviceWorkload(wl)
    announce("graph: single pass")
    capture_and_replay(d, lambda: c128.compress_store(*d.args()))
    ws = c128.fanout_workspace(wl.num_tokens, 4)
    announce("graph: fan-out splits=4")
    capture_and_replay(d, lambda: c128.compress_store_ex(*d.args(), workspace=ws, splits=4))


def test_graph_staged_schedule():
    """8192 tokens: the plain entry point takes the staged schedule."""
    wl = synth.shared_pool_batch("graph staged", 1305, 8192, 2048, 8, 64, 130, 1024)
    d = DeviceWorkload(wl)
    announce("graph: staged schedule (plain entry point, 8192 tokens)")
    capture_and_replay(d, lambda: c128.compress_store(*d.args()))


def test_graph_compacted_schedule():
    wl = synth.varlen_prefill("graph varlen", 1302, 8, 600, 1024, 8 * 208, kv_bs=64,
                              cs_rows=2048)
    d = DeviceWorkload(wl)
    ws = torch.empty(c128.varlen_workspace_bytes(wl.num_tokens), dtype=torch.uint8,
                     device="cuda")
    announce("graph: compacted schedule")
    capture_and_replay(d, lambda: c128.compress_store_varlen(*d.args(), workspace=ws))


def test_graph_c4_and_indexer():
    c4 = synth.c4_decode_batch("graph c4", 1303, 300, 700, 16, 16, kv_bs=16, kv_blocks=40,
                               cs_rows=128)
    d = DeviceWorkload(c4)
    announce("graph: c4")
    capture_and_replay(d, lambda: c128.c4_compress_store(*d.args()))
    ix = synth.indexer_decode_batch("graph indexer", 1304, 300, 700, 16, 16, kv_bs=16,
                                    kv_blocks=40, cs_rows=128)
    d = DeviceWorkload(ix)
    announce("graph: indexer")
    capture_and_replay(d, lambda: c128.indexer_compress_store(*d.args()))
    fx = synth.indexer_decode_batch("graph indexer mxfp4", 1305, 300, 700, 16, 16, kv_bs=16,
                                    kv_blocks=40, cs_rows=128, fp4=True)
    d = DeviceWorkload(fx)
    announce("graph: indexer mxfp4")
    capture_and_replay(d, lambda: c128.indexer_mxfp4_compress_store(*d.args()))


def test_graph_c4_wide_workgroups_and_indexer_runs():
    """9000 tokens: C4 takes its 12-wave workgroups that gate and deal their tokens, and the
    indexer's waves take two tokens each."""
    c4 = synth.c4_decode_batch("graph c4 wide", 1306, 9000, 18008, 16, 16, kv_bs=16,
                               kv_blocks=1125, cs_rows=128)
    d = DeviceWorkload(c4)
    announce("graph: c4 wide workgroups (9000 tokens)")
    capture_and_replay(d, lambda: c128.c4_compress_store(*d.args()))
    ix = synth.indexer_decode_batch("graph indexer 9000", 1307, 9000, 18008, 16, 16, kv_bs=16,
                                    kv_blocks=1125, cs_rows=128)
    d = DeviceWorkload(ix)
    announce("graph: indexer (9000 tokens)")
    capture_and_replay(d, lambda: c128.indexer_compress_store(*d.args()))
