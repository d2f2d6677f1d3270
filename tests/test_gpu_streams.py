"""Entry points keep no state between calls beyond a caller's own workspace, so calls on
different streams may overlap on one device.  Each entry point gets a batch and a stream of its
own (default priority); all calls are launched before one synchronisation, three times over, and
every k_cache must equal the bytes of the same call run alone.  (The allocation-free schedule
shares one array per device and is left out: its calls must be ordered on one stream.)"""

import sys

import pytest
import torch

import paged_kv_cache_fp32_amd as c128
import synth
from synth.device import DeviceWorkload

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def cases():
    """(name, workload, call(d, workspace), workspace bytes or fan-out splits)."""
    return [
        ("single pass, 300 tokens",
         synth.decode_batch("streams single", 7200, 300, 4800, 8, 128, kv_bs=16, kv_blocks=20,
                            cs_rows=1024),
         lambda d, ws: c128.compress_store(*d.args()), None),
        ("staged, 2048 tokens",
         synth.shared_pool_batch("streams staged", 7201, 2048, 2048, 8, 64, 34, 1024),
         lambda d, ws: c128.compress_store(*d.args()), None),
        ("fan-out, 8 splits, 9 tokens",
         synth.decode_batch("streams fanout", 7202, 9, 200, 8, 128, kv_bs=4, kv_blocks=4,
                            cs_rows=1024),
         lambda d, ws: c128.compress_store_ex(*d.args(), workspace=ws, splits=8), "fanout"),
        ("compacted, varlen prefill",
         synth.varlen_prefill("streams varlen", 7203, 16, 512, 2048, 8192, kv_bs=64,
                              cs_rows=4096),
         lambda d, ws: c128.compress_store_varlen(*d.args(), workspace=ws), "varlen"),
        ("C4, 600 tokens",
         synth.c4_decode_batch("streams c4", 7204, 600, 2400, 16, 64, kv_bs=16, kv_blocks=40,
                               cs_rows=256, state_bs=4),
         lambda d, ws: c128.c4_compress_store(*d.args()), None),
        ("indexer, 600 tokens",
         synth.indexer_decode_batch("streams indexer", 7205, 600, 2400, 16, 64, kv_bs=16,
                                    kv_blocks=40, cs_rows=256, state_bs=4),
         lambda d, ws: c128.indexer_compress_store(*d.args()), None),
        ("indexer MXFP4, 600 tokens",
         synth.indexer_decode_batch("streams mxfp4", 7206, 600, 2400, 16, 64, kv_bs=16,
                                    kv_blocks=40, cs_rows=256, state_bs=4, fp4=True),
         lambda d, ws: c128.indexer_mxfp4_compress_store(*d.args()), None),
    ]


def test_entry_points_on_concurrent_streams():
    runs = []
    for name, wl, call, kind in cases():
        d = DeviceWorkload(wl)
        if kind == "fanout":
            ws = c128.fanout_workspace(wl.num_tokens, 8, d.state.device)
        elif kind == "varlen":
            ws = torch.empty(c128.varlen_workspace_bytes(wl.num_tokens), dtype=torch.uint8,
                             device="cuda")
        else:
            ws = None
        runs.append((name, d, call, ws, d.kc_buf.clone()))
    announce("each entry point alone")
    alone = []
    for name, d, call, ws, initial in runs:
        call(d, ws)
        torch.cuda.synchronize()
        assert not torch.equal(d.kc_buf, initial), f"{name}: the call wrote nothing"
        alone.append(d.kc_buf.clone())
    streams = [torch.cuda.Stream() for _ in runs]
    for rep in range(3):
        for _, d, _, _, initial in runs:
            d.kc_buf.copy_(initial)
        torch.cuda.synchronize()
        announce(f"all entry points on {len(streams)} streams, launch {rep}")
        for s, (name, d, call, ws, _) in zip(streams, runs):
            with torch.cuda.stream(s):
                call(d, ws)
        torch.cuda.synchronize()
        for (name, d, _, _, _), ref in zip(runs, alone):
            assert torch.equal(d.kc_buf, ref), f"{name}: bytes differ on concurrent streams"
