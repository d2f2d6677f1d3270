"""Properties of the GPU path that hold at any size, checked without the oracle.

With eps = 0, multiplying every kv value of the state by 2^k multiplies the pooled values by
exactly 2^k (the softmax weights do not change, and fp32 scaling by a power of two is exact), and
RMSNorm divides it out again: the sum of squares scales by 4^k, its square root and the
reciprocal by 2^k and 2^-k, all exactly.  So every record must be byte-identical, on every
schedule and compressor.  The batches are large enough to use each schedule's own kernel (the
staged schedule from 2048 tokens, the fan-out with its splits, the compacted schedule)."""

import sys

import numpy as np
import pytest

import synth
from synth.device import run_gpu

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def scaled(make, kv_cols, k):
    wl = make()
    wl.eps = 0.0
    wl.state[..., :kv_cols] *= np.float32(2.0 ** k)
    return wl


CASES = {
    "single pass, 300 tokens": (
        lambda: synth.decode_batch("prop single", 7100, 300, 4800, 8, 128, kv_bs=16,
                                   kv_blocks=20, cs_rows=1024, score_std=2.0), 512, {}),
    "fan-out, 8 splits, 9 tokens": (
        lambda: synth.decode_batch("prop fanout", 7101, 9, 200, 8, 128, kv_bs=4, kv_blocks=4,
                                   cs_rows=1024), 512, {"splits": 8}),
    "staged, 2048 tokens": (
        lambda: synth.shared_pool_batch("prop staged", 7102, 2048, 2048, 8, 64, 34, 1024),
        512, {}),
    "compacted, varlen prefill": (
        lambda: synth.varlen_prefill("prop varlen", 7103, 16, 512, 2048, 8192, kv_bs=64,
                                     cs_rows=4096), 512, {"varlen": True}),
    "C4, 600 tokens": (
        lambda: synth.c4_decode_batch("prop c4", 7104, 600, 2400, 16, 64, kv_bs=16,
                                      kv_blocks=40, cs_rows=256, state_bs=4), 1024, {}),
    "indexer, 600 tokens": (
        lambda: synth.indexer_decode_batch("prop indexer", 7105, 600, 2400, 16, 64, kv_bs=16,
                                           kv_blocks=40, cs_rows=256, state_bs=4), 256, {}),
    "indexer MXFP4, 600 tokens": (
        lambda: synth.indexer_decode_batch("prop mxfp4", 7106, 600, 2400, 16, 64, kv_bs=16,
                                           kv_blocks=40, cs_rows=256, state_bs=4, fp4=True),
        256, {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_records_invariant_under_power_of_two_kv_scaling(name):
    make, kv_cols, kw = CASES[name]
    announce(f"kv scaling invariance: {name}")
    base, _, ok = run_gpu(scaled(make, kv_cols, 0), debug=False, **kw)
    assert ok
    wl = scaled(make, kv_cols, 0)
    assert int(wl.written_mask().sum()) > 0
    for k in (-9, 7):
        body, _, ok = run_gpu(scaled(make, kv_cols, k), debug=False, **kw)
        assert ok
        assert np.array_equal(body, base), f"records differ after scaling kv by 2^{k}"
