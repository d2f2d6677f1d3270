"""Seeded randomised parity: each case draws a configuration (path, token count, state and
cache block sizes, paddings, score spread, a mix of boundary / non-boundary tokens, negative
state and kv slots), runs it on the GPU and compares against the CPU oracle.  Small sizes, so
the whole file runs in seconds; the seeds are fixed, so a failure names its case."""

import sys

import numpy as np
import pytest

import oracle
import synth
from oracle.compare import compare
from synth.device import run_gpu

pytestmark = pytest.mark.gpu

PATHS = ["single", "fanout", "varlen", "c4", "indexer"]


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def perturb(wl, rng, ratio):
    """Turn a random share of tokens into non-boundary tokens, negative state slots or
    negative kv slots."""
    T = wl.num_tokens
    off = rng.random(T) < rng.uniform(0.0, 0.4)
    wl.positions[off] = np.maximum(wl.positions[off] - rng.integers(1, ratio, off.sum()), 0)
    wl.slot_mapping[rng.random(T) < rng.uniform(0.0, 0.2)] = -1
    wl.kv_slot_mapping[rng.random(T) < rng.uniform(0.0, 0.2)] = -1


def draw(case, path=None):
    """A random batch of one path: ``path`` None takes PATHS[case % len(PATHS)]; "mxfp4" is
    the indexer with its MXFP4 cache."""
    rng = np.random.default_rng(9000 + case)
    path = PATHS[case % len(PATHS)] if path is None else path
    T = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 100, 257]))
    kv_bs = int(rng.choice([1, 2, 5, 16, 64]))
    kv_blocks = -(-2 * T // kv_bs) + 1
    score_std = float(rng.choice([0.5, 2 ** 0.5, 2.0, 4.0]))
    kc_pad = int(rng.choice([0, 8, 40]))
    seed = 9000 + case
    if path in ("single", "fanout", "varlen"):
        k_max = int(rng.integers(1, 9))
        wl = synth.decode_batch(f"fuzz {case}", seed, T, 16 * T + 8, k_max, 16 * k_max + 3,
                                kv_bs=kv_bs, kv_blocks=kv_blocks, cs_rows=128 * k_max,
                                score_std=score_std, row_pad=int(rng.choice([0, 16])),
                                block_pad=int(rng.choice([0, 32])), kc_block_pad=kc_pad)
        perturb(wl, rng, 128)
        kw = {}
        if path == "fanout":
            kw = {"splits": int(rng.choice([0, 2, 4, 8, 16]))}
        elif path == "varlen":
            kw = {"varlen": True}
        return path, wl, kw
    state_bs = int(rng.choice([1, 2, 4, 8, 16]))
    k_max = int(rng.integers(1, 40))
    cols = -(-4 * k_max // state_bs) + 1
    gen = synth.c4_decode_batch if path == "c4" else synth.indexer_decode_batch
    pad = 8 if path == "c4" else 4
    fmt = {"fp4": True} if path == "mxfp4" else {}
    wl = gen(f"fuzz {case}", seed, T, T * (-(-8 // state_bs) + 1) + 4, k_max, cols, kv_bs=kv_bs,
             kv_blocks=kv_blocks, cs_rows=4 * k_max + 4, state_bs=state_bs, score_std=score_std,
             row_pad=int(rng.choice([0, 16])), block_pad=int(rng.choice([0, 32])),
             kc_block_pad=(kc_pad // pad) * pad, **fmt)
    perturb(wl, rng, 4)
    return path, wl, {}


@pytest.mark.parametrize("case", range(40))
def test_fuzz(case):
    path, wl, kw = draw(case)
    announce(f"fuzz case {case}: {path} T={wl.num_tokens} kv_bs={wl.k_cache.shape[1]} "
             f"state_bs={wl.state.shape[1]} {kw}")
    body, comp, guards_ok = run_gpu(wl, debug=True, **kw)
    assert guards_ok, "k_cache guard bands were written"
    rep = compare(wl, body, oracle.run(wl, 4), gpu_compressed=comp)
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("case", range(8))
def test_fuzz_mxfp4(case):
    path, wl, kw = draw(100 + case, "mxfp4")
    announce(f"fuzz case {100 + case}: mxfp4 T={wl.num_tokens} kv_bs={wl.k_cache.shape[1]} "
             f"state_bs={wl.state.shape[1]}")
    body, comp, guards_ok = run_gpu(wl, debug=True, **kw)
    assert guards_ok, "k_cache guard bands were written"
    rep = compare(wl, body, oracle.run(wl, 4), gpu_compressed=comp)
    assert rep.ok(), rep.summary()


def draw_large(case):
    """Batches the plain entry point runs on the staged schedule (2048 tokens and more), on a
    small shared pool, with random paddings and the same gate and slot perturbations."""
    rng = np.random.default_rng(9500 + case)
    T = int(rng.choice([2048, 3001, 5555, 8192, 9001, 12345, 16500]))
    kv_bs = int(rng.choice([1, 7, 16, 64]))
    wl = synth.shared_pool_batch(f"fuzz large {case}", 9500 + case, T, 2048, 8, kv_bs,
                                 -(-T // kv_bs) + 2, 1024,
                                 score_std=float(rng.choice([0.5, 2 ** 0.5, 4.0])),
                                 kc_block_pad=int(rng.choice([0, 8, 40])),
                                 row_pad=int(rng.choice([0, 16])),
                                 block_pad=int(rng.choice([0, 32])))
    perturb(wl, rng, 128)
    return wl


@pytest.mark.parametrize("case", range(8))
def test_fuzz_staged(case):
    wl = draw_large(case)
    announce(f"fuzz staged case {case}: T={wl.num_tokens} kv_bs={wl.k_cache.shape[1]}")
    body, comp, guards_ok = run_gpu(wl, debug=True)
    assert guards_ok, "k_cache guard bands were written"
    rep = compare(wl, body, oracle.run(wl, 8), gpu_compressed=comp)
    assert rep.ok(), rep.summary()
