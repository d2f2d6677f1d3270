"""Seeded synthetic inputs for the compress-store paths (C128, C4, indexer).

This module draws the inputs that both the CPU oracle and the HIP path
consume; it holds none of the compressor's arithmetic.  Every random value
comes from the counter-based generator in ``synth_gen.c`` (SplitMix64
finaliser over (seed, stream, index), Box-Muller normals in fp64 rounded to
fp32), so results do not depend on the thread count.

Shapes and value distributions follow the workloads of the DeepSeek-V4
compressor pages (vLLM ``fused_compress_quant_cache`` API page, "Cache block
layout" of the sparse-attention kernel; vLLM PR 44230, "Summary"):

* state cache: fp32 ``[S, 8, W]`` with ``W >= 1024``; a row is kv[0:512]
  followed by score[512:1024].
* block_table: int32 ``[R, M]`` of state block ids per request.
* k_cache: uint8 ``[B, bs, 584]`` byte container, pre-filled with 0xAB.
  Each block holds ``bs`` token records of 576 bytes, then ``bs`` x 8 scale
  bytes.
* cos_sin: fp32 ``[P, 64]``, cos in columns [0, 32), sin in [32, 64),
  angle ``p * 10000**(-2i/64)`` (computed in fp64, rounded to fp32).
* C4 state: fp32 ``[S, bs, 2048]`` (kv of the previous and current window's
  projections, 2 x 512, then their scores); indexer state ``[S, bs, 512]``
  (2 x 128 each) and indexer cache ``[B, bs, 132]`` (bs records of 128 fp8
  bytes, then bs fp32 scales).
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")

HEAD = 512
ROW = 1024
STATE_BLOCK = 8
WINDOW = 128
ROPE_DIM = 64
RECORD = 576
SCALE_BYTES = 8
SLOT_BYTES = RECORD + SCALE_BYTES  # 584 bytes of a k_cache block per token
FILL = 0xAB

# Seeds: 1000 + workload number, as used by the tests and the bench.
SEED_BASE = 1000


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (host only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC,
             "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_fill_pool.argtypes = [vp, i64, i64, i64, i64, i64, i64, i64, u64, dbl, vp, vp,
                                        dbl, dbl, ctypes.c_int]
        lib.synth_fill_pool.restype = ctypes.c_int
        lib.synth_fill_normal.argtypes = [vp, i64, u64, u64, dbl, dbl]
        lib.synth_fill_normal.restype = ctypes.c_int
        lib.synth_fill_bits.argtypes = [vp, i64, u64, u64]
        lib.synth_fill_bits.restype = ctypes.c_int
        lib.synth_fill_uniform.argtypes = [vp, i64, u64, u64]
        lib.synth_fill_uniform.restype = ctypes.c_int
        lib.synth_bits.argtypes = [u64, u64, u64]
        lib.synth_bits.restype = u64
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# ---------------------------------------------------------------- primitives

def bits(n: int, seed: int, stream: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    if n:
        _load().synth_fill_bits(out.ctypes.data, n, seed, stream)
    return out


def uniform(n: int, seed: int, stream: int) -> np.ndarray:
    """Uniform doubles in (0, 1]."""
    out = np.empty(n, dtype=np.float64)
    if n:
        _load().synth_fill_uniform(out.ctypes.data, n, seed, stream)
    return out


def normal(n: int, seed: int, stream: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().synth_fill_normal(out.ctypes.data, n, seed, stream, mean, std)
    return out


def randint(n: int, lo: int, hi: int, seed: int, stream: int) -> np.ndarray:
    """Integers uniform in [lo, hi] (inclusive)."""
    span = hi - lo + 1
    return (lo + (bits(n, seed, stream) % np.uint64(span)).astype(np.int64)).astype(np.int64)


def permutation(n: int, seed: int, stream: int) -> np.ndarray:
    """A seeded permutation of range(n): argsort of counter-based keys."""
    keys = bits(n, seed, stream)
    return np.argsort(keys, kind="stable").astype(np.int64)


def alloc_state(n_blocks: int, row_width: int = ROW, row_pad: int = 0, block_pad: int = 0,
                rows_per_block: int = STATE_BLOCK):
    """fp32 state view ``[n_blocks, rows_per_block, row_width]``; padding (in floats) between
    rows and blocks."""
    stride1 = row_width + row_pad
    stride0 = rows_per_block * stride1 + block_pad
    base = np.zeros(n_blocks * stride0, dtype=np.float32)
    view = np.lib.stride_tricks.as_strided(
        base, shape=(n_blocks, rows_per_block, row_width), strides=(stride0 * 4, stride1 * 4, 4))
    return base, view


def fill_state(state: np.ndarray, seed: int, kv_std: float = 1.0, score_std: float = 1.0,
               score_mean_per_block=None, score_std_per_block=None, threads: int | None = None,
               width: int = HEAD):
    """kv columns [0, width) ~ N(0, kv_std^2); score columns [width, 2*width) ~ N(mean_b, std_b^2)
    (width = 512 for the C128 state, 1024 for the C4 state with its two overlapping halves)."""
    nb = state.shape[0]
    s0, s1, s2 = (x // 4 for x in state.strides)
    assert s2 == 1 and state.shape[2] >= 2 * width
    mean_ptr = std_ptr = None
    if score_mean_per_block is not None:
        score_mean_per_block = np.ascontiguousarray(score_mean_per_block, dtype=np.float64)
        assert score_mean_per_block.shape == (nb,)
        mean_ptr = score_mean_per_block.ctypes.data
    if score_std_per_block is not None:
        score_std_per_block = np.ascontiguousarray(score_std_per_block, dtype=np.float64)
        assert score_std_per_block.shape == (nb,)
        std_ptr = score_std_per_block.ctypes.data
    rc = _load().synth_fill_pool(
        state.ctypes.data, nb, state.shape[1], s0, s1, width, width, width, seed, kv_std, mean_ptr,
        std_ptr, 0.0, score_std, threads or default_threads())
    assert rc == 0


def rope_table(rows: int, dim: int = ROPE_DIM, base: float = 10000.0) -> np.ndarray:
    """``[rows, dim]`` fp32: cos(p * base**(-2i/dim)) | sin(...), i < dim/2, fp64 then rounded."""
    half = dim // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def alloc_k_cache(n_blocks: int, bs: int, block_pad: int = 0, fill: int = FILL):
    """uint8 k_cache view ``[n_blocks, bs, 584]``, block stride ``bs*584 + block_pad`` bytes."""
    stride0 = bs * SLOT_BYTES + block_pad
    base = np.full(n_blocks * stride0, fill, dtype=np.uint8)
    view = np.lib.stride_tricks.as_strided(
        base, shape=(n_blocks, bs, SLOT_BYTES), strides=(stride0, SLOT_BYTES, 1))
    return base, view


# ---------------------------------------------------------------- workloads

@dataclass
class Workload:
    name: str
    state: np.ndarray
    block_table: np.ndarray
    token_to_req: np.ndarray
    positions: np.ndarray
    slot_mapping: np.ndarray
    rms_w: np.ndarray
    eps: float
    cos_sin: np.ndarray
    k_cache: np.ndarray
    kv_slot_mapping: np.ndarray
    seed: int
    state_base: np.ndarray | None = None
    k_cache_base: np.ndarray | None = None
    info: dict = field(default_factory=dict)
    compress_ratio: int = 128
    overlap: int = 0
    indexer: bool = False
    indexer_fp4: bool = False   # indexer cache in MXFP4 ([bs*64 packed][bs*4 UE8M0] blocks)

    @property
    def num_tokens(self) -> int:
        return int(self.positions.shape[0])

    def active_mask(self) -> np.ndarray:
        p = self.positions.astype(np.int64)
        return (self.slot_mapping >= 0) & (p >= 0) & ((p + 1) % self.compress_ratio == 0)

    def written_mask(self) -> np.ndarray:
        return self.active_mask() & (self.kv_slot_mapping >= 0)


def _rms_weight(seed: int) -> np.ndarray:
    return (1.0 + 0.1 * normal(HEAD, seed, 3).astype(np.float64)).astype(np.float32)


def decode_batch(name: str, seed: int, num_tokens: int, n_blocks: int, k_max: int,
                 table_cols: int, kv_bs: int, kv_blocks: int, cs_rows: int,
                 score_std: float = math.sqrt(2.0), score_mix: bool = False,
                 state=None, window_set: int = 0, row_pad: int = 0, block_pad: int = 0,
                 kc_block_pad: int = 0, pool_seed: int | None = None, k_min: int = 1,
                 threads: int | None = None) -> Workload:
    """One boundary token per request at position 128k-1, k ~ U{k_min..k_max}.

    Each window's 16 state blocks are a disjoint 16-slice of a seeded
    permutation of the pool (slice ``window_set*T + r`` for request r), so
    windows never share a block.  Table entries outside the window hold
    arbitrary valid ids.  kv slots are a seeded injection into
    ``kv_blocks*kv_bs`` slots.  ``state`` may pass a pre-filled pool.
    """
    T = num_tokens
    need = (window_set + 1) * T * 16
    if need > n_blocks:
        raise ValueError(f"pool of {n_blocks} blocks cannot hold {need // 16} disjoint windows")
    if k_max * 16 > table_cols:
        raise ValueError("block table too narrow for k_max")
    if T > kv_blocks * kv_bs:
        raise ValueError("not enough kv slots")
    k = randint(T, k_min, k_max, seed, 10)
    positions = (WINDOW * k - 1).astype(np.int32)
    perm = permutation(n_blocks, seed if pool_seed is None else pool_seed, 11)
    windows = perm[window_set * T * 16:(window_set + 1) * T * 16].reshape(T, 16)
    bt = (bits(T * table_cols, seed, 12) % np.uint64(n_blocks)).astype(np.int32).reshape(
        T, table_cols)
    for r in range(T):
        c0 = 16 * (int(k[r]) - 1)
        bt[r, c0:c0 + 16] = windows[r]
    token_to_req = np.arange(T, dtype=np.int32)
    last_blk = bt[np.arange(T), (positions // STATE_BLOCK)]
    slot_mapping = (last_blk.astype(np.int64) * STATE_BLOCK + positions % STATE_BLOCK).astype(
        np.int32)
    kv_slots = permutation(kv_blocks * kv_bs, seed, 13)[:T].astype(np.int32)

    state_base = None
    if state is None:
        state_base, state = alloc_state(n_blocks, row_pad=row_pad, block_pad=block_pad)
        mean = std = None
        if score_mix:
            # Half of the windows (Bernoulli 1/2) are N(0,1); the others are
            # near-constant c_w + 1e-3 N(0,1) with c_w ~ N(0,1).
            pick = uniform(T, seed, 14) < 0.5
            c_w = normal(T, seed, 15).astype(np.float64)
            mean = np.zeros(n_blocks)
            std = np.full(n_blocks, score_std)
            for r in range(T):
                if not pick[r]:
                    mean[windows[r]] = c_w[r]
                    std[windows[r]] = 1e-3
        fill_state(state, seed if pool_seed is None else pool_seed, 1.0, score_std,
                   mean, std, threads)
    kc_base, kc = alloc_k_cache(kv_blocks, kv_bs, kc_block_pad)
    wl = Workload(name, state, bt, token_to_req, positions, slot_mapping, _rms_weight(seed),
                  1e-6, rope_table(cs_rows), kc, kv_slots, seed, state_base, kc_base)
    wl.info = {"kind": "decode", "tokens": T, "pool_blocks": n_blocks, "k_max": k_max,
               "window_set": window_set}
    return wl


def varlen_prefill(name: str, seed: int, num_reqs: int, max_chunk: int, max_start: int,
                   n_blocks: int, kv_bs: int, cs_rows: int, drop_frac: float = 0.1,
                   score_std: float = math.sqrt(2.0), threads: int | None = None) -> Workload:
    """Chunked prefill: request r holds positions start_r .. start_r + L_r - 1, contiguous,
    request-major; L ~ U{1..max_chunk}, start ~ U{0..max_start}.  Block-table
    entries are all distinct.  A seeded ``drop_frac`` of slot_mapping is -1.
    Every token gets its own distinct kv slot, so slots of inactive tokens
    stay 0xAB."""
    L = randint(num_reqs, 1, max_chunk, seed, 20)
    start = randint(num_reqs, 0, max_start, seed, 21)
    cols = int(-(-(max_start + max_chunk) // STATE_BLOCK))
    if num_reqs * cols > n_blocks:
        raise ValueError("pool too small for distinct block-table entries")
    bt = permutation(n_blocks, seed, 22)[:num_reqs * cols].reshape(num_reqs, cols).astype(np.int32)
    token_to_req = np.concatenate([np.full(int(L[r]), r, np.int32) for r in range(num_reqs)])
    positions = np.concatenate(
        [np.arange(int(start[r]), int(start[r] + L[r]), dtype=np.int64) for r in range(num_reqs)])
    T = positions.shape[0]
    blk = bt[token_to_req, positions // STATE_BLOCK].astype(np.int64)
    slot_mapping = (blk * STATE_BLOCK + positions % STATE_BLOCK)
    drop = uniform(T, seed, 23) < drop_frac
    slot_mapping[drop] = -1
    kv_blocks = int(-(-T // kv_bs))
    kv_slots = permutation(kv_blocks * kv_bs, seed, 24)[:T].astype(np.int32)
    state_base, state = alloc_state(n_blocks)
    fill_state(state, seed, 1.0, score_std, threads=threads)
    kc_base, kc = alloc_k_cache(kv_blocks, kv_bs)
    wl = Workload(name, state, bt, token_to_req, positions.astype(np.int32),
                  slot_mapping.astype(np.int32), _rms_weight(seed), 1e-6, rope_table(cs_rows),
                  kc, kv_slots, seed, state_base, kc_base)
    wl.info = {"kind": "varlen", "tokens": T, "requests": num_reqs, "pool_blocks": n_blocks}
    return wl


def scattered_batch(name: str, seed: int, num_tokens: int, num_reqs: int, n_blocks: int,
                    table_cols: int, kv_bs: int, kv_blocks: int, cs_rows: int,
                    drop_frac: float = 0.1, score_std: float = math.sqrt(2.0)) -> Workload:
    """Tokens of random requests at uniformly random positions 0 .. 8*table_cols - 1, so about
    one token in 128 closes a window; block-table entries uniform over the pool (windows may
    share blocks); a seeded ``drop_frac`` of slot_mapping is -1.  Tokens that close a window
    with slot >= 0 get distinct kv slots; the others get arbitrary slots."""
    T = num_tokens
    req = randint(T, 0, num_reqs - 1, seed, 30).astype(np.int32)
    positions = randint(T, 0, STATE_BLOCK * table_cols - 1, seed, 31)
    bt = (bits(num_reqs * table_cols, seed, 32) % np.uint64(n_blocks)).astype(np.int32).reshape(
        num_reqs, table_cols)
    blk = bt[req, positions // STATE_BLOCK].astype(np.int64)
    slot_mapping = blk * STATE_BLOCK + positions % STATE_BLOCK
    slot_mapping[uniform(T, seed, 33) < drop_frac] = -1
    n_kv = kv_blocks * kv_bs
    kv_slots = randint(T, 0, n_kv - 1, seed, 34).astype(np.int32)
    state_base, state = alloc_state(n_blocks)
    fill_state(state, seed, 1.0, score_std)
    kc_base, kc = alloc_k_cache(kv_blocks, kv_bs)
    wl = Workload(name, state, bt, req, positions.astype(np.int32),
                  slot_mapping.astype(np.int32), _rms_weight(seed), 1e-6, rope_table(cs_rows),
                  kc, kv_slots, seed, state_base, kc_base)
    act = wl.active_mask()
    if int(act.sum()) > n_kv:
        raise ValueError("not enough kv slots for the active tokens")
    wl.kv_slot_mapping[act] = permutation(n_kv, seed, 35)[:int(act.sum())].astype(np.int32)
    wl.info = {"kind": "scattered", "tokens": T, "requests": num_reqs, "pool_blocks": n_blocks}
    return wl



def shared_pool_batch(name: str, seed: int, num_tokens: int, n_blocks: int, k_max: int,
                      kv_bs: int, kv_blocks: int, cs_rows: int,
                      score_std: float = math.sqrt(2.0), kc_block_pad: int = 0,
                      row_pad: int = 0, block_pad: int = 0) -> Workload:
    """Large decode-shaped batches on a small pool: one request per token, each at position
    128k-1 with k ~ U{1..k_max}, block-table entries uniform over an ``n_blocks`` pool (windows
    may share blocks; a window reads 16 of them), kv slots a seeded injection.  Every token
    closes a window; tests perturb gates and indices afterwards."""
    T = num_tokens
    if T > kv_blocks * kv_bs:
        raise ValueError("not enough kv slots")
    cols = 16 * k_max
    k = randint(T, 1, k_max, seed, 50)
    positions = (WINDOW * k - 1).astype(np.int64)
    bt = (bits(T * cols, seed, 51) % np.uint64(n_blocks)).astype(np.int32).reshape(T, cols)
    blk = bt[np.arange(T), positions // STATE_BLOCK].astype(np.int64)
    slot_mapping = (blk * STATE_BLOCK + positions % STATE_BLOCK).astype(np.int32)
    kv_slots = permutation(kv_blocks * kv_bs, seed, 52)[:T].astype(np.int32)
    state_base, state = alloc_state(n_blocks, row_pad=row_pad, block_pad=block_pad)
    fill_state(state, seed, 1.0, score_std)
    kc_base, kc = alloc_k_cache(kv_blocks, kv_bs, kc_block_pad)
    wl = Workload(name, state, bt, np.arange(T, dtype=np.int32), positions.astype(np.int32),
                  slot_mapping, _rms_weight(seed), 1e-6, rope_table(cs_rows), kc, kv_slots, seed,
                  state_base, kc_base)
    wl.info = {"kind": "shared-pool decode", "tokens": T, "pool_blocks": n_blocks}
    return wl


C4_RATIO = 4
C4_ROWS = 2 * C4_RATIO       # window rows: the previous window's 4 and the current 4
C4_ROW = 4 * HEAD            # kv (2 x 512) | score (2 x 512)


def c4_decode_batch(name: str, seed: int, num_tokens: int, n_blocks: int, k_max: int,
                    table_cols: int, kv_bs: int, kv_blocks: int, cs_rows: int, state_bs: int = 8,
                    score_std: float = math.sqrt(2.0), k_min: int = 1, row_pad: int = 0,
                    block_pad: int = 0, kc_block_pad: int = 0,
                    threads: int | None = None) -> Workload:
    """C4 compressor: one boundary token per request at position 4k-1, k ~ U{k_min..k_max}.

    The window is rows pos-7 .. pos (rows before position 0 do not exist when k = 1).  Each
    request's table columns covering its window get state blocks of their own (consecutive
    entries of a seeded permutation of the pool), so windows never share a block; other table
    entries hold arbitrary valid ids.  State rows are [S, state_bs, 2048]: kv of the previous-
    and current-window projections, then their scores."""
    T = num_tokens
    if T > kv_blocks * kv_bs:
        raise ValueError("not enough kv slots")
    k = randint(T, k_min, k_max, seed, 40)
    positions = (C4_RATIO * k - 1).astype(np.int64)
    if int(positions.max(initial=0)) // state_bs >= table_cols:
        raise ValueError("block table too narrow for k_max")
    per_tok = -(-C4_ROWS // state_bs) + 1
    if T * per_tok > n_blocks:
        raise ValueError("pool too small for disjoint windows")
    perm = permutation(n_blocks, seed, 41)
    bt = (bits(T * table_cols, seed, 42) % np.uint64(n_blocks)).astype(np.int32).reshape(
        T, table_cols)
    for r in range(T):
        lo = max(0, int(positions[r]) - (C4_ROWS - 1)) // state_bs
        hi = int(positions[r]) // state_bs
        bt[r, lo:hi + 1] = perm[r * per_tok:r * per_tok + (hi - lo + 1)]
    last_blk = bt[np.arange(T), positions // state_bs].astype(np.int64)
    slot_mapping = (last_blk * state_bs + positions % state_bs).astype(np.int32)
    kv_slots = permutation(kv_blocks * kv_bs, seed, 43)[:T].astype(np.int32)
    state_base, state = alloc_state(n_blocks, row_width=C4_ROW, rows_per_block=state_bs,
                                    row_pad=row_pad, block_pad=block_pad)
    fill_state(state, seed, 1.0, score_std, threads=threads, width=2 * HEAD)
    kc_base, kc = alloc_k_cache(kv_blocks, kv_bs, kc_block_pad)
    wl = Workload(name, state, bt, np.arange(T, dtype=np.int32), positions.astype(np.int32),
                  slot_mapping, _rms_weight(seed), 1e-6, rope_table(cs_rows), kc, kv_slots, seed,
                  state_base, kc_base, compress_ratio=C4_RATIO, overlap=1)
    wl.info = {"kind": "c4 decode", "tokens": T, "pool_blocks": n_blocks, "state_bs": state_bs}
    return wl


def c4_varlen_prefill(name: str, seed: int, num_reqs: int, max_chunk: int, max_start: int,
                      kv_bs: int, cs_rows: int, state_bs: int = 8, drop_frac: float = 0.1,
                      score_std: float = math.sqrt(2.0), threads: int | None = None) -> Workload:
    """C4 chunked prefill: request r holds positions start_r .. start_r + L_r - 1, contiguous,
    request-major, L ~ U{1..max_chunk}, start ~ U{0..max_start}; every fourth position closes a
    window.  Each request's table entries are distinct blocks of a pool sized for them; a seeded
    ``drop_frac`` of slot_mapping is -1; every token gets a distinct kv slot."""
    L = randint(num_reqs, 1, max_chunk, seed, 50)
    start = randint(num_reqs, 0, max_start, seed, 51)
    cols = int(-(-(max_start + max_chunk) // state_bs))
    n_blocks = num_reqs * cols
    bt = permutation(n_blocks, seed, 52).reshape(num_reqs, cols).astype(np.int32)
    token_to_req = np.concatenate([np.full(int(L[r]), r, np.int32) for r in range(num_reqs)])
    positions = np.concatenate(
        [np.arange(int(start[r]), int(start[r] + L[r]), dtype=np.int64) for r in range(num_reqs)])
    T = positions.shape[0]
    blk = bt[token_to_req, positions // state_bs].astype(np.int64)
    slot_mapping = blk * state_bs + positions % state_bs
    slot_mapping[uniform(T, seed, 53) < drop_frac] = -1
    kv_blocks = int(-(-T // kv_bs))
    kv_slots = permutation(kv_blocks * kv_bs, seed, 54)[:T].astype(np.int32)
    state_base, state = alloc_state(n_blocks, row_width=C4_ROW, rows_per_block=state_bs)
    fill_state(state, seed, 1.0, score_std, threads=threads, width=2 * HEAD)
    kc_base, kc = alloc_k_cache(kv_blocks, kv_bs)
    wl = Workload(name, state, bt, token_to_req, positions.astype(np.int32),
                  slot_mapping.astype(np.int32), _rms_weight(seed), 1e-6, rope_table(cs_rows),
                  kc, kv_slots, seed, state_base, kc_base, compress_ratio=C4_RATIO, overlap=1)
    wl.info = {"kind": "c4 varlen", "tokens": T, "requests": num_reqs, "pool_blocks": n_blocks,
               "state_bs": state_bs}
    return wl


INDEXER_HEAD = 128
INDEXER_ROW = 4 * INDEXER_HEAD   # kv (2 x 128) | score (2 x 128)
INDEXER_RECORD = 128             # fp8 bytes per token
INDEXER_SCALE = 4                # one fp32 scale per token
INDEXER_SLOT = INDEXER_RECORD + INDEXER_SCALE
INDEXER_FP4_RECORD = 64          # 128 E2M1 codes, two a byte
INDEXER_FP4_SCALES = 4           # one UE8M0 byte per 32-dim block
INDEXER_FP4_SLOT = INDEXER_FP4_RECORD + INDEXER_FP4_SCALES


def alloc_indexer_cache(n_blocks: int, bs: int, block_pad: int = 0, fill: int = FILL,
                        fp4: bool = False):
    """uint8 indexer k_cache view ``[n_blocks, bs, 132]``: each block holds ``bs`` records of 128
    fp8 bytes, then ``bs`` fp32 scales; block stride ``bs*132 + block_pad`` bytes.  ``fp4``:
    the MXFP4 cache ``[n_blocks, bs, 68]``, ``bs`` records of 64 packed bytes, then ``bs`` x 4
    UE8M0 bytes."""
    slot = INDEXER_FP4_SLOT if fp4 else INDEXER_SLOT
    stride0 = bs * slot + block_pad
    base = np.full(n_blocks * stride0, fill, dtype=np.uint8)
    view = np.lib.stride_tricks.as_strided(
        base, shape=(n_blocks, bs, slot), strides=(stride0, slot, 1))
    return base, view


def indexer_decode_batch(name: str, seed: int, num_tokens: int, n_blocks: int, k_max: int,
                         table_cols: int, kv_bs: int, kv_blocks: int, cs_rows: int,
                         state_bs: int = 8, score_std: float = math.sqrt(2.0), k_min: int = 1,
                         kc_block_pad: int = 0, row_pad: int = 0, block_pad: int = 0,
                         threads: int | None = None, fp4: bool = False) -> Workload:
    """The indexer's compressor: one boundary token per request at position 4k-1, k ~
    U{k_min..k_max}, an 8-row overlapping window as for C4, head 128 (state rows [S, state_bs,
    512]: kv 2 x 128 | score 2 x 128).  Windows get state blocks of their own; kv slots are a
    seeded injection into ``kv_blocks * kv_bs`` slots of a [B, kv_bs, 132] indexer cache
    (``fp4``: the [B, kv_bs, 68] MXFP4 cache; the inputs are the same)."""
    T = num_tokens
    if T > kv_blocks * kv_bs:
        raise ValueError("not enough kv slots")
    k = randint(T, k_min, k_max, seed, 60)
    positions = (C4_RATIO * k - 1).astype(np.int64)
    if int(positions.max(initial=0)) // state_bs >= table_cols:
        raise ValueError("block table too narrow for k_max")
    per_tok = -(-C4_ROWS // state_bs) + 1
    if T * per_tok > n_blocks:
        raise ValueError("pool too small for disjoint windows")
    perm = permutation(n_blocks, seed, 61)
    bt = (bits(T * table_cols, seed, 62) % np.uint64(n_blocks)).astype(np.int32).reshape(
        T, table_cols)
    for r in range(T):
        lo = max(0, int(positions[r]) - (C4_ROWS - 1)) // state_bs
        hi = int(positions[r]) // state_bs
        bt[r, lo:hi + 1] = perm[r * per_tok:r * per_tok + (hi - lo + 1)]
    last_blk = bt[np.arange(T), positions // state_bs].astype(np.int64)
    slot_mapping = (last_blk * state_bs + positions % state_bs).astype(np.int32)
    kv_slots = permutation(kv_blocks * kv_bs, seed, 63)[:T].astype(np.int32)
    state_base, state = alloc_state(n_blocks, row_width=INDEXER_ROW, rows_per_block=state_bs,
                                    row_pad=row_pad, block_pad=block_pad)
    fill_state(state, seed, 1.0, score_std, threads=threads, width=2 * INDEXER_HEAD)
    kc_base, kc = alloc_indexer_cache(kv_blocks, kv_bs, kc_block_pad, fp4=fp4)
    w = (1.0 + 0.1 * normal(INDEXER_HEAD, seed, 3).astype(np.float64)).astype(np.float32)
    wl = Workload(name, state, bt, np.arange(T, dtype=np.int32), positions.astype(np.int32),
                  slot_mapping, w, 1e-6, rope_table(cs_rows), kc, kv_slots, seed, state_base,
                  kc_base, compress_ratio=C4_RATIO, overlap=1, indexer=True, indexer_fp4=fp4)
    wl.info = {"kind": "indexer mxfp4 decode" if fp4 else "indexer decode", "tokens": T,
               "pool_blocks": n_blocks, "state_bs": state_bs}
    return wl


def indexer_varlen_prefill(name: str, seed: int, num_reqs: int, max_chunk: int,
                           max_start: int, kv_bs: int, cs_rows: int, state_bs: int = 8,
                           drop_frac: float = 0.1, score_std: float = math.sqrt(2.0),
                           threads: int | None = None, fp4: bool = False) -> Workload:
    """The indexer's compressor on a chunked prefill, laid out as ``c4_varlen_prefill`` (request
    r holds positions start_r .. start_r + L_r - 1, L ~ U{1..max_chunk}, start ~ U{0..max_start};
    every fourth position closes a window; a seeded ``drop_frac`` of slot_mapping is -1; every
    token gets a distinct kv slot), with head-128 state rows and the indexer cache (``fp4``: the
    MXFP4 one)."""
    L = randint(num_reqs, 1, max_chunk, seed, 70)
    start = randint(num_reqs, 0, max_start, seed, 71)
    cols = int(-(-(max_start + max_chunk) // state_bs))
    n_blocks = num_reqs * cols
    bt = permutation(n_blocks, seed, 72).reshape(num_reqs, cols).astype(np.int32)
    token_to_req = np.concatenate([np.full(int(L[r]), r, np.int32) for r in range(num_reqs)])
    positions = np.concatenate(
        [np.arange(int(start[r]), int(start[r] + L[r]), dtype=np.int64) for r in range(num_reqs)])
    T = positions.shape[0]
    blk = bt[token_to_req, positions // state_bs].astype(np.int64)
    slot_mapping = blk * state_bs + positions % state_bs
    slot_mapping[uniform(T, seed, 73) < drop_frac] = -1
    kv_blocks = int(-(-T // kv_bs))
    kv_slots = permutation(kv_blocks * kv_bs, seed, 74)[:T].astype(np.int32)
    state_base, state = alloc_state(n_blocks, row_width=INDEXER_ROW, rows_per_block=state_bs)
    fill_state(state, seed, 1.0, score_std, threads=threads, width=2 * INDEXER_HEAD)
    kc_base, kc = alloc_indexer_cache(kv_blocks, kv_bs, fp4=fp4)
    w = (1.0 + 0.1 * normal(INDEXER_HEAD, seed, 3).astype(np.float64)).astype(np.float32)
    wl = Workload(name, state, bt, token_to_req, positions.astype(np.int32),
                  slot_mapping.astype(np.int32), w, 1e-6, rope_table(cs_rows), kc, kv_slots,
                  seed, state_base, kc_base, compress_ratio=C4_RATIO, overlap=1, indexer=True,
                  indexer_fp4=fp4)
    wl.info = {"kind": "indexer varlen", "tokens": T, "requests": num_reqs,
               "pool_blocks": n_blocks, "state_bs": state_bs}
    return wl


def config0() -> Workload:
    """Single request, one boundary token at position 127; 16-block pool; KV block size 2,
    kv slot 3; kv ~ N(0,1), score ~ N(0,2); 4096 RoPE rows."""
    seed = SEED_BASE + 0
    state_base, state = alloc_state(16)
    fill_state(state, seed, 1.0, math.sqrt(2.0))
    bt = permutation(16, seed, 11).astype(np.int32).reshape(1, 16)
    positions = np.array([127], np.int32)
    slot = np.array([int(bt[0, 15]) * STATE_BLOCK + 7], np.int32)
    kc_base, kc = alloc_k_cache(4, 2)
    wl = Workload("cfg0 single boundary token", state, bt, np.zeros(1, np.int32), positions, slot,
                  _rms_weight(seed), 1e-6, rope_table(4096), kc, np.array([3], np.int32), seed,
                  state_base, kc_base)
    wl.info = {"kind": "decode", "tokens": 1, "pool_blocks": 16}
    return wl


def config1() -> Workload:
    """128 decode boundary tokens, k ~ U{1..32}, pool 4096 blocks, KV block size 64."""
    return decode_batch("cfg1 decode boundary batch T=128", SEED_BASE + 1, 128, 4096, 32, 512,
                        kv_bs=64, kv_blocks=4, cs_rows=4096)


def config2() -> Workload:
    """64-request varlen chunked prefill (~32.8k tokens), pool 65536 blocks."""
    return varlen_prefill("cfg2 varlen chunked prefill", SEED_BASE + 2, 64, 1024, 4096, 65536,
                          kv_bs=64, cs_rows=8192)


def large_prefill(threads: int | None = None) -> Workload:
    """A large chunked prefill: 32 requests, chunks of up to 16384 tokens starting at positions
    up to 16384 (246,933 tokens, 1,730 of them close a window with a state slot), distinct
    windows in a 131072-block (4.3 GB) pool."""
    return varlen_prefill("large chunked prefill", SEED_BASE + 6, 32, 16384, 16384, 131072,
                          kv_bs=64, cs_rows=32768, threads=threads)


def config3_pool(threads: int | None = None):
    """The shared 65536-block pool of the decode sweep (scores ~ N(0,4))."""
    base, state = alloc_state(65536)
    fill_state(state, SEED_BASE + 3, 1.0, 2.0, threads=threads)
    return base, state


def config3(num_tokens: int, state=None, window_set: int = 0) -> Workload:
    """Decode sweep point: ``num_tokens`` boundary tokens, k ~ U{1..64}, pool 65536 blocks."""
    T = num_tokens
    kv_blocks = max(1, -(-T // 64))
    return decode_batch(f"cfg3 decode sweep T={T}", SEED_BASE + 3 + 7919 * T, T, 65536, 64, 1024,
                        kv_bs=64, kv_blocks=kv_blocks, cs_rows=8192, score_std=2.0, state=state,
                        window_set=window_set, pool_seed=SEED_BASE + 3)


def decode_step(num_tokens: int, state=None, window_set: int = 0) -> Workload:
    """A decode step as a serving loop sees it: the decode sweep's batch of ``num_tokens``
    requests, of which about one in 128 (a seeded draw, at least one) has its new token close a
    window; every other token sits one position before its window's end."""
    wl = config3(num_tokens, state=state, window_set=window_set)
    T = num_tokens
    pick = permutation(T, SEED_BASE + 7 + window_set, 0)[:max(1, T // 128)]
    keep = np.zeros(T, bool)
    keep[pick] = True
    wl.positions[~keep] -= 1
    wl.name = f"decode step T={T}"
    return wl


def config4(threads: int | None = None) -> Workload:
    """16384 boundary tokens over a 262144-block (8.59 GB) pool; every block read once;
    score windows mix N(0,1) and near-constant; KV block size 64, 256 blocks."""
    return decode_batch("cfg4 large boundary batch T=16384", SEED_BASE + 4, 16384, 262144, 64, 1024,
                        kv_bs=64, kv_blocks=256, cs_rows=8192, score_std=1.0, score_mix=True,
                        threads=threads)


def state_bytes_per_token() -> int:
    return WINDOW * ROW * 4
