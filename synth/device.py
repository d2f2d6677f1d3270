"""Place a synth.Workload in device memory (torch tensors; the k_cache view sits between
guard bands), run the library on it and bring the k_cache bytes back.  Used by the GPU
tests, the smoke check and the bench."""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_fp32_amd as c128

GUARD = 4096
GUARD_BYTE = 0x5A


class DeviceWorkload:
    def __init__(self, wl, device="cuda", guard=GUARD, state=None):
        """``state``: an already resident (buffer, view) pair holding the same bytes as
        ``wl.state`` (several workloads can share one device pool)."""
        self.wl = wl
        self.guard = guard
        st = wl.state
        if state is not None:
            self.state_buf, self.state = state
        else:
            base = wl.state_base if wl.state_base is not None else \
                np.ascontiguousarray(st).reshape(-1)
            self.state_buf = torch.from_numpy(base).to(device)
            if wl.state_base is not None:
                s = tuple(x // 4 for x in st.strides)
                self.state = torch.as_strided(self.state_buf, st.shape, s)
            else:
                self.state = self.state_buf.view(st.shape)
        self.block_table = torch.from_numpy(np.ascontiguousarray(wl.block_table)).to(device)
        self.token_to_req = torch.from_numpy(np.ascontiguousarray(wl.token_to_req)).to(device)
        self.positions = torch.from_numpy(np.ascontiguousarray(wl.positions)).to(device)
        self.slot_mapping = torch.from_numpy(np.ascontiguousarray(wl.slot_mapping)).to(device)
        self.kv_slot_mapping = torch.from_numpy(np.ascontiguousarray(wl.kv_slot_mapping)).to(device)
        self.rms_w = torch.from_numpy(np.ascontiguousarray(wl.rms_w)).to(device)
        self.cos_sin = torch.from_numpy(np.ascontiguousarray(wl.cos_sin)).to(device)
        kb = wl.k_cache_base
        self.kc_buf = torch.full((kb.size + 2 * guard,), GUARD_BYTE, dtype=torch.uint8,
                                 device=device)
        self.kc_buf[guard:guard + kb.size].copy_(torch.from_numpy(kb))
        kc = wl.k_cache
        self.k_cache = torch.as_strided(self.kc_buf, kc.shape, kc.strides, guard)
        self.eps = wl.eps

    def args(self):
        return (self.state, self.block_table, self.token_to_req, self.positions,
                self.slot_mapping, self.rms_w, self.eps, self.cos_sin, self.k_cache,
                self.kv_slot_mapping)

    def run(self, debug=False, splits=None, varlen=False):
        """One call; splits None = the plain entry points, else compress_store_ex with that
        split count (0 = automatic) and a workspace of the size it needs; varlen = the
        compacted schedule (compress_store_varlen).  A C4 workload (compress ratio 4) always
        goes to c4_compress_store, an indexer workload to indexer_compress_store (or
        indexer_mxfp4_compress_store for the MXFP4 cache)."""
        comp = None
        indexer = getattr(self.wl, "indexer", False)
        if debug:
            comp = torch.full((self.wl.num_tokens, 128 if indexer else 512), float("nan"),
                              dtype=torch.float32, device=self.state.device)
        if indexer and getattr(self.wl, "indexer_fp4", False):
            c128.indexer_mxfp4_compress_store(*self.args(), compressed_out=comp)
        elif indexer:
            c128.indexer_compress_store(*self.args(), compressed_out=comp)
        elif getattr(self.wl, "compress_ratio", 128) == 4:
            c128.c4_compress_store(*self.args(), compressed_out=comp)
        elif varlen:
            ws = torch.empty(max(c128.varlen_workspace_bytes(self.wl.num_tokens), 16),
                             dtype=torch.uint8, device=self.state.device)
            c128.compress_store_varlen(*self.args(), compressed_out=comp, workspace=ws)
        elif splits is None:
            if debug:
                c128.compress_store_debug(*self.args(), comp)
            else:
                c128.compress_store(*self.args())
        else:
            ws = c128.fanout_workspace(self.wl.num_tokens, splits, self.state.device)
            c128.compress_store_ex(*self.args(), compressed_out=comp, workspace=ws,
                                   splits=splits)
        torch.cuda.synchronize()
        return comp

    def k_cache_bytes(self):
        """(body bytes, guards intact?)"""
        buf = self.kc_buf.cpu().numpy()
        g = self.guard
        guards_ok = bool(np.all(buf[:g] == GUARD_BYTE) and np.all(buf[-g:] == GUARD_BYTE))
        return buf[g:-g].copy(), guards_ok


def relocated_pool(wl, n_blocks, ids, device="cuda"):
    """A device state pool of ``n_blocks`` blocks (the block and row shape of ``wl.state``, no
    padding) that holds block b of ``wl.state`` at id ``ids[b]``; the other blocks stay
    uninitialised, so the block table must send every window read to a relocated block.
    Returns (pool, block table renumbered through ``ids``, as an int32 device tensor)."""
    st = wl.state
    ids = np.asarray(ids, dtype=np.int64)
    assert ids.shape == (st.shape[0],) and len(np.unique(ids)) == ids.size
    assert ids.min() >= 0 and ids.max() < n_blocks
    bt = wl.block_table
    assert bt.min() >= 0 and bt.max() < st.shape[0], "every table entry must name a pool block"
    pool = torch.empty((n_blocks,) + st.shape[1:], dtype=torch.float32, device=device)
    pool[torch.from_numpy(ids).to(device)] = torch.from_numpy(np.ascontiguousarray(st)).to(device)
    table = torch.from_numpy(ids[bt].astype(np.int32)).to(device)
    return pool, table


def run_gpu(wl, debug=True, splits=None, varlen=False):
    d = DeviceWorkload(wl)
    comp = d.run(debug=debug, splits=splits, varlen=varlen)
    body, guards_ok = d.k_cache_bytes()
    return body, (comp.cpu().numpy() if comp is not None else None), guards_ok
