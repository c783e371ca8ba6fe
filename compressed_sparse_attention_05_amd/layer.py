"""Owning wrappers around the C ABI: allocate caches, outputs and workspaces once, then run the
layer's forward (prefill chunks) or decode steps through libcsa.so."""
from __future__ import annotations

import torch

from . import lib


def dims(m: int, D: int, H: int, H_I: int, D_I: int, top_k: int, window: int, sm_scale: float = 0.0) -> lib.Dims:
    return lib.make_dims(m, D, H, H_I, D_I, top_k, window, sm_scale)


def _key_cache(d: lib.Dims, B: int, n_cap: int, dtype, device, fp4: bool):
    """Indexer key cache: rows of the activation dtype, or MXFP4 codes and scales."""
    if fp4:
        return (torch.zeros(B, n_cap, d.D_I // 2, dtype=torch.uint8, device=device),
                torch.zeros(B, n_cap, d.D_I // 32, dtype=torch.uint8, device=device))
    return torch.zeros(B, n_cap, d.D_I, dtype=dtype, device=device), None


class CSAPrefill:
    """Chunked prefill of B sequences: x [B, T, d_model], sequence b at positions pos0[b] .. pos0[b]+T-1.

    Caches (all in the activation dtype): entries [B, n_cap, D], keys [B, n_cap, D_I],
    win [B, window-1+T, D] (row r of sequence b = position pos0[b]-(window-1)+r), halo
    [B, m, 2D+2D_I] (the previous block's cb|zb|icb|izb). Fill the context rows before calling with
    pos0 > 0, or let chain=True carry them from one call to the next: each call then also writes the
    next chunk's halo (halo_out) and the next chunk's window prefix is moved to the front of win, so
    consecutive calls at pos0, pos0 + T, ... prefill one long sequence chunk by chunk.
    fp4_keys=True keeps the indexer keys in MXFP4 (keys: uint8 codes [B, n_cap, D_I/2], key_scales
    [B, n_cap, D_I/32]) and runs the indexer on MXFP4 queries and keys.
    """

    def __init__(self, d: lib.Dims, B: int, T: int, d_model: int, n_cap: int, dtype=torch.bfloat16,
                 out_dtype=torch.float32, device="cuda", records: bool = False, chain: bool = False,
                 fp4_keys: bool = False):
        self.d, self.B, self.T, self.chain = d, B, T, chain
        if chain and T % d.m:
            raise ValueError("chained chunks need T % m == 0")
        if records:  # the entry cache as 584-byte FP8 records
            self.entries = torch.zeros(B, n_cap, lib.ENTRY_RECORD_BYTES, dtype=torch.uint8, device=device)
        else:
            self.entries = torch.zeros(B, n_cap, d.D, dtype=dtype, device=device)
        self.keys, self.key_scales = _key_cache(d, B, n_cap, dtype, device, fp4_keys)
        self.win = torch.zeros(B, d.window - 1 + T, d.D, dtype=dtype, device=device)
        self.halo = torch.zeros(B, d.m, 2 * d.D + 2 * d.D_I, dtype=dtype, device=device)
        self.halo_next = torch.zeros_like(self.halo) if chain else None
        self.out = torch.empty(B, T, d.H, d.D, dtype=out_dtype, device=device)
        self.idx = torch.empty(B, T, d.top_k, dtype=torch.int32, device=device)
        code = lib.CSA_BF16 if dtype == torch.bfloat16 else lib.CSA_F32
        self.fwd = lib.Forward(d, B, T, d_model, n_cap, code, device)
        self._pos = {}

    def positions(self, pos0):
        """pos0 as the device array the library reads (ints cached, so a repeated call launches nothing)."""
        if isinstance(pos0, int):
            if pos0 not in self._pos:
                self._pos[pos0] = lib.positions(self.B, pos0, self.out.device)
            return self._pos[pos0]
        return lib.positions(self.B, pos0, self.out.device)

    def __call__(self, weights: dict, x: torch.Tensor, pos0) -> torch.Tensor:
        pos = self.positions(pos0)
        cache = {"entries": self.entries, "keys": self.keys, "key_scales": self.key_scales, "win": self.win,
                 "halo": self.halo if pos is not None else None,
                 "halo_out": self.halo_next if self.chain else None}
        self.fwd(weights, x, cache, self.out, pos0=pos, out_idx=self.idx)
        if self.chain:
            W1 = self.d.window - 1
            self.win[:, :W1] = self.win[:, self.T:self.T + W1].clone()   # the next chunk's window prefix
            self.halo, self.halo_next = self.halo_next, self.halo
        return self.out


class CSADecode:
    """One decode step of B sequences, sequence b at position L[b] (the caches hold L[b]/m entries and
    the raw KV of positions L[b]-window+1 .. L[b]): indexer + top-k, then sparse attention.

    L: an int (every sequence) or per-sequence positions (a list, or a device int64 [B] tensor).
    fid (optional): QK-norm and partial RoPE, a dict with gamma_q (float32 [D] tensor or None), eps,
    rope_dims, theta. The query is then normalised and rotated at L into a buffer of its own before
    the attention and the output is rotated back by L; the caches are read as stored (already
    normalised and rotated)."""

    def __init__(self, d: lib.Dims, B: int, n_cap: int, idx_dtype: int = lib.CSA_BF16, out_dtype=torch.float32,
                 device="cuda", fid=None, q_dtype=torch.bfloat16):
        self.d, self.B, self.fid = d, B, fid
        self.device = device
        self.q_n = torch.empty(B, 1, d.H, d.D, dtype=q_dtype, device=device) if fid else None
        self.idx = torch.empty(B, 1, d.top_k, dtype=torch.int32, device=device)
        self.out = torch.empty(B, 1, d.H, d.D, dtype=out_dtype, device=device)
        self.ws = lib.workspace(lib.csa_workspace_size(lib.CSA_OP_INDEX_TOPK, d, B, 1, n_cap, 0, idx_dtype), device)
        op = lib.CSA_OP_SPARSE_ATTN_QK if fid else lib.CSA_OP_SPARSE_ATTN
        self.ws_attn = lib.workspace(lib.csa_workspace_size(op, d, B, 1, n_cap, 0, lib.CSA_BF16), device)
        self._pos = {}

    def _positions(self, L):
        """(query positions, window row-0 positions) as device arrays; ints are cached."""
        key = L if isinstance(L, int) else None
        if key is not None and key in self._pos:
            return self._pos[key]
        q = lib.positions(self.B, L, self.device, null_if_zero=False)
        r = q - (self.d.window - 1)
        if key is not None:
            self._pos[key] = (q, r)
        return q, r

    def __call__(self, L, q_idx, w_head, keys, q, entries, kv_raw, q_scale=None, k_scale=None, sink=None):
        f = self.fid
        qp, rp = self._positions(L)
        lib.csa_index_topk(self.d, q_idx, w_head, keys, self.idx, q_pos0=qp, q_scale=q_scale, k_scale=k_scale,
                           ws=self.ws)
        if f and entries.dtype != torch.uint8:
            # the query's norm and rotation and the output's back-rotation inside the attention call
            lib.csa_sparse_attn_qk(self.d, f, q, entries, self.idx, kv_raw, self.out, q_pos0=qp, raw_pos0=rp,
                                   sink=sink, ws=self.ws_attn)
            return self.out
        if f:
            q = lib.csa_norm_rope(q, y=self.q_n, pos0=qp, gamma=f.get("gamma_q"), eps=f.get("eps", 0.0),
                                  rope_dims=f.get("rope_dims", 0), theta=f.get("theta", 10000.0))
        lib.csa_sparse_attn(self.d, q, entries, self.idx, kv_raw, self.out, q_pos0=qp, raw_pos0=rp, sink=sink,
                            ws=self.ws_attn)
        if f and f.get("rope_dims", 0):
            lib.csa_norm_rope(self.out, pos0=qp, rope_dims=f["rope_dims"], theta=f.get("theta", 10000.0),
                              inverse=True)
        return self.out


class CSADecodeState:
    """Token-by-token decode of B sequences over a state cache (entries, indexer keys, a ring of the
    last `window` raw KV rows, the compressor inputs of the previous and current block, block i in
    rows (i % 2) * m ..); when a token completes its block the entry and key are compressed into the
    caches (csa_decode_step). Each sequence advances at its own position. records=True keeps the
    entries as 584-byte FP8 records; fp4_keys=True keeps the indexer keys in MXFP4 (the step quantises
    its q_idx)."""

    def __init__(self, d: lib.Dims, B: int, n_cap: int, dtype=torch.bfloat16, out_dtype=torch.float32,
                 records: bool = False, device="cuda", fp4_keys: bool = False):
        self.d, self.B = d, B
        self.device = device
        if records:
            self.entries = torch.zeros(B, n_cap, lib.ENTRY_RECORD_BYTES, dtype=torch.uint8, device=device)
        else:
            self.entries = torch.zeros(B, n_cap, d.D, dtype=dtype, device=device)
        self.keys, self.key_scales = _key_cache(d, B, n_cap, dtype, device, fp4_keys)
        self.win = torch.zeros(B, d.window, d.D, dtype=dtype, device=device)
        self.block = torch.zeros(B, 2 * d.m, 4 * d.D + 4 * d.D_I, dtype=dtype, device=device)
        self.out = torch.empty(B, d.H, d.D, dtype=out_dtype, device=device)
        self.idx = torch.empty(B, d.top_k, dtype=torch.int32, device=device)
        code = lib.CSA_BF16 if dtype == torch.bfloat16 else lib.CSA_F32
        self.ws = lib.workspace(lib.csa_workspace_size(lib.CSA_OP_DECODE_STEP, d, B, 1, n_cap, 0, code), device)
        self._pos = {}

    def state(self) -> dict:
        return {"entries": self.entries, "keys": self.keys, "key_scales": self.key_scales, "win": self.win,
                "block": self.block}

    def block_rows(self, blk: int) -> slice:
        """The rows of the state's block that hold block `blk`."""
        r0 = (blk % 2) * self.d.m
        return slice(r0, r0 + self.d.m)

    def step(self, weights: dict, pos, q, q_idx, kv, comp):
        """pos: an int (every sequence) or per-sequence positions (a device int64 [B] tensor)."""
        if isinstance(pos, int):
            if pos not in self._pos:
                self._pos[pos] = lib.positions(self.B, pos, self.device, null_if_zero=False)
            pos = self._pos[pos]
        return lib.csa_decode_step(self.d, weights, pos, q, q_idx, kv, comp, self.state(), self.out,
                                   out_idx=self.idx, ws=self.ws)
