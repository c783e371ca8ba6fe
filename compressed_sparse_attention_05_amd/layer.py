"""Owning wrappers around the C ABI: allocate caches, outputs and workspaces once, then run the
layer's forward (prefill chunks) or decode steps through libcsa.so."""
from __future__ import annotations

import torch

from . import lib


def dims(m: int, D: int, H: int, H_I: int, D_I: int, top_k: int, window: int, sm_scale: float = 0.0) -> lib.Dims:
    return lib.make_dims(m, D, H, H_I, D_I, top_k, window, sm_scale)


class CSAPrefill:
    """Chunked prefill of B sequences: x [B, T, d_model] at positions pos0 .. pos0+T-1.

    Caches (all in the activation dtype): entries [B, n_cap, D], keys [B, n_cap, D_I],
    win [B, window-1+T, D] (row r = position pos0-(window-1)+r), halo [B, m, 2D+2D_I] (the previous
    block's cb|zb|icb|izb). Fill the context rows before calling with pos0 > 0.
    """

    def __init__(self, d: lib.Dims, B: int, T: int, d_model: int, n_cap: int, dtype=torch.bfloat16,
                 out_dtype=torch.float32, device="cuda", records: bool = False):
        self.d, self.B, self.T = d, B, T
        if records:  # the entry cache as 584-byte FP8 records
            self.entries = torch.zeros(B, n_cap, lib.ENTRY_RECORD_BYTES, dtype=torch.uint8, device=device)
        else:
            self.entries = torch.zeros(B, n_cap, d.D, dtype=dtype, device=device)
        self.keys = torch.zeros(B, n_cap, d.D_I, dtype=dtype, device=device)
        self.win = torch.zeros(B, d.window - 1 + T, d.D, dtype=dtype, device=device)
        self.halo = torch.zeros(B, d.m, 2 * d.D + 2 * d.D_I, dtype=dtype, device=device)
        self.out = torch.empty(B, T, d.H, d.D, dtype=out_dtype, device=device)
        self.idx = torch.empty(B, T, d.top_k, dtype=torch.int32, device=device)
        code = lib.CSA_BF16 if dtype == torch.bfloat16 else lib.CSA_F32
        self.fwd = lib.Forward(d, B, T, d_model, n_cap, code, device)

    def __call__(self, weights: dict, x: torch.Tensor, pos0: int) -> torch.Tensor:
        cache = {"entries": self.entries, "keys": self.keys, "win": self.win,
                 "halo": self.halo if pos0 > 0 else None}
        return self.fwd(weights, x, cache, self.out, pos0=pos0, out_idx=self.idx)


class CSADecode:
    """One decode step of B sequences at position L (the caches hold L/m entries and the raw KV of
    positions L-window+1 .. L): indexer + top-k, then sparse attention.

    fid (optional): QK-norm and partial RoPE, a dict with gamma_q (float32 [D] tensor or None), eps,
    rope_dims, theta. The query is then normalised and rotated at L into a buffer of its own before
    the attention and the output is rotated back by L; the caches are read as stored (already
    normalised and rotated)."""

    def __init__(self, d: lib.Dims, B: int, n_cap: int, idx_dtype: int = lib.CSA_BF16, out_dtype=torch.float32,
                 device="cuda", fid=None, q_dtype=torch.bfloat16):
        self.d, self.B, self.fid = d, B, fid
        self.q_n = torch.empty(B, 1, d.H, d.D, dtype=q_dtype, device=device) if fid else None
        self.idx = torch.empty(B, 1, d.top_k, dtype=torch.int32, device=device)
        self.out = torch.empty(B, 1, d.H, d.D, dtype=out_dtype, device=device)
        self.ws = lib.workspace(lib.csa_workspace_size(lib.CSA_OP_INDEX_TOPK, d, B, 1, n_cap, 0, idx_dtype), device)
        self.ws_attn = lib.workspace(lib.csa_workspace_size(lib.CSA_OP_SPARSE_ATTN, d, B, 1, n_cap, 0, lib.CSA_BF16),
                                     device)

    def __call__(self, L: int, q_idx, w_head, keys, q, entries, kv_raw, q_scale=None, k_scale=None, sink=None):
        f = self.fid
        if f:
            q = lib.csa_norm_rope(q, y=self.q_n, pos0=L, gamma=f.get("gamma_q"), eps=f.get("eps", 0.0),
                                  rope_dims=f.get("rope_dims", 0), theta=f.get("theta", 10000.0))
        lib.csa_index_topk(self.d, q_idx, w_head, keys, self.idx, q_pos0=L, q_scale=q_scale, k_scale=k_scale,
                           ws=self.ws)
        lib.csa_sparse_attn(self.d, q, entries, self.idx, kv_raw, self.out, q_pos0=L,
                            raw_pos0=L - (self.d.window - 1), sink=sink, ws=self.ws_attn)
        if f and f.get("rope_dims", 0):
            lib.csa_norm_rope(self.out, pos0=L, rope_dims=f["rope_dims"], theta=f.get("theta", 10000.0), inverse=True)
        return self.out


class CSADecodeState:
    """Token-by-token decode of B sequences over a state cache (entries, indexer keys, a ring of the
    last `window` raw KV rows, the compressor inputs of the previous and current block); when a token
    completes its block the entry and key are compressed into the caches (csa_decode_step).
    records=True keeps the entries as 584-byte FP8 records."""

    def __init__(self, d: lib.Dims, B: int, n_cap: int, dtype=torch.bfloat16, out_dtype=torch.float32,
                 records: bool = False, device="cuda"):
        self.d, self.B = d, B
        if records:
            self.entries = torch.zeros(B, n_cap, lib.ENTRY_RECORD_BYTES, dtype=torch.uint8, device=device)
        else:
            self.entries = torch.zeros(B, n_cap, d.D, dtype=dtype, device=device)
        self.keys = torch.zeros(B, n_cap, d.D_I, dtype=dtype, device=device)
        self.win = torch.zeros(B, d.window, d.D, dtype=dtype, device=device)
        self.block = torch.zeros(B, 2 * d.m, 4 * d.D + 4 * d.D_I, dtype=dtype, device=device)
        self.out = torch.empty(B, d.H, d.D, dtype=out_dtype, device=device)
        self.idx = torch.empty(B, d.top_k, dtype=torch.int32, device=device)
        code = lib.CSA_BF16 if dtype == torch.bfloat16 else lib.CSA_F32
        self.ws = lib.workspace(lib.csa_workspace_size(lib.CSA_OP_DECODE_STEP, d, B, 1, n_cap, 0, code), device)

    def state(self) -> dict:
        return {"entries": self.entries, "keys": self.keys, "win": self.win, "block": self.block}

    def step(self, weights: dict, pos: int, q, q_idx, kv, comp):
        return lib.csa_decode_step(self.d, weights, pos, q, q_idx, kv, comp, self.state(), self.out,
                                   out_idx=self.idx, ws=self.ws)

