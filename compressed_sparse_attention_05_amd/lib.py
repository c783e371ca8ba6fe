"""Thin ctypes binding of libcsa.so (include/csa.h) over torch tensors.

Argument marshalling only: every step runs in the HIP kernels of libcsa.so. torch supplies device
memory (tensors, workspaces) and the current HIP stream. There is no CPU fallback: if the library
is missing, importing the entry points fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

CSA_F32, CSA_BF16, CSA_MXFP4 = 0, 1, 2
ENTRY_RECORD_BYTES = 584
CSA_OP_COMPRESS, CSA_OP_INDEX_TOPK, CSA_OP_TOPK_FROM_SCORES, CSA_OP_SPARSE_ATTN, CSA_OP_FORWARD, CSA_OP_DENSE_ATTN, \
    CSA_OP_DECODE_STEP, CSA_OP_HCA_DECODE_STEP, CSA_OP_SPARSE_ATTN_QK = range(9)
EXPORTS = ("csa_version", "csa_last_error", "csa_workspace_size", "csa_compress", "csa_index_topk",
           "csa_topk_from_scores", "csa_sparse_attn", "csa_forward", "csa_hca_compress", "csa_dense_attn",
           "csa_norm_rope", "csa_entry_pack", "csa_sparse_attn_fp8", "csa_decode_step", "csa_dense_attn_fp8",
           "csa_hca_decode_step", "csa_decode_step_noalloc", "csa_mxfp4_quantize", "csa_sparse_attn_qk",
           "csa_projection_gemm")
PROBE_EXPORTS = ("csa_probe_hbm_read", "csa_probe_gather_read", "csa_probe_mfma_bf16", "csa_probe_sink_words")
STATIC_SCRATCH_BYTES = 64 << 20


class CsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"csa error {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32), ("H_I", ctypes.c_int32),
                ("D_I", ctypes.c_int32), ("top_k", ctypes.c_int32), ("window", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [("w_proj", ctypes.c_void_p), ("bias_a", ctypes.c_void_p), ("bias_b", ctypes.c_void_p),
                ("ibias_a", ctypes.c_void_p), ("ibias_b", ctypes.c_void_p), ("w_head", ctypes.c_void_p),
                ("sink", ctypes.c_void_p), ("gamma_q", ctypes.c_void_p), ("gamma_kv", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("rope_dims", ctypes.c_int32), ("rope_theta", ctypes.c_float)]


class Cache(ctypes.Structure):
    _fields_ = [("entries", ctypes.c_void_p), ("keys", ctypes.c_void_p), ("n_cap", ctypes.c_int64),
                ("win", ctypes.c_void_p), ("win_cap", ctypes.c_int64), ("halo", ctypes.c_void_p),
                ("halo_out", ctypes.c_void_p), ("entry_fmt", ctypes.c_int32), ("key_fmt", ctypes.c_int32),
                ("key_scales", ctypes.c_void_p)]


class DecodeState(ctypes.Structure):
    _fields_ = [("entries", ctypes.c_void_p), ("entry_fmt", ctypes.c_int32), ("keys", ctypes.c_void_p),
                ("n_cap", ctypes.c_int64), ("win", ctypes.c_void_p), ("block", ctypes.c_void_p),
                ("key_fmt", ctypes.c_int32), ("key_scales", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """Loads libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m compressed_sparse_attention_05_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.csa_version.restype = i32
    lib.csa_last_error.restype = ctypes.c_char_p
    lib.csa_workspace_size.argtypes = [i32, ctypes.POINTER(Dims), i32, i32, i64, i32, i32, ctypes.POINTER(i64)]
    lib.csa_compress.argtypes = [i32, i32, vp, i32, i32, i32, vp, vp, vp, vp, i64, i64, vp, vp, i64, i64, vp, vp,
                                 vp, i64, i64, i32, vp]
    lib.csa_index_topk.argtypes = [ctypes.POINTER(Dims), i32, i32, vp, i32, vp, i64, i64, vp, vp, i64, vp, i64, vp,
                                   i64, vp, vp, vp, sz, vp]
    lib.csa_topk_from_scores.argtypes = [vp, i64, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.csa_sparse_attn.argtypes = [ctypes.POINTER(Dims), i32, i32, vp, i32, vp, i64, i64, vp, i64, i64, vp, vp,
                                    i64, i64, vp, i64, vp, vp, i32, vp, sz, vp]
    lib.csa_forward.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), i32, i32, vp, i32, i32, vp,
                                ctypes.POINTER(Cache), vp, i32, vp, vp, sz, vp]
    lib.csa_hca_compress.argtypes = [i32, i32, vp, i32, i32, i32, vp, vp, i64, i64, vp, vp, i64, i64, i32, vp]
    lib.csa_dense_attn.argtypes = [ctypes.POINTER(Dims), i32, i32, vp, i32, vp, i64, i64, vp, i64, i64, vp,
                                   i64, i64, vp, i64, vp, vp, i32, vp, sz, vp]
    lib.csa_norm_rope.argtypes = [i32, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, vp, ctypes.c_float, i32,
                                  ctypes.c_float, vp, i64, i64, i32, vp]
    lib.csa_entry_pack.argtypes = [i32, i32, i32, vp, i64, i64, vp, i64, vp]
    lib.csa_decode_step.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), i32, vp, i32, vp, vp, vp, vp,
                                    ctypes.POINTER(DecodeState), vp, i32, vp, vp, sz, vp]
    lib.csa_sparse_attn_fp8.argtypes = lib.csa_sparse_attn.argtypes
    lib.csa_dense_attn_fp8.argtypes = lib.csa_dense_attn.argtypes
    lib.csa_hca_decode_step.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), i32, vp, i32, vp, vp, vp,
                                        ctypes.POINTER(DecodeState), vp, i32, vp, sz, vp]
    lib.csa_decode_step_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), i32, vp, i32, vp, vp, vp,
                                            vp, ctypes.POINTER(DecodeState), vp, i32, vp, vp]
    lib.csa_mxfp4_quantize.argtypes = [i64, i32, i32, vp, i64, vp, vp, vp]
    lib.csa_projection_gemm.argtypes = [i32, i32, i32, i32, vp, i64, vp, i64, vp, i64, i32, vp]
    lib.csa_sparse_attn_qk.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), i32, i32, vp, i32, vp, i64, i64, vp,
                                       i64, i64, vp, vp, i64, i64, vp, i64, vp, i32, vp, sz, vp]
    lib.csa_probe_hbm_read.argtypes = [vp, sz, vp, vp]
    lib.csa_probe_hbm_read.restype = i32
    lib.csa_probe_gather_read.argtypes = [vp, sz, sz, vp, i64, vp, vp]
    lib.csa_probe_gather_read.restype = i32
    lib.csa_probe_mfma_bf16.argtypes = [i32, vp, vp]
    lib.csa_probe_mfma_bf16.restype = i32
    lib.csa_probe_sink_words.argtypes = []
    lib.csa_probe_sink_words.restype = sz
    for f in ("csa_workspace_size", "csa_compress", "csa_index_topk", "csa_topk_from_scores", "csa_sparse_attn",
              "csa_forward", "csa_hca_compress", "csa_dense_attn", "csa_norm_rope", "csa_entry_pack",
              "csa_sparse_attn_fp8", "csa_decode_step", "csa_dense_attn_fp8", "csa_hca_decode_step",
              "csa_decode_step_noalloc", "csa_mxfp4_quantize", "csa_sparse_attn_qk",
           "csa_projection_gemm"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def make_dims(m, D, H, H_I, D_I, top_k, window, sm_scale=0.0) -> Dims:
    return Dims(m, D, H, H_I, D_I, top_k, window, sm_scale)


def _check(rc: int):
    if rc != 0:
        raise CsaError(rc, load().csa_last_error().decode())


def _p(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dt(t) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.uint8:
        return CSA_MXFP4
    raise TypeError(f"unsupported dtype {t.dtype}")


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def workspace(nbytes: int, device="cuda") -> torch.Tensor | None:
    """A byte tensor large enough for an nbytes workspace at a 256-byte aligned address."""
    return _workspace(nbytes, device)


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def positions(B: int, v, device="cuda", null_if_zero: bool = True):
    """Per-sequence positions as the device int64 [B] array the C ABI takes: an int gives every
    sequence that position (None when it is 0 and null_if_zero: the ABI reads NULL as all zeros), a
    sequence gives one per sequence, a tensor is passed as is (int64, [B], contiguous, on the GPU)."""
    if v is None:
        return None
    if isinstance(v, torch.Tensor):
        if v.dtype != torch.int64 or v.numel() != B or not v.is_cuda or not v.is_contiguous():
            raise ValueError("positions must be a contiguous int64 [B] tensor on the GPU")
        return v
    if isinstance(v, (int, np.integer)):
        if v == 0 and null_if_zero:
            return None
        return torch.full((B,), int(v), dtype=torch.int64, device=device)
    t = torch.as_tensor(np.asarray(v, dtype=np.int64), device=device)
    if t.numel() != B:
        raise ValueError(f"{t.numel()} positions for {B} sequences")
    return t.contiguous()


def _aligned_ptr(ws):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    off = (-p) % 256
    return p + off, ws.numel() - off


def csa_version() -> int:
    return load().csa_version()


def csa_workspace_size(op: int, dims: Dims, B: int, T: int, n_cap: int, d_model: int = 0,
                       idx_dtype: int = CSA_BF16) -> int:
    out = ctypes.c_int64(0)
    _check(load().csa_workspace_size(op, ctypes.byref(dims), B, T, n_cap, d_model, idx_dtype, ctypes.byref(out)))
    return out.value


def csa_compress(ca, za, cb, zb, bias_a, bias_b, entries, *, pos0, m: int, halo_cb=None, halo_zb=None):
    """Step 1. ca/za/cb/zb: [B, T, c] views sharing strides; entries: [B, n_cap, c] (rows contiguous);
    pos0: an int or per-sequence positions (see positions())."""
    _require_cuda(ca, za, cb, zb, bias_a, bias_b, entries, halo_cb, halo_zb)
    B, T, c = ca.shape
    for v in (za, cb, zb):
        if v.shape != ca.shape or v.stride() != ca.stride():
            raise ValueError("ca, za, cb, zb must share shape and strides")
    if ca.stride(2) != 1 or entries.stride(2) != 1 or entries.stride(1) != c:
        raise ValueError("channel axes must be contiguous")
    hl = hs = 0
    if halo_cb is not None:
        if halo_cb.stride() != halo_zb.stride() or halo_cb.stride(2) != 1:
            raise ValueError("halo views must share strides with unit channel stride")
        hl, hs = halo_cb.stride(1), halo_cb.stride(0)
    pos = positions(B, pos0, ca.device)
    _check(load().csa_compress(B, T, _p(pos), m, c, _dt(ca), _p(ca), _p(za), _p(cb), _p(zb), ca.stride(1), ca.stride(0),
                               _p(halo_cb), _p(halo_zb), hl, hs, _p(bias_a), _p(bias_b), _p(entries),
                               entries.stride(0), entries.shape[1], _dt(entries), _stream()))
    return entries


def csa_index_topk(dims: Dims, q_idx, w, keys, out_idx, *, q_pos0, q_scale=None, k_scale=None,
                   out_score=None, ws=None):
    """Steps 2+3. q_idx [B, T, H_I, D_I] (MXFP4: uint8 codes [B, T, H_I, D_I/2] + q_scale);
    keys [B, n_cap, D_I] (MXFP4: uint8 [B, n_cap, D_I/2] + k_scale); w [H_I] or per row [B, T, H_I];
    out_idx int32 [B, T, k]."""
    _require_cuda(q_idx, w, keys, out_idx, q_scale, k_scale, out_score)
    B, T = q_idx.shape[0], q_idx.shape[1]
    n_cap = keys.shape[1]
    dt = _dt(q_idx)
    if dt == CSA_MXFP4:
        q_ld = q_ss = 0
        k_ss = 0
    else:
        if q_idx.stride(3) != 1 or q_idx.stride(2) != dims.D_I or keys.stride(2) != 1 or keys.stride(1) != dims.D_I:
            raise ValueError("indexer rows must be contiguous")
        q_ld, q_ss, k_ss = q_idx.stride(1), q_idx.stride(0), keys.stride(0)
    w_ld = 0 if w.dim() == 1 else w.stride(-2)
    if out_idx.shape != (B, T, dims.top_k) or out_idx.dtype != torch.int32 or not out_idx.is_contiguous():
        raise ValueError("out_idx must be a contiguous int32 [B, T, top_k] tensor")
    need = csa_workspace_size(CSA_OP_INDEX_TOPK, dims, B, T, n_cap, 0, dt)
    if ws is None or ws.numel() < need + 256:
        ws = _workspace(need, q_idx.device)
    wp, wn = _aligned_ptr(ws)
    qp = positions(B, q_pos0, q_idx.device)
    _check(load().csa_index_topk(ctypes.byref(dims), B, T, _p(qp), dt, _p(q_idx), q_ld, q_ss, _p(q_scale), _p(w),
                                 w_ld, _p(keys), k_ss, _p(k_scale), n_cap, _p(out_idx), _p(out_score), wp, wn,
                                 _stream()))
    return out_idx


def csa_topk_from_scores(scores, n_valid, k: int, out_idx, out_score=None):
    """Step 3 alone on float32 scores [R, n] with n_valid int32 [R]; out_idx int32 [R, k]."""
    _require_cuda(scores, n_valid, out_idx, out_score)
    R, n = scores.shape
    if scores.stride(1) != 1:
        raise ValueError("score rows must be contiguous")
    d = make_dims(1, 1, 1, 1, 1, k, 1)
    need = csa_workspace_size(CSA_OP_TOPK_FROM_SCORES, d, R, 1, scores.stride(0))
    ws = _workspace(need, scores.device)
    wp, wn = _aligned_ptr(ws)
    _check(load().csa_topk_from_scores(_p(scores), scores.stride(0), _p(n_valid), R, k, _p(out_idx), _p(out_score),
                                       wp, wn, _stream()))
    return out_idx


def csa_sparse_attn(dims: Dims, q, entries, idx, kv_raw, out, *, q_pos0, raw_pos0, sink=None, ws=None):
    """Step 4. q [B, T, H, D]; entries [B, n_cap, D]; idx int32 [B, T, k]; kv_raw [B, R, D] whose row r of
    sequence b is position raw_pos0[b] + r; out [B, T, H, D] (float32 or bfloat16). Positions: ints or
    per-sequence (see positions())."""
    _require_cuda(q, entries, idx, kv_raw, out, sink)
    B, T = q.shape[0], q.shape[1]
    records = entries.dtype == torch.uint8          # [B, n_cap, 584] FP8 entry records
    row = ENTRY_RECORD_BYTES if records else dims.D
    if q.stride(3) != 1 or q.stride(2) != dims.D or entries.stride(2) != 1 or entries.stride(1) != row:
        raise ValueError("q heads and entry rows must be contiguous")
    if kv_raw.stride(2) != 1 or not out.is_contiguous() or not idx.is_contiguous():
        raise ValueError("kv_raw rows, idx and out must be contiguous")
    need = csa_workspace_size(CSA_OP_SPARSE_ATTN, dims, B, T, entries.shape[1], 0, _dt(q))
    if ws is None or ws.numel() < need + 256:
        ws = _workspace(need, q.device)
    wp, wn = _aligned_ptr(ws)
    fn = load().csa_sparse_attn_fp8 if records else load().csa_sparse_attn
    qp, rp = positions(B, q_pos0, q.device), positions(B, raw_pos0, q.device)
    _check(fn(ctypes.byref(dims), B, T, _p(qp), _dt(q), _p(q), q.stride(1), q.stride(0),
              _p(entries), entries.stride(0), entries.shape[1], _p(idx), _p(kv_raw),
              kv_raw.stride(1), kv_raw.stride(0), _p(rp), kv_raw.shape[1], _p(sink), _p(out),
              _dt(out), wp, wn, _stream()))
    return out


def csa_sparse_attn_qk(dims: Dims, fid: dict, q, entries, idx, kv_raw, out, *, q_pos0, raw_pos0, sink=None,
                       ws=None):
    """csa_sparse_attn with QK-norm and partial RoPE of the query and the output's back-rotation (see
    include/csa.h); fid: gamma_q (float32 [D] tensor or None), eps, rope_dims, theta. Entries are rows."""
    _require_cuda(q, entries, idx, kv_raw, out, sink, fid.get("gamma_q"))
    B, T = q.shape[0], q.shape[1]
    if q.stride(3) != 1 or q.stride(2) != dims.D or entries.stride(2) != 1 or entries.stride(1) != dims.D:
        raise ValueError("q heads and entry rows must be contiguous")
    if kv_raw.stride(2) != 1 or not out.is_contiguous() or not idx.is_contiguous():
        raise ValueError("kv_raw rows, idx and out must be contiguous")
    need = csa_workspace_size(CSA_OP_SPARSE_ATTN_QK, dims, B, T, entries.shape[1], 0, _dt(q))
    if ws is None or ws.numel() < need + 256:
        ws = _workspace(need, q.device)
    wp, wn = _aligned_ptr(ws)
    w = Weights(None, None, None, None, None, None, _p(sink), _p(fid.get("gamma_q")), None,
                float(fid.get("eps", 0.0)), int(fid.get("rope_dims", 0)), float(fid.get("theta", 10000.0)))
    qp, rp = positions(B, q_pos0, q.device), positions(B, raw_pos0, q.device)
    _check(load().csa_sparse_attn_qk(ctypes.byref(dims), ctypes.byref(w), B, T, _p(qp), _dt(q), _p(q), q.stride(1),
                                     q.stride(0), _p(entries), entries.stride(0), entries.shape[1], _p(idx),
                                     _p(kv_raw), kv_raw.stride(1), kv_raw.stride(0), _p(rp), kv_raw.shape[1],
                                     _p(out), _dt(out), wp, wn, _stream()))
    return out


def csa_entry_pack(entries, records=None):
    """entries [B, N, 512] (float32 or bfloat16) -> 584-byte FP8 records [B, N, 584] (uint8)."""
    _require_cuda(entries, records)
    B, N, D = entries.shape
    if D != 512 or entries.stride(2) != 1:
        raise ValueError("entries must be [B, N, 512] with contiguous rows")
    if records is None:
        records = torch.empty(B, N, ENTRY_RECORD_BYTES, dtype=torch.uint8, device=entries.device)
    if records.shape != (B, N, ENTRY_RECORD_BYTES) or records.stride(2) != 1 or records.stride(1) != ENTRY_RECORD_BYTES:
        raise ValueError("records must be [B, N, 584] with contiguous rows")
    _check(load().csa_entry_pack(B, N, _dt(entries), _p(entries), entries.stride(1), entries.stride(0), _p(records),
                                 records.stride(0), _stream()))
    return records


def csa_mxfp4_quantize(x, codes=None, scales=None):
    """x [R, D] (float32 or bfloat16, unit stride along D, D % 32 == 0) -> MXFP4 codes uint8 [R, D/2] and
    scales uint8 [R, D/32] (see include/csa.h). Returns (codes, scales)."""
    _require_cuda(x, codes, scales)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [R, D] with unit stride along D")
    R, D = x.shape
    if codes is None:
        codes = torch.empty(R, D // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(R, D // 32, dtype=torch.uint8, device=x.device)
    if not (codes.is_contiguous() and scales.is_contiguous()) or codes.numel() != R * (D // 2) or \
            scales.numel() != R * (D // 32):
        raise ValueError("codes / scales must be contiguous [R, D/2] / [R, D/32]")
    _check(load().csa_mxfp4_quantize(R, D, _dt(x), _p(x), x.stride(0), _p(codes), _p(scales), _stream()))
    return codes, scales


def csa_projection_gemm(a, wt, c):
    """c [M, N] = a [M, K] @ wt [N, K]^T on the library's own GEMM kernels (see include/csa.h); rows of
    each operand must have unit stride."""
    _require_cuda(a, wt, c)
    if a.stride(1) != 1 or wt.stride(1) != 1 or c.stride(1) != 1 or a.dtype != wt.dtype:
        raise ValueError("operands need unit stride along rows and one input dtype")
    M, K = a.shape
    N = wt.shape[0]
    if wt.shape[1] != K or tuple(c.shape) != (M, N):
        raise ValueError("shapes do not match")
    _check(load().csa_projection_gemm(M, N, K, _dt(a), _p(a), a.stride(0), _p(wt), wt.stride(0), _p(c), c.stride(0),
                                      _dt(c), _stream()))
    return c


def probe_sink(device="cuda") -> torch.Tensor:
    """A sink buffer for the ceiling probes (include/csa_probe.h)."""
    return torch.empty(load().csa_probe_sink_words(), dtype=torch.int32, device=device)


def probe_hbm_read(buf: torch.Tensor, sink: torch.Tensor):
    """Reads all of buf (a contiguous device tensor, 16-byte aligned, nbytes % 16 == 0) once."""
    _check(load().csa_probe_hbm_read(_p(buf), buf.numel() * buf.element_size(), _p(sink), _stream()))


def probe_gather_read(buf: torch.Tensor, row_bytes: int, idx: torch.Tensor, sink: torch.Tensor):
    """Reads the rows idx (int32 device tensor) of buf, each row_bytes long, once (see include/csa_probe.h)."""
    _check(load().csa_probe_gather_read(_p(buf), buf.numel() * buf.element_size(), row_bytes, _p(idx), idx.numel(),
                                        _p(sink), _stream()))


def probe_mfma_bf16(iters: int, sink: torch.Tensor) -> int:
    """Runs the MFMA probe; returns its FLOP count."""
    _check(load().csa_probe_mfma_bf16(iters, _p(sink), _stream()))
    return (load().csa_probe_sink_words() // 64) * 4 * 32768 * iters


def csa_hca_compress(cv, z, bias, entries, *, pos0, m: int):
    """HCA compressor. cv, z: [B, T, c] views sharing strides; bias float32 [m, c]; entries [B, n_cap, c]."""
    _require_cuda(cv, z, bias, entries)
    B, T, c = cv.shape
    if z.shape != cv.shape or z.stride() != cv.stride():
        raise ValueError("cv and z must share shape and strides")
    if cv.stride(2) != 1 or entries.stride(2) != 1 or entries.stride(1) != c:
        raise ValueError("channel axes must be contiguous")
    pos = positions(B, pos0, cv.device)
    _check(load().csa_hca_compress(B, T, _p(pos), m, c, _dt(cv), _p(cv), _p(z), cv.stride(1), cv.stride(0), _p(bias),
                                   _p(entries), entries.stride(0), entries.shape[1], _dt(entries), _stream()))
    return entries


def csa_norm_rope(x, *, pos0, pos_step: int = 1, pos_off: int = 0, gamma=None, eps: float = 0.0,
                  rope_dims: int = 0, theta: float = 10000.0, inverse: bool = False, y=None):
    """QK-norm and partial RoPE on x [B, R, H, D] (or [B, R, D]: one head), row r of sequence b at position
    pos0[b] + pos_off + r * pos_step (pos0: an int or per-sequence positions); into y (same shape and
    dtype) or in place. gamma float32 [D] or None."""
    _require_cuda(x, y, gamma)
    y = x if y is None else y
    if x.dim() == 3:
        B, R, D = x.shape
        H = 1
    else:
        B, R, H, D = x.shape
    for t in (x, y):
        if t.stride(-1) != 1 or (t.dim() == 4 and t.stride(2) != D):
            raise ValueError("head vectors must be contiguous")
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("y must match x")
    if isinstance(pos0, (int, np.integer)):  # a common position goes in pos_off (no device array)
        pos_off, pos0 = pos_off + int(pos0), None
    pos = positions(B, pos0, x.device)
    _check(load().csa_norm_rope(B, R, H, D, _dt(x), _p(x), x.stride(1), x.stride(0), _p(y), y.stride(1), y.stride(0),
                                _p(gamma), eps, rope_dims, theta, _p(pos), pos_off, pos_step, 1 if inverse else 0,
                                _stream()))
    return y


def csa_dense_attn(dims: Dims, q, entries, kv_raw, out, *, q_pos0, raw_pos0, sink=None, ws=None):
    """HCA attention over every visible entry plus the window. q [B, T, H, D]; entries [B, n_cap, D];
    kv_raw [B, R, D] whose row r is position raw_pos0 + r; out [B, T, H, D] (float32 or bfloat16)."""
    _require_cuda(q, entries, kv_raw, out, sink)
    B, T = q.shape[0], q.shape[1]
    records = entries.dtype == torch.uint8          # [B, n_cap, 584] FP8 entry records
    row = ENTRY_RECORD_BYTES if records else dims.D
    if q.stride(3) != 1 or q.stride(2) != dims.D or entries.stride(2) != 1 or entries.stride(1) != row:
        raise ValueError("q heads and entry rows must be contiguous")
    if kv_raw.stride(2) != 1 or not out.is_contiguous():
        raise ValueError("kv_raw rows and out must be contiguous")
    need = csa_workspace_size(CSA_OP_DENSE_ATTN, dims, B, T, entries.shape[1], 0, _dt(q))
    if ws is None or ws.numel() < need + 256:
        ws = _workspace(need, q.device)
    wp, wn = _aligned_ptr(ws)
    fn = load().csa_dense_attn_fp8 if records else load().csa_dense_attn
    qp, rp = positions(B, q_pos0, q.device), positions(B, raw_pos0, q.device)
    _check(fn(ctypes.byref(dims), B, T, _p(qp), _dt(q), _p(q), q.stride(1), q.stride(0),
              _p(entries), entries.stride(0), entries.shape[1], _p(kv_raw), kv_raw.stride(1),
              kv_raw.stride(0), _p(rp), kv_raw.shape[1], _p(sink), _p(out), _dt(out), wp, wn, _stream()))
    return out


def weights_struct(weights: dict) -> Weights:
    return Weights(_p(weights.get("w_proj")), _p(weights["bias_a"]), _p(weights["bias_b"]), _p(weights["ibias_a"]),
                   _p(weights["ibias_b"]), _p(weights["w_head"]), _p(weights.get("sink")),
                   _p(weights.get("gamma_q")), _p(weights.get("gamma_kv")), float(weights.get("norm_eps", 0.0)),
                   int(weights.get("rope_dims", 0)), float(weights.get("rope_theta", 10000.0)))


def _state_struct(state: dict, keys: bool = True) -> DecodeState:
    """The C decode state of a dict of tensors: entries (rows, or uint8 records), keys (rows, or uint8
    MXFP4 codes when key_scales is given), win, block."""
    ent = state["entries"]
    ks = state.get("key_scales") if keys else None
    return DecodeState(_p(ent), 1 if ent.dtype == torch.uint8 else 0, _p(state["keys"]) if keys else None,
                       ent.shape[1], _p(state["win"]), _p(state["block"]), 1 if ks is not None else 0, _p(ks))


def csa_decode_step(dims: Dims, weights: dict, pos, q, q_idx, kv, comp, state: dict, out, *, out_idx=None,
                    ws=None):
    """One decode step of B sequences, sequence b at position pos[b] (an int: all at pos), over a decode
    state (see include/csa.h):
    q [B, H, D], q_idx [B, H_I, D_I], kv [B, D], comp [B, 4D + 4D_I]; state holds entries (rows, or
    uint8 records [B, n_cap, 584]), keys (rows, or uint8 MXFP4 codes [B, n_cap, D_I/2] with key_scales
    [B, n_cap, D_I/32]), win [B, window, D], block [B, 2m, 4D + 4D_I]."""
    _require_cuda(q, q_idx, kv, comp, out, out_idx)
    for t in (q, q_idx, kv, comp, out):
        if not t.is_contiguous():
            raise ValueError("decode step tensors must be contiguous")
    B = q.shape[0]
    ent = state["entries"]
    st = _state_struct(state)
    need = csa_workspace_size(CSA_OP_DECODE_STEP, dims, B, 1, ent.shape[1], 0, _dt(q))
    if ws is None or ws.numel() < need + 256:
        ws = _workspace(need, q.device)
    wp, wn = _aligned_ptr(ws)
    w = weights_struct(weights)
    pt = positions(B, pos, q.device, null_if_zero=False)
    _check(load().csa_decode_step(ctypes.byref(dims), ctypes.byref(w), B, _p(pt), _dt(q), _p(q), _p(q_idx), _p(kv),
                                  _p(comp), ctypes.byref(st), _p(out), _dt(out), _p(out_idx), wp, wn, _stream()))
    return out


def csa_decode_step_noalloc(dims: Dims, weights: dict, pos, q, q_idx, kv, comp, state: dict, out, *, out_idx=None):
    """csa_decode_step with the scratch the library holds on the GPU (no workspace; see include/csa.h).
    pos must be a device int64 [B] tensor: building one here would allocate."""
    _require_cuda(q, q_idx, kv, comp, out, out_idx)
    for t in (q, q_idx, kv, comp, out):
        if not t.is_contiguous():
            raise ValueError("decode step tensors must be contiguous")
    if not isinstance(pos, torch.Tensor):
        raise TypeError("pos must be a device int64 [B] tensor")
    B = q.shape[0]
    pt = positions(B, pos, q.device)
    st = _state_struct(state)
    w = weights_struct(weights)
    _check(load().csa_decode_step_noalloc(ctypes.byref(dims), ctypes.byref(w), B, _p(pt), _dt(q), _p(q), _p(q_idx),
                                          _p(kv), _p(comp), ctypes.byref(st), _p(out), _dt(out), _p(out_idx),
                                          _stream()))
    return out


def csa_hca_decode_step(dims: Dims, weights: dict, pos, q, kv, comp, state: dict, out, *, ws=None):
    """One HCA decode step (see include/csa.h): q [B, H, D], kv [B, D], comp [B, 2D]; state holds entries
    (rows, or uint8 records), win [B, window, D], block [B, m, 2D]; weights: bias_a [m, D] (the pooling
    biases), sink and the QK-norm / RoPE fields."""
    _require_cuda(q, kv, comp, out)
    for t in (q, kv, comp, out):
        if not t.is_contiguous():
            raise ValueError("decode step tensors must be contiguous")
    B = q.shape[0]
    ent = state["entries"]
    st = _state_struct(state, keys=False)
    need = csa_workspace_size(CSA_OP_HCA_DECODE_STEP, dims, B, 1, ent.shape[1], 0, _dt(q))
    if ws is None or ws.numel() < need + 256:
        ws = _workspace(need, q.device)
    wp, wn = _aligned_ptr(ws)
    w = Weights(None, _p(weights["bias_a"]), None, None, None, None, _p(weights.get("sink")),
                _p(weights.get("gamma_q")), _p(weights.get("gamma_kv")), float(weights.get("norm_eps", 0.0)),
                int(weights.get("rope_dims", 0)), float(weights.get("rope_theta", 10000.0)))
    pt = positions(B, pos, q.device, null_if_zero=False)
    _check(load().csa_hca_decode_step(ctypes.byref(dims), ctypes.byref(w), B, _p(pt), _dt(q), _p(q), _p(kv), _p(comp),
                                      ctypes.byref(st), _p(out), _dt(out), wp, wn, _stream()))
    return out


class Forward:
    """csa_forward with a reusable workspace (allocated once per shape, outside the timed call)."""

    def __init__(self, dims: Dims, B: int, T: int, d_model: int, n_cap: int, dtype: int, device):
        self.dims, self.B, self.T, self.d_model, self.dtype = dims, B, T, d_model, dtype
        need = csa_workspace_size(CSA_OP_FORWARD, dims, B, T, n_cap, d_model, dtype)
        self._ws = _workspace(need, device)
        self._wp, self._wn = _aligned_ptr(self._ws)

    def projection(self) -> torch.Tensor:
        """The projection x @ w_proj^T of the last call, [B*T, n_tot], as a view of the workspace."""
        d = self.dims
        n_tot = 4 * d.D + 4 * d.D_I + d.H * d.D + d.H_I * d.D_I + d.D
        es = 4 if self.dtype == CSA_F32 else 2
        off = self._wp - self._ws.data_ptr()
        raw = self._ws[off:off + self.B * self.T * n_tot * es]
        return raw.view(torch.float32 if es == 4 else torch.bfloat16).view(self.B * self.T, n_tot)

    def __call__(self, weights: dict, x, cache: dict, out, *, pos0, out_idx=None):
        """pos0: an int (every sequence) or per-sequence positions (see positions())."""
        w = weights_struct(weights)
        pos = positions(self.B, pos0, x.device)
        ks = cache.get("key_scales")
        c = Cache(_p(cache["entries"]), _p(cache["keys"]), cache["entries"].shape[1], _p(cache["win"]),
                  cache["win"].shape[1], _p(cache.get("halo")), _p(cache.get("halo_out")),
                  1 if cache["entries"].dtype == torch.uint8 else 0, 1 if ks is not None else 0, _p(ks))
        _check(load().csa_forward(ctypes.byref(self.dims), ctypes.byref(w), self.B, self.T, _p(pos), self.d_model,
                                  self.dtype, _p(x), ctypes.byref(c), _p(out), _dt(out), _p(out_idx), self._wp,
                                  self._wn, _stream()))
        return out


def csa_forward(dims: Dims, weights: dict, x, cache: dict, out, *, pos0, out_idx=None):
    """The whole layer on x [B, T, d_model]; see include/csa.h for the cache layout."""
    _require_cuda(x, out)
    B, T, d = x.shape
    f = Forward(dims, B, T, d, cache["entries"].shape[1], _dt(x), x.device)
    return f(weights, x, cache, out, pos0=pos0, out_idx=out_idx)
