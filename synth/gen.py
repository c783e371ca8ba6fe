"""Seeded input generation for the named CSA workloads.

Recipe (the same bits feed the oracle and the GPU path):

* Every named tensor has its own counter-style stream: element chunk c of tensor `name` is drawn
  from ``PCG64(SeedSequence(seed, spawn_key=(crc32(name), c)))``, so the bits depend neither on the
  order tensors are drawn in nor on how many threads draw them.
* Normal draws are float32 standard normals scaled by the stated standard deviation.
* bf16 tensors are those float32 draws rounded to nearest-even bf16 and kept as raw uint16 bits.
* MXFP4 tensors (OCP Microscaling v1.0): per 32 consecutive elements an e8m0 scale
  2**(floor(log2(max|x|)) - 2) and e2m1 codes rounded to nearest-even with saturation at 6;
  two codes per byte, the even-indexed element in the low nibble.

Distributions, per the workload descriptions: activations x ~ N(0, 1); projection weights
~ N(0, 1/d); position biases ~ N(0, 0.1) (variance 0.1); indexer head weights w = softmax over the
heads of N(0, 1) draws; pre-built caches (compressed entries, indexer keys, raw window KV, queries)
~ N(0, 1).
"""
from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import Workload

CHUNK = 1 << 22           # elements per independent random stream
_THREADS = 8


def _stream(seed: int, name: str, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(zlib.crc32(name.encode()), chunk))
    return np.random.Generator(np.random.PCG64(ss))


def normal_f32(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draws of the given shape, chunked into independent streams."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        _stream(seed, name, c).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nchunks)))
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for lo in range(0, flat_u.size, step):
        v = flat_u[lo:lo + step].astype(np.uint64)
        v = (v + 0x7FFF + ((v >> 16) & 1)) >> 16
        flat_o[lo:lo + step] = v.astype(np.uint16)
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_E2M1_EDGES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def mxfp4_encode(x: np.ndarray):
    """float32 [..., D] (D % 32 == 0) -> (codes uint8 [..., D/2], scales uint8 [..., D/32])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (D // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    scales = (e + 127).astype(np.uint8)
    v = blocks / np.exp2(e.astype(np.float32))[..., None]
    mag = np.abs(v)
    code = np.zeros(mag.shape, dtype=np.uint8)
    for j, edge in enumerate(_E2M1_EDGES):
        # a value exactly on an edge goes to the even code (j + 1 is even when j is odd)
        passed = (mag > edge) | ((mag == edge) & (j % 2 == 1))
        code += passed.astype(np.uint8)
    code |= np.where((v < 0) & (code > 0), 8, 0).astype(np.uint8)
    code = code.reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, scales


def _act(seed, name, shape, wl: Workload, std=1.0):
    a = normal_f32(seed, name, shape, std)
    return f32_to_bf16_bits(a) if wl.dtype == "bf16" else a


def _softmax_weights(seed, name, n):
    z = normal_f32(seed, name, (n,)).astype(np.float64)
    e = np.exp(z - z.max())
    return (e / e.sum()).astype(np.float32)


def make_inputs(wl: Workload) -> dict:
    """All inputs of one workload as numpy arrays (bf16 tensors as uint16 bits)."""
    s = wl.seed
    B, m, D, DI = wl.B, wl.m, wl.D, wl.D_I
    out = {"w_head": _softmax_weights(s, "w_head", wl.H_I)}
    if wl.kind == "prefill":
        d = wl.d
        out["x"] = _act(s, "x", (B, wl.T, d), wl)
        out["W"] = _act(s, "W", (wl.n_tot, d), wl, std=1.0 / np.sqrt(d))
        bstd = float(np.sqrt(0.1))
        out["bias_a"] = normal_f32(s, "bias_a", (m, D), bstd)
        out["bias_b"] = normal_f32(s, "bias_b", (m, D), bstd)
        out["ibias_a"] = normal_f32(s, "ibias_a", (m, DI), bstd)
        out["ibias_b"] = normal_f32(s, "ibias_b", (m, DI), bstd)
        if wl.L > 0:
            assert wl.L % m == 0
            n0 = wl.L // m
            out["entries_prefix"] = _act(s, "entries_prefix", (B, n0, D), wl)
            if wl.idx_dtype == "mxfp4":
                out["keys_prefix_codes"], out["keys_prefix_scales"] = mxfp4_encode(
                    normal_f32(s, "keys_prefix", (B, n0, DI)))
            else:
                out["keys_prefix"] = _act(s, "keys_prefix", (B, n0, DI), wl)
            out["win_prefix"] = _act(s, "win_prefix", (B, wl.W - 1, D), wl)
            out["halo"] = _act(s, "halo", (B, m, 2 * D + 2 * DI), wl)
    else:
        assert wl.T == 1 and wl.L % m == 0
        N = wl.L // m
        out["entries"] = _act(s, "entries", (B, N, D), wl)
        out["kv_raw"] = _act(s, "kv_raw", (B, wl.W, D), wl)
        out["q"] = _act(s, "q", (B, 1, wl.H, D), wl)
        if wl.idx_dtype == "mxfp4":
            out["keys_codes"], out["keys_scales"] = mxfp4_encode(
                normal_f32(s, "keys", (B, N, DI)))
            out["q_idx_codes"], out["q_idx_scales"] = mxfp4_encode(
                normal_f32(s, "q_idx", (B, 1, wl.H_I, DI)))
        else:
            out["keys"] = _act(s, "keys", (B, N, DI), wl)
            out["q_idx"] = _act(s, "q_idx", (B, 1, wl.H_I, DI), wl)
    return out


def dyadic_projection(inp: dict, wl: Workload) -> dict:
    """The inputs with x and W moved to coarse power-of-two grids (x in multiples of 1/4 within [-2, 2],
    W in multiples of 1/128 within [-1/16, 1/16]), so that every projected value is exact in float32
    whatever the summation order: products are multiples of 2**-9 below 2**-3 in magnitude, and d_model
    of them need at most 24 significant bits. Used where a quantiser decides codes from the projected
    values, so that both sides quantise the same numbers."""
    out = dict(inp)
    x = np.clip(np.rint(normal_f32(wl.seed, "x", (wl.B, wl.T, wl.d)) * 4), -8, 8) / 4
    W = np.clip(np.rint(normal_f32(wl.seed, "W", (wl.n_tot, wl.d), std=1.0 / np.sqrt(wl.d)) * 128), -8, 8) / 128
    assert wl.d * 2 ** -3 < 2 ** 15, "projection sums must stay exact in float32"
    conv = f32_to_bf16_bits if wl.dtype == "bf16" else (lambda a: a)
    out["x"] = conv(x.astype(np.float32))
    out["W"] = conv(W.astype(np.float32))
    return out
