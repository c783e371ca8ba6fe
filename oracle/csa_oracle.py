"""Plain CPU oracle of the Compressed Sparse Attention (CSA) forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run this module: only the
tests, the smoke check and the CPU-baseline leg of the benchmark use it. It shares no code with the
HIP library.

Everything is computed in float64 with NumPy, one definition at a time, in the order the pages give
the steps. Where the GPU path stores an intermediate in bf16 (projected activations, compressed
entries, indexer keys) the oracle rounds to bf16 at that same point (round to nearest, ties to even,
straight from float64); fp32 workloads round nothing.

Sources (pages as titled):
  [EXR]  "The Exchange Rates of a Million Tokens", section 3 "Rate #2: bytes buy budget, and spend
         recall": two overlapping series Ca/Cb under one joint softmax; an indexer of ReLU-gated dot
         products that selects the top-k compressed blocks.
  [ANAT] "Anatomy of a Frontier Model: Reading DeepSeek-V4 Through Part V":
         "The skeleton, and what's kept": one key-value head shared by all query heads, and each
         cached entry is both the key and the value;
         "The attention: compress, then select", bullet "Compressed Sparse Attention (CSA)": every 4
         tokens become one entry by a per-channel softmax-weighted pooling with learned position
         biases, each entry pooling its own block and the one before; a 64-head x 128-dim indexer
         ranks entries and each query keeps 1,024 (512 in Flash);
         bullet "A sliding window in every layer": an entry exists only once its block is complete,
         and every layer also attends directly to the last 128 tokens;
         bullet "An attention sink": a per-head learned logit whose exponential joins the softmax
         denominator;
         section "Precision: FP8 everywhere, FP4 experts": the indexer's query-key path in FP4.
  The indexer score is s[t, i] = sum_h w_h * ReLU(q_I[t, h] . k_I[i]).

Readings where the pages are silent (each is listed with its reason in the design notes):
  series a pools the entry's own block and series b the previous block; entry 0 has no previous
  block and pools only its own m tokens; an entry i is visible to the query at position p iff its
  block is complete, (i+1)*m - 1 <= p, so n_vis(p) = floor((p+1)/m); the window is the W raw tokens
  [max(0, p-W+1), p] including p itself; selected entries and window tokens share one softmax with
  scale 1/sqrt(D); top-k ties break toward the smaller entry index; fewer than k visible entries
  means all of them are kept and the index list is padded with -1.

Entry records ([ANAT] "The KV cache, recomputed"): e4m3_encode / e4m3_decode (OCP FP8 E4M3) and
entry_pack / entry_unpack, the 584-byte record of 448 FP8 dims with 7 UE8M0 scales plus 64 bf16
RoPE dims (readings: byte order, and the smallest power-of-two scale that keeps a 64-dim group
within 448).

QK-norm and partial RoPE ([ANAT] bullet "QK-norm and partial RoPE"): rms_norm and rope, applied by
prefill/decode when their fid argument is given (readings: a per-dim gain, adjacent-pair rotation
with base theta, entries rotated at the last token of their block, the window's raw KV normalised
and rotated like an entry at its token's position).

FP4 indexer ([ANAT] "The KV cache, recomputed" and "Precision: FP8 everywhere, FP4 experts"):
mxfp4_quantize / mxfp4_decode (OCP MXFP4: e2m1 elements, one e8m0 scale per 32); prefill quantises
the chunk's new keys and its indexer queries when the workload's indexer storage is MXFP4 (reading:
quantise the stored bf16 values, the sign bit copies the input's sign).

HCA ([ANAT] bullet "Heavily Compressed Attention (HCA)"): hca_compress pools each block of m = 128
tokens with no overlap (reading: the CSA pooling over the entry's own block); dense_attention
attends to every visible entry plus the window.

Parity status: every function here is pinned by the CPU tests (closed forms, invariants, a dense
attention routine, hand-worked examples, the MXFP4 table and conversion rule of the OCP spec). What the pages leave open
(the readings above) cannot be pinned against DeepSeek's own layer: that part is parity unpinned.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------------------
# Storage formats
# --------------------------------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact values as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits, ties to even).

    bf16 keeps float32's 8-bit exponent and 7 stored mantissa bits. For a normal x = f * 2**e with
    0.5 <= |f| < 1, the bf16 grid spacing is 2**(e - 8); below the smallest normal (2**-126) it is
    fixed at 2**-133. Overflow past the largest finite bf16 goes to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)                      # subnormal range keeps the spacing 2**-133
    spacing = np.ldexp(1.0, e - 8)
    y = np.rint(x / spacing) * spacing           # np.rint rounds half to even
    big = 3.3895313892515355e38                  # largest finite bf16
    y = np.where(np.abs(y) > big, np.copysign(np.inf, y), y)
    return y


# e2m1 magnitudes for codes 0..7 (OCP Microscaling Formats v1.0, FP4 E2M1): exponent bias 1,
# subnormal 0.5, largest normal 6.
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    """4-bit e2m1 codes (bit 3 = sign, bits 2-1 = exponent, bit 0 = mantissa) -> float64."""
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_MAGNITUDE[code & 7]
    return np.where(code & 8, -mag, mag)


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 block format -> float64.

    codes [..., D/2] hold two e2m1 elements per byte, the even-indexed element in the low nibble;
    scales [..., D/32] are e8m0 exponents, one per 32 consecutive elements: scale = 2**(E - 127).
    The FP4 indexer path is the one the pages run in FP4 ([ANAT] "Precision"); the block of 32 with a
    one-byte scale is the cache layout of [ANAT] "The KV cache, recomputed".
    """
    codes = np.asarray(codes, dtype=np.uint8)
    lo = e2m1_decode(codes & 0x0F)
    hi = e2m1_decode(codes >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    E = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    if np.any(E == 255):
        raise ValueError("e8m0 NaN scale")
    scale = np.ldexp(1.0, E - 127)
    D = vals.shape[-1]
    vals = vals.reshape(vals.shape[:-1] + (D // 32, 32)) * scale[..., None]
    return vals.reshape(vals.shape[:-2] + (D,))


def mxfp4_quantize(x: np.ndarray):
    """float values [..., D] (D % 32 == 0) -> MXFP4 (codes [..., D/2], scales [..., D/32]), the layout
    of mxfp4_decode.

    The conversion of a block of 32 values in the OCP Microscaling Formats v1.0 spec: the shared scale
    is 2**X with X = floor(log2(max |x|)) - 2, 2 being the largest exponent an e2m1 element has, kept
    inside the e8m0 range [-127, 127] (a block of zeros takes X = -127); every element x / 2**X goes to
    the nearest e2m1 value, ties to the one whose mantissa bit is 0, and magnitudes past 6 saturate to
    6. The pages keep indexer keys as 128 FP4 numbers plus one scale byte per 32 ([ANAT] "The KV cache,
    recomputed") and run the indexer's query-key product in FP4 ([ANAT] "Precision: FP8 everywhere,
    FP4 experts").
    Readings: the sign bit is the sign of x, so a negative value that rounds to zero is stored as -0
    (code 8); the values quantised are those of the storage type (bf16-rounded where the layer stores
    bf16), as a separate pass over the stored keys would see them.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % 32:
        raise ValueError("MXFP4 blocks need D % 32 == 0")
    blocks = x.reshape(x.shape[:-1] + (D // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)                     # amax = f * 2**e, f in [0.5, 1): floor(log2 amax) = e - 1
    X = np.where(amax > 0, e.astype(np.int64) - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    v = blocks / np.ldexp(1.0, X)[..., None]  # exact: a power of two
    dist = np.abs(np.abs(v)[..., None] - E2M1_MAGNITUDE)       # [..., 32, 8]
    nearest = dist == dist.min(axis=-1, keepdims=True)
    even = nearest & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), nearest.argmax(axis=-1)).astype(np.uint8)
    code |= np.where(np.signbit(blocks), 8, 0).astype(np.uint8)
    code = code.reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def mxfp4_round(x: np.ndarray) -> np.ndarray:
    """The values x takes once stored as MXFP4 (mxfp4_quantize, then mxfp4_decode)."""
    return mxfp4_decode(*mxfp4_quantize(x))


# e4m3 (OCP 8-bit Floating Point Specification, E4M3): bit 7 sign, bits 6-3 exponent (bias 7), bits
# 2-0 mantissa. Normal values 2^(e-7) * (1 + m/8) for e = 1..15, except e = 15, m = 7 (NaN);
# subnormals (e = 0) 2^-6 * m/8; no infinities; the largest finite magnitude is 448.
E4M3_MAX = 448.0


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """8-bit e4m3 codes -> float64 (NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> the nearest e4m3 code, ties to the even code (mantissa bit 0 clear); magnitudes
    above 448 saturate to 448; the sign bit is the sign of x (so -0.0 gives 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("NaN has no e4m3 code here")
    mags = e4m3_decode(np.arange(0x7F, dtype=np.uint8))     # codes 0x00..0x7E, ascending magnitudes
    a = np.minimum(np.abs(x), E4M3_MAX)
    i = np.clip(np.searchsorted(mags, a), 1, 0x7E)          # mags[i-1] < a <= mags[i] (or a == 0)
    lo, hi = mags[i - 1], mags[i]
    up = (hi - a < a - lo) | ((hi - a == a - lo) & (i % 2 == 0))
    code = np.where(up, i, i - 1).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


# The compressed-entry record ([ANAT] "The KV cache, recomputed" and bullet "QK-norm and partial
# RoPE"): 512 numbers, the 448 position-free ones in FP8 and the 64 RoPE dims in BF16, with seven
# one-byte UE8M0 scales and one pad byte, 584 bytes. Byte order (a reading: the pages give the sizes
# only): e4m3 codes of dims 0..447 | bf16 of dims 448..511, little-endian | 7 scale exponents, one per
# 64 consecutive FP8 dims | a zero pad byte.
ENTRY_FP8_DIMS, ENTRY_GROUP, ENTRY_BYTES = 448, 64, 584


def entry_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """UE8M0 exponent E (scale 2^(E-127)) of a group: the smallest power of two s with amax / s <=
    448, so that no element saturates (reading); an all-zero group takes E = 127."""
    amax = np.asarray(amax, dtype=np.float64)
    q = np.where(amax > 0, amax, 1.0) / E4M3_MAX
    f, e = np.frexp(q)                                     # q = f * 2^e, 0.5 <= f < 1
    k = np.where(f == 0.5, e - 1, e)                       # ceil(log2(q))
    E = np.where(amax > 0, k + 127, 127)
    if np.any((E < 0) | (E > 254)):
        raise ValueError("group magnitude outside the UE8M0 range")
    return E.astype(np.int64)


def entry_pack(e: np.ndarray) -> np.ndarray:
    """Entries [..., 512] (dims 448..511 on the bf16 grid) -> records [..., 584] uint8."""
    e = np.asarray(e, dtype=np.float64)
    if e.shape[-1] != 512:
        raise ValueError("entry records hold 512 dims")
    lead = e.shape[:-1]
    fp = e[..., :ENTRY_FP8_DIMS].reshape(lead + (ENTRY_FP8_DIMS // ENTRY_GROUP, ENTRY_GROUP))
    E = entry_scale_exponent(np.abs(fp).max(axis=-1))
    codes = e4m3_encode(fp / np.ldexp(1.0, E - 127)[..., None]).reshape(lead + (ENTRY_FP8_DIMS,))
    rope = e[..., ENTRY_FP8_DIMS:]
    if not np.array_equal(round_bf16(rope), rope):
        raise ValueError("RoPE dims must be bf16 values")
    bits = (rope.astype(np.float32).view(np.uint32) >> 16).astype("<u2")
    out = np.zeros(lead + (ENTRY_BYTES,), dtype=np.uint8)
    out[..., :448] = codes
    out[..., 448:576] = bits.view(np.uint8).reshape(lead + (128,))
    out[..., 576:583] = E.astype(np.uint8)
    return out


def entry_unpack(rec: np.ndarray) -> np.ndarray:
    """Records [..., 584] uint8 -> entries [..., 512] float64 (exact values of the stored format)."""
    rec = np.asarray(rec, dtype=np.uint8)
    lead = rec.shape[:-1]
    E = rec[..., 576:583].astype(np.int64)
    if np.any(E == 255):
        raise ValueError("UE8M0 NaN scale")
    fp = e4m3_decode(rec[..., :448]).reshape(lead + (7, 64)) * np.ldexp(1.0, E - 127)[..., None]
    bits = np.ascontiguousarray(rec[..., 448:576]).view("<u2").reshape(lead + (64,))
    return np.concatenate([fp.reshape(lead + (448,)), bf16_bits_to_f64(bits)], axis=-1)


# --------------------------------------------------------------------------------------------------
# The CSA steps
# --------------------------------------------------------------------------------------------------


def n_visible(p, m: int):
    """Compressed entries visible to the query at absolute position p.

    [ANAT] "A sliding window in every layer": an entry is formed only once its block is complete.
    Entry i covers tokens [i*m, (i+1)*m); it is complete at position p iff (i+1)*m - 1 <= p.
    """
    return (np.asarray(p, dtype=np.int64) + 1) // m


def compress(ca, za, cb, zb, bias_a, bias_b, m: int, first_entry: int,
             halo_cb=None, halo_zb=None, return_weights: bool = False):
    """CSA compressor: one entry per complete block of m tokens.

    [EXR] section 3 and [ANAT] bullet "Compressed Sparse Attention (CSA)". For entry i (block
    [i*m, (i+1)*m)) and channel j, with the previous block [(i-1)*m, i*m):
        logits  = { za[i*m + r, j] + bias_a[r, j] : r < m }  U  { zb[(i-1)*m + r, j] + bias_b[r, j] : r < m }
        p       = softmax(logits)            (one joint softmax over the 2m logits of channel j)
        E[i, j] = sum_r p_a[r] * ca[i*m + r, j] + sum_r p_b[r] * cb[(i-1)*m + r, j]
    Entry 0 has no previous block: its softmax runs over its own m logits only.

    ca, za, cb, zb: [T, c] rows for the tokens of this call, whose first token is the first token of
    block `first_entry`. halo_cb, halo_zb: [m, c] rows of block first_entry - 1 (needed iff
    first_entry > 0). Only complete blocks produce entries: floor(T / m) of them.
    Returns entries [n, c] (and, if asked, the weights [n, 2m, c]: own block, then previous block).
    """
    ca, za, cb, zb = (np.asarray(a, dtype=np.float64) for a in (ca, za, cb, zb))
    bias_a = np.asarray(bias_a, dtype=np.float64)
    bias_b = np.asarray(bias_b, dtype=np.float64)
    T, c = ca.shape
    n = T // m
    entries = np.zeros((n, c))
    weights = np.zeros((n, 2 * m, c))
    for e in range(n):
        i = first_entry + e
        own = slice(e * m, (e + 1) * m)
        la = za[own] + bias_a                                  # [m, c]
        va = ca[own]
        if e >= 1:
            prev = slice((e - 1) * m, e * m)
            lb, vb = zb[prev] + bias_b, cb[prev]
        elif i >= 1:
            if halo_cb is None or halo_zb is None:
                raise ValueError("entry %d needs the previous block (halo)" % i)
            lb = np.asarray(halo_zb, dtype=np.float64) + bias_b
            vb = np.asarray(halo_cb, dtype=np.float64)
        else:
            lb, vb = None, None
        if lb is None:
            logits, vals = la, va
        else:
            logits, vals = np.concatenate([la, lb], axis=0), np.concatenate([va, vb], axis=0)
        mx = logits.max(axis=0, keepdims=True)
        ex = np.exp(logits - mx)
        p = ex / ex.sum(axis=0, keepdims=True)
        entries[e] = (p * vals).sum(axis=0)
        weights[e, :p.shape[0]] = p
    return (entries, weights) if return_weights else entries


def index_scores(q_idx, keys, w, n_vis):
    """Lightning indexer scores for every query against every entry it can see.

    [EXR] section 3 (cheap ReLU-gated dot products) and [ANAT] bullet "Compressed Sparse Attention":
        s[t, i] = sum_h w[h] * max(0, q_idx[t, h, :] . keys[i, :])        for i < n_vis[t]
    Entries the query cannot see get -inf.
    q_idx [T, H_I, D_I]; keys [N, D_I]; w [H_I] shared by all queries, or [T, H_I] per query.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, N = q_idx.shape[0], keys.shape[0]
    s = np.full((T, N), -np.inf)
    for t in range(T):
        nv = int(min(n_vis[t], N))
        if nv == 0:
            continue
        dots = q_idx[t] @ keys[:nv].T                        # [H_I, nv]
        wt = w if w.ndim == 1 else w[t]
        s[t, :nv] = wt @ np.maximum(dots, 0.0)
    return s


def topk_select(scores_row, n_vis: int, k: int):
    """Top-k of one query's visible entries.

    [ANAT] bullet "Compressed Sparse Attention (CSA)": each query keeps the k most relevant entries.
    Order: larger score first, ties toward the smaller entry index (and -0 equals +0). When fewer
    than k entries are visible all of them are kept. Returned sorted ascending, padded with -1.
    """
    scores_row = np.asarray(scores_row, dtype=np.float64)
    nv = int(n_vis)
    cand = np.arange(nv)
    order = np.lexsort((cand, -scores_row[:nv]))         # primary: -score, secondary: index
    chosen = np.sort(cand[order[:min(k, nv)]])
    out = np.full(k, -1, dtype=np.int64)
    out[:chosen.size] = chosen
    return out


def sparse_attention(q, entries, idx, raw, raw_pos0: int, q_pos, W: int, scale=None, sink=None):
    """Single-KV-head attention over the selected entries plus the raw-token window.

    [ANAT] "The skeleton, and what's kept" (one KV head for all query heads, the entry is both key
    and value), bullet "Compressed Sparse Attention (CSA)" (the selected entries) and bullet "A
    sliding window in every layer" (the last W raw tokens). One softmax runs over the union; the
    optional sink ([ANAT] bullet "An attention sink") adds exp(sink[h]) to the denominator.
        keys_t   = [entries[idx[t, j]] for valid j] ++ [raw row of position u, u in max(0,p-W+1)..p]
        logit    = scale * q[t, h] . key                 (scale = 1/sqrt(D) by default)
        o[t, h]  = sum_key softmax(logit) * key
    raw [R, D] holds positions raw_pos0 .. raw_pos0 + R - 1; the window must lie inside it.
    """
    q = np.asarray(q, dtype=np.float64)
    entries = np.asarray(entries, dtype=np.float64)
    raw = np.asarray(raw, dtype=np.float64)
    T, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((T, H, D))
    for t in range(T):
        p = int(q_pos[t])
        sel = idx[t][idx[t] >= 0]
        lo = max(0, p - W + 1)
        if lo < raw_pos0 or p - raw_pos0 >= raw.shape[0]:
            raise ValueError("window [%d, %d] not inside the raw buffer" % (lo, p))
        keys = np.concatenate([entries[sel], raw[lo - raw_pos0:p - raw_pos0 + 1]], axis=0)
        logits = scale * (q[t] @ keys.T)                    # [H, n_keys]
        mx = logits.max(axis=1)
        if sink is not None:
            mx = np.maximum(mx, np.asarray(sink, dtype=np.float64))
        ex = np.exp(logits - mx[:, None])
        den = ex.sum(axis=1)
        if sink is not None:
            den = den + np.exp(np.asarray(sink, dtype=np.float64) - mx)
        out[t] = (ex @ keys) / den[:, None]
    return out


def hca_compress(c, z, bias, m: int, first_entry: int = 0):
    """HCA compressor: one entry per complete block of m tokens (m = 128), without overlap.

    [ANAT] bullet "Heavily Compressed Attention (HCA)": every 128 tokens become one entry, with no
    overlap between entries. The pages name no other pooling, so the entry pools its own block with
    the CSA compressor's per-channel softmax over learned position biases (one series):
        logits  = { z[i*m + r, j] + bias[r, j] : r < m }
        E[i, j] = sum_r softmax(logits)[r] * c[i*m + r, j]
    c, z: [T, c] rows of this call, whose first token is the first token of block `first_entry`.
    Only complete blocks produce entries: floor(T / m) of them. Returns entries [n, c].
    """
    c = np.asarray(c, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    T, ch = c.shape
    n = T // m
    entries = np.zeros((n, ch))
    for e in range(n):
        own = slice(e * m, (e + 1) * m)
        logits = z[own] + bias                                 # [m, c]
        ex = np.exp(logits - logits.max(axis=0, keepdims=True))
        entries[e] = (ex / ex.sum(axis=0, keepdims=True) * c[own]).sum(axis=0)
    return entries


def dense_attention(q, entries, raw, raw_pos0: int, q_pos, m: int, W: int, scale=None, sink=None):
    """HCA attention: every visible entry plus the raw-token window, one softmax.

    [ANAT] bullet "Heavily Compressed Attention (HCA)": queries attend to all entries densely;
    bullet "A sliding window in every layer"; bullet "An attention sink". It is sparse_attention
    with the selection replaced by every entry visible at p: idx[t] = 0 .. n_vis(p_t) - 1 (capped at
    the entries given).
    """
    entries = np.asarray(entries, dtype=np.float64)
    N = entries.shape[0]
    q_pos = np.asarray(q_pos, dtype=np.int64)
    nv = np.minimum(n_visible(q_pos, m), N)
    width = int(max(nv.max(initial=0), 1))
    idx = np.full((len(q_pos), width), -1, dtype=np.int64)
    for t, n in enumerate(nv):
        idx[t, :n] = np.arange(n)
    return sparse_attention(q, entries, idx, raw, raw_pos0, q_pos, W, scale=scale, sink=sink)


# --------------------------------------------------------------------------------------------------
# QK-norm and partial RoPE ([ANAT] bullet "QK-norm and partial RoPE")
# --------------------------------------------------------------------------------------------------


def rms_norm(x, gamma, eps: float):
    """RMS normalisation of each head vector (the last axis), then the learned per-dim gain:
        y = x / sqrt(mean(x^2) + eps) * gamma
    [ANAT] bullet "QK-norm and partial RoPE": queries and compressed entries are RMS-normalised per
    head. The gain vector and eps are readings (the pages name the norm only)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(gamma, dtype=np.float64)


def rope(x, pos, rope_dims: int, theta: float, inverse: bool = False):
    """Rotary position embedding on the last rope_dims dims of each vector (the last axis).

    [ANAT] bullet "QK-norm and partial RoPE": RoPE rotates only the last 64 of the 512 dims; the
    output is rotated back by the query's own position. Reading: the rotated slice is taken in
    adjacent pairs (2i, 2i+1), pair i turns by the angle pos * theta^(-2i/rope_dims), i.e.
        (a, b) -> (a cos - b sin, a sin + b cos)
    and inverse=True turns by the negative angle. pos broadcasts against x.shape[:-1] from the left
    (pos [T] with x [T, H, D] gives every head of row t the position pos[t])."""
    y = np.array(x, dtype=np.float64, copy=True)
    if rope_dims == 0:
        return y
    D = y.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)
    freq = float(theta) ** (-2.0 * np.arange(rope_dims // 2) / rope_dims)
    ang = pos.reshape(pos.shape + (1,) * (y.ndim - 1 - pos.ndim)) [..., None] * freq
    if inverse:
        ang = -ang
    c, s = np.cos(ang), np.sin(ang)
    a = y[..., D - rope_dims::2].copy()
    b = y[..., D - rope_dims + 1::2].copy()
    y[..., D - rope_dims::2] = a * c - b * s
    y[..., D - rope_dims + 1::2] = a * s + b * c
    return y


def entry_positions(first_entry: int, n: int, m: int):
    """Position at which RoPE turns entry i: the last token of its block, (i+1)*m - 1 (reading: the
    position at which the entry becomes visible; the pages give none)."""
    return (np.arange(first_entry, first_entry + n) + 1) * m - 1


# --------------------------------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------------------------------


def projection_columns(D, D_I, H, H_I):
    """Column ranges of the fused projection x @ W^T.

    The pages do not give the projections; the layer needs, per token, the two pooled series and
    their logits for the entries (dim D) and for the indexer keys (dim D_I), the queries, the indexer
    queries and the raw KV of the window. Column order: [Ca Za Cb Zb | Ca' Za' Cb' Zb' | q | q_I | kv].
    """
    cols, off = {}, 0
    for name, width in (("ca", D), ("za", D), ("cb", D), ("zb", D),
                        ("ica", D_I), ("iza", D_I), ("icb", D_I), ("izb", D_I),
                        ("q", H * D), ("q_idx", H_I * D_I), ("kv", D)):
        cols[name] = (off, off + width)
        off += width
    return cols, off


def _store(a, bf16: bool):
    return round_bf16(a) if bf16 else a


def _val(a, bf16: bool):
    return bf16_bits_to_f64(a) if bf16 else np.asarray(a, dtype=np.float64)


def prefill(inp: dict, wl, b: int = 0, query_rows=None, sink=None, fid=None):
    """The CSA layer over a chunk of T tokens whose context holds L earlier tokens (sequence b).

    Steps in the pages' order: projections, compressor (entries and indexer keys), indexer scores,
    top-k, sparse attention over entries + window. query_rows selects which query rows to finish
    (all by default); every row still feeds the compressor and the window.
    Returns a dict with the projected parts, new entries/keys, scores, idx and out for query_rows.
    With an MXFP4 indexer (wl.idx_dtype == "mxfp4") the key cache holds the MXFP4 form of every key
    (the context's as generated, the chunk's new keys quantised from their stored values) and the
    indexer queries are quantised the same way before the scores; keys_new stays the unquantised
    stored key and keys_new_fp4 holds its (codes, scales); q_idx is what the indexer multiplies and
    q_idx_stored the query before quantisation.
    fid (optional) turns on QK-norm and partial RoPE: a dict with gamma_q, gamma_kv [D], eps,
    rope_dims, theta. Queries, new entries and the chunk's raw KV are then RMS-normalised and
    rotated (queries at their positions, raw KV at its token's position, entries at
    entry_positions) and stored again; the output is rotated back by the query position. Context
    caches (prefix entries and window rows) are taken as stored, i.e. already normalised and
    rotated.
    """
    bf = wl.dtype == "bf16"
    m, D, DI, H, HI = wl.m, wl.D, wl.D_I, wl.H, wl.H_I
    T, L = wl.T, wl.L
    rows = np.arange(T) if query_rows is None else np.asarray(query_rows)
    x = _val(inp["x"][b], bf)                              # [T, d]
    Wt = _val(inp["W"], bf)                                # [n_tot, d]
    cols, _ = projection_columns(D, DI, H, HI)

    def proj(name, r=None):
        lo, hi = cols[name]
        xr = x if r is None else x[r]
        return _store(xr @ Wt[lo:hi].T, bf)

    parts = {n: proj(n) for n in ("ca", "za", "cb", "zb", "ica", "iza", "icb", "izb", "kv")}
    q = proj("q", rows).reshape(len(rows), H, D)
    q_idx = proj("q_idx", rows).reshape(len(rows), HI, DI)
    if fid is not None:
        q = _store(rope(rms_norm(q, fid["gamma_q"], fid["eps"]), L + rows, fid["rope_dims"], fid["theta"]), bf)
        parts["kv"] = _store(rope(rms_norm(parts["kv"], fid["gamma_kv"], fid["eps"]), L + np.arange(T),
                                  fid["rope_dims"], fid["theta"]), bf)

    first = L // m
    halo = _val(inp["halo"][b], bf) if L > 0 else None
    hcb = halo[:, 0:D] if L > 0 else None
    hzb = halo[:, D:2 * D] if L > 0 else None
    hicb = halo[:, 2 * D:2 * D + DI] if L > 0 else None
    hizb = halo[:, 2 * D + DI:2 * D + 2 * DI] if L > 0 else None
    new_e = _store(compress(parts["ca"], parts["za"], parts["cb"], parts["zb"], inp["bias_a"],
                            inp["bias_b"], m, first, hcb, hzb), bf)
    new_k = _store(compress(parts["ica"], parts["iza"], parts["icb"], parts["izb"], inp["ibias_a"],
                            inp["ibias_b"], m, first, hicb, hizb), bf)
    if fid is not None:
        new_e = _store(rope(rms_norm(new_e, fid["gamma_kv"], fid["eps"]), entry_positions(first, len(new_e), m),
                            fid["rope_dims"], fid["theta"]), bf)
    fp4 = wl.idx_dtype == "mxfp4"
    new_k_fp4 = mxfp4_quantize(new_k) if fp4 else None
    keys_new = mxfp4_decode(*new_k_fp4) if fp4 else new_k   # what the key cache holds
    q_idx_stored = q_idx
    if fp4:
        q_idx = mxfp4_round(q_idx)
    if L > 0:
        entries = np.concatenate([_val(inp["entries_prefix"][b], bf), new_e], axis=0)
        kp = (mxfp4_decode(inp["keys_prefix_codes"][b], inp["keys_prefix_scales"][b]) if fp4
              else _val(inp["keys_prefix"][b], bf))
        keys = np.concatenate([kp, keys_new], axis=0)
        raw = np.concatenate([_val(inp["win_prefix"][b], bf), parts["kv"]], axis=0)
        raw_pos0 = L - (wl.W - 1)
    else:
        entries, keys, raw, raw_pos0 = new_e, keys_new, parts["kv"], 0

    q_pos = L + rows
    nv = n_visible(q_pos, m)
    scores = index_scores(q_idx, keys, inp["w_head"], nv)
    idx = np.stack([topk_select(scores[i], nv[i], wl.k) for i in range(len(rows))])
    out = sparse_attention(q, entries, idx, raw, raw_pos0, q_pos, wl.W, sink=sink)
    if fid is not None:
        out = rope(out, q_pos, fid["rope_dims"], fid["theta"], inverse=True)
    return dict(parts=parts, q=q, q_idx=q_idx, q_idx_stored=q_idx_stored, entries_new=new_e, keys_new=new_k,
                keys_new_fp4=new_k_fp4,
                entries=entries, keys=keys, raw=raw, raw_pos0=raw_pos0, rows=rows, q_pos=q_pos,
                n_vis=nv, scores=scores, idx=idx, out=out)


def decode(inp: dict, wl, b: int, sink=None, fid=None, fp8_entries=False):
    """One decode step of sequence b: the new token sits at position L (it opens a new block, so
    no compression runs), the caches hold L/m entries and the raw KV of positions L-W+1..L.
    fid (see prefill): the query is RMS-normalised and rotated at L (then stored), the caches are
    taken as stored, and the output is rotated back by L.
    fp8_entries: the entry cache holds the 584-byte records of the given entries (entry_pack), so
    the attention sees their stored values (entry_unpack)."""
    bf = wl.dtype == "bf16"
    L, m = wl.L, wl.m
    entries = _val(inp["entries"][b], bf)
    if fp8_entries:
        entries = entry_unpack(entry_pack(entries))
    if wl.idx_dtype == "mxfp4":
        keys = mxfp4_decode(inp["keys_codes"][b], inp["keys_scales"][b])
        q_idx = mxfp4_decode(inp["q_idx_codes"][b], inp["q_idx_scales"][b])
    else:
        keys = _val(inp["keys"][b], bf)
        q_idx = _val(inp["q_idx"][b], bf)
    q = _val(inp["q"][b], bf)
    raw = _val(inp["kv_raw"][b], bf)
    q_pos = np.array([L])
    if fid is not None:
        q = _store(rope(rms_norm(q, fid["gamma_q"], fid["eps"]), q_pos, fid["rope_dims"], fid["theta"]), bf)
    nv = n_visible(q_pos, m)
    scores = index_scores(q_idx, keys, inp["w_head"], nv)
    idx = topk_select(scores[0], nv[0], wl.k)[None]
    out = sparse_attention(q, entries, idx, raw, L - (wl.W - 1), q_pos, wl.W, sink=sink)
    if fid is not None:
        out = rope(out, q_pos, fid["rope_dims"], fid["theta"], inverse=True)
    return dict(scores=scores, idx=idx, out=out, n_vis=nv, keys=keys, entries=entries, q=q,
                q_idx=q_idx, raw=raw)
