"""GPU parity of the HCA steps ("Anatomy of a Frontier Model", bullet "Heavily Compressed Attention
(HCA)"): the compressor over 128-token blocks without overlap, and dense attention over every
visible entry plus the window, against the oracle on seeded inputs."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_05_amd import lib
from synth import gen as G
from synth.torch_io import to_device
from tests.csa_testlib import O, TOL, max_err, tensor_f64

pytestmark = pytest.mark.gpu

M, D, H, W = 128, 512, 128, 128


def _bf16(seed, name, shape, std=1.0):
    """(device bf16 tensor, its exact float64 values)"""
    bits = G.f32_to_bf16_bits(G.normal_f32(seed, name, shape, std))
    return to_device(bits, "bf16"), O.bf16_bits_to_f64(bits)


def _dims(m=M, h=H, d=D, w=W):
    return lib.make_dims(m, d, h, 64, 128, 0, w)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hca_compress(dtype):
    B, c, first = 2, D, 5
    T = 3 * M + 77                                   # the trailing 77 tokens make no entry
    n_cap = first + 4
    if dtype == "bf16":
        cv, c64 = _bf16(50, "hca_c", (B, T, c))
        z, z64 = _bf16(50, "hca_z", (B, T, c), std=2.0)
        out = torch.zeros(B, n_cap, c, dtype=torch.bfloat16, device="cuda")
    else:
        c64 = G.normal_f32(50, "hca_c", (B, T, c)).astype(np.float64)
        z64 = G.normal_f32(50, "hca_z", (B, T, c), std=2.0).astype(np.float64)
        cv, z = to_device(c64, "f32"), to_device(z64, "f32")
        out = torch.zeros(B, n_cap, c, device="cuda")
    bias = G.normal_f32(50, "hca_bias", (M, c), std=0.5)
    lib.csa_hca_compress(cv, z, to_device(bias, "f32"), out, pos0=first * M, m=M)
    got = tensor_f64(out)
    for b in range(B):
        want = O.hca_compress(c64[b], z64[b], bias.astype(np.float64), M)
        assert max_err(got[b, first:first + 3], want) <= TOL[dtype]
        assert np.all(got[b, :first] == 0) and np.all(got[b, first + 3:] == 0)   # nothing else written


def _dense_case(seed, B, T, q_pos0, n_cap, sink=False, h=H):
    q, q64 = _bf16(seed, "q", (B, T, h, D))
    ent, e64 = _bf16(seed, "ent", (B, n_cap, D))
    raw_pos0 = max(0, q_pos0 - W + 1)
    R = q_pos0 + T - raw_pos0
    raw, r64 = _bf16(seed, "raw", (B, R, D))
    sk = np.linspace(-1.0, 2.0, h) if sink else None
    out = torch.empty(B, T, h, D, dtype=torch.bfloat16, device="cuda")
    lib.csa_dense_attn(_dims(h=h), q, ent, raw, out, q_pos0=q_pos0, raw_pos0=raw_pos0,
                       sink=None if sk is None else to_device(sk.astype(np.float32), "f32"))
    return out, q64, e64, r64, raw_pos0, sk


@pytest.mark.parametrize("q_pos0,T,n_cap", [(128 * 40 - 100, 200, 64), (128 * 300 + 7, 96, 320)])
def test_dense_attn_prefill_bf16(q_pos0, T, n_cap):
    # 128 heads, T >= 8 rows: one workgroup per row over all its keys
    out, q64, e64, r64, raw_pos0, _ = _dense_case(60, 1, T, q_pos0, n_cap)
    got = tensor_f64(out[0])
    want = O.dense_attention(q64[0], e64[0], r64[0], raw_pos0, q_pos0 + np.arange(T), M, W)
    assert max_err(got, want) <= TOL["bf16"]


@pytest.mark.parametrize("B,q_pos0,n_cap,rows", [(3, 128 * 3000 + 50, 3100, None), (64, 128 * 3100, 3200, 8)])
def test_dense_attn_decode_splits_bf16(B, q_pos0, n_cap, rows):
    # one query row per sequence: the key list is cut into fixed splits and merged, sink in the merge
    out, q64, e64, r64, raw_pos0, sk = _dense_case(61, B, 1, q_pos0, n_cap, sink=True)
    got = tensor_f64(out)
    for b in (range(B) if rows is None else np.linspace(0, B - 1, rows).astype(int)):
        want = O.dense_attention(q64[b], e64[b], r64[b], raw_pos0, [q_pos0], M, W, sink=sk)
        assert max_err(got[b], want) <= TOL["bf16"]


def test_dense_attn_decode_batch_invariance():
    B, q_pos0, n_cap = 5, 128 * 2000 + 3, 2100
    out, *_ = _dense_case(62, B, 1, q_pos0, n_cap)
    q, _ = _bf16(62, "q", (B, 1, H, D))
    ent, _ = _bf16(62, "ent", (B, n_cap, D))
    raw, _ = _bf16(62, "raw", (B, W, D))
    one = torch.empty(1, 1, H, D, dtype=torch.bfloat16, device="cuda")
    lib.csa_dense_attn(_dims(), q[3:4].contiguous(), ent[3:4].contiguous(), raw[3:4].contiguous(), one,
                       q_pos0=q_pos0, raw_pos0=q_pos0 - W + 1)
    assert torch.equal(one[0], out[3])


def test_dense_attn_fp32_small():
    # fp32 operands take the generic kernel
    rng = np.random.default_rng(63)
    m, h, d, w, T, q_pos0, n_cap = 4, 3, 32, 6, 40, 17, 20
    q64 = rng.standard_normal((1, T, h, d))
    e64 = rng.standard_normal((1, n_cap, d))
    r64 = rng.standard_normal((1, q_pos0 + T, d))
    out = torch.empty(1, T, h, d, device="cuda")
    f = lambda a: to_device(a.astype(np.float32), "f32")
    lib.csa_dense_attn(_dims(m=m, h=h, d=d, w=w), f(q64), f(e64), f(r64), out, q_pos0=q_pos0, raw_pos0=0)
    want = O.dense_attention(q64[0].astype(np.float32), e64[0].astype(np.float32), r64[0].astype(np.float32), 0,
                             q_pos0 + np.arange(T), m, w)
    assert max_err(tensor_f64(out[0]), want) <= TOL["f32"]


@pytest.mark.parametrize("h", [H, 64])
@pytest.mark.parametrize("B,T,q_pos0,n_cap", [(2, 1, 128 * 2000 + 5, 2100), (1, 40, 128 * 300 + 11, 320)])
def test_dense_attn_over_records(B, T, q_pos0, n_cap, h):
    # HCA entries in the 584-byte record format: decode splits (T = 1) and whole rows; 128 heads in
    # the 8-wave pairs kernel, 64 in the 4-wave one
    q, q64 = _bf16(64, "q", (B, T, h, D))
    ent, e64 = _bf16(64, "ent", (B, n_cap, D))
    raw_pos0 = max(0, q_pos0 - W + 1)
    raw, r64 = _bf16(64, "raw", (B, q_pos0 + T - raw_pos0, D))
    rec = lib.csa_entry_pack(ent)
    out = torch.empty(B, T, h, D, dtype=torch.float32, device="cuda")
    lib.csa_dense_attn(_dims(h=h), q, rec, raw, out, q_pos0=q_pos0, raw_pos0=raw_pos0)
    stored = O.entry_unpack(O.entry_pack(e64))
    got = tensor_f64(out)
    for b in range(B):
        want = O.dense_attention(q64[b], stored[b], r64[b], raw_pos0, q_pos0 + np.arange(T), M, W)
        assert max_err(got[b], want) <= TOL["bf16"]


@pytest.mark.parametrize("variant", ["plain", "fid_records"])
def test_hca_decode_steps(variant):
    # token-by-token HCA decode over a state: every step equals the oracle's row, and the entry the
    # step at a block's last token pools equals the oracle's
    B, L0, T = 2, 2 * M, 3 * M + 40                 # steps at 256 .. 423, the block ending at 383 completes
    fid = variant != "plain"
    records = fid
    cv, c64 = _bf16(70, "hd_c", (B, T, D))
    z, z64 = _bf16(70, "hd_z", (B, T, D), std=2.0)
    kvd, kv64 = _bf16(70, "hd_kv", (B, T, D))
    qd, q64 = _bf16(70, "hd_q", (B, T, H, D))
    bias = G.normal_f32(70, "hd_bias", (M, D), std=0.5)
    gq = (1.0 + 0.2 * G.normal_f32(70, "hd_gq", (D,))).astype(np.float32)
    gk = (1.0 + 0.2 * G.normal_f32(70, "hd_gk", (D,))).astype(np.float32)
    n_cap = T // M + 1
    # oracle side: entries, window rows and queries as the layer stores them
    ent = [O.round_bf16(O.hca_compress(c64[b], z64[b], bias.astype(np.float64), M)) for b in range(B)]
    raw = [kv64[b] for b in range(B)]
    qs = [q64[b] for b in range(B)]
    if fid:
        g_q, g_k = gq.astype(np.float64), gk.astype(np.float64)
        ent = [O.round_bf16(O.rope(O.rms_norm(e, g_k, float(np.float32(1e-6))), O.entry_positions(0, len(e), M), 64,
                                   10000.0)) for e in ent]
        raw = [O.round_bf16(O.rope(O.rms_norm(r, g_k, float(np.float32(1e-6))), np.arange(T), 64, 10000.0)) for r in raw]
        qs = [O.round_bf16(O.rope(O.rms_norm(q, g_q, float(np.float32(1e-6))), np.arange(T), 64, 10000.0)) for q in qs]
    seen = [O.entry_unpack(O.entry_pack(e)) if records else e for e in ent]
    # GPU state: entries of the two complete blocks, window rows of positions L0-W+1 .. L0-1
    dims = _dims()
    bits = lambda a: to_device(G.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)), "bf16")
    ent_dev = torch.zeros(B, n_cap, D, dtype=torch.bfloat16, device="cuda")
    ent_dev[:, :2] = bits(np.stack([e[:2] for e in ent]))
    if records:
        ent_state = torch.zeros(B, n_cap, lib.ENTRY_RECORD_BYTES, dtype=torch.uint8, device="cuda")
        lib.csa_entry_pack(ent_dev[:, :2].contiguous(), ent_state[:, :2])
    else:
        ent_state = ent_dev
    win = torch.zeros(B, W, D, dtype=torch.bfloat16, device="cuda")
    for p in range(L0 - W + 1, L0):
        win[:, p % W] = bits(np.stack([r[p] for r in raw]))
    block = torch.zeros(B, M, 2 * D, dtype=torch.bfloat16, device="cuda")
    state = {"entries": ent_state, "win": win, "block": block}
    weights = {"bias_a": to_device(bias, "f32")}
    if fid:
        weights.update({"gamma_q": to_device(gq, "f32"), "gamma_kv": to_device(gk, "f32"), "norm_eps": 1e-6,
                        "rope_dims": 64, "rope_theta": 10000.0})
    out = torch.empty(B, H, D, dtype=torch.float32, device="cuda")
    worst = 0.0
    for p in range(L0, T):
        comp = torch.cat([cv[:, p], z[:, p]], dim=1).contiguous()
        lib.csa_hca_decode_step(dims, weights, p, qd[:, p].contiguous(), kvd[:, p].contiguous(), comp, state, out)
        if p % 16 == 0 or p in (L0, 3 * M - 1, 3 * M, T - 1):
            torch.cuda.synchronize()
            got = tensor_f64(out)
            for b in range(B):
                o = O.dense_attention(qs[b][p:p + 1], seen[b], raw[b], 0, np.array([p]), M, W)
                if fid:
                    o = O.rope(o, np.array([p]), 64, 10000.0, inverse=True)
                worst = max(worst, max_err(got[b], o[0]))
    assert worst <= TOL["bf16"], worst
    # the entry of the block that completed at 383
    torch.cuda.synchronize()
    if records:
        np.testing.assert_allclose(O.entry_unpack(ent_state[:, 2].cpu().numpy()), np.stack([s[2] for s in seen]),
                                   rtol=2 ** -3, atol=1e-2)
    else:
        assert max_err(tensor_f64(ent_state[:, 2]), np.stack([e[2] for e in ent])) <= TOL["bf16"]
