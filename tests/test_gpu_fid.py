"""GPU parity of QK-norm and partial RoPE ("Anatomy of a Frontier Model", bullet "QK-norm and partial
RoPE"): csa_norm_rope against the oracle's rms_norm / rope, and the layer with the norm and the
rotation on (csa_forward, decode) against the oracle's prefill / decode with the same options."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_05_amd import lib
from synth.torch_io import act, to_device
from synth.workloads import get
from tests.csa_testlib import (O, G, TOL, check_idx_rows, decode_tensors, max_err, run_decode, run_prefill,
                               tensor_f64, weights_to_device)

pytestmark = pytest.mark.gpu


def _fid(D, seed, rope_dims):
    """gains from the seeded generator (the same float32 bits for both sides)"""
    gq = (1.0 + 0.2 * G.normal_f32(seed, "gamma_q", (D,))).astype(np.float32)
    gk = (1.0 + 0.2 * G.normal_f32(seed, "gamma_kv", (D,))).astype(np.float32)
    host = {"gamma_q": gq.astype(np.float64), "gamma_kv": gk.astype(np.float64), "eps": float(np.float32(1e-6)),
            "rope_dims": rope_dims, "theta": 10000.0}
    dev = {"gamma_q": to_device(gq, "f32"), "gamma_kv": to_device(gk, "f32"), "norm_eps": 1e-6,
           "rope_dims": rope_dims, "rope_theta": 10000.0}
    return host, dev


@pytest.mark.parametrize("dtype,D,rope_dims,pos0,step", [("bf16", 512, 64, 1_048_000, 1), ("f32", 512, 64, 131_000, 4),
                                                         ("f32", 32, 16, 5, 1), ("bf16", 192, 0, 0, 1),
                                                         ("f32", 96, 96, 777_777, 3), ("f32", 256, 64, 999_999, 1),
                                                         ("bf16", 1024, 192, 65_537, 2)])
def test_norm_rope_matches_oracle(dtype, D, rope_dims, pos0, step):
    B, R, H = 2, 7, 3
    x64 = G.normal_f32(90, "nr_x", (B, R, H, D)).astype(np.float64) * 3.0
    if dtype == "bf16":
        bits = G.f32_to_bf16_bits(x64.astype(np.float32))
        x, x64 = to_device(bits, "bf16"), O.bf16_bits_to_f64(bits)
    else:
        x = to_device(x64.astype(np.float32), "f32")
        x64 = x64.astype(np.float32).astype(np.float64)
    host, dev = _fid(D, 91, rope_dims)
    pos = pos0 + step * np.arange(R)
    want = O.rope(O.rms_norm(x64, host["gamma_q"], host["eps"]), np.broadcast_to(pos, (B, R)), rope_dims, 10000.0)
    y = torch.empty_like(x)
    lib.csa_norm_rope(x, y=y, pos0=pos0, pos_step=step, gamma=dev["gamma_q"], eps=1e-6, rope_dims=rope_dims)
    got = tensor_f64(y)
    rel = 2.0 ** -8 if dtype == "bf16" else 2e-6
    assert np.all(np.abs(got - want) <= rel * np.abs(want) + 1e-6), max_err(got, want)
    # in place, then rotated back (no norm): the normalised vectors again
    lib.csa_norm_rope(x, pos0=pos0, pos_step=step, gamma=dev["gamma_q"], eps=1e-6, rope_dims=rope_dims)
    assert torch.equal(x, y)
    lib.csa_norm_rope(y, pos0=pos0, pos_step=step, rope_dims=rope_dims, inverse=True)
    back = O.rms_norm(x64, host["gamma_q"], host["eps"])
    # a rotated pair carries the rounding of both members: bound by the pair's magnitude
    mag = np.abs(back)
    if rope_dims:
        rs = D - rope_dims
        hyp = np.hypot(back[..., rs::2], back[..., rs + 1::2])
        mag[..., rs::2] = hyp
        mag[..., rs + 1::2] = hyp
    assert np.all(np.abs(tensor_f64(y) - back) <= 2 * rel * mag + 1e-5)


def test_norm_rope_argument_errors():
    x = torch.zeros(1, 2, 3, 8, device="cuda")
    with pytest.raises(lib.CsaError):
        lib.csa_norm_rope(x, pos0=0, rope_dims=3)             # odd
    with pytest.raises(lib.CsaError):
        lib.csa_norm_rope(x, pos0=0, rope_dims=10)            # > D
    with pytest.raises(lib.CsaError):
        lib.csa_norm_rope(x, pos0=0, gamma=torch.ones(8, device="cuda"), inverse=True)


def _check_fid_prefill(wl, host, dev, tol, max_differ):
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl, fid=host)
    w = weights_to_device(wl, inp)
    w.update(dev)
    st = run_prefill(wl, inp, weights=w)
    first = wl.L // wl.m
    n_new = wl.T // wl.m
    assert max_err(tensor_f64(st.entries[0, first:first + n_new]), r["entries_new"]) <= tol
    assert max_err(tensor_f64(st.win[0, wl.W - 1:wl.W - 1 + wl.T]), r["parts"]["kv"]) <= tol
    gidx = st.idx[0].cpu().numpy()
    differ = check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
    assert len(differ) <= max_differ
    ref = r["out"].copy()
    for t in differ:
        o = O.sparse_attention(r["q"][t:t + 1], r["entries"], gidx[t:t + 1], r["raw"], r["raw_pos0"],
                               r["q_pos"][t:t + 1], wl.W)
        ref[t] = O.rope(o, r["q_pos"][t:t + 1], host["rope_dims"], host["theta"], inverse=True)[0]
    assert max_err(tensor_f64(st.out[0]), ref) <= tol


def test_fid_forward_tiny_fp32():
    wl = get("tiny")
    host, dev = _fid(wl.D, 92, 16)
    _check_fid_prefill(wl, host, dev, TOL["f32"], 0)


def test_fid_forward_bf16_chunk_with_context():
    # a chunk after L tokens of context: positions of queries, window rows and new entries are absolute
    wl = get("chunk1m").with_(L=2048, T=264, d=512)
    host, dev = _fid(wl.D, 93, 64)
    _check_fid_prefill(wl, host, dev, TOL["bf16"], wl.T // 20)


def test_fid_decode_bf16():
    wl = get("decode128k").with_(B=3, L=4 * 3000)
    host, dev = _fid(wl.D, 94, 64)
    inp = G.make_inputs(wl)
    t = decode_tensors(wl, inp)
    from compressed_sparse_attention_05_amd import layer
    from tests.csa_testlib import dims_of
    st = layer.CSADecode(dims_of(wl), wl.B, wl.L // wl.m, idx_dtype=lib.CSA_BF16,
                         fid={"gamma_q": dev["gamma_q"], "eps": 1e-6, "rope_dims": 64, "theta": 10000.0})
    st(wl.L, t["q_idx"], t["w_head"], t["keys"], t["q"], t["entries"], t["kv_raw"])
    torch.cuda.synchronize()
    for b in range(wl.B):
        r = O.decode(inp, wl, b, fid=host)
        gidx = st.idx[b].cpu().numpy()
        differ = check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
        ref = r["out"]
        if differ:
            o = O.sparse_attention(r["q"], r["entries"], gidx, r["raw"], wl.L - (wl.W - 1), np.array([wl.L]), wl.W)
            ref = O.rope(o, np.array([wl.L]), 64, 10000.0, inverse=True)
        assert max_err(tensor_f64(st.out[b]), ref) <= TOL["bf16"]


@pytest.mark.parametrize("case", ["fused_sink", "gamma_unaligned", "rope_only", "f32"])
def test_sparse_attn_qk_matches_oracle(case):
    """csa_sparse_attn_qk over the oracle's selection: the query normalised and rotated inside the attention
    (bf16, 128 heads) or by a pass of its own (a gain that is not 16-byte aligned, float32 queries), with no
    norm (rotation only), and with a sink."""
    wl = get("decode128k").with_(B=2, L=4 * 2500, **({"dtype": "f32"} if case == "f32" else {}))
    bf = wl.dtype == "bf16"
    host, dev = _fid(wl.D, 95, 64)
    inp = G.make_inputs(wl)
    t = decode_tensors(wl, inp)
    sink_h = G.normal_f32(96, "qk_sink", (wl.H,)) if case == "fused_sink" else None
    fid = {"gamma_q": dev["gamma_q"], "eps": 1e-6, "rope_dims": 64, "theta": 10000.0}
    if case == "gamma_unaligned":
        buf = torch.empty(wl.D + 1, dtype=torch.float32, device="cuda")
        buf[1:] = dev["gamma_q"]
        fid["gamma_q"] = buf[1:]
    elif case == "rope_only":
        fid["gamma_q"] = None
    refs = [O.decode(inp, wl, b, sink=None if sink_h is None else sink_h.astype(np.float64), fid=host)
            for b in range(wl.B)]
    idx = to_device(np.stack([r["idx"] for r in refs]).astype(np.int32), "i32").view(wl.B, 1, wl.k)
    out = torch.empty(wl.B, 1, wl.H, wl.D, dtype=torch.float32, device="cuda")
    from tests.csa_testlib import dims_of
    lib.csa_sparse_attn_qk(dims_of(wl), fid, t["q"], t["entries"], idx, t["kv_raw"], out, q_pos0=wl.L,
                           raw_pos0=wl.L - (wl.W - 1),
                           sink=None if sink_h is None else to_device(sink_h.astype(np.float32), "f32"))
    torch.cuda.synchronize()
    for b, r in enumerate(refs):
        ref = r["out"]
        if case == "rope_only":
            qpos = np.array([wl.L])
            q = O.rope(O._val(inp["q"][b], bf), qpos, 64, 10000.0)
            q = O.round_bf16(q) if bf else q
            o = O.sparse_attention(q, r["entries"], r["idx"], r["raw"], wl.L - (wl.W - 1), qpos, wl.W)
            ref = O.rope(o, qpos, 64, 10000.0, inverse=True)
        assert max_err(tensor_f64(out[b]), ref) <= TOL[wl.dtype], (case, b)


@pytest.mark.parametrize("dtype,T", [("bf16", 40), ("bf16", 7), ("f32", 12)])
def test_sparse_attn_qk_chunk_rows(dtype, T):
    """csa_sparse_attn_qk over a chunk of T query rows (8 or more: the prefill plan, the norm and rotation
    inside the 128-head kernel for bf16; fewer: the split plan, turned back in the merge; float32: the
    separate passes), two sequences at different positions, on seeded selections."""
    B, H, D, k, W, m = 2, 128, 512, 64, 128, 4
    n_cap = 600
    rng = np.random.default_rng(T)
    host, dev = _fid(D, 97, 64)
    pos0 = np.array([2000, 1555])
    bf = dtype == "bf16"

    def make(name, shape, scale=1.0):
        x = G.normal_f32(98, name, shape) * np.float32(scale)
        if bf:
            bits = G.f32_to_bf16_bits(x)
            return to_device(bits, "bf16"), O.bf16_bits_to_f64(bits)
        return to_device(x, "f32"), x.astype(np.float64)
    q_d, q_h = make(f"qk_q{T}", (B, T, H, D))
    ent_d, ent_h = make(f"qk_e{T}", (B, n_cap, D))
    R = T + W - 1
    raw_d, raw_h = make(f"qk_r{T}", (B, R, D))
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            nv = min(n_cap, (int(pos0[b]) + t + 1) // m)
            sel = np.sort(rng.choice(nv, size=min(k - 3 * (t % 3), nv), replace=False))
            idx[b, t, :sel.size] = sel
    out = torch.empty(B, T, H, D, dtype=torch.float32, device="cuda")
    d = lib.make_dims(m, D, H, 64, 128, k, W)
    fid = {"gamma_q": dev["gamma_q"], "eps": 1e-6, "rope_dims": 64, "theta": 10000.0}
    lib.csa_sparse_attn_qk(d, fid, q_d, ent_d, to_device(idx, "i32"), raw_d, out,
                           q_pos0=torch.tensor(pos0, dtype=torch.int64, device="cuda"),
                           raw_pos0=torch.tensor(pos0 - (W - 1), dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    got = tensor_f64(out)
    for b in range(B):
        qp = pos0[b] + np.arange(T)
        qn = O.rope(O.rms_norm(q_h[b], host["gamma_q"], host["eps"]), qp, 64, 10000.0)
        qn = O.round_bf16(qn) if bf else qn
        o = O.sparse_attention(qn, ent_h[b], idx[b], raw_h[b], int(pos0[b]) - (W - 1), qp, W)
        ref = O.rope(o, qp, 64, 10000.0, inverse=True)
        assert max_err(got[b], ref) <= TOL[dtype], (dtype, T, b)
