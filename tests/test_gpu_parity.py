"""GPU parity: every step of the HIP path against the CPU oracle on the same seeded inputs.

Small cases are compared element by element; the named full-size workloads are run in the launch
configuration the benchmark times and compared on sampled rows / sequences.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_05_amd import lib
from synth.torch_io import act, to_device
from synth.workloads import get
from tests.csa_testlib import (O, G, TOL, check_idx_rows, decode_tensors, dims_of, max_err, run_decode, run_prefill,
                               tensor_f64)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------------ selection


def _oracle_topk_rows(s32, nv, k):
    return np.stack([O.topk_select(s32[r].astype(np.float64), nv[r], k) for r in range(s32.shape[0])])


@pytest.mark.parametrize("R,n,k,tie", [(7, 100, 16, False), (5, 3000, 512, True), (3, 5000, 1024, False),
                                       (2, 40000, 1024, True), (4, 70000, 100, False), (6, 64, 64, True),
                                       # one workgroup per row (rows of 16K..32K scores), odd and full lengths
                                       (3, 20001, 1024, True), (7, 32768, 512, False), (5, 24000, 2048, True),
                                       # rows past 32K scores (the three-launch path) with many rows
                                       (40, 32769, 1024, True), (33, 49152, 512, False), (32, 40001, 2048, True),
                                       (31, 40000, 1024, False), (32, 49153, 1024, False),
                                       # rows past 4 x 32K scores: group maxima, candidates, final selection
                                       (3, 200000, 1024, True), (5, 140000, 512, False)])
def test_topk_from_scores_bit_exact(R, n, k, tie):
    rng = np.random.default_rng(R * 1000 + n)
    s = rng.standard_normal((R, n)).astype(np.float32)
    if tie:
        s = (np.round(s * 4) / 4).astype(np.float32)
        s[:, ::3] = 0.0
        s[:, 1::7] = -0.0
    nv = np.resize(np.array([n, n // 2, 0, 1, min(n, k - 1), n - 1, 5], dtype=np.int32), R)
    idx = torch.empty(R, k, dtype=torch.int32, device="cuda")
    sc = torch.empty(R, k, dtype=torch.float32, device="cuda")
    lib.csa_topk_from_scores(to_device(s, "f32"), to_device(nv, "i32"), k, idx, out_score=sc)
    got = idx.cpu().numpy()
    want = _oracle_topk_rows(s, nv, k)
    np.testing.assert_array_equal(got, want)
    gs = sc.cpu().numpy()
    for r in range(R):
        v = want[r] >= 0
        np.testing.assert_array_equal(gs[r][v], s[r][want[r][v]])


def test_topk_from_scores_negative_infinity_scores():
    # valid entries scored -inf rank below every finite score and among themselves by index; rows split
    # into pieces (few rows) must not let a short piece's padding outrank them
    R, n, k = 4, 12288, 1024
    rng = np.random.default_rng(77)
    s = rng.standard_normal((R, n)).astype(np.float32)
    s[:, 300:] = -np.inf                       # 300 finite scores, then -inf
    s[1, :] = -np.inf                          # every score -inf
    s[2, 5000:5100] = 1.0                      # finite scores in a later piece
    nv = np.array([n, n, n - 7, 2500], dtype=np.int32)
    idx = torch.empty(R, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_from_scores(to_device(s, "f32"), to_device(nv, "i32"), k, idx)
    np.testing.assert_array_equal(idx.cpu().numpy(), _oracle_topk_rows(s, nv, k))


@pytest.mark.parametrize("n", [20000, 32768, 50000])
def test_topk_from_scores_constant_rows(n):
    # every score equal: the top-k is the first k entries (ties go to the smaller index)
    R, k = 3, 1024
    s = np.full((R, n), 0.75, dtype=np.float32)
    s[1] = -2.0
    s[2, : n // 2] = 0.0
    s[2, n // 2:] = -0.0
    nv = np.array([n, n - 3, n], dtype=np.int32)
    idx = torch.empty(R, k, dtype=torch.int32, device="cuda")
    lib.csa_topk_from_scores(to_device(s, "f32"), to_device(nv, "i32"), k, idx)
    np.testing.assert_array_equal(idx.cpu().numpy(), _oracle_topk_rows(s, nv, k))
    np.testing.assert_array_equal(idx.cpu().numpy(), np.tile(np.arange(k, dtype=np.int32), (R, 1)))


# ------------------------------------------------------------------------------------ tiny fp32


def test_tiny_forward_fp32_end_to_end():
    wl = get("tiny")
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    st = run_prefill(wl, inp)
    np.testing.assert_allclose(tensor_f64(st.entries[0]), r["entries"], atol=TOL["f32"], rtol=0)
    np.testing.assert_allclose(tensor_f64(st.keys[0]), r["keys"], atol=TOL["f32"], rtol=0)
    gidx = st.idx[0].cpu().numpy()
    differ = check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
    ref = r["out"].copy()
    for t in differ:
        ref[t] = O.sparse_attention(r["q"][t:t + 1], r["entries"], gidx[t:t + 1], r["raw"], r["raw_pos0"],
                                    r["q_pos"][t:t + 1], wl.W)[0]
    assert max_err(tensor_f64(st.out[0]), ref) <= TOL["f32"]


def test_tiny_steps_fp32_on_oracle_inputs():
    wl = get("tiny")
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    d = dims_of(wl)
    p = r["parts"]
    f = lambda a: to_device(a.astype(np.float32), "f32")
    # step 1
    ent = torch.zeros(1, wl.n_cap, wl.D, device="cuda")
    lib.csa_compress(f(p["ca"])[None], f(p["za"])[None], f(p["cb"])[None], f(p["zb"])[None],
                     f(inp["bias_a"]), f(inp["bias_b"]), ent, pos0=0, m=wl.m)
    assert max_err(tensor_f64(ent[0]), r["entries"]) <= TOL["f32"]
    # steps 2+3
    idx = torch.empty(1, wl.T, wl.k, dtype=torch.int32, device="cuda")
    lib.csa_index_topk(d, f(r["q_idx"])[None], f(inp["w_head"]), f(r["keys"])[None], idx, q_pos0=0)
    check_idx_rows(idx[0].cpu().numpy(), r["idx"], r["scores"], r["n_vis"])
    # step 4 with the oracle's selection
    out = torch.empty(1, wl.T, wl.H, wl.D, device="cuda")
    lib.csa_sparse_attn(d, f(r["q"])[None], f(r["entries"])[None], to_device(r["idx"], "i32")[None],
                        f(r["raw"])[None], out, q_pos0=0, raw_pos0=0)
    assert max_err(tensor_f64(out[0]), r["out"]) <= TOL["f32"]


def test_attention_sink_fp32():
    wl = get("tiny")
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    sink = np.linspace(-1.0, 2.0, wl.H)
    want = O.sparse_attention(r["q"], r["entries"], r["idx"], r["raw"], 0, r["q_pos"], wl.W, sink=sink)
    f = lambda a: to_device(np.asarray(a, dtype=np.float32), "f32")
    out = torch.empty(1, wl.T, wl.H, wl.D, device="cuda")
    lib.csa_sparse_attn(dims_of(wl), f(r["q"])[None], f(r["entries"])[None], to_device(r["idx"], "i32")[None],
                        f(r["raw"])[None], out, q_pos0=0, raw_pos0=0, sink=f(sink))
    assert max_err(tensor_f64(out[0]), want) <= TOL["f32"]


# ------------------------------------------------------------------------------------ bf16 prefill


def _bf16_small(**kw):
    base = dict(T=1000, d=1024)   # ragged T: not a multiple of 8 (rows per workgroup) or 64 (key tile)
    base.update(kw)
    return get("prefill8k").with_(**base)


def _assert_bf16_close(got, want, frac_exact=0.99):
    assert max_err(got, want) <= TOL["bf16"]
    assert np.mean(got == want) >= frac_exact


def test_bf16_prefill_end_to_end_small():
    wl = _bf16_small()
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    st = run_prefill(wl, inp)
    _assert_bf16_close(tensor_f64(st.entries[0]), r["entries"])
    _assert_bf16_close(tensor_f64(st.keys[0]), r["keys"])
    gidx = st.idx[0].cpu().numpy()
    differ = check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
    assert len(differ) <= wl.T // 20
    ref = r["out"].copy()
    for t in differ:
        ref[t] = O.sparse_attention(r["q"][t:t + 1], r["entries"], gidx[t:t + 1], r["raw"], 0, r["q_pos"][t:t + 1],
                                    wl.W)[0]
    assert max_err(tensor_f64(st.out[0]), ref) <= TOL["bf16"]


def test_bf16_steps_on_oracle_inputs():
    wl = _bf16_small(T=520)
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    d = dims_of(wl)
    bits = lambda a: to_device(G.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)), "bf16")  # exact: on bf16 grid
    p = r["parts"]
    ent = torch.zeros(1, wl.n_cap, wl.D, dtype=torch.bfloat16, device="cuda")
    lib.csa_compress(bits(p["ca"])[None], bits(p["za"])[None], bits(p["cb"])[None], bits(p["zb"])[None],
                     to_device(inp["bias_a"], "f32"), to_device(inp["bias_b"], "f32"), ent, pos0=0, m=wl.m)
    _assert_bf16_close(tensor_f64(ent[0]), r["entries"])
    idx = torch.empty(1, wl.T, wl.k, dtype=torch.int32, device="cuda")
    lib.csa_index_topk(d, bits(r["q_idx"])[None], to_device(inp["w_head"], "f32"), bits(r["keys"])[None], idx,
                       q_pos0=0)
    check_idx_rows(idx[0].cpu().numpy(), r["idx"], r["scores"], r["n_vis"])
    out = torch.empty(1, wl.T, wl.H, wl.D, device="cuda")
    lib.csa_sparse_attn(d, bits(r["q"])[None], bits(r["entries"])[None], to_device(r["idx"], "i32")[None],
                        bits(r["raw"])[None], out, q_pos0=0, raw_pos0=0)
    assert max_err(tensor_f64(out[0]), r["out"]) <= TOL["bf16"]


def test_bf16_selection_bit_exact_on_oracle_scores():
    wl = _bf16_small(T=300, d=512)
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    s32 = np.where(np.isfinite(r["scores"]), r["scores"], 0).astype(np.float32)
    nv = r["n_vis"].astype(np.int32)
    idx = torch.empty(wl.T, wl.k, dtype=torch.int32, device="cuda")
    lib.csa_topk_from_scores(to_device(s32, "f32"), to_device(nv, "i32"), wl.k, idx)
    np.testing.assert_array_equal(idx.cpu().numpy(), _oracle_topk_rows(s32, nv, wl.k))


def test_bf16_chunked_prefill_with_context():
    # a chunk after L tokens of context: prefix entries/keys, window rows and halo come from the cache
    wl = get("chunk1m").with_(L=2048, T=264, d=512)
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    st = run_prefill(wl, inp)
    _assert_bf16_close(tensor_f64(st.entries[0]), r["entries"])
    gidx = st.idx[0].cpu().numpy()
    differ = check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
    ref = r["out"].copy()
    for t in differ:
        ref[t] = O.sparse_attention(r["q"][t:t + 1], r["entries"], gidx[t:t + 1], r["raw"], r["raw_pos0"],
                                    r["q_pos"][t:t + 1], wl.W)[0]
    assert max_err(tensor_f64(st.out[0]), ref) <= TOL["bf16"]


def test_bf16_short_sequence_window_only():
    # T < k and the first m-1 rows see no entry at all: padding and the window-only path
    wl = _bf16_small(T=40, d=512)
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    st = run_prefill(wl, inp)
    gidx = st.idx[0].cpu().numpy()
    assert np.all(gidx[:3] == -1)
    check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
    assert max_err(tensor_f64(st.out[0]), r["out"]) <= TOL["bf16"]


def test_bf16_forward_is_deterministic():
    wl = _bf16_small(T=256, d=512)
    inp = G.make_inputs(wl)
    a = run_prefill(wl, inp)
    o1, i1 = a.out.clone(), a.idx.clone()
    b = run_prefill(wl, inp)
    assert torch.equal(o1, b.out) and torch.equal(i1, b.idx)


# ------------------------------------------------------------------------------------ decode


def _decode_check(wl, inp, st, seqs):
    gidx = st.idx.cpu().numpy()
    gout = st.out.float().cpu().numpy()
    for b in seqs:
        r = O.decode(inp, wl, b)
        differ = check_idx_rows(gidx[b], r["idx"], r["scores"], r["n_vis"])
        ref = r["out"]
        if differ:
            ref = O.sparse_attention(r["q"], r["entries"], gidx[b], r["raw"], wl.L - wl.W + 1, [wl.L], wl.W)
        assert max_err(gout[b], ref) <= TOL["bf16"], f"sequence {b}"


@pytest.mark.parametrize("H", [128, 64])   # 64 heads: the 16-head-per-wave kernel and its split merge
def test_decode_bf16_small(H):
    wl = get("decode128k").with_(B=3, L=4096 + 2048, H=H)
    inp = G.make_inputs(wl)
    st = run_decode(wl, decode_tensors(wl, inp))
    _decode_check(wl, inp, st, range(wl.B))


def test_decode_fewer_entries_than_k():
    wl = get("decode128k").with_(B=2, L=1000)        # 250 entries < k = 1024: all kept, padded
    inp = G.make_inputs(wl)
    st = run_decode(wl, decode_tensors(wl, inp))
    assert np.all(st.idx.cpu().numpy()[:, 0, 250:] == -1)
    _decode_check(wl, inp, st, range(wl.B))


def test_decode_mxfp4_small():
    wl = get("decode1m_fp4").with_(B=2, L=4 * 20000)
    inp = G.make_inputs(wl)
    st = run_decode(wl, decode_tensors(wl, inp))
    _decode_check(wl, inp, st, range(wl.B))


@pytest.mark.parametrize("B,L,b", [(8, 4 * 9000, 5), (64, 4 * 2000, 37)])
def test_decode_batch_invariance(B, L, b):
    # a sequence decoded alone gives the bits it gets inside a batch, whatever the batch size
    wl = get("decode128k").with_(B=B, L=L)
    inp = G.make_inputs(wl)
    t = decode_tensors(wl, inp)
    full = run_decode(wl, t)
    o_full, i_full = full.out.clone(), full.idx.clone()
    one = {k: (v[b:b + 1] if (v is not None and k != "w_head") else v) for k, v in t.items()}
    solo = run_decode(wl.with_(B=1), one)
    assert torch.equal(solo.out[0], o_full[b]) and torch.equal(solo.idx[0], i_full[b])


# ------------------------------------------------------------------------------------ full-size workloads


def _sampled_prefill(name, rows):
    wl = get(name)
    inp = G.make_inputs(wl)
    st = run_prefill(wl, inp)
    r = O.prefill(inp, wl, query_rows=rows)
    n_new = wl.T // wl.m
    first = wl.L // wl.m
    _assert_bf16_close(tensor_f64(st.entries[0, first:first + n_new]), r["entries_new"])
    _assert_bf16_close(tensor_f64(st.keys[0, first:first + n_new]), r["keys_new"])
    gidx = st.idx[0].cpu().numpy()[rows]
    differ = check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
    ref = r["out"].copy()
    for j in differ:
        ref[j] = O.sparse_attention(r["q"][j:j + 1], r["entries"], gidx[j:j + 1], r["raw"], r["raw_pos0"],
                                    r["q_pos"][j:j + 1], wl.W)[0]
    assert max_err(tensor_f64(st.out[0, rows]), ref) <= TOL["bf16"]


def test_full_prefill8k_sampled():
    # rows at the 8-row workgroup and 64-entry key-tile seams as well as the ends
    _sampled_prefill("prefill8k", np.array([0, 3, 4, 7, 8, 63, 64, 127, 128, 1000, 1023, 1024, 3071, 3072, 4095, 4096,
                                            6001, 8190, 8191]))


def test_full_chunk1m_sampled():
    _sampled_prefill("chunk1m", np.array([0, 1, 2, 3, 7, 8, 63, 64, 777, 1023, 1024, 2048, 3071, 3072, 4094, 4095]))


def test_full_decode128k_sampled():
    wl = get("decode128k")
    inp = G.make_inputs(wl)
    st = run_decode(wl, decode_tensors(wl, inp))
    _decode_check(wl, inp, st, [0, 7, 8, 17, 31, 32, 63])


def test_full_decode1m_fp4():
    wl = get("decode1m_fp4")
    inp = G.make_inputs(wl)
    st = run_decode(wl, decode_tensors(wl, inp))
    _decode_check(wl, inp, st, [0, 3])


def test_decode_sink_split_kv():
    # few (row, head group) pairs: the key list is split across workgroups and merged; the sink
    # enters once, in the merge
    wl = get("decode128k").with_(B=2, L=4 * 3000)
    inp = G.make_inputs(wl)
    t = decode_tensors(wl, inp)
    sink = np.linspace(-2.0, 3.0, wl.H)
    from compressed_sparse_attention_05_amd import layer
    code = lib.CSA_BF16
    st = layer.CSADecode(dims_of(wl), wl.B, wl.L // wl.m, idx_dtype=code)
    st(wl.L, t["q_idx"], t["w_head"], t["keys"], t["q"], t["entries"], t["kv_raw"],
       sink=to_device(sink.astype(np.float32), "f32"))
    torch.cuda.synchronize()
    gidx = st.idx.cpu().numpy()
    gout = st.out.float().cpu().numpy()
    for b in range(wl.B):
        r = O.decode(inp, wl, b, sink=sink)
        check_idx_rows(gidx[b], r["idx"], r["scores"], r["n_vis"])
        ref = O.sparse_attention(r["q"], r["entries"], gidx[b], r["raw"], wl.L - wl.W + 1, [wl.L], wl.W, sink=sink)
        assert max_err(gout[b], ref) <= TOL["bf16"]


def test_sparse_attn_prefill_batch_invariance():
    # 128 query rows of 128 heads: each sequence of a batch of 2 gives the bits it gets alone
    B, T, H, D, k, n_cap, q_pos0 = 2, 128, 128, 512, 512, 1500, 4 * 1500 - 128
    d = dims_of(get("decode128k").with_(k=k))
    mk = lambda name, shape: to_device(G.f32_to_bf16_bits(G.normal_f32(71, name, shape)), "bf16")
    q, ent = mk("q", (B, T, H, D)), mk("ent", (B, n_cap, D))
    raw_pos0 = q_pos0 - 127
    raw = mk("raw", (B, q_pos0 + T - raw_pos0, D))
    rng = np.random.default_rng(71)
    idx = np.stack([np.stack([np.sort(rng.choice(n_cap, k, replace=False)) for _ in range(T)]) for _ in range(B)])
    idx = to_device(idx.astype(np.int32), "i32")
    out = torch.empty(B, T, H, D, dtype=torch.float32, device="cuda")
    lib.csa_sparse_attn(d, q, ent, idx, raw, out, q_pos0=q_pos0, raw_pos0=raw_pos0)
    for b in range(B):
        one = torch.empty(1, T, H, D, dtype=torch.float32, device="cuda")
        lib.csa_sparse_attn(d, q[b:b + 1].contiguous(), ent[b:b + 1].contiguous(), idx[b:b + 1].contiguous(),
                            raw[b:b + 1].contiguous(), one, q_pos0=q_pos0, raw_pos0=raw_pos0)
        assert torch.equal(one[0], out[b])


@pytest.mark.parametrize("H", [128, 64])
def test_sparse_attn_bf16_output_alignment(H):
    # a bf16 output that is not 16-byte aligned takes the element-wise store path; both paths give
    # the same bits as the LDS-staged row stores
    T, D, k, n_cap, q_pos0 = 64, 512, 512, 1500, 4 * 1500 - 64
    d = dims_of(get("decode128k").with_(k=k, H=H))
    mk = lambda name, shape: to_device(G.f32_to_bf16_bits(G.normal_f32(72, name, shape)), "bf16")
    q, ent = mk("q", (1, T, H, D)), mk("ent", (1, n_cap, D))
    raw_pos0 = q_pos0 - 127
    raw = mk("raw", (1, q_pos0 + T - raw_pos0, D))
    rng = np.random.default_rng(72)
    idx = to_device(np.stack([np.sort(rng.choice(n_cap, k, replace=False)) for _ in range(T)])[None].astype(np.int32), "i32")
    out = torch.empty(1, T, H, D, dtype=torch.bfloat16, device="cuda")
    lib.csa_sparse_attn(d, q, ent, idx, raw, out, q_pos0=q_pos0, raw_pos0=raw_pos0)
    buf = torch.empty(T * H * D + 8, dtype=torch.bfloat16, device="cuda")
    odd = buf[1:1 + T * H * D].view(1, T, H, D)
    assert odd.data_ptr() % 16 != 0
    lib.csa_sparse_attn(d, q, ent, idx, raw, odd, q_pos0=q_pos0, raw_pos0=raw_pos0)
    assert torch.equal(odd, out)
    ref = torch.empty(1, T, H, D, dtype=torch.float32, device="cuda")
    lib.csa_sparse_attn(d, q, ent, idx, raw, ref, q_pos0=q_pos0, raw_pos0=raw_pos0)
    assert torch.equal(ref.bfloat16(), out)


@pytest.mark.parametrize("n_cap,L", [(40001, 4 * 30000), (40000, 4 * 24000), (70001, 4 * 50000)])
def test_decode_index_capacity_beyond_visible(n_cap, L):
    # a key cache with more slots than the query sees: the selection covers the visible prefix (one
    # pass while it fits a workgroup, 16K pieces of it otherwise), whatever the row stride
    B, H_I, D_I, k = 2, 64, 128, 1024
    d = dims_of(get("decode128k").with_(k=k))
    mk = lambda name, shape: G.f32_to_bf16_bits(G.normal_f32(73, name, shape))
    qb, kb = mk("iq", (B, 1, H_I, D_I)), mk("ik", (B, n_cap, D_I))
    w = G.normal_f32(73, "iw", (H_I,))
    out_idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    lib.csa_index_topk(d, to_device(qb, "bf16"), to_device(w, "f32"), to_device(kb, "bf16"), out_idx, q_pos0=L)
    got = out_idx.cpu().numpy()
    nv = min((L + 1) // 4, n_cap)
    for b in range(B):
        s = O.index_scores(O.bf16_bits_to_f64(qb[b, 0])[None], O.bf16_bits_to_f64(kb[b]), w.astype(np.float64), [nv])
        check_idx_rows(got[b], O.topk_select(s[0], nv, k)[None], s, [nv])


@pytest.mark.parametrize("T,n_cap,q_pos0", [
    (16, 2000, 256 * 5 - 16),   # the last workgroup sees exactly 5 whole 64-entry tiles
    (16, 2000, 256 * 5 - 12),   # ... and one entry of a sixth
    (16, 2000, 256 * 6 - 20),   # ... and 63 entries of a sixth
    (16, 320, 4000),            # every row capped at n_cap = 5 whole tiles
    (24, 321, 4000),            # every row capped one entry past them
    (16, 2000, 150),            # rows that see fewer than k entries keep them all
    (16, 100, 0),               # rows from position 0: no entries, then one or two
])
def test_fused_bf16_prefill_index_tile_edges(T, n_cap, q_pos0):
    # the fused bf16 indexer loads whole key tiles from one base address and clamps the rows of the
    # last, partial tile: rows at and around the 64-entry tile edges, by position and by capacity
    H_I, D_I, k = 64, 128, 64
    d = dims_of(get("chunk1m").with_(k=k))
    mk = lambda name, shape: G.f32_to_bf16_bits(G.normal_f32(91, name, shape))
    qb, kb = mk("eq", (1, T, H_I, D_I)), mk("ek", (1, n_cap, D_I))
    w = G.normal_f32(91, "ew", (H_I,))
    idx = torch.empty(1, T, k, dtype=torch.int32, device="cuda")
    lib.csa_index_topk(d, to_device(qb, "bf16"), to_device(w, "f32"), to_device(kb, "bf16"), idx, q_pos0=q_pos0)
    got = idx[0].cpu().numpy()
    nv = np.minimum(O.n_visible(q_pos0 + np.arange(T), 4), n_cap)
    s = O.index_scores(O.bf16_bits_to_f64(qb[0]), O.bf16_bits_to_f64(kb[0]), w.astype(np.float64), nv)
    ora = np.stack([O.topk_select(s[t], nv[t], k) for t in range(T)])
    differ = check_idx_rows(got, ora, s, nv)
    assert len(differ) <= 1, differ
