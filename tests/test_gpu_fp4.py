"""GPU parity of the MXFP4 indexer path ("Anatomy of a Frontier Model", sections "The KV cache,
recomputed": indexer keys as 128 FP4 values plus a scale byte per 32; "Precision: FP8 everywhere, FP4
experts": the indexer's query-key product in FP4).

  * csa_mxfp4_quantize: codes and scales bit-exact against the oracle's quantiser (ties, saturation,
    signed zeros, tiny and huge blocks, strided and unaligned rows, f32 and bf16 inputs);
  * the fused MXFP4 prefill indexer (many query rows, no score matrix) on generated FP4 queries and
    keys: index sets against the oracle's scores under the near-tie rule, several tiles and a ragged
    tail, rows with fewer visible entries than k;
  * csa_forward with an MXFP4 key cache: the compressor epilogue's codes equal csa_mxfp4_quantize of
    the keys a bf16 cache stores, and the oracle's codes wherever the stored bf16 keys agree; the
    chunk's indices and outputs match the oracle. The projection inputs sit on a dyadic grid so that
    q_I is exact on both sides (an FP4 code is a step function of q_I: a last-bit difference in a GEMM
    sum can move it by a whole e2m1 step);
  * decode steps over an MXFP4 key state equal the oracle's rows, and the keys the steps compress
    equal the oracle's codes.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_05_amd import layer, lib
from synth.torch_io import act, to_device
from synth.workloads import get
from tests.csa_testlib import O, G, TOL, check_idx_rows, dims_of, max_err, run_prefill, tensor_f64, \
    weights_to_device

pytestmark = pytest.mark.gpu


def _quant_rows(seed):
    """Generated rows of 256 values at scales 2**-30 .. 2**29, and rows built from the cases the rule
    singles out: exact rounding midpoints, saturation, zeros of both signs, subnormal and huge blocks."""
    x = G.normal_f32(seed, "mx", (240, 256)) * np.exp2((np.arange(240) % 60) - 30).astype(np.float32)[:, None]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    edge = np.zeros((16, 256), np.float32)
    for r in range(8):
        s = np.float32(2.0 ** (3 * r - 12))
        blk = np.concatenate([mids, -mids, mids * 1.0009765625, [7.0, -7.5, 0.0, -0.0, 6.5, 8.0 - 1 / 64, 0.1, -0.1]])
        edge[r] = np.tile(blk.astype(np.float32) * s, 256 // 32)
    edge[8] = 0.0
    edge[9, ::3] = -0.0
    edge[10] = np.float32(2.0 ** -130) * np.sign(G.normal_f32(seed, "sg", (256,)))   # subnormal values
    edge[11, ::2] = np.float32(2.0 ** -127)
    edge[12] = np.float32(1.5 * 2.0 ** 127) * np.sign(G.normal_f32(seed, "sg2", (256,)))
    edge[13] = np.float32(2.0 ** -125)
    edge[14] = G.normal_f32(seed, "e14", (256,)) * np.float32(2.0 ** 100)
    edge[15] = G.normal_f32(seed, "e15", (256,)) * np.float32(2.0 ** -120)
    return np.concatenate([x, edge])


@pytest.mark.parametrize("dtype,layout", [("f32", "contiguous"), ("bf16", "contiguous"), ("bf16", "strided"),
                                          ("bf16", "unaligned"), ("f32", "unaligned")])
def test_quantize_bit_exact(dtype, layout):
    x32 = _quant_rows(21)
    R, D = x32.shape
    if dtype == "bf16":
        bits = G.f32_to_bf16_bits(x32)
        host = O.bf16_bits_to_f64(bits)
        src = to_device(bits, "bf16")
    else:
        host = x32.astype(np.float64)
        src = to_device(x32, "f32")
    if layout == "contiguous":
        dev = src
    else:
        # a wider buffer: rows 320 apart; "unaligned" starts one element in (not 16-byte aligned)
        off = 1 if layout == "unaligned" else 0
        wide = torch.zeros(R, 320, dtype=src.dtype, device=src.device)
        wide[:, off:off + D] = src
        dev = wide[:, off:off + D]
    codes, scales = lib.csa_mxfp4_quantize(dev)
    torch.cuda.synchronize()
    oc, os_ = O.mxfp4_quantize(host)
    np.testing.assert_array_equal(scales.cpu().numpy(), os_)
    np.testing.assert_array_equal(codes.cpu().numpy(), oc)


def _fp4_index_case(T, n_cap, k, seed, q_pos0):
    wl = get("decode1m_fp4").with_(T=T, seed=seed)
    qc, qs = G.mxfp4_encode(G.normal_f32(seed, "qi", (1, T, wl.H_I, wl.D_I)))
    kc, ks = G.mxfp4_encode(G.normal_f32(seed, "ki", (1, n_cap, wl.D_I)))
    w = G.normal_f32(seed, "w", (wl.H_I,))
    w = np.exp(w - w.max()) / np.exp(w - w.max()).sum()
    d = layer.dims(4, wl.D, wl.H, wl.H_I, wl.D_I, k, wl.W)
    idx = torch.empty(1, T, k, dtype=torch.int32, device="cuda")
    lib.csa_index_topk(d, to_device(qc, "u8"), to_device(w.astype(np.float32), "f32"), to_device(kc, "u8"), idx,
                       q_pos0=q_pos0, q_scale=to_device(qs, "u8"), k_scale=to_device(ks, "u8"))
    torch.cuda.synchronize()
    q = O.mxfp4_decode(qc[0], qs[0])
    keys = O.mxfp4_decode(kc[0], ks[0])
    nv = np.minimum(O.n_visible(q_pos0 + np.arange(T), 4), n_cap)
    scores = O.index_scores(q, keys, w.astype(np.float64), nv)
    ora = np.stack([O.topk_select(scores[t], nv[t], k) for t in range(T)])
    return idx[0].cpu().numpy(), ora, scores, nv


@pytest.mark.parametrize("T,n_cap,k,q_pos0", [(44, 3000, 256, 11000), (20, 700, 512, 500), (9, 130, 64, 0),
                                               (16, 5000, 64, 512 * 5 - 16), (16, 5000, 64, 512 * 5 - 12),
                                               (16, 640, 64, 4000), (16, 641, 64, 4000)])
def test_fused_fp4_prefill_index(T, n_cap, k, q_pos0):
    # T >= 8 rows per sequence take the fused MXFP4 kernel: several 128-entry tiles, a ragged last tile,
    # a ragged last workgroup of rows, (second case) rows that see fewer than k entries, and (the last
    # four) a last workgroup that sees exactly 5 whole tiles or one entry more, by position or capacity
    assert lib.csa_workspace_size(lib.CSA_OP_INDEX_TOPK, layer.dims(4, 512, 128, 64, 128, k, 128), 1, T, n_cap,
                                  0, lib.CSA_MXFP4) == 0
    gidx, ora, scores, nv = _fp4_index_case(T, n_cap, k, 40 + T, q_pos0)
    differ = check_idx_rows(gidx, ora, scores, nv)
    assert len(differ) <= max(2, T // 10), differ


def _fp4_forward(fid_host=None):
    # a 260-token chunk after 2048 tokens of context (577 entries: 5 key tiles, the last ragged; the last
    # workgroup of query rows holds 4), k = 64 so that the selection has a choice
    wl = get("chunk1m").with_(L=2048, T=260, d=512, B=1, k=64, idx_dtype="mxfp4")
    inp = G.dyadic_projection(G.make_inputs(wl), wl)
    ref = O.prefill(inp, wl)
    st = run_prefill(wl, inp)
    wl16 = wl.with_(idx_dtype="bf16")
    inp16 = dict(inp)
    inp16["keys_prefix"] = G.f32_to_bf16_bits(O.mxfp4_decode(inp["keys_prefix_codes"], inp["keys_prefix_scales"])
                                              .astype(np.float32))
    st16 = run_prefill(wl16, inp16)
    return wl, inp, ref, st, st16


def test_forward_fp4_keys_and_parity():
    wl, inp, r, st, st16 = _fp4_forward()
    n0, n1 = wl.L // wl.m, wl.n_cap
    # the fused epilogue equals quantising the keys a bf16 cache stores
    c16, s16 = lib.csa_mxfp4_quantize(st16.keys[0, n0:n1].contiguous())
    torch.cuda.synchronize()
    gc, gs = st.keys[0, n0:n1].cpu().numpy(), st.key_scales[0, n0:n1].cpu().numpy()
    np.testing.assert_array_equal(gc, c16.cpu().numpy())
    np.testing.assert_array_equal(gs, s16.cpu().numpy())
    # and the oracle's codes wherever the stored bf16 keys agree (whole blocks of 32)
    oc, os_ = r["keys_new_fp4"]
    k16 = tensor_f64(st16.keys[0, n0:n1])
    same = (k16 == r["keys_new"]).reshape(n1 - n0, -1, 32).all(axis=-1)        # [entries, blocks]
    assert same.mean() > 0.95, same.mean()
    np.testing.assert_array_equal(gs[same], os_[same])
    cb = gc.reshape(n1 - n0, -1, 16)
    ob = oc.reshape(n1 - n0, -1, 16)
    np.testing.assert_array_equal(cb[same], ob[same])
    # the context rows are untouched
    np.testing.assert_array_equal(st.keys[0, :n0].cpu().numpy(), inp["keys_prefix_codes"][0])
    # indices (near-tie rule against the oracle's FP4 scores) and outputs
    gidx = st.idx[0].cpu().numpy()
    differ = check_idx_rows(gidx, r["idx"], r["scores"], r["n_vis"])
    ref = r["out"].copy()
    for t in differ:
        ref[t] = O.sparse_attention(r["q"][t:t + 1], r["entries"], gidx[t:t + 1], r["raw"], r["raw_pos0"],
                                    r["q_pos"][t:t + 1], wl.W)[0]
    assert max_err(tensor_f64(st.out[0]), ref) <= TOL["bf16"]
    assert len(differ) <= 8, differ


def _bf(a):
    return to_device(G.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)), "bf16")


def test_decode_steps_over_fp4_keys():
    # token-by-token decode at positions 200 .. 299 over an MXFP4 key state equals the oracle's prefill
    # rows; the steps quantise their q_idx and the keys of the blocks they complete
    wl = get("chunk1m").with_(L=0, T=300, d=512, k=64, B=2, idx_dtype="mxfp4")
    L0, T, m, W = 200, wl.T, wl.m, wl.W
    inp = G.make_inputs(wl)
    refs = [O.prefill(inp, wl, b=b) for b in range(wl.B)]
    d = dims_of(wl)
    n_cap = T // m + 2
    st = layer.CSADecodeState(d, wl.B, n_cap, fp4_keys=True)
    weights = {"bias_a": to_device(inp["bias_a"], "f32"), "bias_b": to_device(inp["bias_b"], "f32"),
               "ibias_a": to_device(inp["ibias_a"], "f32"), "ibias_b": to_device(inp["ibias_b"], "f32"),
               "w_head": to_device(inp["w_head"], "f32")}
    cols = ["ca", "za", "cb", "zb", "ica", "iza", "icb", "izb"]
    comp = [np.concatenate([r["parts"][c] for c in cols], axis=1) for r in refs]
    n0 = L0 // m
    st.entries[:, :n0] = _bf(np.stack([r["entries"][:n0] for r in refs]))
    st.keys[:, :n0] = to_device(np.stack([r["keys_new_fp4"][0][:n0] for r in refs]), "u8")
    st.key_scales[:, :n0] = to_device(np.stack([r["keys_new_fp4"][1][:n0] for r in refs]), "u8")
    for p in range(L0 - W + 1, L0):
        st.win[:, p % W] = _bf(np.stack([r["raw"][p] for r in refs]))
    st.block[:, st.block_rows(L0 // m - 1)] = _bf(np.stack([c[L0 - m:L0] for c in comp]))
    pc = O.projection_columns(wl.D, wl.D_I, wl.H, wl.H_I)[0]
    Wt = O.bf16_bits_to_f64(inp["W"])
    xs = [O.bf16_bits_to_f64(inp["x"][b]) for b in range(wl.B)]
    q_all = [O.round_bf16(x @ Wt[slice(*pc["q"])].T).reshape(T, wl.H, wl.D) for x in xs]
    kv_all = [O.round_bf16(x @ Wt[slice(*pc["kv"])].T) for x in xs]
    worst, n_differ = 0.0, 0
    for p in range(L0, T):
        q = _bf(np.stack([qa[p] for qa in q_all]))
        q_idx = _bf(np.stack([r["q_idx_stored"][p] for r in refs]))
        kv = _bf(np.stack([ka[p] for ka in kv_all]))
        cp = _bf(np.stack([c[p] for c in comp]))
        st.step(weights, p, q, q_idx, kv, cp)
        torch.cuda.synchronize()
        gidx = st.idx.cpu().numpy()
        got = tensor_f64(st.out)
        for b, r in enumerate(refs):
            differ = check_idx_rows(gidx[b:b + 1], r["idx"][p:p + 1], r["scores"][p:p + 1], r["n_vis"][p:p + 1])
            if differ:
                n_differ += 1
                want = O.sparse_attention(r["q"][p:p + 1], r["entries"], gidx[b:b + 1], r["raw"], r["raw_pos0"],
                                          r["q_pos"][p:p + 1], W)[0]
            else:
                want = r["out"][p]
            worst = max(worst, max_err(got[b], want))
    assert worst <= TOL["bf16"], worst
    assert n_differ <= 10, n_differ
    # the keys the steps compressed: the oracle's codes (blocks whose stored bf16 keys could differ by a
    # last bit are rare; at most a few blocks may differ, each by one e2m1 step)
    n1 = T // m
    blocks = total = 0
    for b, r in enumerate(refs):
        gc = st.keys[b, n0:n1].cpu().numpy()
        gs = st.key_scales[b, n0:n1].cpu().numpy()
        oc, os_ = r["keys_new_fp4"][0][n0:n1], r["keys_new_fp4"][1][n0:n1]
        eq = (gc.reshape(n1 - n0, -1, 16) == oc.reshape(n1 - n0, -1, 16)).all(axis=-1) & (gs == os_)
        blocks += int((~eq).sum())
        total += eq.size
        dv = np.abs(O.mxfp4_decode(gc, gs) - O.mxfp4_decode(oc, os_))
        step = np.repeat(np.ldexp(1.0, os_.astype(int) - 127), 32, axis=-1)
        assert np.all(dv <= 2 * step + 1e-30)
    assert blocks <= max(2, total // 100), (blocks, total)
