"""GPU parity of token-by-token decode over a state cache (csa_decode_step): every step equals the
oracle's prefill row at that position, and the entries / indexer keys that steps compress when they
complete a block equal the oracle's. Variants: plain bf16 entries, QK-norm + partial RoPE on, and
QK-norm + RoPE with the entries kept as 584-byte FP8 records."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_05_amd import layer, lib
from synth.torch_io import to_device
from synth.workloads import get
from tests.csa_testlib import O, G, TOL, check_idx_rows, dims_of, max_err, tensor_f64

pytestmark = pytest.mark.gpu


def _bf(a):
    return to_device(G.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)), "bf16")   # exact: on the bf16 grid


@pytest.mark.parametrize("variant", ["plain", "fid", "fid_records"])
def test_decode_steps_equal_prefill_rows(variant):
    wl = get("chunk1m").with_(L=0, T=300, d=512, k=64, B=2)
    L0, T = 200, wl.T                       # the context holds 200 tokens; steps at 200 .. 299
    fid = variant != "plain"
    records = variant == "fid_records"
    inp = G.make_inputs(wl)
    host = dev = None
    if fid:
        gq = (1.0 + 0.2 * G.normal_f32(120, "gamma_q", (wl.D,))).astype(np.float32)
        gk = (1.0 + 0.2 * G.normal_f32(120, "gamma_kv", (wl.D,))).astype(np.float32)
        host = {"gamma_q": gq.astype(np.float64), "gamma_kv": gk.astype(np.float64), "eps": float(np.float32(1e-6)),
                "rope_dims": 64, "theta": 10000.0}
        dev = {"gamma_q": to_device(gq, "f32"), "gamma_kv": to_device(gk, "f32"), "norm_eps": 1e-6, "rope_dims": 64,
               "rope_theta": 10000.0}
    refs = [O.prefill(inp, wl, b=b, fid=host) for b in range(wl.B)]
    d = dims_of(wl)
    m, W = wl.m, wl.W
    n_cap = T // m + 2
    st = layer.CSADecodeState(d, wl.B, n_cap, records=records)
    weights = {"bias_a": to_device(inp["bias_a"], "f32"), "bias_b": to_device(inp["bias_b"], "f32"),
               "ibias_a": to_device(inp["ibias_a"], "f32"), "ibias_b": to_device(inp["ibias_b"], "f32"),
               "w_head": to_device(inp["w_head"], "f32")}
    if fid:
        weights.update(dev)
    cols = ["ca", "za", "cb", "zb", "ica", "iza", "icb", "izb"]
    comp = [np.concatenate([r["parts"][c] for c in cols], axis=1) for r in refs]       # [T, 4D + 4D_I]
    # context: entries and keys of the first L0/m blocks, raw KV of the last W-1 positions, the previous block
    n0 = L0 // m
    ent0 = _bf(np.stack([r["entries"][:n0] for r in refs]))
    if records:
        lib.csa_entry_pack(ent0, st.entries[:, :n0])
    else:
        st.entries[:, :n0] = ent0
    st.keys[:, :n0] = _bf(np.stack([r["keys"][:n0] for r in refs]))
    for p in range(L0 - W + 1, L0):
        st.win[:, p % W] = _bf(np.stack([r["raw"][p] for r in refs]))
    st.block[:, st.block_rows(L0 // m - 1)] = _bf(np.stack([c[L0 - m:L0] for c in comp]))   # the previous block
    # the projected query and raw KV rows (before any norm: the step applies it), computed as the
    # oracle computes its projections
    pc = O.projection_columns(wl.D, wl.D_I, wl.H, wl.H_I)[0]
    Wt = O.bf16_bits_to_f64(inp["W"])
    xs = [O.bf16_bits_to_f64(inp["x"][b]) for b in range(wl.B)]
    q_all = [O.round_bf16(x @ Wt[slice(*pc["q"])].T).reshape(T, wl.H, wl.D) for x in xs]
    kv_all = [O.round_bf16(x @ Wt[slice(*pc["kv"])].T) for x in xs]
    worst = 0.0
    for p in range(L0, T):
        q = _bf(np.stack([qa[p] for qa in q_all]))
        q_idx = _bf(np.stack([r["q_idx"][p] for r in refs]))
        kv = _bf(np.stack([ka[p] for ka in kv_all]))
        cp = _bf(np.stack([c[p] for c in comp]))
        st.step(weights, p, q, q_idx, kv, cp)
        torch.cuda.synchronize()
        gidx = st.idx.cpu().numpy()
        got = tensor_f64(st.out)
        for b, r in enumerate(refs):
            differ = check_idx_rows(gidx[b:b + 1], r["idx"][p:p + 1], r["scores"][p:p + 1], r["n_vis"][p:p + 1])
            ents = O.entry_unpack(O.entry_pack(r["entries"])) if records else r["entries"]
            if differ or records:
                o = O.sparse_attention(r["q"][p:p + 1], ents, gidx[b:b + 1], r["raw"], r["raw_pos0"],
                                       r["q_pos"][p:p + 1], W)
                want = O.rope(o, r["q_pos"][p:p + 1], 64, 10000.0, inverse=True)[0] if fid else o[0]
            else:
                want = r["out"][p]
            worst = max(worst, max_err(got[b], want))
    assert worst <= TOL["bf16"], worst
    # entries and keys the steps compressed (blocks ending at 203, 207, ..., 299)
    n1 = T // m
    for b, r in enumerate(refs):
        if records:
            gotr = st.entries[b, n0:n1].cpu().numpy()
            np.testing.assert_allclose(O.entry_unpack(gotr), O.entry_unpack(O.entry_pack(r["entries"][n0:n1])),
                                       atol=TOL["bf16"] * 8, rtol=2 ** -3)
        else:
            assert max_err(tensor_f64(st.entries[b, n0:n1]), r["entries"][n0:n1]) <= TOL["bf16"]
        assert max_err(tensor_f64(st.keys[b, n0:n1]), r["keys"][n0:n1]) <= TOL["bf16"]
