"""csa_decode_step_noalloc (the decode step whose scratch is the array the library holds on the GPU)
against csa_decode_step with a caller workspace: the same outputs, selections and state updates, bit
for bit, on two calls in a row, the second with a smaller batch (the array keeps the first call's
contents)."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_05_amd import layer, lib
from synth import gen as G
from synth.torch_io import to_device

pytestmark = pytest.mark.gpu

M, D, H, H_I, D_I, K, W = 4, 512, 128, 64, 128, 1024, 128


def _bf(seed, name, shape):
    return to_device(G.f32_to_bf16_bits(G.normal_f32(seed, name, shape)), "bf16")


def _state(seed, B, n_cap, records):
    st = layer.CSADecodeState(lib.make_dims(M, D, H, H_I, D_I, K, W), B, n_cap, records=records)
    ent = _bf(seed, "ent", (B, n_cap, D))
    if records:
        lib.csa_entry_pack(ent, st.entries)
    else:
        st.entries.copy_(ent)
    st.keys.copy_(_bf(seed, "keys", (B, n_cap, D_I)))
    st.win.copy_(_bf(seed, "win", tuple(st.win.shape)))
    st.block.copy_(_bf(seed, "block", tuple(st.block.shape)))
    return st


def _weights(seed, fid):
    f = lambda name, shape, std: to_device(G.normal_f32(seed, name, shape, std), "f32")
    w = {"bias_a": f("ba", (M, D), 0.3), "bias_b": f("bb", (M, D), 0.3), "ibias_a": f("iba", (M, D_I), 0.3),
         "ibias_b": f("ibb", (M, D_I), 0.3),
         "w_head": to_device(np.full(H_I, 1.0 / H_I, dtype=np.float32), "f32")}
    if fid:
        w.update({"gamma_q": to_device((1 + 0.2 * G.normal_f32(seed, "gq", (D,))).astype(np.float32), "f32"),
                  "gamma_kv": to_device((1 + 0.2 * G.normal_f32(seed, "gk", (D,))).astype(np.float32), "f32"),
                  "norm_eps": 1e-6, "rope_dims": 64, "rope_theta": 10000.0})
    return w


@pytest.mark.parametrize("first", ["records_fid", "rows"])
def test_noalloc_decode_step_matches_workspace_step(first):
    n_cap = 3000
    d = lib.make_dims(M, D, H, H_I, D_I, K, W)
    # call 1: four sequences (two of them complete a block); call 2: two sequences, plain rows
    calls = [(4, [4 * 2500 - 1, 4 * 2000 + 1, 4 * 2900 + 3, 700], first == "records_fid"),
             (2, [4 * 1000 + 3, 4 * 2600 + 2], False)]
    for c, (B, posl, opt) in enumerate(calls):
        seed = 200 + c
        a, b = _state(seed, B, n_cap, opt), _state(seed, B, n_cap, opt)
        w = _weights(seed, opt)
        q, qi = _bf(seed, "q", (B, H, D)), _bf(seed, "qi", (B, H_I, D_I))
        kv, comp = _bf(seed, "kv", (B, D)), _bf(seed, "comp", (B, 4 * D + 4 * D_I))
        pos = torch.tensor(posl, dtype=torch.int64, device="cuda")
        a.step(w, pos, q, qi, kv, comp)
        out = torch.empty_like(a.out)
        idx = torch.empty_like(a.idx)
        lib.csa_decode_step_noalloc(d, w, pos, q, qi, kv, comp, b.state(), out, out_idx=idx)
        torch.cuda.synchronize()
        assert torch.equal(out, a.out), f"call {c}: outputs differ"
        assert torch.equal(idx, a.idx), f"call {c}: selections differ"
        for name in ("entries", "keys", "win", "block"):
            assert torch.equal(getattr(a, name), getattr(b, name)), f"call {c}: state {name} differs"


def test_noalloc_decode_step_replays_in_a_captured_graph():
    # the caller this entry point is for: a serving loop that captures the step once (nothing may
    # allocate under capture) and replays it. Replaying the same step rewrites the same state rows with
    # the same values, so every replay, with eager work between replays, equals the eager call.
    B, n_cap, seed = 4, 3000, 210
    d = lib.make_dims(M, D, H, H_I, D_I, K, W)
    st = _state(seed, B, n_cap, True)
    w = _weights(seed, True)
    q, qi = _bf(seed, "q", (B, H, D)), _bf(seed, "qi", (B, H_I, D_I))
    kv, comp = _bf(seed, "kv", (B, D)), _bf(seed, "comp", (B, 4 * D + 4 * D_I))
    pos = torch.tensor([4 * 2500 - 1, 4 * 2000 + 1, 4 * 2900 + 3, 700], dtype=torch.int64, device="cuda")
    out, idx = torch.empty_like(st.out), torch.empty_like(st.idx)
    state = st.state()
    step = lambda: lib.csa_decode_step_noalloc(d, w, pos, q, qi, kv, comp, state, out, out_idx=idx)
    step()
    torch.cuda.synchronize()
    ref_out, ref_idx = out.clone(), idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: outputs differ"
        assert torch.equal(idx, ref_idx), f"replay {r}: selections differ"
