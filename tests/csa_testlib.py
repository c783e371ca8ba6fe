"""Shared helpers of the GPU parity tests: upload generated inputs, run the layer through the C ABI,
compare with the oracle under the parity rules.

Rules (from the layer's acceptance bar):
  * top-k sets: bit-exact when the selection is fed the oracle's own scores; end to end the GPU set
    may differ from the oracle's only at near-ties, |s_a - s_b| <= 1e-3 * max(|s_a|, |s_b|) + floor,
    scores taken from the oracle in float64 (floor: 1e-6 of the row's largest score, for exact zeros);
  * outputs: max abs error <= 1e-4 (fp32 layers) / 2e-2 (bf16 layers); where the sets differ the
    oracle's attention is recomputed on the GPU's set.
"""
from __future__ import annotations

import numpy as np
import torch

from compressed_sparse_attention_05_amd import layer, lib
from oracle import csa_oracle as O
from synth import gen as G
from synth.torch_io import act, to_device

TOL = {"f32": 1e-4, "bf16": 2e-2}


def dims_of(wl) -> lib.Dims:
    return layer.dims(wl.m, wl.D, wl.H, wl.H_I, wl.D_I, wl.k, wl.W)


def torch_dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def weights_to_device(wl, inp) -> dict:
    return {
        "w_proj": act(inp["W"], wl),
        "bias_a": to_device(inp["bias_a"], "f32"),
        "bias_b": to_device(inp["bias_b"], "f32"),
        "ibias_a": to_device(inp["ibias_a"], "f32"),
        "ibias_b": to_device(inp["ibias_b"], "f32"),
        "w_head": to_device(inp["w_head"], "f32"),
    }


def run_prefill(wl, inp, weights=None, out_dtype=torch.float32):
    """csa_forward over the workload's chunk; returns the CSAPrefill holding out/idx/caches."""
    d = dims_of(wl)
    w = weights or weights_to_device(wl, inp)
    fp4 = wl.idx_dtype == "mxfp4"
    st = layer.CSAPrefill(d, wl.B, wl.T, wl.d, wl.n_cap, dtype=torch_dtype(wl), out_dtype=out_dtype, fp4_keys=fp4)
    if wl.L > 0:
        n0 = wl.L // wl.m
        st.entries[:, :n0] = act(inp["entries_prefix"], wl)
        if fp4:
            st.keys[:, :n0] = to_device(inp["keys_prefix_codes"], "u8")
            st.key_scales[:, :n0] = to_device(inp["keys_prefix_scales"], "u8")
        else:
            st.keys[:, :n0] = act(inp["keys_prefix"], wl)
        st.win[:, : wl.W - 1] = act(inp["win_prefix"], wl)
        st.halo.copy_(act(inp["halo"], wl))
    x = act(inp["x"], wl)
    st(w, x, wl.L)
    torch.cuda.synchronize()
    return st


def decode_tensors(wl, inp) -> dict:
    t = {"entries": act(inp["entries"], wl), "kv_raw": act(inp["kv_raw"], wl), "q": act(inp["q"], wl),
         "w_head": to_device(inp["w_head"], "f32")}
    if wl.idx_dtype == "mxfp4":
        t["keys"] = to_device(inp["keys_codes"], "u8")
        t["k_scale"] = to_device(inp["keys_scales"], "u8")
        t["q_idx"] = to_device(inp["q_idx_codes"], "u8")
        t["q_scale"] = to_device(inp["q_idx_scales"], "u8")
    else:
        t["keys"] = act(inp["keys"], wl)
        t["q_idx"] = act(inp["q_idx"], wl)
        t["k_scale"] = t["q_scale"] = None
    return t


def run_decode(wl, t, out_dtype=torch.float32):
    d = dims_of(wl)
    code = lib.CSA_MXFP4 if wl.idx_dtype == "mxfp4" else (lib.CSA_BF16 if wl.dtype == "bf16" else lib.CSA_F32)
    st = layer.CSADecode(d, wl.B, wl.L // wl.m, idx_dtype=code, out_dtype=out_dtype)
    st(wl.L, t["q_idx"], t["w_head"], t["keys"], t["q"], t["entries"], t["kv_raw"], q_scale=t["q_scale"],
       k_scale=t["k_scale"])
    torch.cuda.synchronize()
    return st


def near_tie_ok(gpu_row, ora_row, scores_row):
    """The GPU's set may differ from the oracle's only by swaps of near-tied entries."""
    g = set(int(i) for i in gpu_row if i >= 0)
    o = set(int(i) for i in ora_row if i >= 0)
    if len(g) != len(o):
        return False, f"set sizes {len(g)} vs {len(o)}"
    only_g, only_o = sorted(g - o), sorted(o - g)
    if not only_g:
        return True, ""
    fin = scores_row[np.isfinite(scores_row)]
    floor = 1e-6 * (np.abs(fin).max() if fin.size else 1.0)
    sg = scores_row[only_g]
    so = scores_row[only_o]
    if not np.all(np.isfinite(sg)):
        return False, "GPU selected an invisible entry"
    # every swapped-in entry must be within the tolerance of every swapped-out one
    gap = np.abs(sg[:, None] - so[None, :])
    tol = 1e-3 * np.maximum(np.abs(sg)[:, None], np.abs(so)[None, :]) + floor
    ok = bool(np.all(gap <= tol))
    return ok, "" if ok else f"{len(only_g)} swaps, worst gap {(gap - tol).max():.3g} above tolerance"


def check_idx_rows(gpu_idx, ora_idx, scores, n_vis):
    """gpu_idx, ora_idx: [R, k]; scores: [R, N] oracle float64; returns rows whose sets differ."""
    differ = []
    for r in range(gpu_idx.shape[0]):
        g = gpu_idx[r]
        valid = g[g >= 0]
        assert np.all(np.diff(valid) > 0), f"row {r}: indices not ascending/unique"
        assert np.all(g[len(valid):] == -1), f"row {r}: padding not -1"
        assert len(valid) == min(len(g), int(n_vis[r])), f"row {r}: {len(valid)} selected, n_vis {n_vis[r]}"
        assert np.all(valid < n_vis[r]), f"row {r}: non-causal entry selected"
        if not np.array_equal(g, ora_idx[r]):
            ok, msg = near_tie_ok(g, ora_idx[r], scores[r])
            assert ok, f"row {r}: {msg}"
            differ.append(r)
    return differ


def max_err(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)))) if np.size(a) else 0.0


def tensor_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_inputs(wl):
    return G.make_inputs(wl)


__all__ = ["O", "G", "TOL", "dims_of", "run_prefill", "run_decode", "decode_tensors", "check_idx_rows",
           "max_err", "tensor_f64", "weights_to_device", "near_tie_ok", "make_inputs", "torch_dtype"]
