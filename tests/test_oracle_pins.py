"""Pins for the CPU oracle: each check ties the oracle to something other than itself.

Hand-worked examples (tests/golden/*.json, each citing its source), closed forms, invariants,
special cases that reduce to a library routine (torch's scaled_dot_product_attention in float64,
torch's float32 -> bfloat16 rounding) and brute-force properties on small inputs.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synth import gen as G
from synth.workloads import get

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------- formats


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-30).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        # exact halfway cases: 1 + odd multiples of 2**-8
        (1.0 + (2 * np.arange(64) + 1) * 2.0 ** -8).astype(np.float32),
    ])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x32.astype(np.float64)), ref)


def test_bf16_round_ties_to_even_by_hand():
    # 1 + 2**-8 lies halfway between 1 and 1 + 2**-7: the even mantissa (1.0) wins.
    assert O.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2**-8 lies halfway between 1 + 2**-7 (odd) and 1 + 2**-6 (even).
    assert O.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above the halfway point rounds up
    assert O.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7


def test_bf16_generator_bits_decode_to_their_value():
    x = G.normal_f32(3, "t", (4096,))
    bits = G.f32_to_bf16_bits(x)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(bits), O.round_bf16(x.astype(np.float64)))


def test_mxfp4_table_from_spec():
    g = _gold("mxfp4_e2m1.json")
    for code, val in g["e2m1_code_to_value"].items():
        got = O.e2m1_decode(np.array([int(code)]))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)
    for E, s in g["e8m0_scale"].items():
        codes = np.zeros(16, dtype=np.uint8)
        codes[0] = 0x02                        # element 0 = +1.0, element 1 = 0
        codes[1] = 0x70                        # element 2 = 0,    element 3 = +6.0
        vals = O.mxfp4_decode(codes[None], np.array([[int(E)]], dtype=np.uint8))[0]
        assert vals[0] == 1.0 * s and vals[1] == 0.0 and vals[2] == 0.0 and vals[3] == 6.0 * s


def test_mxfp4_each_block_has_its_own_scale():
    codes = np.full((1, 64), 0x22, dtype=np.uint8)        # every element +1.0
    scales = np.array([[127, 128, 126, 130]], dtype=np.uint8)
    v = O.mxfp4_decode(codes, scales)[0]
    np.testing.assert_array_equal(v, np.repeat([1.0, 2.0, 0.5, 8.0], 32))


def test_mxfp4_encoder_roundtrip_error_bound():
    x = G.normal_f32(5, "q", (64, 128))
    codes, scales = G.mxfp4_encode(x)
    y = O.mxfp4_decode(codes, scales)
    # The scale puts max|x| / scale in [4, 8): below 6 the error is at most half an e2m1 step
    # (steps are at most 2 scales wide); above 6 saturation costs at most 8 - 6 = 2 scales.
    scale = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=-1)
    err = np.abs(y - x) / scale
    assert np.all(err <= 2.0)
    assert np.all(err[np.abs(x) <= 6 * scale] <= 1.0)


def _unpack_codes(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    return np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))


def test_mxfp4_quantize_hand_blocks():
    # blocks worked by hand from the OCP conversion rule: scale choice, ties to even, saturation,
    # signed zero, clamping of the shared exponent at both ends of the e8m0 range
    g = _gold("mxfp4_quantize_hand.json")
    for i, blk in enumerate(g["blocks"]):
        codes, scales = O.mxfp4_quantize(np.array(blk["x"], dtype=np.float64)[None])
        assert scales[0, 0] == blk["scale"], (i, scales[0, 0])
        np.testing.assert_array_equal(_unpack_codes(codes)[0], blk["codes"], err_msg=f"block {i}")


def test_mxfp4_quantize_fixed_points():
    # every MXFP4 value is its own quantisation: a block holding all 16 codes (its largest magnitude
    # 6 * 2**X puts the shared exponent back at X) comes back unchanged, for every finite scale byte
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    for s in range(0, 254):
        x = O.mxfp4_decode(packed[None], np.array([[s]], dtype=np.uint8))
        c2, s2 = O.mxfp4_quantize(x)
        assert s2[0, 0] == s
        np.testing.assert_array_equal(c2[0], packed)


def test_mxfp4_quantize_is_a_nearest_rounding_brute_force():
    # each element goes to a nearest value among all 16 codes under the block's scale; on an exact
    # tie the chosen code has mantissa bit 0; past 6 * scale it saturates to 6 * scale
    rng = np.random.default_rng(11)
    x = rng.standard_normal((400, 64)) * np.exp2(rng.integers(-20, 20, size=(400, 1)))
    # exact halfway points and saturating values, placed inside blocks whose max sets a known scale
    x[:50, :8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * np.exp2(rng.integers(-5, 5, size=(50, 1)))
    x[:50, 8:32] = 0.0
    codes, scales = O.mxfp4_quantize(x)
    got = O.mxfp4_decode(codes, scales)
    scale = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=-1)
    allv = O.e2m1_decode(np.arange(16))                          # [16]
    cand = allv[None, None, :] * scale[..., None]                # [R, D, 16]
    d = np.abs(cand - x[..., None])
    best = d.min(axis=-1)
    np.testing.assert_array_equal(np.abs(got - x), best)
    c = _unpack_codes(codes)
    n_near = ((d == best[..., None]) & (np.abs(cand) != 0)).sum(axis=-1)   # +-0 count once
    tie = n_near >= 2
    assert tie.sum() > 50
    assert np.all((c[tie] & 1) == 0)
    # the scale is the one the rule fixes: max |x| / 2**X in [4, 8)
    amax = np.abs(x.reshape(400, 2, 32)).max(axis=-1)
    ratio = amax / np.ldexp(1.0, scales.astype(int) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))


def test_mxfp4_quantize_sign_and_scale_symmetry():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 128))
    c, s = O.mxfp4_quantize(x)
    cn, sn = O.mxfp4_quantize(-x)
    np.testing.assert_array_equal(sn, s)
    np.testing.assert_array_equal(cn, c ^ 0x88)
    for j in (-9, -1, 1, 7):
        cj, sj = O.mxfp4_quantize(x * 2.0 ** j)
        np.testing.assert_array_equal(cj, c)
        np.testing.assert_array_equal(sj.astype(int), s.astype(int) + j)


def test_mxfp4_quantize_agrees_with_the_generator_encoder_on_values():
    # the generator's encoder is a separate implementation (edge comparisons instead of a nearest
    # search); they may differ only in the sign of a zero
    x = G.normal_f32(13, "k", (256, 128)).astype(np.float64)
    co, so = O.mxfp4_quantize(x)
    cg, sg = G.mxfp4_encode(x.astype(np.float32))
    np.testing.assert_array_equal(so, sg)
    np.testing.assert_array_equal(O.mxfp4_decode(co, so), O.mxfp4_decode(cg, sg))


# ---------------------------------------------------------------------------------- compressor


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_compress_hand_example():
    g = _gold("compress_hand.json")
    e = O.compress(g["ca"], g["za"], g["cb"], g["zb"], g["bias_a"], g["bias_b"], g["m"], 0)
    np.testing.assert_allclose(e, g["expected_entries"], rtol=0, atol=1e-12)


def test_compress_weights_sum_to_one_and_entry0_pools_own_block_only():
    rng = np.random.default_rng(0)
    T, c, m = 40, 7, 4
    ca, za, cb, zb = (_rand(rng, T, c) * 3 for _ in range(4))
    ba, bb = _rand(rng, m, c), _rand(rng, m, c)
    e, p = O.compress(ca, za, cb, zb, ba, bb, m, 0, return_weights=True)
    assert e.shape == (T // m, c)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[0, m:] == 0.0)            # entry 0: no previous block
    assert np.all(p[1:, m:] > 0.0)            # later entries: both blocks take part


def test_compress_zero_logits_give_plain_mean():
    rng = np.random.default_rng(1)
    T, c, m = 24, 5, 4
    ca, cb = _rand(rng, T, c), _rand(rng, T, c)
    z = np.zeros((T, c))
    b0 = np.zeros((m, c))
    e = O.compress(ca, z, cb, z, b0, b0, m, 0)
    np.testing.assert_allclose(e[0], ca[0:4].mean(axis=0), atol=1e-12)
    for i in range(1, T // m):
        want = (ca[i * m:(i + 1) * m].sum(axis=0) + cb[(i - 1) * m:i * m].sum(axis=0)) / (2 * m)
        np.testing.assert_allclose(e[i], want, atol=1e-12)


@pytest.mark.parametrize("series,r", [("a", 0), ("a", 3), ("b", 1), ("b", 2)])
def test_compress_one_hot_bias_selects_that_token(series, r):
    rng = np.random.default_rng(2)
    T, c, m = 20, 3, 4
    ca, za, cb, zb = (_rand(rng, T, c) for _ in range(4))
    ba, bb = np.zeros((m, c)), np.zeros((m, c))
    (ba if series == "a" else bb)[r, :] = 1e4
    e = O.compress(ca, za, cb, zb, ba, bb, m, 0)
    for i in range(1, T // m):
        want = ca[i * m + r] if series == "a" else cb[(i - 1) * m + r]
        np.testing.assert_allclose(e[i], want, atol=1e-9)


def test_compress_constant_values():
    rng = np.random.default_rng(3)
    T, c, m = 16, 4, 4
    za, zb = _rand(rng, T, c), _rand(rng, T, c)
    ba, bb = _rand(rng, m, c), _rand(rng, m, c)
    const = np.tile(np.array([1.5, -2.0, 0.25, 7.0]), (T, 1))
    e = O.compress(const, za, const, zb, ba, bb, m, 0)
    np.testing.assert_allclose(e, const[: T // m], atol=1e-12)


def test_compress_with_halo_equals_compress_of_whole_sequence():
    rng = np.random.default_rng(4)
    T, c, m, split = 32, 6, 4, 12
    ca, za, cb, zb = (_rand(rng, T, c) for _ in range(4))
    ba, bb = _rand(rng, m, c), _rand(rng, m, c)
    whole = O.compress(ca, za, cb, zb, ba, bb, m, 0)
    tail = O.compress(ca[split:], za[split:], cb[split:], zb[split:], ba, bb, m, split // m,
                      halo_cb=cb[split - m:split], halo_zb=zb[split - m:split])
    np.testing.assert_allclose(tail, whole[split // m:], atol=1e-12)


def test_compress_drops_incomplete_trailing_block():
    rng = np.random.default_rng(5)
    ca, za, cb, zb = (_rand(rng, 10, 2) for _ in range(4))
    e = O.compress(ca, za, cb, zb, np.zeros((4, 2)), np.zeros((4, 2)), 4, 0)
    assert e.shape == (2, 2)


def test_compress_single_series_special_case():
    # With identical series and biases the two readings coincide: entry i is a softmax over the
    # 8 consecutive tokens [(i-1)m, (i+1)m) of z + bias[token mod m].
    rng = np.random.default_rng(6)
    T, c, m = 24, 3, 4
    cc, zz = _rand(rng, T, c), _rand(rng, T, c)
    bias = _rand(rng, m, c)
    e = O.compress(cc, zz, cc, zz, bias, bias, m, 0)
    for i in range(1, T // m):
        rows = np.arange((i - 1) * m, (i + 1) * m)
        lg = zz[rows] + bias[rows % m]
        w = np.exp(lg - lg.max(axis=0))
        w /= w.sum(axis=0)
        np.testing.assert_allclose(e[i], (w * cc[rows]).sum(axis=0), atol=1e-12)


def test_hca_compress_closed_forms():
    # [ANAT] bullet "HCA": one entry per block of m tokens, no overlap
    rng = np.random.default_rng(40)
    T, c, m = 3 * 128 + 50, 6, 128
    cc, zz = _rand(rng, T, c), _rand(rng, T, c) * 4
    bias = _rand(rng, m, c)
    e = O.hca_compress(cc, zz, bias, m)
    assert e.shape == (3, c)                                   # the tail block produces nothing
    z0 = np.zeros((T, c))
    np.testing.assert_allclose(O.hca_compress(cc, z0, np.zeros((m, c)), m),
                               cc[:3 * m].reshape(3, m, c).mean(axis=1), atol=1e-12)
    hot = np.zeros((m, c))
    hot[77] = 1e4
    np.testing.assert_allclose(O.hca_compress(cc, zz, hot, m), cc[77:3 * m:m], atol=1e-9)
    const = np.tile(np.linspace(-3, 3, c), (T, 1))
    np.testing.assert_allclose(O.hca_compress(const, zz, bias, m), const[:3], atol=1e-12)
    # entries are convex combinations of their own block only
    for i in range(3):
        blk = cc[i * m:(i + 1) * m]
        assert np.all(e[i] <= blk.max(axis=0) + 1e-12) and np.all(e[i] >= blk.min(axis=0) - 1e-12)


def test_dense_attention_equals_sdpa_with_causal_entries_and_window():
    rng = np.random.default_rng(41)
    T, H, D, m, W, p0 = 29, 3, 8, 4, 6, 40
    N = (p0 + T) // m
    q = _rand(rng, T, H, D)
    ent = _rand(rng, N, D)
    raw = _rand(rng, p0 + T, D)
    q_pos = p0 + np.arange(T)
    sink = rng.standard_normal(H)
    o = O.dense_attention(q, ent, raw, 0, q_pos, m, W, sink=sink)
    nv = O.n_visible(q_pos, m)
    keys = torch.from_numpy(np.concatenate([ent, raw, np.zeros((1, D))], axis=0))   # + sink slot
    L = keys.shape[0]
    mask = torch.zeros(T, L, dtype=torch.bool)
    for t in range(T):
        p = int(q_pos[t])
        mask[t, :nv[t]] = True
        mask[t, N + max(0, p - W + 1):N + p + 1] = True
    mask[:, L - 1] = True
    scale = 1.0 / np.sqrt(D)
    logits = torch.einsum("thd,ld->htl", torch.from_numpy(q), keys) * scale
    logits[:, :, L - 1] = torch.from_numpy(sink)[:, None]           # the sink's logit, value row 0
    logits = logits.masked_fill(~mask.unsqueeze(0), float("-inf"))
    ref = torch.softmax(logits, dim=-1) @ keys                          # [H, T, D]
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------------- indexer


def test_index_hand_example():
    g = _gold("index_hand.json")
    s = O.index_scores(g["q_idx"], g["keys"], g["w"], np.array(g["n_vis"]))
    np.testing.assert_allclose(s, g["expected_scores"], atol=1e-12)


def test_index_single_head_is_relu_dot():
    rng = np.random.default_rng(7)
    q, k = _rand(rng, 5, 1, 8), _rand(rng, 9, 8)
    s = O.index_scores(q, k, np.array([1.0]), np.full(5, 9))
    for t in range(5):
        for i in range(9):
            assert s[t, i] == pytest.approx(max(0.0, float(np.dot(q[t, 0], k[i]))), abs=1e-12)


def test_index_nonnegative_and_invisible_masked():
    rng = np.random.default_rng(8)
    q, k = _rand(rng, 6, 3, 4), _rand(rng, 10, 4)
    w = np.abs(_rand(rng, 3))
    nv = np.array([0, 1, 3, 5, 10, 12])
    s = O.index_scores(q, k, w, nv)
    for t in range(6):
        v = min(nv[t], 10)
        assert np.all(s[t, :v] >= 0)
        assert np.all(np.isneginf(s[t, v:]))


def test_index_per_query_weights():
    rng = np.random.default_rng(9)
    q, k = _rand(rng, 3, 2, 4), _rand(rng, 5, 4)
    w = np.abs(_rand(rng, 3, 2))
    s = O.index_scores(q, k, w, np.full(3, 5))
    for t in range(3):
        s1 = O.index_scores(q[t:t + 1], k, w[t], np.array([5]))
        np.testing.assert_allclose(s[t], s1[0], atol=1e-12)


def test_n_visible_matches_block_completion_by_enumeration():
    m = 4
    for p in range(0, 50):
        complete = sum(1 for i in range(100) if (i + 1) * m - 1 <= p)
        assert O.n_visible(p, m) == complete
    assert O.n_visible(2, 4) == 0 and O.n_visible(3, 4) == 1 and O.n_visible(131072, 4) == 32768


# ---------------------------------------------------------------------------------- top-k


def test_topk_hand_cases():
    for c in _gold("topk_hand.json")["cases"]:
        got = O.topk_select(np.array(c["scores"]), c["n_vis"], c["k"])
        assert got.tolist() == c["expected"], c


def _check_topk_properties(s, nv, k, idx):
    sel = idx[idx >= 0]
    assert sel.size == min(k, nv)
    assert np.all(np.diff(sel) > 0)                       # ascending, distinct
    assert np.all(idx[sel.size:] == -1)
    assert np.all(sel < nv)                               # causal: nothing invisible
    rest = np.setdiff1d(np.arange(nv), sel)
    if sel.size and rest.size:
        kth = s[sel].min()
        assert np.all(s[rest] <= kth)                     # everything kept beats everything left
        ties = rest[s[rest] == kth]
        tied_sel = sel[s[sel] == kth]
        assert ties.size == 0 or tied_sel.max() < ties.min()   # ties go to smaller indices


@pytest.mark.parametrize("seed", range(6))
def test_topk_properties_random_and_tied(seed):
    rng = np.random.default_rng(seed)
    N = 300
    s = rng.standard_normal(N) if seed % 2 else np.round(rng.standard_normal(N) * 2) / 2
    if seed == 4:
        s[:] = 0.0
        s[::7] = -0.0
    for nv in (0, 1, 17, 150, 300):
        for k in (1, 16, 64, 400):
            _check_topk_properties(s, nv, k, O.topk_select(s, nv, k))


def test_topk_all_equal_takes_first_k():
    assert O.topk_select(np.zeros(50), 50, 8).tolist() == list(range(8))


# ---------------------------------------------------------------------------------- attention


def test_attention_hand_example():
    g = _gold("attention_hand.json")
    q = np.array(g["q"])
    o = O.sparse_attention(q, np.array(g["entries"]), np.array(g["idx"]), np.array(g["raw"]), 0,
                           [g["p"]], g["W"])
    np.testing.assert_allclose(o, g["expected_out"], atol=1e-12)
    o = O.sparse_attention(q, np.array(g["entries"]), np.array(g["idx"]), np.array(g["raw"]), 0,
                           [g["p"]], g["W"], sink=np.array(g["sink"]))
    np.testing.assert_allclose(o, g["expected_out_sink"], atol=1e-12)


def test_attention_dense_equivalence_with_sdpa():
    # With k >= N and W >= T the layer is masked dense attention over [entries ; raw tokens].
    rng = np.random.default_rng(10)
    T, H, D, m = 37, 3, 8, 4
    N = T // m
    q = _rand(rng, T, H, D)
    ent = _rand(rng, N, D)
    raw = _rand(rng, T, D)
    q_pos = np.arange(T)
    nv = O.n_visible(q_pos, m)
    idx = np.stack([O.topk_select(rng.standard_normal(N), nv[t], N) for t in range(T)])
    o = O.sparse_attention(q, ent, idx, raw, 0, q_pos, W=T)
    keys = torch.from_numpy(np.concatenate([ent, raw], axis=0))        # [N + T, D]
    mask = torch.zeros(T, N + T, dtype=torch.bool)
    for t in range(T):
        mask[t, :nv[t]] = True
        mask[t, N:N + t + 1] = True
    qq = torch.from_numpy(q).permute(1, 0, 2)                          # [H, T, D]
    kk = keys.unsqueeze(0).expand(H, -1, -1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk, attn_mask=mask)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_attention_window_only_returns_own_raw_row():
    rng = np.random.default_rng(11)
    T, H, D = 3, 2, 5                    # p < m - 1: no entries are visible yet
    q, raw = _rand(rng, T, H, D), _rand(rng, T, D)
    idx = np.full((T, 4), -1)
    o = O.sparse_attention(q, np.zeros((0, D)), idx, raw, 0, np.arange(T), W=1)
    for t in range(T):
        np.testing.assert_allclose(o[t], np.tile(raw[t], (H, 1)), atol=1e-15)


def test_attention_zero_query_is_uniform_mean():
    rng = np.random.default_rng(12)
    T, H, D = 1, 2, 6
    ent, raw = _rand(rng, 10, D), _rand(rng, 20, D)
    idx = np.array([[1, 4, 7, -1]])
    o = O.sparse_attention(np.zeros((T, H, D)), ent, idx, raw, 0, [15], W=5)
    want = np.concatenate([ent[[1, 4, 7]], raw[11:16]]).mean(axis=0)
    np.testing.assert_allclose(o[0], np.tile(want, (H, 1)), atol=1e-12)


def test_attention_sink_limits():
    rng = np.random.default_rng(13)
    q, ent, raw = _rand(rng, 2, 3, 4), _rand(rng, 8, 4), _rand(rng, 12, 4)
    idx = np.array([[0, 2, 5], [1, 3, -1]])
    base = O.sparse_attention(q, ent, idx, raw, 0, [9, 11], W=4)
    none = O.sparse_attention(q, ent, idx, raw, 0, [9, 11], W=4, sink=np.full(3, -np.inf))
    np.testing.assert_allclose(none, base, atol=1e-15)
    huge = O.sparse_attention(q, ent, idx, raw, 0, [9, 11], W=4, sink=np.full(3, 60.0))
    assert np.abs(huge).max() < 1e-20


# ---------------------------------------------------------------------------------- whole layer


def _tiny(**kw):
    return get("tiny").with_(**kw)


def test_prefill_dense_equivalence_end_to_end():
    wl = _tiny(T=64, k=64, W=64)
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    T, H, D, N = wl.T, wl.H, wl.D, r["entries"].shape[0]
    keys = torch.from_numpy(np.concatenate([r["entries"], r["raw"]], axis=0))
    mask = torch.zeros(T, N + T, dtype=torch.bool)
    for t in range(T):
        mask[t, :r["n_vis"][t]] = True
        mask[t, N:N + t + 1] = True
    qq = torch.from_numpy(r["q"]).permute(1, 0, 2)
    kk = keys.unsqueeze(0).expand(H, -1, -1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk, attn_mask=mask)
    np.testing.assert_allclose(r["out"], ref.permute(1, 0, 2).numpy(), atol=1e-12)


def _prefix_inputs_from_full(inp_full, wl_full, r_full, L):
    """Build chunked-prefill inputs whose context is the first L tokens of a full run."""
    wl = wl_full.with_(L=L, T=wl_full.T - L)
    m, D, DI = wl.m, wl.D, wl.D_I
    cols, _ = O.projection_columns(D, DI, wl.H, wl.H_I)
    p = r_full["parts"]
    inp = dict(inp_full)
    inp["x"] = inp_full["x"][:, L:]
    inp["entries_prefix"] = r_full["entries"][None, : L // m]
    inp["keys_prefix"] = r_full["keys"][None, : L // m]
    inp["win_prefix"] = p["kv"][None, L - (wl.W - 1):L]
    hb = slice(L - m, L)
    inp["halo"] = np.concatenate([p["cb"][hb], p["zb"][hb], p["icb"][hb], p["izb"][hb]], axis=1)[None]
    return wl, inp


def test_chunked_prefill_equals_one_shot():
    wl_full = _tiny(T=96)
    inp = G.make_inputs(wl_full)
    full = O.prefill(inp, wl_full)
    wl, inp2 = _prefix_inputs_from_full(inp, wl_full, full, L=48)
    part = O.prefill(inp2, wl)
    np.testing.assert_allclose(part["entries"], full["entries"], atol=1e-12)
    np.testing.assert_allclose(part["out"], full["out"][48:], atol=1e-12)
    np.testing.assert_array_equal(part["idx"], full["idx"][48:])


def test_decode_equals_prefill_of_the_last_token():
    wl_full = _tiny(T=97)                       # the last token sits at p = 96 = L
    inp = G.make_inputs(wl_full)
    full = O.prefill(inp, wl_full)
    L = 96
    wl = wl_full.with_(kind="decode", L=L, T=1, d=0)
    dec = {
        "entries": full["entries"][None, : L // 4],
        "keys": full["keys"][None, : L // 4],
        "kv_raw": full["parts"]["kv"][None, L - wl.W + 1:L + 1],
        "q": full["q"][None, L:L + 1],
        "q_idx": full["q_idx"][None, L:L + 1],
        "w_head": inp["w_head"],
    }
    wl = wl.with_(dtype="f32", idx_dtype="f32")
    r = O.decode(dec, wl, 0)
    np.testing.assert_array_equal(r["idx"][0], full["idx"][L])
    np.testing.assert_allclose(r["out"][0], full["out"][L], atol=1e-12)


def test_prefill_invariants_bf16_tiny():
    wl = _tiny(dtype="bf16", idx_dtype="bf16")
    inp = G.make_inputs(wl)
    r = O.prefill(inp, wl)
    # stored tensors sit on the bf16 grid
    for a in (r["entries"], r["keys"], r["q"], r["raw"]):
        np.testing.assert_array_equal(O.round_bf16(a), a)
    for t in range(wl.T):
        _check_topk_properties(r["scores"][t], r["n_vis"][t], wl.k, r["idx"][t])


# ---------------------------------------------------------------------------------- QK-norm, partial RoPE


def test_rms_norm_closed_forms():
    # hand-worked: x = (3, 4): mean of squares 12.5, so y = x / sqrt(12.5)
    np.testing.assert_allclose(O.rms_norm([3.0, 4.0], [1.0, 1.0], 0.0), [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)],
                               rtol=0, atol=1e-15)
    rng = np.random.default_rng(80)
    x = rng.standard_normal((5, 3, 64))
    y = O.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-13)        # unit RMS per head vector
    np.testing.assert_allclose(O.rms_norm(7.5 * x, np.ones(64), 0.0), y, atol=1e-13)   # scale invariance
    g = rng.uniform(0.5, 2.0, 64)
    np.testing.assert_allclose(O.rms_norm(x, g, 0.0), y * g, atol=1e-13)        # the gain is per dim
    assert np.all(O.rms_norm(np.zeros(8), np.ones(8), 1e-6) == 0)               # eps keeps zero finite
    np.testing.assert_allclose(O.rms_norm([1e-4] * 4, [1.0] * 4, 1e-6), [1e-4 / np.sqrt(1e-8 + 1e-6)] * 4, rtol=1e-14)


def test_rope_closed_forms():
    p = 3.0
    # pair 0 of the rotated slice turns at frequency 1: (1, 0) -> (cos p, sin p); other dims untouched
    y = O.rope([5.0, -2.0, 1.0, 0.0], p, 2, 10000.0)
    np.testing.assert_allclose(y, [5.0, -2.0, np.cos(p), np.sin(p)], atol=1e-15)
    # pair 1 of a 4-dim slice with theta = 100 turns at 100^(-1/2) = 0.1: (0, 1) -> (-sin, cos)
    y = O.rope([0.0, 0.0, 0.0, 1.0], p, 4, 100.0)
    np.testing.assert_allclose(y, [0.0, 0.0, -np.sin(0.1 * p), np.cos(0.1 * p)], atol=1e-15)
    # the rotation of each pair is the complex product (a + ib) e^{i angle}
    rng = np.random.default_rng(81)
    x = rng.standard_normal(512)
    pos = 123457.0
    y = O.rope(x, pos, 64, 10000.0)
    z = (x[448::2] + 1j * x[449::2]) * np.exp(1j * pos * 10000.0 ** (-np.arange(32) / 32.0))
    np.testing.assert_allclose(y[448::2], z.real, atol=1e-9)
    np.testing.assert_allclose(y[449::2], z.imag, atol=1e-9)
    np.testing.assert_array_equal(y[:448], x[:448])
    # norm preserved, position 0 is the identity, the inverse undoes it
    np.testing.assert_allclose(np.linalg.norm(y), np.linalg.norm(x), rtol=1e-14)
    np.testing.assert_array_equal(O.rope(x, 0.0, 64, 10000.0), x)
    np.testing.assert_allclose(O.rope(y, pos, 64, 10000.0, inverse=True), x, atol=1e-12)


def test_rope_logits_depend_on_relative_position_only():
    rng = np.random.default_rng(82)
    q, k = rng.standard_normal(512), rng.standard_normal(512)
    a = O.rope(q, 1000.0, 64, 10000.0) @ O.rope(k, 37.0, 64, 10000.0)
    b = O.rope(q, 1000.0 + 65536.0, 64, 10000.0) @ O.rope(k, 37.0 + 65536.0, 64, 10000.0)
    c = O.rope(q, 1001.0, 64, 10000.0) @ O.rope(k, 37.0, 64, 10000.0)
    assert abs(a - b) < 1e-9 and abs(a - c) > 1e-6


def test_rotated_attention_output_is_shift_invariant():
    # entries and raw KV rotated at their positions, queries at theirs, the output rotated back by the
    # query position: shifting every position by the same amount leaves the output unchanged, and
    # leaving out the back-rotation does not
    rng = np.random.default_rng(83)
    m, D, H, W, N, T = 4, 64, 3, 8, 40, 5
    q0, e0 = rng.standard_normal((T, H, D)), rng.standard_normal((N, D))
    idx = np.stack([np.sort(rng.choice(N, 12, replace=False)) for _ in range(T)])

    def run(shift, back=True):
        L = 4 * N + shift
        q_pos = L + np.arange(T)
        raw_pos0 = L - W + 1
        raw0 = np.random.default_rng(84).standard_normal((W - 1 + T, D))
        e = O.rope(e0, O.entry_positions(shift // m, N, m), 16, 10000.0)
        raw = O.rope(raw0, raw_pos0 + np.arange(len(raw0)), 16, 10000.0)
        q = O.rope(q0, q_pos, 16, 10000.0)
        out = O.sparse_attention(q, e, idx, raw, raw_pos0, q_pos, W)
        return O.rope(out, q_pos, 16, 10000.0, inverse=True) if back else out

    np.testing.assert_allclose(run(4 * 1000), run(0), atol=1e-12)
    assert np.abs(run(4 * 1000, back=False) - run(0, back=False)).max() > 1e-3


def _fid(D, seed=85, rope_dims=16):
    rng = np.random.default_rng(seed)
    return {"gamma_q": rng.uniform(0.5, 1.5, D), "gamma_kv": rng.uniform(0.5, 1.5, D), "eps": 1e-6,
            "rope_dims": rope_dims, "theta": 10000.0}


def test_fid_chunked_prefill_equals_one_shot():
    # positions of queries, raw KV and new entries follow the absolute token positions of the chunk
    wl_full = _tiny(T=96)
    fid = _fid(wl_full.D)
    inp = G.make_inputs(wl_full)
    full = O.prefill(inp, wl_full, fid=fid)
    wl, inp2 = _prefix_inputs_from_full(inp, wl_full, full, L=48)
    part = O.prefill(inp2, wl, fid=fid)
    np.testing.assert_allclose(part["entries"], full["entries"], atol=1e-12)
    np.testing.assert_allclose(part["out"], full["out"][48:], atol=1e-12)
    np.testing.assert_array_equal(part["idx"], full["idx"][48:])
    # the fid layer is not the plain one
    assert np.abs(O.prefill(inp, wl_full)["out"] - full["out"]).max() > 1e-3


def test_fid_decode_equals_prefill_of_the_last_token():
    wl_full = _tiny(T=97)
    fid = _fid(wl_full.D)
    inp = G.make_inputs(wl_full)
    full = O.prefill(inp, wl_full, fid=fid)
    L = 96
    wl = wl_full.with_(kind="decode", L=L, T=1, d=0, dtype="f32", idx_dtype="f32")
    cols, _ = O.projection_columns(wl.D, wl.D_I, wl.H, wl.H_I)
    x = np.asarray(inp["x"][0], dtype=np.float64)
    lo, hi = cols["q"]
    q_raw = (x[L:L + 1] @ np.asarray(inp["W"], dtype=np.float64)[lo:hi].T).reshape(1, wl.H, wl.D)
    dec = {
        "entries": full["entries"][None, : L // 4],
        "keys": full["keys"][None, : L // 4],
        "kv_raw": full["parts"]["kv"][None, L - wl.W + 1:L + 1],
        "q": q_raw[None],                         # before the norm: decode normalises and rotates it
        "q_idx": full["q_idx"][None, L:L + 1],
        "w_head": inp["w_head"],
    }
    r = O.decode(dec, wl, 0, fid=fid)
    np.testing.assert_allclose(r["q"][0], full["q"][L], atol=1e-12)
    np.testing.assert_array_equal(r["idx"][0], full["idx"][L])
    np.testing.assert_allclose(r["out"][0], full["out"][L], atol=1e-12)


# ---------------------------------------------------------------------------------- FP8 entry records


def test_e4m3_table_closed_forms():
    dec = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    # spot values from the E4M3 definition
    assert dec[0x00] == 0.0 and dec[0x01] == 2.0 ** -9 and dec[0x07] == 7 * 2.0 ** -9
    assert dec[0x08] == 2.0 ** -6 and dec[0x38] == 1.0 and dec[0x3C] == 1.5 and dec[0x7E] == 448.0
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    np.testing.assert_array_equal(dec[0x80:0xFF], -dec[0x00:0x7F])
    assert np.all(np.diff(dec[:0x7F]) > 0)                  # codes 0x00..0x7E ascend
    # each binade of a normal exponent holds 8 evenly spaced values
    for e in range(1, 15):
        v = dec[8 * e:8 * e + 8]
        np.testing.assert_allclose(np.diff(v), 2.0 ** (e - 10), rtol=0)


def test_e4m3_encode_rounding():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_decode(finite)
    np.testing.assert_array_equal(O.e4m3_encode(vals), finite)           # every value encodes to its code
    # midpoints go to the even code, the rest to the nearest
    assert O.e4m3_encode(np.array([1.0625]))[0] == 0x38                  # between 1.0 (0x38) and 1.125
    assert O.e4m3_encode(np.array([1.1875]))[0] == 0x3A                  # between 1.125 and 1.25 (0x3A)
    assert O.e4m3_encode(np.array([1.0625 + 1e-9]))[0] == 0x39
    assert O.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00              # half the smallest subnormal
    assert O.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02          # 1.5 subnormal steps -> even
    assert O.e4m3_encode(np.array([500.0, -1e9]))[0] == 0x7E and O.e4m3_encode(np.array([-1e9]))[0] == 0xFE
    assert O.e4m3_encode(np.array([-0.0]))[0] == 0x80
    # brute force: the nearest finite value, ties to the even code
    rng = np.random.default_rng(86)
    x = np.concatenate([rng.standard_normal(4000) * 50, rng.standard_normal(1000) * 0.01])
    got = O.e4m3_decode(O.e4m3_encode(x))
    pos = vals[vals >= 0][:127]
    for xi, gi in zip(x, got):
        d = np.abs(pos - min(abs(xi), 448.0))
        best = pos[d == d.min()]
        assert abs(gi) in best


def test_entry_record_golden():
    g = _gold("entry_fp8_record.json")
    e = np.zeros(512)
    for k, v in g["nonzero_dims"].items():
        e[int(k)] = v
    e[448:] = g["rope_dims_value"]
    r = O.entry_pack(e)
    assert r.shape == (584,)
    for k, v in g["expected_bytes"].items():
        assert r[int(k)] == v, k
    assert list(r[448:452]) == g["expected_rope_bytes_first4"]
    assert list(r[576:584]) == g["expected_scales_and_pad"]
    np.testing.assert_array_equal(O.entry_unpack(r), e)                  # these values are exact in the format


def test_entry_record_error_bound_and_scale_choice():
    rng = np.random.default_rng(87)
    e = O.round_bf16(O.rms_norm(rng.standard_normal((50, 512)) * rng.uniform(0.01, 100, (50, 1)), np.ones(512), 0))
    r = O.entry_pack(e)
    u = O.entry_unpack(r)
    np.testing.assert_array_equal(u[:, 448:], e[:, 448:])                # RoPE dims kept in bf16
    E = r[:, 576:583].astype(np.int64)
    s = np.ldexp(1.0, E - 127)                                           # [50, 7]
    amax = np.abs(e[:, :448]).reshape(50, 7, 64).max(axis=-1)
    assert np.all(amax / s <= 448) and np.all(amax / (s / 2) > 448)      # the smallest such power of two
    x = e[:, :448].reshape(50, 7, 64) / s[..., None]
    err = np.abs(u[:, :448].reshape(50, 7, 64) / s[..., None] - x)
    binade = np.floor(np.log2(np.maximum(np.abs(x), 1e-300)))
    half_ulp = np.where(np.abs(x) >= 2.0 ** -6, 2.0 ** (binade - 4), 2.0 ** -10)
    assert np.all(err <= half_ulp * (1 + 1e-12))
    assert np.all(r[:, 583] == 0)


def test_entry_rotation_position_is_the_last_token_of_its_block():
    # reading: entry i turns at the position of its block's last token, (i+1)m - 1, so a query on
    # that token meets the entry at relative distance 0 (m = 4: entries 0, 1, 2 at 3, 7, 11)
    assert list(O.entry_positions(0, 3, 4)) == [3, 7, 11]
    assert list(O.entry_positions(5, 2, 128)) == [767, 895]
    rng = np.random.default_rng(88)
    v = rng.standard_normal(64)
    q = O.rope(v, 7.0, 16, 10000.0)
    e = O.rope(v, O.entry_positions(1, 1, 4)[0], 16, 10000.0)
    assert abs(q @ e - v @ v) < 1e-9                       # rotations cancel at distance 0
    assert abs(q @ O.rope(v, 4.0, 16, 10000.0) - v @ v) > 1e-3
