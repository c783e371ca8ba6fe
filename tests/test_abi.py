"""Host-side checks of the C ABI: the library loads, exports every declared entry point, sizes its
workspaces and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from compressed_sparse_attention_05_amd import layer, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="csa.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_steps_and_helpers():
    names = _declared()
    for n in ("csa_compress", "csa_index_topk", "csa_topk_from_scores", "csa_sparse_attn", "csa_forward",
              "csa_workspace_size", "csa_last_error", "csa_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = lib.load()
    for n in _declared():
        assert hasattr(L, n), n
    assert set(lib.EXPORTS) == set(_declared())
    assert lib.csa_version() == 3
    # the ceiling probes of include/csa_probe.h
    for n in _declared("csa_probe.h"):
        assert hasattr(L, n), n
    assert set(lib.PROBE_EXPORTS) == set(_declared("csa_probe.h"))
    assert os.listdir(os.path.join(ROOT, "include")) and \
        sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == ["csa.h", "csa_probe.h"]


def _d(**kw):
    base = dict(m=4, D=512, H=64, H_I=64, D_I=128, top_k=512, window=128)
    base.update(kw)
    return lib.make_dims(**base)


def test_workspace_sizes():
    d = _d()
    assert lib.csa_workspace_size(lib.CSA_OP_COMPRESS, d, 1, 8192, 2048) == 0
    assert lib.csa_workspace_size(lib.CSA_OP_SPARSE_ATTN, d, 1, 8192, 2048) == 0
    # prefill (many rows per sequence): fused streaming selection, no score matrix
    assert lib.csa_workspace_size(lib.CSA_OP_INDEX_TOPK, d, 1, 8192, 2048) == 0
    # decode: scores of every (row, entry) pass through the workspace
    nb = lib.csa_workspace_size(lib.CSA_OP_INDEX_TOPK, _d(top_k=1024), 64, 1, 32768)
    assert nb >= 64 * 32768 * 4
    # MXFP4 prefill is fused too; MXFP4 decode rows pass their scores through the workspace
    assert lib.csa_workspace_size(lib.CSA_OP_INDEX_TOPK, d, 1, 8192, 2048, 0, lib.CSA_MXFP4) == 0
    assert lib.csa_workspace_size(lib.CSA_OP_INDEX_TOPK, _d(top_k=1024), 4, 1, 262144, 0,
                                  lib.CSA_MXFP4) >= 4 * 262144 * 4
    fw = lib.csa_workspace_size(lib.CSA_OP_FORWARD, d, 1, 8192, 2048, 4096)
    n_tot = 4 * 512 + 4 * 128 + 64 * 512 + 64 * 128 + 512
    assert fw >= 8192 * n_tot * 2 + 8192 * 512 * 4


def _err(rc):
    return rc, lib.load().csa_last_error().decode()


def test_compress_rejects_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    pos = ctypes.c_void_p(4096)  # a device position array (8-byte aligned)
    # per-sequence positions without the previous block
    rc, msg = _err(L.csa_compress(1, 8, pos, 4, 16, lib.CSA_BF16, p, p, p, p, 16, 128, None, None, 0, 0, p, p, p,
                                  64, 8, lib.CSA_BF16, None))
    assert rc == -1 and "halo" in msg
    # a misaligned position array
    rc, msg = _err(L.csa_compress(1, 8, ctypes.c_void_p(4100), 4, 16, lib.CSA_BF16, p, p, p, p, 16, 128, p, p, 16,
                                  64, p, p, p, 64, 8, lib.CSA_BF16, None))
    assert rc == -1 and "aligned" in msg
    # entries beyond capacity (every sequence at 0)
    rc, msg = _err(L.csa_compress(1, 64, None, 4, 16, lib.CSA_BF16, p, p, p, p, 16, 1024, None, None, 0, 0, p, p, p,
                                  64, 8, lib.CSA_BF16, None))
    assert rc == -1 and "n_cap" in msg
    # bad dtype
    rc, _ = _err(L.csa_compress(1, 8, None, 4, 16, 7, p, p, p, p, 16, 128, None, None, 0, 0, p, p, p, 64, 8,
                                lib.CSA_BF16, None))
    assert rc == -1
    # nothing to do is fine
    assert L.csa_compress(1, 3, None, 4, 16, lib.CSA_BF16, p, p, p, p, 16, 128, None, None, 0, 0, p, p, p, 64, 8,
                          lib.CSA_BF16, None) == 0


def test_index_topk_rejects_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(256)
    d = _d()
    rc, msg = _err(L.csa_index_topk(ctypes.byref(_d(top_k=0)), 1, 8, None, lib.CSA_BF16, p, 8192, 65536, None, p, 0,
                                    p, 262144, None, 2048, p, None, None, 0, None))
    assert rc == -1 and "top_k" in msg
    rc, msg = _err(L.csa_index_topk(ctypes.byref(d), 1, 8, None, lib.CSA_MXFP4, p, 0, 0, None, p, 0, p, 0, None,
                                    2048, p, None, None, 0, None))
    assert rc == -1 and "scale" in msg
    # MXFP4 key scales are read four bytes at a time
    rc, msg = _err(L.csa_index_topk(ctypes.byref(d), 1, 8, None, lib.CSA_MXFP4, p, 0, 0, p, p, 0, p, 0,
                                    ctypes.c_void_p(258), 2048, p, None, None, 0, None))
    assert rc == -1 and "4-byte aligned" in msg
    rc, msg = _err(L.csa_index_topk(ctypes.byref(d), 1, 8, None, lib.CSA_BF16, p, 100, 800, None, p, 0, p, 262144,
                                    None, 2048, p, None, None, 0, None))
    assert rc == -1 and "q_ld" in msg
    # decode shape needs a workspace
    rc, msg = _err(L.csa_index_topk(ctypes.byref(d), 64, 1, ctypes.c_void_p(4096), lib.CSA_BF16, ctypes.c_void_p(4096), 8192,
                                    8192, None, p, 0, ctypes.c_void_p(4096), 32768 * 128, None, 32768, p, None,
                                    None, 0, None))
    assert rc == -3 and "workspace" in msg


def test_sparse_attn_rejects_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(4096)
    d = _d()
    # no raw row at all (the window always holds the query's own token)
    rc, msg = _err(L.csa_sparse_attn(ctypes.byref(d), 1, 16, p, lib.CSA_BF16, p, 32768, 0, p, 0, 256, p, p, 512,
                                     0, p, 0, None, p, lib.CSA_F32, None, 0, None))
    assert rc == -1 and "row" in msg
    # misaligned position arrays
    rc, msg = _err(L.csa_sparse_attn(ctypes.byref(d), 1, 16, ctypes.c_void_p(4100), lib.CSA_BF16, p, 32768, 0, p, 0,
                                     256, p, p, 512, 0, p, 200, None, p, lib.CSA_F32, None, 0, None))
    assert rc == -1 and "aligned" in msg
    # q rows shorter than H*D
    rc, msg = _err(L.csa_sparse_attn(ctypes.byref(d), 1, 16, p, lib.CSA_BF16, p, 100, 0, p, 0, 256, p, p, 512,
                                     0, p, 200, None, p, lib.CSA_F32, None, 0, None))
    assert rc == -1 and "q_ld" in msg


def test_topk_from_scores_rejects_bad_k():
    L = lib.load()
    p = ctypes.c_void_p(256)
    rc, _ = _err(L.csa_topk_from_scores(p, 100, p, 4, 0, p, None, None, 0, None))
    assert rc == -1
    rc, _ = _err(L.csa_topk_from_scores(p, 100, p, 4, 5000, p, None, None, 0, None))
    assert rc == -1
    assert L.csa_topk_from_scores(p, 100, p, 0, 4, p, None, None, 0, None) == 0


def test_forward_rejects_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(4096)
    d = _d()
    w = lib.Weights(4096, 4096, 4096, 4096, 4096, 4096, None)
    # every sequence at 0 and more blocks than entry slots
    c = lib.Cache(4096, 4096, 100, 4096, 9000, None, None)
    rc, msg = _err(L.csa_forward(ctypes.byref(d), ctypes.byref(w), 1, 8192, None, 4096, lib.CSA_BF16, p,
                                 ctypes.byref(c), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "n_cap" in msg
    # per-sequence positions without the previous block
    c = lib.Cache(4096, 4096, 4000, 4096, 9000, None, None)
    rc, msg = _err(L.csa_forward(ctypes.byref(d), ctypes.byref(w), 1, 8192, p, 4096, lib.CSA_BF16, p,
                                 ctypes.byref(c), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "halo" in msg
    # the window rows do not fit
    c = lib.Cache(4096, 4096, 4000, 4096, 1000, None, None)
    rc, msg = _err(L.csa_forward(ctypes.byref(d), ctypes.byref(w), 1, 8192, None, 4096, lib.CSA_BF16, p,
                                 ctypes.byref(c), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "win_cap" in msg


def test_norm_rope_entry_pack_and_fp8_attention_reject_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(4096)
    # odd rope_dims, rope_dims beyond D, a norm on the inverse rotation, D beyond the kernel's limit
    for args in ((1, 2, 3, 8, lib.CSA_F32, p, 24, 48, p, 24, 48, None, 0.0, 3, 10000.0, None, 0, 1, 0, None),
                 (1, 2, 3, 8, lib.CSA_F32, p, 24, 48, p, 24, 48, None, 0.0, 10, 10000.0, None, 0, 1, 0, None),
                 (1, 2, 3, 8, lib.CSA_F32, p, 24, 48, p, 24, 48, p, 0.0, 4, 10000.0, None, 0, 1, 1, None),
                 (1, 2, 1, 8192, lib.CSA_F32, p, 8192, 16384, p, 8192, 16384, None, 0.0, 0, 10000.0, None, 0, 1, 0,
                  None),
                 (1, 2, 3, 8, lib.CSA_F32, p, 8, 48, p, 24, 48, None, 0.0, 4, 10000.0, None, 0, 1, 0, None),
                 (1, 2, 3, 8, lib.CSA_F32, p, 24, 48, p, 24, 48, None, 0.0, 4, 10000.0, ctypes.c_void_p(4100), 0, 1, 0,
                  None)):
        rc, _ = _err(L.csa_norm_rope(*args))
        assert rc == -1, args
    assert L.csa_norm_rope(0, 2, 3, 8, lib.CSA_F32, None, 24, 48, None, 24, 48, None, 0.0, 4, 10000.0, None, 0, 1,
                           0, None) == 0
    # records: misaligned, short sequence stride, bad dtype
    rc, msg = _err(L.csa_entry_pack(2, 4, lib.CSA_BF16, p, 512, 2048, ctypes.c_void_p(4100), 4 * 584, None))
    assert rc == -1 and "align" in msg
    rc, msg = _err(L.csa_entry_pack(2, 4, lib.CSA_BF16, p, 512, 2048, p, 100, None))
    assert rc == -1 and "stride" in msg
    rc, _ = _err(L.csa_entry_pack(2, 4, lib.CSA_MXFP4, p, 512, 2048, p, 4 * 584, None))
    assert rc == -1
    # attention over records needs D = 512 and a byte stride of whole records
    d = _d(D=256)
    rc, msg = _err(L.csa_sparse_attn_fp8(ctypes.byref(d), 1, 1, p, lib.CSA_BF16, p, 64 * 256, 0, p, 0, 256, p,
                                         p, 256, 0, p, 128, None, p, lib.CSA_F32, None, 0, None))
    assert rc == -1 and "512" in msg


def test_decode_step_rejects_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(4096)
    d = _d(H=128, top_k=1024)
    w = lib.Weights(None, 4096, 4096, 4096, 4096, 4096, None, None, None, 0.0, 0, 10000.0)
    st = lib.DecodeState(4096, 0, 4096, 100, 4096, 4096)
    # the positions are required (each sequence decodes at its own)
    rc, msg = _err(L.csa_decode_step(ctypes.byref(d), ctypes.byref(w), 2, None, lib.CSA_BF16, p, p, p, p,
                                     ctypes.byref(st), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "pos" in msg
    # MXFP4 is not an activation dtype
    rc, _ = _err(L.csa_decode_step(ctypes.byref(d), ctypes.byref(w), 2, p, lib.CSA_MXFP4, p, p, p, p,
                                   ctypes.byref(st), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1
    # records need D = 512
    st2 = lib.DecodeState(4096, 1, 4096, 100, 4096, 4096)
    d2 = _d(D=256, H=128, top_k=1024)
    rc, msg = _err(L.csa_decode_step(ctypes.byref(d2), ctypes.byref(w), 2, p, lib.CSA_BF16, p, p, p, p,
                                     ctypes.byref(st2), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "512" in msg
    # no workspace
    rc, msg = _err(L.csa_decode_step(ctypes.byref(d), ctypes.byref(w), 2, p, lib.CSA_BF16, p, p, p, p,
                                     ctypes.byref(st), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -3 and "workspace" in msg
    assert lib.csa_workspace_size(lib.CSA_OP_DECODE_STEP, d, 2, 1, 100, 0, lib.CSA_BF16) > 0


def test_decode_step_noalloc_rejects_a_step_beyond_its_scratch():
    # checked on the host before any HIP call: 64 sequences over 2M entry slots need more scratch than
    # the library holds (their scores alone are 512 MiB)
    L = lib.load()
    p = ctypes.c_void_p(4096)
    d = _d(H=128, top_k=1024)
    w = lib.Weights(None, 4096, 4096, 4096, 4096, 4096, None, None, None, 0.0, 0, 10000.0)
    st = lib.DecodeState(4096, 0, 4096, 1 << 21, 4096, 4096)
    need = lib.csa_workspace_size(lib.CSA_OP_DECODE_STEP, d, 64, 1, 1 << 21, 0, lib.CSA_BF16)
    assert need > lib.STATIC_SCRATCH_BYTES
    rc, msg = _err(L.csa_decode_step_noalloc(ctypes.byref(d), ctypes.byref(w), 64, p, lib.CSA_BF16, p, p, p, p,
                                             ctypes.byref(st), p, lib.CSA_F32, None, None))
    assert rc == -3 and "scratch" in msg
    # the decode128k batch fits
    assert lib.csa_workspace_size(lib.CSA_OP_DECODE_STEP, d, 64, 1, 32768, 0, lib.CSA_BF16) <= lib.STATIC_SCRATCH_BYTES


def test_mxfp4_quantize_rejects_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(4096)
    for args, what in (((4, 48, lib.CSA_BF16, p, 48, p, p, None), "multiple of 32"),
                       ((4, 64, lib.CSA_BF16, p, 32, p, p, None), "ld"),
                       ((4, 64, lib.CSA_MXFP4, p, 64, p, p, None), "dtype"),
                       ((4, 64, lib.CSA_BF16, p, 64, ctypes.c_void_p(4098), p, None), "align"),
                       ((4, 64, lib.CSA_BF16, None, 64, p, p, None), "NULL")):
        rc, msg = _err(L.csa_mxfp4_quantize(*args))
        assert rc == -1 and what in msg, (args, msg)
    assert L.csa_mxfp4_quantize(0, 64, lib.CSA_BF16, None, 64, None, None, None) == 0


def test_mxfp4_key_caches_need_their_scales():
    L = lib.load()
    p = ctypes.c_void_p(4096)
    d = _d()
    w = lib.Weights(4096, 4096, 4096, 4096, 4096, 4096, None)
    c = lib.Cache(4096, 4096, 4000, 4096, 9000, None, None, 0, 1, None)
    rc, msg = _err(L.csa_forward(ctypes.byref(d), ctypes.byref(w), 1, 8192, None, 4096, lib.CSA_BF16, p,
                                 ctypes.byref(c), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "key_scales" in msg
    c = lib.Cache(4096, 4096, 4000, 4096, 9000, None, None, 0, 2, p)
    rc, msg = _err(L.csa_forward(ctypes.byref(d), ctypes.byref(w), 1, 8192, None, 4096, lib.CSA_BF16, p,
                                 ctypes.byref(c), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "key_fmt" in msg
    d = _d(H=128, top_k=1024)
    wd = lib.Weights(None, 4096, 4096, 4096, 4096, 4096, None, None, None, 0.0, 0, 10000.0)
    st = lib.DecodeState(4096, 0, 4096, 100, 4096, 4096, 1, None)
    rc, msg = _err(L.csa_decode_step(ctypes.byref(d), ctypes.byref(wd), 2, p, lib.CSA_BF16, p, p, p, p,
                                     ctypes.byref(st), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "key_scales" in msg
    st = lib.DecodeState(4096, 0, ctypes.c_void_p(4104), 100, 4096, 4096, 1, p)
    rc, msg = _err(L.csa_decode_step(ctypes.byref(d), ctypes.byref(wd), 2, p, lib.CSA_BF16, p, p, p, p,
                                     ctypes.byref(st), p, lib.CSA_F32, None, None, 0, None))
    assert rc == -1 and "aligned" in msg


def test_probes_reject_bad_arguments():
    L = lib.load()
    rc, msg = _err(L.csa_probe_hbm_read(ctypes.c_void_p(4100), 4096, ctypes.c_void_p(4096), None))
    assert rc == -1 and "aligned" in msg
    rc, msg = _err(L.csa_probe_mfma_bf16(0, ctypes.c_void_p(4096), None))
    assert rc == -1 and "iters" in msg
    p = ctypes.c_void_p(4096)
    for args in ((p, 1 << 20, 1000, p, 8, p), (p, 512, 1024, p, 8, p), (ctypes.c_void_p(4104), 1 << 20, 1024, p, 8, p),
                 (p, 1 << 20, 1024, ctypes.c_void_p(4098), 8, p), (p, 1 << 20, 1024, p, -1, p)):
        rc, msg = _err(L.csa_probe_gather_read(*args, None))
        assert rc == -1 and "gather" in msg, args
    assert L.csa_probe_gather_read(p, 1 << 20, 1024, p, 0, p, None) == 0  # nothing to read: no launch


def test_projection_gemm_rejects_bad_arguments():
    L = lib.load()
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rc, msg = _err(L.csa_projection_gemm(-1, 8, 64, lib.CSA_BF16, p, 64, p, 64, p, 8, lib.CSA_BF16, None))
    assert rc == -1 and ">= 0" in msg
    rc, msg = _err(L.csa_projection_gemm(4, 8, 64, lib.CSA_MXFP4, p, 64, p, 64, p, 8, lib.CSA_BF16, None))
    assert rc == -1 and "dtype" in msg
    rc, msg = _err(L.csa_projection_gemm(4, 8, 64, lib.CSA_BF16, p, 64, p, 63, p, 8, lib.CSA_BF16, None))
    assert rc == -1 and "stride" in msg
    rc, msg = _err(L.csa_projection_gemm(4, 8, 64, lib.CSA_BF16, None, 64, p, 64, p, 8, lib.CSA_F32, None))
    assert rc == -1 and "NULL" in msg
    assert L.csa_projection_gemm(0, 8, 64, lib.CSA_BF16, None, 64, None, 64, None, 8, lib.CSA_F32, None) == 0


def test_sparse_attn_qk_rejects_bad_arguments():
    L = lib.load()
    d = layer.dims(4, 512, 128, 64, 128, 1024, 128)
    p = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    args = lambda w: (ctypes.byref(d), w, 1, 1, p, lib.CSA_BF16, p, 128 * 512, 128 * 512, p, 1024 * 512, 1024, p, p,
                      512, 128 * 512, p, 128, p, lib.CSA_F32, None, 0, None)
    rc, msg = _err(L.csa_sparse_attn_qk(*args(None)))
    assert rc == -1 and "weights" in msg
    w = lib.Weights(None, None, None, None, None, None, None, None, None, 1e-6, 63, 10000.0)
    rc, msg = _err(L.csa_sparse_attn_qk(*args(ctypes.byref(w))))
    assert rc == -1 and "rope_dims" in msg
    w = lib.Weights(None, None, None, None, None, None, None, None, None, 1e-6, 64, 0.0)
    rc, msg = _err(L.csa_sparse_attn_qk(*args(ctypes.byref(w))))
    assert rc == -1 and "rope_theta" in msg
