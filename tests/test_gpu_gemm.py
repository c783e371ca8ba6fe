"""GPU parity of the layer's fused input projection on the library's own kernels (csa_projection_gemm:
the 128 x 128-tile matrix-core kernel for aligned bf16 operands, the one-output-per-thread kernel
otherwise), the GEMM csa_forward runs when hipBLASLt declines a shape. The reference is the float64
product of the same stored inputs; the bound is fp32 accumulation over K plus the output rounding."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_05_amd import lib
from synth.torch_io import to_device
from tests.csa_testlib import G, O, tensor_f64

pytestmark = pytest.mark.gpu


def _operand(seed, name, shape, dtype, scale):
    x = G.normal_f32(seed, name, shape) * np.float32(scale)
    if dtype == "bf16":
        bits = G.f32_to_bf16_bits(x)
        return to_device(bits, "bf16"), O.bf16_bits_to_f64(bits)
    return to_device(x, "f32"), x.astype(np.float64)


# (in, out, M, N, K): tile grids that are and are not a multiple of the 8 XCDs, ragged M / N edges,
# K not a multiple of the 64-deep K step (scalar kernel), and float32 operands
@pytest.mark.parametrize("din,dout,M,N,K", [("bf16", "bf16", 384, 1024, 1024), ("bf16", "bf16", 300, 392, 512),
                                           ("bf16", "f32", 129, 1000, 4096), ("bf16", "f32", 1, 128, 64),
                                           ("bf16", "bf16", 65, 130, 96), ("f32", "f32", 33, 70, 100),
                                           ("f32", "bf16", 17, 256, 64)])
def test_projection_gemm_matches_float64_product(din, dout, M, N, K):
    a, a64 = _operand(70, "gemm_a", (M, K), din, 1.0)
    w, w64 = _operand(71, "gemm_w", (N, K), din, 1.0 / np.sqrt(K))
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16 if dout == "bf16" else torch.float32, device="cuda")
    lib.csa_projection_gemm(a, w, c)
    torch.cuda.synchronize()
    got = tensor_f64(c)
    ref = a64 @ w64.T
    mag = np.abs(a64) @ np.abs(w64).T
    tol = 3e-5 * mag + (2.0 ** -8 * np.abs(ref) if dout == "bf16" else 0.0)
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))


def test_projection_gemm_strided_rows_and_rejections():
    # row strides above the row length (a view into wider buffers) take the same kernels
    M, N, K = 200, 256, 128
    abuf, a64 = _operand(72, "gemm_sa", (M, K + 64), "bf16", 1.0)
    wbuf, w64 = _operand(73, "gemm_sw", (N, K + 8), "bf16", 1.0 / np.sqrt(K))
    cbuf = torch.zeros(M, N + 32, dtype=torch.float32, device="cuda")
    lib.csa_projection_gemm(abuf[:, :K], wbuf[:, :K], cbuf[:, :N])
    torch.cuda.synchronize()
    ref = a64[:, :K] @ w64[:, :K].T
    got = tensor_f64(cbuf)
    assert np.all(np.abs(got[:, :N] - ref) <= 3e-5 * (np.abs(a64[:, :K]) @ np.abs(w64[:, :K]).T))
    assert np.all(got[:, N:] == 0.0)  # nothing written past the rows
    # a row stride below the row length is refused before any launch
    rc = lib.load().csa_projection_gemm(M, N, K, lib.CSA_BF16, abuf.data_ptr(), K - 1, wbuf.data_ptr(), K + 8,
                                        cbuf.data_ptr(), N + 32, lib.CSA_F32, None)
    assert rc == -1  # CSA_ERR_ARG
