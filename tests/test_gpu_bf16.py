"""GPU parity of the bfloat16 variant (W4A16_BF16: bf16 activations, scales,
outputs; weight RNE_bf16((q - z) * s)) against the CPU oracle's bf16 mode.

Bit-exact: dequant (over every finite bf16 scale and every (q, z)) and Y on
the exact-arithmetic family, through both GEMM kernels.  Y elsewhere within
|y - y_ref| <= 2^-7 ||x_m|| ||w_n|| + ulp_bf16(y_ref), element by element,
including K split across workgroups and the benchmark's full sizes on
sampled rows.  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_int4_02_amd as w4
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PATHS = ("small_m", "large_m")


def bf(bits):
    """bf16 bit patterns (uint16 numpy) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_weight(c):
    partial = c.K % c.g != 0
    return w4.quantized_weight(torch.from_numpy(c.codes).cuda(), bf(c.scales),
                               None if c.symmetric else torch.from_numpy(c.zeros).cuda(), c.g,
                               partial=partial)


def oracle_y(c, rows=None):
    return oracle.gemm_rows_bf16(c.X, oracle.pack(c.codes), c.scales,
                                 None if c.symmetric else oracle.pack(c.zeros), c.K, c.g,
                                 c.symmetric, rows=rows)


def assert_close(y_bits, c, rows=None, what=""):
    y_ref, wn2 = oracle_y(c, rows)
    yg = y_bits if rows is None else y_bits[:, rows]
    ok, worst = oracle.check_y_bf16(yg, c.X, y_ref, wn2)
    assert ok, f"{what}: worst |err|/bound = {worst:.3f}"


def test_bf16_dequant_exhaustive_scales():
    """Every finite bf16 scale x every (q, z): row n has zero n, column k code
    k % 16, group j the j-th finite scale."""
    b = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (b << 16).view(np.float32)
    sb = b[np.isfinite(v)].astype(np.uint16)
    G, N, g = sb.size, 16, 32
    K = G * g
    codes = np.tile((np.arange(K) % 16).astype(np.uint8), (N, 1))
    zeros = np.repeat(np.arange(N, dtype=np.uint8)[:, None], G, 1)
    scales = np.tile(sb, (N, 1))
    qp, zp = oracle.pack(codes), oracle.pack(zeros)
    W = w4.dequant(torch.from_numpy(qp.view(np.int32)).cuda(), bf(scales),
                   torch.from_numpy(zp.view(np.int32)).cuda(), K, g)
    assert W.dtype == torch.bfloat16
    assert np.array_equal(bits(W), oracle.dequant_bf16(qp, scales, zp, K, g, False))


@pytest.mark.parametrize("N,K,g,sym", [(512, 512, 128, False), (288, 288, 256, False),
                                       (40, 136, 32, True), (33, 4096, 64, False)])
def test_bf16_dequant_bit_exact(N, K, g, sym):
    c = workloads.draw_bf16(1, N, K, g, sym, seed=N + K + g)
    qp = oracle.pack(c.codes)
    zp = None if sym else oracle.pack(c.zeros)
    W = w4.dequant(torch.from_numpy(qp.view(np.int32)).cuda(), bf(c.scales),
                   None if sym else torch.from_numpy(zp.view(np.int32)).cuda(), K, g,
                   symmetric=sym, partial=K % g != 0)
    assert np.array_equal(bits(W), oracle.dequant_bf16(qp, c.scales, zp, K, g, sym))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,N,K,g,sym", [
    (1, 288, 288, 256, False), (7, 288, 288, 256, True), (33, 288, 288, 256, False),
    (1, 40, 136, 32, False), (5, 300, 520, 64, False), (16, 48, 4096, 128, False),
    (17, 64, 1024, 128, True), (130, 136, 392, 32, False), (257, 512, 1024, 256, False)])
def test_bf16_gemm_small_shapes(path, M, N, K, g, sym):
    c = workloads.draw_bf16(M, N, K, g, sym, seed=M * 131 + N * 7 + K + g)
    y = w4.gemm(bf(c.X), gpu_weight(c), path=path)
    assert y.dtype == torch.bfloat16
    assert_close(bits(y), c, what=f"{path} M{M} N{N} K{K} g{g}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,N,K,g,sym", [
    (4, 512, 512, 128, False), (33, 288, 288, 256, True), (7, 1024, 4096, 32, False),
    (16, 160, 11008, 256, False), (130, 200, 1032, 64, False), (2, 64, 28672, 128, False)])
def test_bf16_gemm_exact_family_bit_exact(path, M, N, K, g, sym):
    c = workloads.exact_family_bf16(M, N, K, g, sym, seed=M + N + K)
    y = w4.gemm(bf(c.X), gpu_weight(c), path=path)
    y_exact, _ = oracle_y(c)
    want = np.array([oracle.f64_to_bf16_bits(float(v)) for v in y_exact.ravel()],
                    np.uint16).reshape(y_exact.shape)
    assert np.array_equal(bits(y), want)


@pytest.mark.parametrize("M,N,K,g,sym", [(520, 4112, 1024, 32, False), (520, 4112, 1024, 128, True),
                                         (2048, 4096, 4096, 128, False),
                                         (1000, 9000, 1024, 128, False)])
def test_bf16_large_m_tiles_exact_family(M, N, K, g, sym):
    """The large-M kernel at its 128 x 256 tile (M = 2048), at g = 32, at the
    128 x 128 tile (M = 520, g = 128) and at the 128 x 384 tile (M = 1000,
    N = 9000), bit-exact on sampled rows of the exact family."""
    c = workloads.exact_family_bf16(M, N, K, g, sym, seed=M + N + K + g)
    y = bits(w4.gemm(bf(c.X), gpu_weight(c), path="large_m"))
    rng = np.random.default_rng(N + g)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 24, replace=False)]))
    y_exact, _ = oracle_y(c, rows)
    want = np.array([oracle.f64_to_bf16_bits(float(v)) for v in y_exact.ravel()],
                    np.uint16).reshape(y_exact.shape)
    assert np.array_equal(y[:, rows], want)


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (16, 22016, 4096), (32, 4096, 11008),
                                   (128, 4096, 11008), (2048, 4096, 4096)])
def test_bf16_gemm_full_size_sampled_rows(M, N, K):
    c = workloads.draw_bf16(M, N, K, 128, False, seed=workloads.shape_seed("bf16", N, K, 128, False))
    y = bits(w4.gemm(bf(c.X), gpu_weight(c)))
    rng = np.random.default_rng(N + K)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 24, replace=False)]))
    assert_close(y, c, rows=rows, what=f"M{M} N{N} K{K}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ("bf16", "f16"))
@pytest.mark.parametrize("M,N,K,g", [(1, 512, 4096, 128), (4, 2048, 1024, 64),
                                     (33, 288, 288, 256), (16, 96, 11008, 128)])
def test_zero_weight_rows_give_exact_zeros(path, dtype, M, N, K, g):
    """Rows whose codes equal their zeros (w = 0 throughout, the quantizer's
    image of an all-zero row) give y = 0 exactly, in both 16-bit formats and
    both kernels (split K included); the other rows stay within the bound."""
    if dtype == "bf16":
        c = workloads.draw_bf16(M, N, K, g, False, seed=M + N + K + g)
    else:
        c = workloads.draw(M, N, K, g, False, seed=M + N + K + g)
    dead = np.arange(0, N, 3)
    codes = c.codes.copy()
    codes[dead] = np.repeat(c.zeros[dead], g, axis=1)[:, :K]
    c = type(c)(c.X, codes, c.zeros, c.scales, c.K, c.g, c.symmetric)
    if dtype == "bf16":
        y = bits(w4.gemm(bf(c.X), gpu_weight(c), path=path))
        assert_close(y, c, what=f"{path} M{M} N{N} K{K}")
    else:
        wq = w4.quantized_weight(torch.from_numpy(codes).cuda(), torch.from_numpy(c.scales).cuda(),
                                 torch.from_numpy(c.zeros).cuda(), g, partial=K % g != 0)
        y = w4.gemm(torch.from_numpy(c.X).cuda(), wq, path=path).cpu().view(torch.int16).numpy()
    assert not (y[:, dead] & 0x7FFF).any(), "a zero weight row gave a nonzero output"
    assert y[:, np.setdiff1d(np.arange(N), dead)].any()


def test_bf16_symmetric_equals_explicit_eights():
    c = workloads.draw_bf16(5, 96, 640, 64, True, seed=11)
    ws = gpu_weight(c)
    c8 = workloads.CaseBF16(c.X, c.codes, np.full((96, 10), 8, np.uint8), c.scales, c.K, c.g, False)
    wa = gpu_weight(c8)
    for path in PATHS:
        assert np.array_equal(bits(w4.gemm(bf(c.X), ws, path=path)),
                              bits(w4.gemm(bf(c.X), wa, path=path)))


def test_bf16_and_fp16_do_not_mix():
    c = workloads.draw_bf16(2, 64, 256, 128, False, seed=3)
    w = gpu_weight(c)
    with pytest.raises(TypeError):
        w4.gemm(torch.zeros((2, 256), dtype=torch.float16, device="cuda"), w)
    with pytest.raises(TypeError):
        w4.quantize(torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda"), 128)
