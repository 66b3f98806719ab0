"""w4a16_gemm_noalloc (the GEMM entry point that allocates nothing, its split-K
partial sums in the library's static scratch) against w4a16_gemm with a
caller-owned workspace, through the C ABI: bit-identical outputs, on two calls
in a row with the second smaller than the first, for plans that split K on
both kernels (so the scratch is really used) and for plans that do not; the
exact family also against the oracle.  Every plan's split-K workspace fits
the library's scratch."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_int4_02_amd as w4
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weight(c, bf16=False):
    scales = dev(c.scales.view(np.int16)).view(torch.bfloat16) if bf16 else dev(c.scales)
    return w4.quantized_weight(dev(c.codes), scales, None if c.symmetric else dev(c.zeros), c.g,
                               partial=c.K % c.g != 0)


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# (M first call, M second call, N, K, g, path): K split on the small-M kernel
# (N = 2048, K = 11008 at M = 16: 8 slices), on the large-M kernel (o_proj at
# M = 256 on the forced large-M path: 4 slices, 16 MiB of partial sums; qkv at
# M = 128: 4 slices of the 128 x 192 tiles, 24 MiB), forced paths with many
# slices, and plans without a split (the scratch is not touched).
CASES = [(16, 5, 2048, 11008, 128, None), (32, 17, 4096, 4096, 128, None),
         (256, 130, 4096, 4096, 128, "large_m"), (128, 65, 12288, 4096, 128, None),
         (17, 3, 33, 16384, 128, "small_m"), (65, 40, 4095, 4096, 128, "large_m"),
         (1, 1, 22016, 4096, 128, None), (2048, 512, 4096, 4096, 128, None),
         (33, 7, 288, 288, 256, None)]


@pytest.mark.parametrize("M1,M2,N,K,g,path", CASES)
def test_noalloc_matches_gemm_twice(M1, M2, N, K, g, path):
    flags = {None: 0, "small_m": w4.PATH_SMALL_M, "large_m": w4.PATH_LARGE_M}[path]
    flags |= w4.PARTIAL_LAST_GROUP if K % g else 0
    print(f"noalloc M={M1}->{M2} N={N} K={K} g={g} path={path} "
          f"ws={w4.workspace_size(M1, N, K, g, flags)}", flush=True)
    r = workloads.draw(M1, N, K, g, False, seed=M1 + N + K)
    w = weight(r)
    X = dev(r.X)
    for M in (M1, M2):   # the second call smaller than the first
        ref = w4.gemm(X[:M], w, path=path)
        got = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        w4.gemm_noalloc(X[:M], w, path=path, out=got)
        assert np.array_equal(bits(got), bits(ref)), f"M={M}"
    e = workloads.exact_family(M1, N, K, g, False, seed=M1 + N + K + 1)
    we = weight(e)
    Xe = dev(e.X)
    qp, zp = oracle.pack(e.codes), oracle.pack(e.zeros)
    y_exact = oracle.gemm_dense(e.X, qp, e.scales, zp, K, g, False)
    for M in (M1, M2):
        got = w4.gemm_noalloc(Xe[:M], we, path=path)
        assert np.array_equal(bits(got), oracle.f64_to_f16_bits_array(y_exact[:M])), f"M={M}"


def test_noalloc_bf16_split():
    assert w4.gemm_kernel(16, 2048, 11008, 128, w4.BF16)[1] > 1
    c = workloads.draw_bf16(16, 2048, 11008, 128, False, seed=9)
    w = weight(c, bf16=True)
    X = dev(c.X.view(np.int16)).view(torch.bfloat16)
    for M in (16, 9):
        ref = w4.gemm(X[:M], w)
        got = w4.gemm_noalloc(X[:M], w)
        assert np.array_equal(bits(got), bits(ref))


def test_every_plan_fits_the_scratch():
    """The static scratch covers every split-K workspace the plan makes:
    Llama-2 7B / 70B shapes at every M up to 4096, every group size, fp16 and
    bf16, both forced paths (so no call is refused for its size)."""
    shapes = list(workloads.LLAMA7B_SHAPES.values()) + list(workloads.LLAMA70B_SHAPES.values())
    worst = 0
    for M in list(range(1, 257)) + list(range(257, 4097, 61)):
        for N, K in shapes:
            for g in (32, 128, 256):
                for fl in (0, w4.BF16, w4.PATH_SMALL_M, w4.PATH_LARGE_M):
                    worst = max(worst, w4.workspace_size(M, N, K, g, fl))
    assert 0 < worst <= w4.NOALLOC_SCRATCH_BYTES
