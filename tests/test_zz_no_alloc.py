"""w4a16_gemm_noalloc (the GEMM entry point that allocates nothing, its split-K
partial sums in the library's static scratch) against w4a16_gemm with a
caller-owned workspace, through the C ABI: bit-identical outputs, on two calls
in a row with the second smaller than the first, for plans that split K on
both kernels (so the scratch is really used) and for plans that do not; the
exact family also against the oracle.  A call whose plan needs more scratch
than the library holds is refused before anything is enqueued."""
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
# (Llama-2-7B down at M = 16: 4 slices), on the large-M kernel (o_proj at M =
# 256: 4 slices, 16 MiB of partial sums), forced paths with many slices, and
# plans without a split (the scratch is not touched).
CASES = [(16, 5, 4096, 11008, 128, None), (32, 17, 4096, 4096, 128, None),
         (256, 130, 4096, 4096, 128, None), (128, 65, 12288, 4096, 128, None),
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
    c = workloads.draw_bf16(16, 4096, 11008, 128, False, seed=9)
    w = weight(c, bf16=True)
    X = dev(c.X.view(np.int16)).view(torch.bfloat16)
    for M in (16, 9):
        ref = w4.gemm(X[:M], w)
        got = w4.gemm_noalloc(X[:M], w)
        assert np.array_equal(bits(got), bits(ref))


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    """A call whose split-K partial sums would not fit in the static scratch
    is refused with W4A16_ERR_WORKSPACE, naming both sizes, and nothing is
    written."""
    # Llama-2-7B down at M = 1024: 2 slices of 1024 x 4096 fp32 partial sums
    M, N, K, path = 1024, 4096, 11008, None
    assert w4.workspace_size(M, N, K, 128, 0) > w4.NOALLOC_SCRATCH_BYTES
    c = workloads.draw(1, N, K, 128, False, seed=3)
    w = weight(c)
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4A16ArgumentError) as e:
        w4.gemm_noalloc(X, w, path=path, out=out)
    assert e.value.status == w4.ERR_WORKSPACE
    msg = w4.lib().w4a16_last_hip_error().decode()
    assert str(w4.NOALLOC_SCRATCH_BYTES) in msg
    assert str(w4.workspace_size(M, N, K, 128, 0)) in msg
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
