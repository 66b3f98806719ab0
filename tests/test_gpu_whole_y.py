"""Whole-output parity at the benchmark's own sizes: every (M, shape) of the
Llama-2-7B decode and prefill sweeps, the 70B-class GQA configuration, the
group-size / edge configuration and the tiny configuration, each through the
kernel and tile the library's plan picks for it, on the exact family
(integer X in [-3, 3], power-of-two scales).  There every partial sum is
exact in fp32 for any order and any K split, so every element of Y must be
RNE_16(y_exact), bit for bit; y_exact is the oracle's fp64 product
(oracle.gemm_dense, pinned to the sequential oracle sum on the CPU).

Weights and X are drawn once per shape at the largest M, and each M uses the
first M rows of X, so one fp64 product serves every M of a shape.  Every case
prints its name before it runs."""
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


def check_shape(N, K, g, sym, ms, seed, bf16=False, expect=None):
    """Runs every M of `ms` with the library's own plan and compares all of Y
    with the exact result.  expect: {M: (path, splits)} the plan must pick."""
    mx = max(ms)
    if bf16:
        c = workloads.exact_family_bf16(mx, N, K, g, sym, seed=seed)
    else:
        c = workloads.exact_family(mx, N, K, g, sym, seed=seed)
    qp = oracle.pack(c.codes)
    zp = None if sym else oracle.pack(c.zeros)
    y_exact = oracle.gemm_dense(c.X, qp, c.scales, zp, K, g, sym, bf16=bf16)
    if bf16:
        want = oracle.f64_to_bf16_bits_array(y_exact)
        scales = dev(c.scales.view(np.int16)).view(torch.bfloat16)
        X = dev(c.X.view(np.int16)).view(torch.bfloat16)
    else:
        want = oracle.f64_to_f16_bits_array(y_exact)
        scales = dev(c.scales)
        X = dev(c.X)
    w = w4.quantized_weight(dev(c.codes), scales, None if sym else dev(c.zeros), g,
                            partial=K % g != 0)
    flags = (w4.BF16 if bf16 else 0) | (w4.SYMMETRIC if sym else 0) | \
        (w4.PARTIAL_LAST_GROUP if K % g else 0)
    for M in ms:
        plan = w4.gemm_kernel(M, N, K, g, flags)
        print(f"whole-Y M={M} N={N} K={K} g={g} sym={sym} bf16={bf16} plan={plan}", flush=True)
        if expect and M in expect:
            assert plan == expect[M], (M, plan)
        y = w4.gemm(X[:M], w).cpu().view(torch.int16).numpy().view(np.uint16)
        bad = np.argwhere(y != want[:M])
        assert bad.size == 0, f"M={M} N={N} K={K}: {len(bad)} elements differ, first at {bad[0]}"


@pytest.mark.parametrize("name", list(workloads.LLAMA7B_SHAPES))
def test_whole_y_llama7b(name):
    """Decode M in {1, 4, 8, 16, 32} and prefill M in {64, ..., 2048}: the
    small-M shapes (LDS-staged at M <= 4, 3/6/8-tile one-per-CU shapes, K
    splits and the reduce) and the large-M tiles (32 x 256, 128 x 128 from
    four 128 x 32 waves with a K split, 128 x 192, 128 x 256 from four 128 x
    64 waves, 128 x 384 from eight 128 x 48 waves at gate+up M = 512 and qkv
    M = 2048, 128 x 512 from eight 128 x 64 waves at gate+up M = 2048)."""
    N, K = workloads.LLAMA7B_SHAPES[name]
    check_shape(N, K, 128, False, workloads.DECODE_M + workloads.PREFILL_M,
                seed=workloads.shape_seed("whole-y/7b", N, K, 128, False))


def test_whole_y_plan_covers_the_named_tiles():
    """The instances the prefill and decode sweeps must exercise are the ones
    the plan picks at these sizes (kernel, K splits)."""
    f = lambda M, N, K: w4.gemm_kernel(M, N, K, 128, 0)
    assert f(2048, 22016, 4096) == ("large_m", 1)    # 128 x 512 tiles
    assert f(2048, 4096, 4096) == ("large_m", 1)     # 128 x 256, four 128 x 64 waves
    assert f(128, 12288, 4096)[0] == "large_m" and f(128, 12288, 4096)[1] > 1  # 128 x 128, split
    assert f(16, 22016, 4096) == ("small_m", 1)      # eight waves, three weight tiles
    assert f(32, 22016, 4096) == ("small_m", 1)
    assert f(16, 4096, 11008) == ("small_m", 1)      # one weight tile per workgroup
    assert f(16, 2048, 11008)[1] > 1                 # K split + reduce
    assert f(32, 4096, 4096) == ("small_m", 1)       # two weight tiles, no split
    assert f(32, 2048, 4096)[1] > 1


@pytest.mark.parametrize("name", list(workloads.LLAMA70B_SHAPES))
def test_whole_y_70b(name):
    N, K = workloads.LLAMA70B_SHAPES[name]
    check_shape(N, K, 128, False, workloads.L70B_M,
                seed=workloads.shape_seed("whole-y/70b", N, K, 128, False))


@pytest.mark.parametrize("g", workloads.EDGE_G)
@pytest.mark.parametrize("sym", [False, True])
def test_whole_y_group_sizes(g, sym):
    check_shape(4096, 4096, g, sym, workloads.EDGE_M,
                seed=workloads.shape_seed("whole-y/edge", 4096, 4096, g, sym))


@pytest.mark.parametrize("N,K,g", [(288, 288, 256), (4096, 11008, 256)])
def test_whole_y_partial_and_odd_group_count(N, K, g):
    check_shape(N, K, g, False, workloads.EDGE_M,
                seed=workloads.shape_seed("whole-y/edge", N, K, g, False))


def test_whole_y_tiny():
    check_shape(512, 512, 128, False, (4,), seed=0)


@pytest.mark.parametrize("name", ["o_proj", "gate_up", "down"])
def test_whole_y_llama7b_bf16(name):
    N, K = workloads.LLAMA7B_SHAPES[name]
    check_shape(N, K, 128, False, (1, 4, 16, 32, 128, 512, 2048),
                seed=workloads.shape_seed("whole-y/7b-bf16", N, K, 128, False), bf16=True)


@pytest.mark.parametrize("N,K,ms", [(4096, 4000, (17, 32, 33, 50, 100, 128, 200, 384)),
                                    (22016, 4000, (33, 47, 64)),
                                    (12288, 4000, (17, 30, 33, 64))])
def test_whole_y_activation_stages_through_lds(N, K, ms):
    """The small-M shapes that copy each wave's activation stage through LDS
    (eight waves of four weight tiles at M = 17..384 for N = 4096; four waves
    at two activation tiles for N = 22016, M = 33..64; eight waves of six
    tiles at M = 17..32 and of eight at M = 33..64 for N = 12288): ragged M
    inside a block, and a last 128-column tile that ends inside K (K = 4000,
    a partial last group), whose copies mask the columns past K."""
    check_shape(N, K, 128, False, ms, seed=workloads.shape_seed("whole-y/xl", N, K, 128, False))


# The large-M epilogue stages each wave's output tile through LDS and writes
# 16-byte pieces of rows when it can: 16-bit results without a K split when
# N % 8 == 0, fp32 partial sums with a split when N % 4 == 0 (tiles whose
# staged rows fit); every other case stores element by element.
EPILOGUE_CASES = [
    (1000, 8200, 2048),   # no split, N % 8 == 0: staged 16-bit rows, ragged last row block
    (1000, 8196, 2048),   # no split, N % 8 == 4: element stores
    (1000, 8199, 2048),   # no split, odd N: element stores
    (2050, 4104, 1024),   # no split, 256-row blocks, two rows past the last full block
    (300, 4104, 4096),    # K split, N % 8 == 0: staged fp32 partial sums
    (130, 4100, 4096),    # K split, N % 4 == 0: staged fp32 partial sums, 2 rows past 128
    (300, 4099, 4096),    # K split, odd N: element stores
]


@pytest.mark.parametrize("M,N,K", EPILOGUE_CASES)
def test_whole_y_large_m_epilogue_forms(M, N, K):
    """Every element of Y through each form of the large-M epilogue, bit-exact
    on the exact family."""
    c = workloads.exact_family(M, N, K, 128, False, seed=workloads.shape_seed("whole-y/epi", N, K, 128, False))
    qp, zp = oracle.pack(c.codes), oracle.pack(c.zeros)
    want = oracle.f64_to_f16_bits_array(oracle.gemm_dense(c.X, qp, c.scales, zp, K, 128, False))
    w = w4.quantized_weight(dev(c.codes), dev(c.scales), dev(c.zeros), 128)
    print(f"epilogue M={M} N={N} K={K} plan={w4.gemm_kernel(M, N, K, 128, w4.PATH_LARGE_M)}", flush=True)
    y = w4.gemm(dev(c.X), w, path="large_m").cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} elements differ, first at {bad[0]}"


# The large-M kernel's 128-row waves on a K that ends inside a 128-column
# tile (the last stage's activation columns past K read zeros) and with a
# partial last group: every tile shape the plan can pick there, forced onto
# the large-M path, bit-exact on the exact family.
RAGGED_K_CASES = [
    (300, 4104, 4000, 128, False),    # 128 x 128, K split
    (1000, 8200, 4000, 128, False),   # 128 x 384, ragged M and N
    (2050, 22016, 1000, 128, True),   # 128 x 384, symmetric
    (130, 4100, 8000, 128, False),    # K split, last slice ragged
    (520, 4104, 4000, 256, False),    # 128 x 192, partial last group (4000 = 15 x 256 + 160)
    (2000, 21992, 1000, 128, False),  # 128 x 512: ragged M, N ending inside a 16-row weight tile
    (2000, 21992, 1000, 128, True),   # the same, symmetric
]


@pytest.mark.parametrize("M,N,K,g,sym", RAGGED_K_CASES)
def test_whole_y_large_m_ragged_k(M, N, K, g, sym):
    c = workloads.exact_family(M, N, K, g, sym,
                               seed=workloads.shape_seed("whole-y/ragged-k", N, K, g, sym))
    qp = oracle.pack(c.codes)
    zp = None if sym else oracle.pack(c.zeros)
    want = oracle.f64_to_f16_bits_array(oracle.gemm_dense(c.X, qp, c.scales, zp, K, g, sym))
    w = w4.quantized_weight(dev(c.codes), dev(c.scales), None if sym else dev(c.zeros), g,
                            partial=K % g != 0)
    flags = (w4.SYMMETRIC if sym else 0) | (w4.PARTIAL_LAST_GROUP if K % g else 0)
    print(f"ragged-K M={M} N={N} K={K} g={g} sym={sym} "
          f"plan={w4.gemm_kernel(M, N, K, g, flags | w4.PATH_LARGE_M)}", flush=True)
    y = w4.gemm(dev(c.X), w, path="large_m").cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} elements differ, first at {bad[0]}"
