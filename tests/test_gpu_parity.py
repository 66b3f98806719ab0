"""GPU parity: every result of the HIP path against the CPU oracle.

Bit-exact: pack, repack, dequant (over the whole finite fp16 scale domain),
and Y on the exact-arithmetic family.  Y elsewhere: |y - y_ref| <=
2e-3 * ||x_m|| * ||w_n|| + ulp16(y_ref), element by element, through both GEMM
kernels, at small sizes in full and at the benchmark's full sizes on sampled
weight rows.  All calls go through the C ABI (ctypes binding).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_int4_02_amd as w4
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PATHS = ("small_m", "large_m")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def gpu_weight(c: workloads.Case, partial=None):
    if partial is None:
        partial = c.K % c.g != 0
    return w4.quantized_weight(dev(c.codes), dev(c.scales),
                               None if c.symmetric else dev(c.zeros), c.g, partial=partial)


def oracle_y(c: workloads.Case, rows=None):
    qp = oracle.pack(c.codes)
    zp = None if c.symmetric else oracle.pack(c.zeros)
    return oracle.gemm_rows(c.X, qp, c.scales, zp, c.K, c.g, c.symmetric, rows=rows)


def assert_y_close(y_gpu, c, rows=None, what=""):
    y_ref, wn2 = oracle_y(c, rows)
    yg = y_gpu if rows is None else y_gpu[:, rows]
    ok, worst = oracle.check_y(yg, c.X, y_ref, wn2)
    assert ok, f"{what}: worst |err|/bound = {worst:.3f}"
    assert np.all(np.isfinite(yg.astype(np.float32)))
    return worst


# ---------------------------------------------------------------------------
# pack / repack / dequant: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,C", [(1, 8), (3, 13), (17, 101), (512, 512), (4096, 11008 // 8), (288, 2)])
def test_pack_bit_exact(R, C):
    rng = np.random.default_rng(R * 7 + C)
    codes = rng.integers(0, 256, (R, C), dtype=np.uint8)   # high bits must be dropped
    got = u32(w4.pack(dev(codes)))
    assert np.array_equal(got, oracle.pack(codes))


@pytest.mark.parametrize("N,K,g,sym", [(512, 512, 128, False), (288, 288, 256, False),
                                       (40, 136, 32, True), (4096, 11008, 256, False),
                                       (33, 4096, 64, False), (17, 1024, 128, True)])
def test_repack_bit_exact(N, K, g, sym):
    c = workloads.draw(1, N, K, g, sym, seed=N + K + g)
    w = gpu_weight(c)
    qd, sd, zd = oracle.repack(oracle.pack(c.codes), c.scales,
                               None if sym else oracle.pack(c.zeros), K, g, sym)
    torch.cuda.synchronize()
    assert np.array_equal(w.q.cpu().numpy().view(np.uint32), qd)
    assert np.array_equal(w.s.cpu().numpy().view(np.uint16), sd.view(np.uint16))
    if sym:
        assert w.z is None
    else:
        assert np.array_equal(u32(w.z), zd)
    assert np.array_equal(oracle.unrepack_q(w.q.cpu().numpy().view(np.uint32), N, K),
                          oracle.pack(c.codes))


def test_dequant_exhaustive_fp16_scales():
    """Every finite fp16 scale x every (q, z) pair: 16.25 M values."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = bits.view(np.float16)
    s = s[np.isfinite(s)]
    N, K, g = s.size, 256, 32
    # K = 256 with g = 32 gives 8 groups; two rows per scale cover all 16 zeros
    codes = np.tile(np.arange(16, dtype=np.uint8), (2 * N, 16))
    zeros = np.concatenate([np.tile(np.arange(8, dtype=np.uint8), (N, 1)),
                            np.tile(np.arange(8, 16, dtype=np.uint8), (N, 1))], 0)
    scales = np.repeat(np.concatenate([s, s])[:, None], 8, 1)
    qp, zp = oracle.pack(codes), oracle.pack(zeros)
    want = oracle.dequant(qp, scales, zp, K, g, False)
    got = w4.dequant(dev(qp.view(np.int32)), dev(scales), dev(zp.view(np.int32)), K, g)
    got = got.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("N,K,g,sym", [(512, 512, 128, False), (288, 288, 256, False),
                                       (64, 4096, 32, True), (4096, 11008, 256, False)])
def test_dequant_bit_exact(N, K, g, sym):
    c = workloads.draw(1, N, K, g, sym, seed=3 * N + K)
    qp = oracle.pack(c.codes)
    zp = None if sym else oracle.pack(c.zeros)
    want = oracle.dequant(qp, c.scales, zp, K, g, sym)
    got = w4.dequant(dev(qp.view(np.int32)), dev(c.scales),
                     None if sym else dev(zp.view(np.int32)), K, g, symmetric=sym,
                     partial=K % g != 0).cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


# ---------------------------------------------------------------------------
# GEMM: tolerance parity, both kernels
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", PATHS)
def test_gemm_tiny_case(path):
    c = workloads.tiny_case()
    w = gpu_weight(c)
    y = w4.gemm(dev(c.X), w, path=path).cpu().numpy()
    assert_y_close(y, c, what=f"tiny {path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,N,K,g,sym", [
    (1, 288, 288, 256, False), (7, 288, 288, 256, True), (33, 288, 288, 256, False),
    (1, 40, 136, 32, False), (5, 300, 520, 64, False), (16, 48, 4096, 128, False),
    (17, 64, 1024, 128, True), (130, 136, 392, 32, False), (257, 512, 1024, 256, False),
    (3, 4096, 11008, 256, False), (1, 300, 520, 64, True), (1, 4096, 4096, 128, True),
    (2, 17000, 1024, 32, False)])
def test_gemm_small_shapes(path, M, N, K, g, sym):
    c = workloads.draw(M, N, K, g, sym, seed=M * 131 + N * 7 + K + g)
    w = gpu_weight(c)
    y = w4.gemm(dev(c.X), w, path=path).cpu().numpy()
    assert_y_close(y, c, what=f"{path} M{M} N{N} K{K} g{g} sym{sym}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,N,K,g,sym", [
    (4, 512, 512, 128, False), (1, 288, 288, 256, False), (33, 288, 288, 256, True),
    (7, 4096 // 4, 4096, 32, False), (16, 160, 11008, 256, False), (130, 200, 1032, 64, False),
    (2, 64, 28672, 128, False)])
def test_gemm_exact_family_bit_exact(path, M, N, K, g, sym):
    """Integer X and power-of-two scales: every partial sum is exact in fp32,
    so Y must be RNE_fp16 of the exact result, bit for bit."""
    c = workloads.exact_family(M, N, K, g, sym, seed=M + N + K)
    w = gpu_weight(c)
    y = w4.gemm(dev(c.X), w, path=path).cpu().numpy()
    y_exact, _ = oracle_y(c)
    assert np.array_equal(y.view(np.uint16), y_exact.astype(np.float16).view(np.uint16))


# The large-M kernel at sizes where the plan picks its 128 x 256 tile (four
# 128 x 64 waves with loader waves at g >= 128, eight 64 x 64 waves without
# them at g < 128) or its 256 x 256 tile (eight 128 x 64 waves, no loader
# waves), K split across workgroups at the smaller size; ragged M, N and K.
# Exact family, sampled rows (the last 40 columns included).
LARGE_TILES = ([(520, 4112, 1024, g, sym) for g in (32, 64, 128, 256) for sym in (False, True)]
               + [(2048, 4096, 4096, 32, False), (2048, 4096, 4096, 64, True),
                  (2048, 4096, 4096, 128, False),
                  # 128 x 256 from 128 x 64 waves at ragged M, N and K
                  (1000, 4112, 1160, 128, False),
                  # 256 x 256: ragged M, N and K, g = 128 and 256
                  (1000, 9000, 1160, 128, False), (1000, 9000, 1280, 256, True),
                  (512, 22016, 1024, 128, False),
                  # 256 x 256 at exactly one 256-row block, ragged N
                  (256, 40000, 512, 128, False),
                  # 256 x 256 with one or two 128-column stages (the second
                  # partial): the two-stage ring with nothing or one stage to copy
                  (512, 22016, 128, 128, False), (512, 22016, 200, 128, True),
                  # 128 x 192 (four 128 x 48 waves): ragged M, N and K, with
                  # and without a K split, symmetric and g = 256
                  (300, 7000, 1160, 128, False), (300, 12300, 1032, 128, True),
                  (130, 12288, 4096, 256, False)])


@pytest.mark.parametrize("M,N,K,g,sym", LARGE_TILES)
def test_large_m_tiles_exact_family(M, N, K, g, sym):
    c = workloads.exact_family(M, N, K, g, sym, seed=M + N + K + g)
    y = w4.gemm(dev(c.X), gpu_weight(c), path="large_m").cpu().numpy()
    rng = np.random.default_rng(N + g)
    rows = np.unique(np.concatenate([[0], np.arange(N - 40, N), rng.choice(N, 24, replace=False)]))
    y_exact, _ = oracle_y(c, rows)
    assert np.array_equal(y[:, rows].view(np.uint16),
                          y_exact.astype(np.float16).view(np.uint16))


# The small-M kernel's wide shapes: eight weight tiles per workgroup (M =
# 17..32 over more than 1536 weight tiles); one workgroup per compute unit with
# 3 or 6 weight tiles (qkv- and gate+up-like N at M = 5..32, one or two
# activation tiles; ragged N, M, K and last block); one activation tile per
# workgroup with K split (M = 17..32 over <= 256 weight tiles).
@pytest.mark.parametrize("M,N,K,g,sym", [(32, 32000, 1024, 128, False), (32, 16400, 1024, 128, False),
                                         (17, 16400, 2048, 256, True), (13, 12280, 1000, 128, False),
                                         (9, 22008, 2048, 128, True), (27, 12280, 1024, 256, False),
                                         (32, 4096, 4096, 128, False), (20, 4000, 11008, 128, False)])
def test_small_m_wide_shapes_exact_family(M, N, K, g, sym):
    c = workloads.exact_family(M, N, K, g, sym, seed=M + N + K + g)
    y = w4.gemm(dev(c.X), gpu_weight(c), path="small_m").cpu().numpy()
    rng = np.random.default_rng(N + g)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 24, replace=False)]))
    y_exact, _ = oracle_y(c, rows)
    assert np.array_equal(y[:, rows].view(np.uint16),
                          y_exact.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("path", PATHS)
def test_symmetric_equals_explicit_eights(path):
    c = workloads.draw(5, 96, 640, 64, True, seed=11)
    ws = gpu_weight(c)
    c8 = workloads.Case(c.X, c.codes, np.full((96, 10), 8, np.uint8), c.scales, c.K, c.g, False)
    wa = gpu_weight(c8)
    X = dev(c.X)
    ys = w4.gemm(X, ws, path=path).cpu().numpy()
    ya = w4.gemm(X, wa, path=path).cpu().numpy()
    assert np.array_equal(ys.view(np.uint16), ya.view(np.uint16))


def test_partial_group_equals_zero_padding():
    """K = 288 with a 32-wide last group == K = 512, X zero-padded (exact family)."""
    c = workloads.exact_family(9, 288, 288, 256, False, seed=5)
    rng = np.random.default_rng(6)
    codes_p = np.concatenate([c.codes, rng.integers(0, 16, (288, 224), dtype=np.uint8)], 1)
    Xp = np.concatenate([c.X, np.zeros((9, 224), np.float16)], 1)
    cp = workloads.Case(Xp, codes_p, c.zeros, c.scales, 512, 256, False)
    for path in PATHS:
        y = w4.gemm(dev(c.X), gpu_weight(c), path=path).cpu().numpy()
        yp = w4.gemm(dev(Xp), gpu_weight(cp), path=path).cpu().numpy()
        assert np.array_equal(y.view(np.uint16), yp.view(np.uint16))


def test_paths_agree_and_are_deterministic():
    c = workloads.draw(16, 1024, 2048, 128, False, seed=21)
    w = gpu_weight(c)
    X = dev(c.X)
    a1 = w4.gemm(X, w, path="small_m").cpu().numpy()
    a2 = w4.gemm(X, w, path="small_m").cpu().numpy()
    b1 = w4.gemm(X, w, path="large_m").cpu().numpy()
    b2 = w4.gemm(X, w, path="large_m").cpu().numpy()
    assert np.array_equal(a1.view(np.uint16), a2.view(np.uint16))
    assert np.array_equal(b1.view(np.uint16), b2.view(np.uint16))
    assert_y_close(a1, c, what="small")
    assert_y_close(b1, c, what="large")


@pytest.mark.parametrize("path", PATHS)
def test_no_writes_outside_y(path):
    """Guard bands around Y keep their poison pattern."""
    c = workloads.draw(7, 200, 392, 64, False, seed=8)
    w = gpu_weight(c)
    M, N = 7, 200
    pad = 4096
    buf = torch.full((pad + M * N + pad,), 0x5A5A, dtype=torch.int16, device="cuda")
    out = buf[pad:pad + M * N].view(torch.float16).view(M, N)
    w4.gemm(dev(c.X), w, path=path, out=out)
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 0x5A5A) and np.all(host[pad + M * N:] == 0x5A5A)
    assert_y_close(out.cpu().numpy(), c, what="guarded")


# Calls whose plan splits K across workgroups (fp32 partial sums in the
# workspace, then the reduce kernel), on both kernels: poisoned guard bands
# around the workspace keep their pattern, and the workspace is given exactly
# the bytes w4a16_gemm_workspace_size asks for.
WS_CASES = [(16, 2048, 11008, None), (32, 2048, 4096, None), (17, 33, 16384, "small_m"),
            (256, 4096, 4096, "large_m"), (256, 4096, 11008, None), (128, 12288, 4096, None), (65, 4095, 4096, "large_m"),
            (100, 1023, 1024, "small_m")]


@pytest.mark.parametrize("M,N,K,path", WS_CASES)
def test_no_writes_outside_the_workspace(M, N, K, path):
    flags = {None: 0, "small_m": w4.PATH_SMALL_M, "large_m": w4.PATH_LARGE_M}[path]
    need = w4.workspace_size(M, N, K, 128, flags)
    assert need > 0 and need % 16 == 0
    c = workloads.exact_family(M, N, K, 128, False, seed=M + N + K + 5)
    w = gpu_weight(c)
    pad = 1 << 16
    buf = torch.full((pad + need + pad,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = buf[pad:pad + need]
    ypad = 4096
    ybuf = torch.full((ypad + M * N + ypad,), 0x5A5A, dtype=torch.int16, device="cuda")
    out = ybuf[ypad:ypad + M * N].view(torch.float16).view(M, N)
    for _ in range(2):
        w4.gemm(dev(c.X), w, path=path, out=out, workspace=ws)
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 0xA5) and np.all(host[pad + need:] == 0xA5)
    yh = ybuf.cpu().numpy()
    assert np.all(yh[:ypad] == 0x5A5A) and np.all(yh[ypad + M * N:] == 0x5A5A)
    y_exact, _ = oracle_y(c)
    assert np.array_equal(out.cpu().numpy().view(np.uint16),
                          oracle.f64_to_f16_bits_array(y_exact))


# ---------------------------------------------------------------------------
# Full benchmark sizes, sampled rows
# ---------------------------------------------------------------------------

FULL = [("decode7b", M, N, K) for (N, K) in workloads.LLAMA7B_SHAPES.values() for M in (1, 16, 32)] + \
       [("prefill7b", 2048, 4096, 4096), ("prefill7b", 512, 22016, 4096),
        ("prefill7b", 64, 22016, 4096), ("prefill7b", 128, 4096, 11008),
        ("prefill7b", 128, 12288, 4096), ("prefill7b", 256, 4096, 4096),
        ("gqa70b", 1, 57344, 8192), ("gqa70b", 16, 8192, 28672), ("gqa70b", 1024, 10240, 8192),
        ("gqa70b", 1, 8192, 28672), ("gqa70b", 4, 57344, 8192)]


@pytest.mark.parametrize("family,M,N,K", FULL)
def test_gemm_full_size_sampled_rows(family, M, N, K):
    c = workloads.draw(M, N, K, 128, False, seed=workloads.shape_seed(family, N, K, 128, False),
                       outliers=family == "prefill7b")
    w = gpu_weight(c)
    y = w4.gemm(dev(c.X), w).cpu().numpy()
    rng = np.random.default_rng(N + K)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 30, replace=False)]))
    assert_y_close(y, c, rows=rows, what=f"{family} M{M} N{N} K{K}")


def test_errors_raise_without_launch():
    c = workloads.tiny_case()
    w = gpu_weight(c)
    with pytest.raises(ValueError):
        w4.gemm(dev(c.X[:, :256]), w)
    bad = w4.PackedWeight(w.q, w.s, w.z, w.N, w.K, 100, w.flags)
    with pytest.raises(w4.W4A16ArgumentError) as e:
        w4.gemm(dev(c.X), bad)
    assert e.value.status == w4.ERR_GROUP
    # device-layout tensors smaller than the weight's shape needs are refused
    # on the host (the kernels would read past them)
    for bad in (w4.PackedWeight(w.q[:-16], w.s, w.z, w.N, w.K, w.g, w.flags),
                w4.PackedWeight(w.q, w.s[:-1], w.z, w.N, w.K, w.g, w.flags),
                w4.PackedWeight(w.q, w.s, w.z[:-1], w.N, w.K, w.g, w.flags),
                w4.PackedWeight(w.q, w.s, w.z, w.N + 16, w.K, w.g, w.flags)):
        with pytest.raises(ValueError):
            w4.gemm(dev(c.X), bad)
    with pytest.raises(TypeError):
        w4.gemm(dev(c.X), w4.PackedWeight(w.q, w.s, None, w.N, w.K, w.g, w.flags))
    qp, zp = oracle.pack(c.codes), oracle.pack(c.zeros)
    with pytest.raises(ValueError):
        w4.dequant(dev(qp.view(np.int32)), dev(c.scales), dev(zp.view(np.int32)[:-1]), c.K, c.g)
    w4.device_check()


# The split-K reduce: slices summed in batches of 2, 4 or 8 loads, more than
# one batch from 16 slices on, four elements per thread where M N is a
# multiple of 4 and one otherwise (odd M and N).  (M, N, K, path, slices the
# plan picks.)
REDUCE_CASES = [(17, 33, 1024, "small_m", 8), (17, 511, 4096, "small_m", 16),
                (20, 511, 4096, "small_m", 16), (17, 33, 16384, "small_m", 128),
                (65, 33, 1024, "large_m", 2), (65, 4095, 4096, "large_m", 4),
                (65, 16, 8192, "large_m", 16), (100, 1023, 1024, "small_m", 4)]


@pytest.mark.parametrize("M,N,K,path,splits", REDUCE_CASES)
def test_split_k_reduce_batches(M, N, K, path, splits):
    flags = w4.PATH_SMALL_M if path == "small_m" else w4.PATH_LARGE_M
    assert w4.gemm_kernel(M, N, K, 128, flags) == (path, splits)
    c = workloads.exact_family(M, N, K, 128, False, seed=M + N + K)
    y = w4.gemm(dev(c.X), gpu_weight(c), path=path).cpu().numpy()
    y_exact, _ = oracle_y(c)
    assert np.array_equal(y.view(np.uint16), y_exact.astype(np.float16).view(np.uint16))
    r = workloads.draw(M, N, K, 128, False, seed=M + N + K + 1)
    yr = w4.gemm(dev(r.X), gpu_weight(r), path=path).cpu().numpy()
    assert_y_close(yr, r, what=f"reduce M{M} N{N} K{K} {path} x{splits}")


def test_split_k_workspace_shared_across_shapes():
    """Shapes whose K is split across workgroups (fp32 partial sums in the
    workspace, then a reduce kernel) share the binding's cached workspace in
    turn with different partial layouts, between calls that split nothing;
    repeated rounds stay correct and bit-identical."""
    shapes = [(16, 1024, 2048), (8, 512, 4096), (1, 4096, 11008), (33, 288, 4096), (4, 4096, 4096),
              (32, 4096, 11008), (17, 288, 520), (16, 4096, 11008), (64, 4096, 4096)]
    cases = [workloads.draw(M, N, K, 128, False, seed=M + N + K) for M, N, K in shapes]
    weights = [gpu_weight(c) for c in cases]
    first = []
    for rnd in range(3):
        for idx, (c, w) in enumerate(zip(cases, weights)):
            y = w4.gemm(dev(c.X), w).cpu().numpy()
            if rnd == 0:
                assert_y_close(y, c, what=f"split M{c.M} N{c.N} K{c.K}")
                first.append(y)
            else:
                assert np.array_equal(y.view(np.uint16), first[idx].view(np.uint16))
