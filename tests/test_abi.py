"""C-ABI tests that need no GPU: the library loads, every symbol the header
declares resolves (the undefined-symbol failure on lmdeploy PR "[Feature]
Blazing fast W4A16 inference" is the failure mode guarded against), and every
argument error is reported through the pure-host check functions.  No compute
entry point is called here."""
import ctypes
import os
import re

import pytest

import weight_only_int4_02_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int32_t)\s*(w4a16_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(w4.LIB_PATH):
        from weight_only_int4_02_amd import build
        build.build_library()
    return w4.lib()


def test_every_declared_symbol_resolves(L):
    names = header_functions()
    assert len(names) == 18
    assert set(names) == set(w4.EXPORTS)
    for n in names:
        assert getattr(L, n) is not None
    # resolved through dlsym on a fresh handle as well
    h = ctypes.CDLL(w4.LIB_PATH)
    for n in names:
        assert ctypes.cast(getattr(h, n), ctypes.c_void_p).value


def test_status_strings(L):
    for code in range(0, -9, -1):
        s = w4.status_str(code)
        assert s.startswith("W4A16_")
    assert w4.status_str(-100) == "unknown status"
    assert w4.status_str(w4.ERR_GROUP).startswith("W4A16_ERR_GROUP")


A = 1 << 20          # a 16-byte-aligned stand-in address (never dereferenced)


def P(off=0):
    return ctypes.c_void_p(A + off)


def gemm_args(**kw):
    args = dict(X=P(), M=4, K=512, q=P(0x1000), s=P(0x2000), z=P(0x3000), N=512, g=128,
                flags=0, Y=P(0x100000), ws=None, wsb=0)
    args.update(kw)
    return args


def check_gemm(L, **kw):
    a = gemm_args(**kw)
    return L.w4a16_check_gemm_args(a["X"], a["M"], a["K"], a["q"], a["s"], a["z"], a["N"],
                                   a["g"], a["flags"], a["Y"], a["ws"], a["wsb"])


def test_gemm_args_ok(L):
    assert check_gemm(L) == w4.OK
    assert check_gemm(L, flags=w4.SYMMETRIC, z=None) == w4.OK
    assert check_gemm(L, K=288, N=288, g=256, flags=w4.PARTIAL_LAST_GROUP) == w4.OK
    for g in (32, 64, 128, 256):
        assert check_gemm(L, g=g) == w4.OK


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), w4.ERR_NULL),
    (dict(q=None), w4.ERR_NULL),
    (dict(s=None), w4.ERR_NULL),
    (dict(z=None), w4.ERR_NULL),            # zeros needed unless symmetric
    (dict(Y=None), w4.ERR_NULL),
    (dict(M=0), w4.ERR_SHAPE),
    (dict(M=-3), w4.ERR_SHAPE),
    (dict(N=0), w4.ERR_SHAPE),
    (dict(K=0), w4.ERR_SHAPE),
    (dict(K=100), w4.ERR_SHAPE),            # K % 8 != 0
    (dict(g=16), w4.ERR_GROUP),
    (dict(g=100), w4.ERR_GROUP),
    (dict(K=288, N=288, g=256), w4.ERR_GROUP),   # the 288 x 288 weight vs g = 256
    (dict(K=11008 + 8, g=128), w4.ERR_GROUP),
    (dict(X=P(2)), w4.ERR_ALIGN),
    (dict(q=P(0x1004)), w4.ERR_ALIGN),
    (dict(s=P(0x2008)), w4.ERR_ALIGN),
    (dict(z=P(0x3001)), w4.ERR_ALIGN),
    (dict(Y=P(0x100002)), w4.ERR_ALIGN),
    (dict(flags=0x400), w4.ERR_FLAGS),
    (dict(flags=w4.PATH_SMALL_M | w4.PATH_LARGE_M), w4.ERR_FLAGS),
    (dict(Y=P(0x10)), w4.ERR_SHAPE),         # Y overlaps X
])
def test_gemm_arg_errors(L, kw, status):
    assert check_gemm(L, **kw) == status


def test_stream_read_refuses_bad_ranges(L):
    """The measurement read checks its ranges before any HIP call."""
    sink = P(0x5000)
    f = L.w4a16_stream_read
    assert f(P(0x1000), 16, None, 0, None, 0, 1, None, None) == w4.ERR_NULL
    assert f(None, 16, None, 0, None, 0, 1, sink, None) == w4.ERR_NULL
    assert f(P(0x1000), 0, None, 0, None, 0, 1, sink, None) == w4.ERR_SHAPE
    assert f(P(0x1000), 24, None, 0, None, 0, 1, sink, None) == w4.ERR_SHAPE
    assert f(P(0x1008), 16, None, 0, None, 0, 1, sink, None) == w4.ERR_ALIGN
    assert f(P(0x1000), 16, P(0x2004), 16, None, 0, 1, sink, None) == w4.ERR_ALIGN


def test_gemm_k_limit(L):
    """K must stay below 2^22: the large-M kernel forms the byte size of a
    256-row activation slice, 256 * K * 2, in 32 bits."""
    big = dict(M=256, N=16, g=128, X=P(1 << 40), Y=P(1 << 44), ws=P(1 << 46), wsb=1 << 40)
    assert check_gemm(L, K=(1 << 22) - 128, **big) == w4.OK
    assert check_gemm(L, K=1 << 22, **big) == w4.ERR_SHAPE
    for flags in (0, w4.PATH_LARGE_M, w4.PATH_SMALL_M):
        b = ctypes.c_size_t(0)
        assert L.w4a16_gemm_workspace_size(256, 16, 1 << 22, 128, flags, ctypes.byref(b)) == w4.ERR_SHAPE
        assert L.w4a16_gemm_workspace_size(256, 16, (1 << 22) - 128, 128, flags,
                                           ctypes.byref(b)) == w4.OK
    q, sb, zb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.w4a16_repack_size(16, 1 << 22, 128, 0, ctypes.byref(q), ctypes.byref(sb),
                               ctypes.byref(zb)) == w4.ERR_SHAPE


def test_gemm_workspace_rules(L):
    for M, N, K in [(1, 4096, 4096), (16, 22016, 4096), (512, 4096, 11008), (7, 288, 288)]:
        for flags in (0, w4.PATH_SMALL_M, w4.PATH_LARGE_M):
            f = flags | (w4.PARTIAL_LAST_GROUP if K == 288 else 0)
            g = 256 if K == 288 else 128
            b = ctypes.c_size_t(123)
            assert L.w4a16_gemm_workspace_size(M, N, K, g, f, ctypes.byref(b)) == w4.OK
            need = b.value
            if need:
                assert check_gemm(L, M=M, N=N, K=K, g=g, flags=f, Y=P(1 << 28)) == w4.ERR_NULL
                assert check_gemm(L, M=M, N=N, K=K, g=g, flags=f, Y=P(1 << 28), ws=P(1 << 30),
                                  wsb=need - 1) == w4.ERR_WORKSPACE
                assert check_gemm(L, M=M, N=N, K=K, g=g, flags=f, Y=P(1 << 28), ws=P(8 + (1 << 30)),
                                  wsb=need + 64) == w4.ERR_ALIGN
            assert check_gemm(L, M=M, N=N, K=K, g=g, flags=f, Y=P(1 << 28), ws=P(1 << 30),
                              wsb=need) == w4.OK
    assert L.w4a16_gemm_workspace_size(1, 64, 64, 128, 0, None) == w4.ERR_NULL


def test_gemm_kernel_choice(L):
    """w4a16_gemm_kernel reports the plan w4a16_gemm runs: the small-M kernel
    to M = 64, to M = 128 for weights of at most 4096 rows, and to M = 384
    for fp16 ones with K <= 4096 (g >= 128); path flags win; K is split
    exactly when a workspace is needed, which is then splits * M * N * 4
    bytes."""
    assert w4.gemm_kernel(1, 4096, 4096, 128, 0)[0] == "small_m"
    assert w4.gemm_kernel(64, 22016, 4096, 128, 0)[0] == "small_m"
    assert w4.gemm_kernel(65, 22016, 4096, 128, 0)[0] == "large_m"
    assert w4.gemm_kernel(128, 4096, 4096, 128, 0)[0] == "small_m"
    assert w4.gemm_kernel(128, 4096, 11008, 128, 0)[0] == "small_m"
    assert w4.gemm_kernel(129, 4096, 4096, 128, 0)[0] == "small_m"
    assert w4.gemm_kernel(384, 4096, 4096, 128, 0)[0] == "small_m"
    assert w4.gemm_kernel(385, 4096, 4096, 128, 0)[0] == "large_m"
    assert w4.gemm_kernel(129, 4096, 11008, 128, 0)[0] == "large_m"
    assert w4.gemm_kernel(256, 4096, 4096, 64, 0)[0] == "large_m"      # g < 128
    assert w4.gemm_kernel(256, 4096, 4096, 128, w4.BF16)[0] == "large_m"
    assert w4.gemm_kernel(128, 4112, 4096, 128, 0)[0] == "large_m"   # 257 row tiles
    assert w4.gemm_kernel(128, 4096, 4096, 128, w4.BF16)[0] == "small_m"
    assert w4.gemm_kernel(129, 4096, 4096, 128, w4.BF16)[0] == "large_m"
    assert w4.gemm_kernel(2048, 4096, 4096, 128, 0)[0] == "large_m"
    assert w4.gemm_kernel(2048, 4096, 4096, 128, w4.PATH_SMALL_M)[0] == "small_m"
    assert w4.gemm_kernel(1, 4096, 4096, 128, w4.PATH_LARGE_M)[0] == "large_m"
    for M in (1, 16, 32, 64, 96, 128, 256, 512, 2048):
        for N, K in ((4096, 4096), (12288, 4096), (22016, 4096), (4096, 11008)):
            for flags in (0, w4.BF16, w4.PATH_SMALL_M, w4.PATH_LARGE_M):
                _, splits = w4.gemm_kernel(M, N, K, 128, flags)
                ws = w4.workspace_size(M, N, K, 128, flags)
                assert splits >= 1
                assert ws == (splits * M * N * 4 if splits > 1 else 0)
    path, splits = ctypes.c_int32(), ctypes.c_int32()
    assert L.w4a16_gemm_kernel(4, 512, 512, 100, 0, ctypes.byref(path),
                               ctypes.byref(splits)) == w4.ERR_GROUP
    assert L.w4a16_gemm_kernel(0, 512, 512, 128, 0, ctypes.byref(path),
                               ctypes.byref(splits)) == w4.ERR_SHAPE
    assert L.w4a16_gemm_kernel(4, 512, 512, 128, 0, None, ctypes.byref(splits)) == w4.ERR_NULL
    assert L.w4a16_gemm_kernel(4, 512, 512, 128, w4.PATH_SMALL_M | w4.PATH_LARGE_M,
                               ctypes.byref(path), ctypes.byref(splits)) == w4.ERR_FLAGS


def test_repack_size_and_args(L):
    q, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    r = L.w4a16_repack_size(4096, 4096, 128, 0, ctypes.byref(q), ctypes.byref(s), ctypes.byref(z))
    assert r == w4.OK
    assert q.value == 4096 * 4096 // 2                  # 16 x 128 tiles, no padding
    assert s.value == 4096 * 32 * 2
    assert z.value == 4096 * 4 * 4                      # ceil(32 / 8) words per row
    r = L.w4a16_repack_size(288, 288, 256, w4.PARTIAL_LAST_GROUP | w4.SYMMETRIC,
                            ctypes.byref(q), ctypes.byref(s), ctypes.byref(z))
    assert r == w4.OK
    assert q.value == 18 * 3 * 1024 and s.value == 18 * 2 * 32 and z.value == 0
    assert L.w4a16_repack_size(288, 288, 256, 0, ctypes.byref(q), ctypes.byref(s),
                               ctypes.byref(z)) == w4.ERR_GROUP
    ok = L.w4a16_check_repack_args(P(), P(0x100), P(0x200), 64, 256, 128, 0, P(0x300),
                                   P(0x400), P(0x500))
    assert ok == w4.OK
    assert L.w4a16_check_repack_args(P(), P(0x100), None, 64, 256, 128, 0, P(0x300),
                                     P(0x400), P(0x500)) == w4.ERR_NULL
    assert L.w4a16_check_repack_args(P(), P(0x100), None, 64, 256, 128, w4.SYMMETRIC,
                                     P(0x300), P(0x400), None) == w4.OK
    assert L.w4a16_check_repack_args(P(), P(0x100), P(0x200), 64, 256, 128, w4.PATH_SMALL_M,
                                     P(0x300), P(0x400), P(0x500)) == w4.ERR_FLAGS


def test_dequant_and_pack_args(L):
    assert L.w4a16_check_dequant_args(P(), P(0x100), P(0x200), 64, 256, 64, 0, P(0x400)) == w4.OK
    assert L.w4a16_check_dequant_args(P(), P(0x100), P(0x200), 64, 250, 64, 0, P(0x400)) == w4.ERR_SHAPE
    assert L.w4a16_check_dequant_args(P(), P(0x100), P(0x200), 64, 256, 48, 0, P(0x400)) == w4.ERR_GROUP
    assert L.w4a16_check_dequant_args(P(), P(0x100), P(0x200), 64, 256, 64, 0, P(0x402)) == w4.ERR_ALIGN
    assert L.w4a16_check_pack_args(P(3), 5, 7, P(0x100)) == w4.OK      # codes: any alignment
    assert L.w4a16_check_pack_args(P(3), 0, 7, P(0x100)) == w4.ERR_SHAPE
    assert L.w4a16_check_pack_args(None, 5, 7, P(0x100)) == w4.ERR_NULL
    assert L.w4a16_check_pack_args(P(), 5, 7, P(0x104)) == w4.ERR_ALIGN


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        w4.pack(torch.zeros((2, 8), dtype=torch.uint8))


def test_quantize_args(L):
    Q = L.w4a16_check_quantize_args
    # W, N, K, g, flags, qpacked, scales, zeros
    assert Q(P(), 64, 256, 64, 0, P(0x100), P(0x200), P(0x400)) == w4.OK
    assert Q(P(), 64, 256, 64, w4.SYMMETRIC, P(0x100), P(0x200), None) == w4.OK
    assert Q(P(), 64, 256, 64, 0, P(0x100), P(0x200), None) == w4.ERR_NULL
    assert Q(None, 64, 256, 64, 0, P(0x100), P(0x200), P(0x400)) == w4.ERR_NULL
    assert Q(P(), 64, 250, 64, 0, P(0x100), P(0x200), P(0x400)) == w4.ERR_SHAPE
    assert Q(P(), 0, 256, 64, 0, P(0x100), P(0x200), P(0x400)) == w4.ERR_SHAPE
    assert Q(P(), 288, 288, 256, 0, P(0x100), P(0x200), P(0x400)) == w4.ERR_GROUP
    assert Q(P(), 288, 288, 256, w4.PARTIAL_LAST_GROUP, P(0x100), P(0x200), P(0x400)) == w4.OK
    assert Q(P(), 64, 256, 48, 0, P(0x100), P(0x200), P(0x400)) == w4.ERR_GROUP
    assert Q(P(0x8), 64, 256, 64, 0, P(0x100), P(0x200), P(0x400)) == w4.ERR_ALIGN
    assert Q(P(), 64, 256, 64, 0x10, P(0x100), P(0x200), P(0x400)) == w4.ERR_FLAGS
    assert Q(P(), 64, 256, 64, w4.BF16, P(0x100), P(0x200), P(0x400)) == w4.ERR_FLAGS
    # the bf16 flag is accepted by repack, dequant and gemm
    assert L.w4a16_check_dequant_args(P(), P(0x100), P(0x200), 64, 256, 64, w4.BF16,
                                      P(0x400)) == w4.OK


def test_build_rejects_spilling_kernels():
    """The build's guard reads the compiler's resource-usage remarks: a kernel
    with scratch or spilled vector registers is reported, scalar spills (into
    lanes of a reserved vector register) and clean kernels are not."""
    from weight_only_int4_02_amd.build import spilled_kernels
    remarks = "\n".join([
        "k.hpp:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "k.hpp:1:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "k.hpp:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "k.hpp:1:1: remark:     SGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]",
        "k.hpp:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "k.hpp:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "k.hpp:9:1: remark:     ScratchSize [bytes/lane]: 36 [-Rpass-analysis=kernel-resource-usage]",
        "k.hpp:9:1: remark:     VGPRs Spill: 9 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert spilled_kernels(remarks) == [("kern_b", "ScratchSize [bytes/lane]", 36),
                                        ("kern_b", "VGPRs Spill", 9)]
