"""CPU oracle for the W4A16 group-quantized GEMM  Y = X . dequant(Q)^T.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package.  It shares no code with the GPU library
(``weight_only_int4_02_amd``) and imports nothing from it.

Two independent implementations of the same definitions live here:

* ``liboracle_w4a16.so`` -- plain C, fp64 (``w4a16_oracle.c``), wrapped below
  with ctypes.  This is *the* oracle.
* a numpy twin (functions prefixed ``np_``), used by the CPU tests to pin the
  C oracle: numpy's float64 -> float16 cast and BLAS matmul are textbook
  routines the C code does not use.

Citations (the source pages):
  [W4A16]     lmdeploy PR "[Feature] Blazing fast W4A16 inference": 4-bit
              weights x 16-bit activations; AWQ-format conversion with
              ``--group_size 128`` (group-wise quantization).
  [FP16xINT4] the Marlin post on the "KPD" Telegram channel: fp16 x int4
              mixed-precision linear layer.
  [PARTIAL]   torchchat issue "linear:int4 quantization regression testing":
              288x288 weight vs group size 256; option 2, a groupwise GEMM
              whose last group is not full; option 1, padding.

Readings where the pages are silent (dequant formula, nibble order, zero and
scale storage, error bound) are those stated in ``w4a16_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_w4a16.so")
_lib = None

SYMMETRIC_ZERO = 8


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP) into liboracle_w4a16.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I32 = ctypes.c_int32
        L.o_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.o_f16_to_f64.restype = ctypes.c_double
        L.o_f64_to_f16_rne.argtypes = [ctypes.c_double]
        L.o_f64_to_f16_rne.restype = ctypes.c_uint16
        L.o_pack.argtypes = [P, I64, I64, P]
        L.o_unpack.argtypes = [P, I64, I64, P]
        L.o_dequant.argtypes = [P, P, P, I64, I64, I32, ctypes.c_int, P]
        L.o_gemm_rows.argtypes = [P, I64, I64, P, P, P, I32, ctypes.c_int, P,
                                  I64, P, P]
        L.o_num_threads.restype = ctypes.c_int
        L.o_f64_to_16_array.argtypes = [P, I64, ctypes.c_int, P]
        L.o_f64_to_16_array.restype = None
        L.o_set_num_threads.argtypes = [ctypes.c_int]
        L.o_set_num_threads.restype = None
        L.o_repack.argtypes = [P, P, P, I64, I64, I32, ctypes.c_int, P, P, P]
        L.o_unrepack_q.argtypes = [P, I64, I64, P]
        L.o_quantize.argtypes = [P, I64, I64, I32, ctypes.c_int, P, P, P]
        L.o_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.o_bf16_to_f64.restype = ctypes.c_double
        L.o_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        L.o_f64_to_bf16_rne.restype = ctypes.c_uint16
        L.o_dequant_fmt.argtypes = [P, P, P, I64, I64, I32, ctypes.c_int, ctypes.c_int, P]
        L.o_gemm_rows_fmt.argtypes = [P, I64, I64, P, P, P, I32, ctypes.c_int, ctypes.c_int,
                                      P, I64, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------------------
# C oracle wrappers
# ---------------------------------------------------------------------------

def f16_bits_to_f64(bits: int) -> float:
    return lib().o_f16_to_f64(bits)


def f64_to_f16_bits(v: float) -> int:
    return lib().o_f64_to_f16_rne(v)


def pack(codes: np.ndarray) -> np.ndarray:
    """uint8 [R, C] -> uint32 [R, ceil(C/8)], low nibble first. [W4A16]"""
    codes = _c(codes, np.uint8)
    R, C = codes.shape
    out = np.empty((R, (C + 7) // 8), np.uint32)
    lib().o_pack(_p(codes), R, C, _p(out))
    return out


def unpack(words: np.ndarray, C: int) -> np.ndarray:
    words = _c(words, np.uint32)
    R = words.shape[0]
    out = np.empty((R, C), np.uint8)
    lib().o_unpack(_p(words), R, C, _p(out))
    return out


def n_groups(K: int, g: int) -> int:
    return (K + g - 1) // g


def dequant(qp, scales, zp, K: int, g: int, symmetric: bool) -> np.ndarray:
    """Canonical packed weight -> W fp16 [N, K], RNE((q - z) * s). [W4A16]"""
    qp = _c(qp, np.uint32)
    s = _c(scales, np.float16)
    zp = None if symmetric else _c(zp, np.uint32)
    N = qp.shape[0]
    W = np.empty((N, K), np.float16)
    lib().o_dequant(_p(qp), _p(s), _p(zp), N, K, g, int(symmetric), _p(W))
    return W


def gemm_rows(X, qp, scales, zp, K: int, g: int, symmetric: bool, rows=None):
    """fp64 Y for the selected weight rows: returns (y [M, len(rows)],
    wnorm2 [len(rows)]).  rows=None means every row. [W4A16] [FP16xINT4]"""
    X = _c(X, np.float16)
    qp = _c(qp, np.uint32)
    s = _c(scales, np.float16)
    zp = None if symmetric else _c(zp, np.uint32)
    M = X.shape[0]
    assert X.shape[1] == K
    N = qp.shape[0]
    if rows is None:
        rows = np.arange(N, dtype=np.int64)
    rows = _c(rows, np.int64)
    y = np.empty((M, rows.size), np.float64)
    wn = np.empty(rows.size, np.float64)
    lib().o_gemm_rows(_p(X), M, K, _p(qp), _p(s), _p(zp), g, int(symmetric),
                      _p(rows), rows.size, _p(y), _p(wn))
    return y, wn


def gemm_dense(X, qp, scales, zp, K: int, g: int, symmetric: bool, bf16: bool = False):
    """The same fp64 product as gemm_rows, every row, with the sum over k done
    by a library matmul (numpy, fp64) of X and the oracle's dequantized W.
    Only the order of the fp64 additions differs from gemm_rows, so the two
    are equal bit for bit wherever every partial sum is exact in fp64 -- the
    exact family (integer X, power-of-two scales), used to check whole
    outputs at sizes the sequential loop would take minutes over.  X and the
    scales are fp16 arrays, or bfloat16 bit patterns with bf16=True."""
    if bf16:
        W = bf16_bits_to_f64_array(dequant_bf16(qp, scales, zp, K, g, symmetric))
        Xd = bf16_bits_to_f64_array(X)
    else:
        W = dequant(qp, scales, zp, K, g, symmetric).astype(np.float64)
        Xd = np.asarray(X, np.float16).astype(np.float64)
    return Xd @ W.T


def bf16_bits_to_f64(bits: int) -> float:
    return lib().o_bf16_to_f64(bits)


def f64_to_bf16_bits(v: float) -> int:
    return lib().o_f64_to_bf16_rne(v)


def f64_to_bf16_bits_array(v) -> np.ndarray:
    """RNE_bf16 of every element of an fp64 array, as bit patterns (uint16)."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().o_f64_to_16_array(_p(v), v.size, 1, _p(out))
    return out


def f64_to_f16_bits_array(v) -> np.ndarray:
    """RNE_fp16 of every element of an fp64 array, as bit patterns (uint16)."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().o_f64_to_16_array(_p(v), v.size, 0, _p(out))
    return out


def dequant_bf16(qp, scales_bits, zp, K: int, g: int, symmetric: bool) -> np.ndarray:
    """bf16 variant of dequant: scales and W as bfloat16 bit patterns
    (uint16).  W = RNE_bf16((q - z) * s)."""
    qp = _c(qp, np.uint32)
    s = _c(scales_bits, np.uint16)
    zp = None if symmetric else _c(zp, np.uint32)
    N = qp.shape[0]
    W = np.empty((N, K), np.uint16)
    lib().o_dequant_fmt(_p(qp), _p(s), _p(zp), N, K, g, int(symmetric), 1, _p(W))
    return W


def gemm_rows_bf16(X_bits, qp, scales_bits, zp, K: int, g: int, symmetric: bool, rows=None):
    """bf16 variant of gemm_rows: X and scales as bfloat16 bit patterns."""
    X = _c(X_bits, np.uint16)
    qp = _c(qp, np.uint32)
    s = _c(scales_bits, np.uint16)
    zp = None if symmetric else _c(zp, np.uint32)
    M = X.shape[0]
    assert X.shape[1] == K
    N = qp.shape[0]
    if rows is None:
        rows = np.arange(N, dtype=np.int64)
    rows = _c(rows, np.int64)
    y = np.empty((M, rows.size), np.float64)
    wn = np.empty(rows.size, np.float64)
    lib().o_gemm_rows_fmt(_p(X), M, K, _p(qp), _p(s), _p(zp), g, int(symmetric), 1,
                          _p(rows), rows.size, _p(y), _p(wn))
    return y, wn


def quantize(W, g: int, symmetric: bool):
    """Round-to-nearest group quantizer (see o_quantize).  W fp16 [N, K] (any
    K; the last group may be partial) -> (codes uint8 [N, K], scales fp16
    [N, G], zeros uint8 [N, G])."""
    Wb = np.ascontiguousarray(np.asarray(W, dtype=np.float16)).view(np.uint16)
    N, K = Wb.shape
    G = n_groups(K, g)
    codes = np.empty((N, K), np.uint8)
    sc = np.empty((N, G), np.uint16)
    zr = np.empty((N, G), np.uint8)
    lib().o_quantize(_p(Wb), N, K, g, int(symmetric), _p(codes), _p(sc), _p(zr))
    return codes, sc.view(np.float16), zr


def num_threads() -> int:
    return lib().o_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the OpenMP loops use from now on (at least 1)."""
    lib().o_set_num_threads(int(n))


def repack_sizes(N: int, K: int, g: int, symmetric: bool):
    """Element counts of (q_dev uint32, s_dev fp16, z_dev uint32)."""
    NT, KT = (N + 15) // 16, (K + 127) // 128
    G = n_groups(K, g)
    GW = (G + 7) // 8
    return NT * KT * 256, NT * G * 16, 0 if symmetric else NT * GW * 16


def repack(qp, scales, zp, K: int, g: int, symmetric: bool):
    """Canonical -> the 16x128 tile device layout (see w4a16_oracle.c)."""
    qp = _c(qp, np.uint32)
    s = _c(scales, np.float16)
    zp = None if symmetric else _c(zp, np.uint32)
    N = qp.shape[0]
    nq, ns, nz = repack_sizes(N, K, g, symmetric)
    qd = np.empty(nq, np.uint32)
    sd = np.empty(ns, np.float16)
    zd = np.empty(max(nz, 1), np.uint32)
    lib().o_repack(_p(qp), _p(s), _p(zp), N, K, g, int(symmetric), _p(qd),
                   _p(sd), _p(zd))
    return qd, sd, (None if symmetric else zd[:nz])


def unrepack_q(qd, N: int, K: int) -> np.ndarray:
    qd = _c(qd, np.uint32)
    out = np.empty((N, (K + 7) // 8), np.uint32)
    lib().o_unrepack_q(_p(qd), N, K, _p(out))
    return out


# ---------------------------------------------------------------------------
# Error bound of the GEMM result
# ---------------------------------------------------------------------------

def ulp16(v: np.ndarray) -> np.ndarray:
    """Spacing of binary16 values at |v| (v kept in fp64): 2^(floor(log2|v|)
    - 10) for |v| >= 2^-14, else the subnormal quantum 2^-24."""
    a = np.abs(np.asarray(v, np.float64))
    out = np.full(a.shape, 2.0 ** -24)
    big = a >= 2.0 ** -14
    _, e = np.frexp(a[big])          # a = f * 2^e, f in [0.5, 1)
    out[big] = np.ldexp(1.0, e - 1 - 10)
    return out


def y_bound(X, y_ref, wnorm2, rows=None):
    """|y - y_ref| <= 2e-3 * ||x_m||_2 * ||w_n||_2 + ulp16(y_ref), norms in
    fp64 over the fp16 X row and the fp16 dequantized W row."""
    xn = np.sqrt((np.asarray(X, np.float16).astype(np.float64) ** 2).sum(1))
    return 2e-3 * xn[:, None] * np.sqrt(wnorm2)[None, :] + ulp16(y_ref)


def check_y(y_gpu, X, y_ref, wnorm2):
    """Returns (ok, worst_ratio) for fp16 y_gpu [M, R] against fp64 y_ref."""
    err = np.abs(np.asarray(y_gpu, np.float16).astype(np.float64) - y_ref)
    b = y_bound(X, y_ref, wnorm2)
    ratio = err / b
    return bool(np.all(err <= b)), float(ratio.max()) if ratio.size else 0.0


def bf16_bits_to_f64_array(bits) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns (the upper half of binary32)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |v|: 2^(floor(log2|v|) - 7) for
    |v| >= 2^-126, else the subnormal quantum 2^-133."""
    a = np.abs(np.asarray(v, np.float64))
    out = np.full(a.shape, 2.0 ** -133)
    big = a >= 2.0 ** -126
    _, e = np.frexp(a[big])
    out[big] = np.ldexp(1.0, e - 1 - 7)
    return out


def y_bound_bf16(X_bits, y_ref, wnorm2):
    """|y - y_ref| <= 2^-7 * ||x_m||_2 * ||w_n||_2 + ulp_bf16(y_ref): the fp16
    bound's construction (four units of the dequantized weight's rounding,
    2e-3 ~ 4 * 2^-11 there, plus one unit of the output format) carried to
    bfloat16's 8-bit significand."""
    xn = np.sqrt((bf16_bits_to_f64_array(X_bits) ** 2).sum(1))
    return 2.0 ** -7 * xn[:, None] * np.sqrt(wnorm2)[None, :] + ulp_bf16(y_ref)


def check_y_bf16(y_gpu_bits, X_bits, y_ref, wnorm2):
    """Returns (ok, worst_ratio) for bf16 y_gpu (bit patterns) against y_ref."""
    err = np.abs(bf16_bits_to_f64_array(y_gpu_bits) - y_ref)
    b = y_bound_bf16(X_bits, y_ref, wnorm2)
    ratio = err / b
    return bool(np.all(err <= b)), float(ratio.max()) if ratio.size else 0.0


# ---------------------------------------------------------------------------
# numpy twin (pins the C oracle; not used as the oracle itself)
# ---------------------------------------------------------------------------

def np_unpack(words, C):
    words = np.asarray(words, np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    nibs = (words[:, :, None] >> shifts[None, None, :]) & 0xF
    return nibs.reshape(words.shape[0], -1)[:, :C].astype(np.uint8)


def np_dequant(qp, scales, zp, K, g, symmetric):
    q = np_unpack(qp, K).astype(np.int64)
    G = n_groups(K, g)
    if symmetric:
        z = np.full((q.shape[0], G), SYMMETRIC_ZERO, np.int64)
    else:
        z = np_unpack(zp, G).astype(np.int64)
    gi = np.arange(K) // g
    s = np.asarray(scales, np.float16).astype(np.float64)
    return ((q - z[:, gi]).astype(np.float64) * s[:, gi]).astype(np.float16)
