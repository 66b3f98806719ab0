"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a closed form, a hand-worked
example (tests/golden), exact integer arithmetic, numpy's correctly rounded
float64 -> float16 cast over the whole finite fp16 domain, or a brute-force
numpy fp64 matmul.
"""
import os
import zlib

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# fp16 <-> fp64 (IEEE binary16 definition vs numpy's conversions)
# --------------------------------------------------------------------------

def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_bits_to_f64(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.signbit(oracle.f16_bits_to_f64(0x8000))


def test_f16_round_all_finite_values_and_midpoints():
    fin = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = fin.view(np.float16)
    fin = fin[np.isfinite(v)]
    vals = fin.view(np.float16).astype(np.float64)
    # every finite fp16 value encodes to itself
    got = np.array([oracle.f64_to_f16_bits(float(x)) for x in vals], np.uint16)
    assert np.array_equal(got, fin)
    # midpoints between neighbours (ties to even) and points just around them
    pos = np.sort(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2
    for probe in (mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)):
        want = probe.astype(np.float16).view(np.uint16)
        got = np.array([oracle.f64_to_f16_bits(float(x)) for x in probe], np.uint16)
        assert np.array_equal(got, want)


def test_f16_round_overflow_underflow_special():
    f = oracle.f64_to_f16_bits
    assert f(65504.0) == 0x7BFF
    assert f(65519.999) == 0x7BFF          # below the midpoint to 2^16
    assert f(65520.0) == 0x7C00            # the tie rounds to even -> inf
    assert f(-1e10) == 0xFC00
    assert f(2.0 ** -25) == 0x0000         # tie between 0 and 2^-24 -> even (0)
    assert f(2.0 ** -25 * 1.5) == 0x0001
    assert f(-0.0) == 0x8000
    assert f(float("inf")) == 0x7C00
    assert (f(float("nan")) & 0x7C00) == 0x7C00 and (f(float("nan")) & 0x3FF)


def test_f16_round_random_doubles():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000))
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16_bits(float(a)) for a in x], np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# pack / unpack (closed form: low nibble first)
# --------------------------------------------------------------------------

def test_pack_closed_form():
    codes = np.arange(8, dtype=np.uint8)[None, :]
    assert oracle.pack(codes)[0, 0] == 0x76543210
    codes = np.array([[0xF, 0, 0, 0, 0, 0, 0, 0xA]], np.uint8)
    assert oracle.pack(codes)[0, 0] == 0xA000000F


def test_pack_all_single_nibble_words():
    for pos in range(8):
        for v in range(16):
            codes = np.zeros((1, 8), np.uint8)
            codes[0, pos] = v
            assert oracle.pack(codes)[0, 0] == v << (4 * pos)


def test_pack_keeps_low_four_bits_and_pads_tail():
    codes = np.array([[0x1F, 0xF2, 3]], np.uint8)  # C = 3: one word
    assert oracle.pack(codes)[0, 0] == 0x32F
    codes = np.arange(10, dtype=np.uint8)[None, :]  # C = 10: two words
    w = oracle.pack(codes)
    assert w.shape == (1, 2) and w[0, 0] == 0x76543210 and w[0, 1] == 0x98


def test_pack_roundtrip_random():
    rng = np.random.default_rng(2)
    for R, C in [(3, 8), (5, 40), (17, 101), (64, 512)]:
        codes = rng.integers(0, 16, (R, C), dtype=np.uint8)
        w = oracle.pack(codes)
        assert np.array_equal(oracle.unpack(w, C), codes)
        assert np.array_equal(oracle.np_unpack(w, C), codes)


# --------------------------------------------------------------------------
# E1: the hand-worked 2 x 8 x 8 example
# --------------------------------------------------------------------------

def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *vals = line.split()
                out[key] = vals
    return out


def _e1_inputs():
    n = np.arange(8)[:, None]
    k = np.arange(8)[None, :]
    codes = ((n + k) % 16).astype(np.uint8)
    zeros = np.stack([np.full(8, 8), np.arange(8)], 1).astype(np.uint8)
    scales = np.tile(np.array([1.0, 0.5], np.float16), (8, 1))
    X = np.zeros((2, 8), np.float16)
    X[0, 0] = 1
    X[1] = np.arange(1, 9)
    return codes, zeros, scales, X


def test_e1_worked_example():
    gold = _golden("e1_worked_2x8x8.txt")
    codes, zeros, scales, X = _e1_inputs()
    qp = oracle.pack(codes)
    zp = oracle.pack(zeros)
    assert [int(v, 16) for v in gold["packed_words"]] == list(qp[:, 0])
    assert [int(v, 16) for v in gold["packed_zeros"]] == list(zp[:, 0])
    assert [int(v, 16) for v in gold["scales_bits"]] == list(scales[0].view(np.uint16))
    W = oracle.dequant(qp, scales, zp, 8, 4, False)
    for nn in range(8):
        want = [float(eval(t.replace("n", str(nn)))) for t in gold["W_row_n"]]
        assert list(W[nn].astype(np.float64)) == want
    y, _ = oracle.gemm_rows(X, qp, scales, zp, 8, 4, False)
    assert list(y[0]) == [float(v) for v in gold["Y_row0"]]
    assert list(y[1]) == [float(v) for v in gold["Y_row1"]]


def test_e1_detects_planted_mistakes():
    """The golden values tell apart the likely misreadings (checked on a
    deliberately wrong numpy variant, never on the GPU path)."""
    gold = _golden("e1_worked_2x8x8.txt")
    codes, zeros, scales, X = _e1_inputs()
    # high-nibble-first reading of the packed words: code k read from nibble 7-k
    qp = oracle.pack(codes)
    zp = oracle.pack(zeros)
    qp_wrong = oracle.pack(codes[:, ::-1])
    W = oracle.np_dequant(qp_wrong, scales, zp, 8, 4, False)
    y0 = X[0].astype(np.float64) @ W.astype(np.float64).T
    assert list(y0) == [-1.0, 0, 1, 2, 3, 4, 5, 6]
    assert list(y0) != [float(v) for v in gold["Y_row0"]]
    # scales read as [G][N] instead of [N][G]
    s_t = scales.reshape(-1).reshape(2, 8).T
    W = oracle.np_dequant(qp, s_t, zp, 8, 4, False)
    y0 = X[0].astype(np.float64) @ W.astype(np.float64).T
    assert list(y0) != [float(v) for v in gold["Y_row0"]]


# --------------------------------------------------------------------------
# E2: z = 8, s = 1 reproduces X . (q - 8)^T exactly (integer matmul)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,g", [(3, 24, 64, 32), (5, 17, 288, 256), (1, 40, 512, 128)])
def test_e2_identity_against_int64(M, N, K, g):
    rng = np.random.default_rng(M * 1000 + N)
    codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
    X = rng.integers(-64, 65, (M, K)).astype(np.float16)
    G = -(-K // g)
    scales = np.ones((N, G), np.float16)
    qp = oracle.pack(codes)
    for sym in (True, False):
        zp = None if sym else oracle.pack(np.full((N, G), 8, np.uint8))
        y, _ = oracle.gemm_rows(X, qp, scales, zp, K, g, sym)
        want = X.astype(np.int64) @ (codes.astype(np.int64) - 8).T
        assert np.array_equal(y, want.astype(np.float64))


# --------------------------------------------------------------------------
# E3: the exact family -- integer X, power-of-two scales -- vs int64
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,g,sym", [(4, 32, 512, 128, False), (3, 16, 288, 256, False),
                                         (2, 20, 256, 32, True), (7, 9, 11008 // 8, 64, False)])
def test_e3_exact_family_against_int64(M, N, K, g, sym):
    c = workloads.exact_family(M, N, K, g, sym, seed=K + N)
    zeros = np.full((N, c.G), 8, np.int64) if sym else c.zeros.astype(np.int64)
    e = -np.log2(c.scales.astype(np.float64))
    assert np.all(e == np.round(e))
    gi = np.arange(K) // g
    # w * 2^7 = (q - z) * 2^(7 - e), an integer
    w7 = (c.codes.astype(np.int64) - zeros[:, gi]) * (2 ** (7 - e.astype(np.int64)))[:, gi]
    want = (c.X.astype(np.int64) @ w7.T).astype(np.float64) / 128.0
    qp = oracle.pack(c.codes)
    zp = None if sym else oracle.pack(c.zeros)
    y, _ = oracle.gemm_rows(c.X, qp, c.scales, zp, K, g, sym)
    assert np.array_equal(y, want)


def test_array_encoders_match_the_scalar_ones_and_numpy():
    """The array forms of the fp16 / bf16 encoders agree element by element
    with the scalar encoders, and the fp16 one with numpy's correctly rounded
    float64 -> float16 cast, on random values, exact midpoints and ties."""
    rng = np.random.default_rng(16)
    v = np.concatenate([rng.standard_normal(4000) * np.ldexp(1.0, rng.integers(-30, 20, 4000)),
                        (np.arange(-300, 300) + 0.5) * 2.0 ** -10,      # fp16 ties
                        (np.arange(-300, 300) + 0.5) * 2.0 ** -7,       # bf16 ties
                        [0.0, -0.0, 65520.0, 1e300, -1e-300]])
    f16 = oracle.f64_to_f16_bits_array(v)
    assert f16.tolist() == [oracle.f64_to_f16_bits(float(x)) for x in v]
    with np.errstate(over="ignore"):
        assert np.array_equal(f16, v.astype(np.float16).view(np.uint16))
    bf = oracle.f64_to_bf16_bits_array(v)
    assert bf.tolist() == [oracle.f64_to_bf16_bits(float(x)) for x in v]


@pytest.mark.parametrize("M,N,K,g,sym", [(4, 32, 512, 128, False), (3, 16, 288, 256, False),
                                         (2, 20, 256, 32, True), (7, 9, 11008 // 8, 64, False)])
def test_gemm_dense_equals_the_sequential_sum_on_the_exact_family(M, N, K, g, sym):
    """gemm_dense (a library fp64 matmul of the dequantized weight) gives the
    int64-exact result of E3, bit for bit, in fp16 and in bf16; on random
    data it differs from gemm_rows only by the order of fp64 additions."""
    c = workloads.exact_family(M, N, K, g, sym, seed=K + N)
    qp = oracle.pack(c.codes)
    zp = None if sym else oracle.pack(c.zeros)
    y, _ = oracle.gemm_rows(c.X, qp, c.scales, zp, K, g, sym)
    assert np.array_equal(oracle.gemm_dense(c.X, qp, c.scales, zp, K, g, sym), y)
    b = workloads.exact_family_bf16(M, N, K, g, sym, seed=K + N)
    zb = None if sym else oracle.pack(b.zeros)
    yb, _ = oracle.gemm_rows_bf16(b.X, oracle.pack(b.codes), b.scales, zb, K, g, sym)
    assert np.array_equal(oracle.gemm_dense(b.X, oracle.pack(b.codes), b.scales, zb, K, g, sym,
                                            bf16=True), yb)
    r = workloads.draw(M, N, K, g, sym, seed=K + N + 1)
    zr = None if sym else oracle.pack(r.zeros)
    yr, _ = oracle.gemm_rows(r.X, oracle.pack(r.codes), r.scales, zr, K, g, sym)
    W = oracle.dequant(oracle.pack(r.codes), r.scales, zr, K, g, sym).astype(np.float64)
    scale = np.abs(r.X.astype(np.float64)) @ np.abs(W).T
    assert np.all(np.abs(oracle.gemm_dense(r.X, oracle.pack(r.codes), r.scales, zr, K, g, sym) - yr)
                  <= 1e-12 * scale)


# --------------------------------------------------------------------------
# E4: partial last group == zero-padding to whole groups
# --------------------------------------------------------------------------

def test_e4_partial_group_equals_padding():
    rng = np.random.default_rng(4)
    M, N, K, g, Kp = 3, 288, 288, 256, 512
    c = workloads.draw(M, N, K, g, False, seed=44)
    # padded problem: codes beyond K arbitrary, X zero beyond K, same s and z
    codes_p = np.concatenate([c.codes, rng.integers(0, 16, (N, Kp - K), dtype=np.uint8)], 1)
    Xp = np.concatenate([c.X, np.zeros((M, Kp - K), np.float16)], 1)
    y, _ = oracle.gemm_rows(c.X, oracle.pack(c.codes), c.scales, oracle.pack(c.zeros), K, g, False)
    yp, _ = oracle.gemm_rows(Xp, oracle.pack(codes_p), c.scales, oracle.pack(c.zeros), Kp, g, False)
    assert np.array_equal(y, yp)
    # the last group is 32 wide: columns 256..287 use group 1
    W = oracle.dequant(oracle.pack(c.codes), c.scales, oracle.pack(c.zeros), K, g, False)
    z1 = c.zeros[:, 1].astype(np.float64)
    s1 = c.scales[:, 1].astype(np.float64)
    want = ((c.codes[:, 256:].astype(np.float64) - z1[:, None]) * s1[:, None]).astype(np.float16)
    assert np.array_equal(W[:, 256:], want)


# --------------------------------------------------------------------------
# E5: brute force on tiny shapes vs numpy's fp64 matmul
# --------------------------------------------------------------------------

def test_e5_brute_force_tiny():
    rng = np.random.default_rng(5)
    n_cases = 0
    for M in range(1, 6):
        for K in range(8, 97, 8):
            for g in (32, 64):
                for sym in (False, True):
                    N = int(rng.integers(1, 41))
                    c = workloads.draw(M, N, K, g, sym, seed=int(rng.integers(1 << 30)))
                    qp = oracle.pack(c.codes)
                    zp = None if sym else oracle.pack(c.zeros)
                    W = oracle.dequant(qp, c.scales, zp, K, g, sym)
                    assert np.array_equal(W.view(np.uint16),
                                          oracle.np_dequant(qp, c.scales, zp, K, g, sym).view(np.uint16))
                    y, wn = oracle.gemm_rows(c.X, qp, c.scales, zp, K, g, sym)
                    ref = c.X.astype(np.float64) @ W.astype(np.float64).T
                    scale = np.abs(c.X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
                    assert np.all(np.abs(y - ref) <= 1e-12 * scale + 1e-300)
                    assert np.allclose(wn, (W.astype(np.float64) ** 2).sum(1), rtol=1e-14)
                    n_cases += 1
    assert n_cases == 5 * 12 * 2 * 2


def test_gemm_rows_subset_matches_full():
    c = workloads.draw(3, 50, 160, 32, False, seed=9)
    qp, zp = oracle.pack(c.codes), oracle.pack(c.zeros)
    y, wn = oracle.gemm_rows(c.X, qp, c.scales, zp, 160, 32, False)
    rows = np.array([49, 0, 17, 17, 3])
    ys, wns = oracle.gemm_rows(c.X, qp, c.scales, zp, 160, 32, False, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(wns, wn[rows])


# --------------------------------------------------------------------------
# E6: dequant over the whole finite fp16 scale domain x all (q, z) pairs
# --------------------------------------------------------------------------

def test_e6_dequant_exhaustive_against_numpy_cast():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = bits.view(np.float16)
    s = s[np.isfinite(s)]
    assert s.size == 63488
    N, K, g = s.size, 256, 16            # group j holds q = 0..15 with zero z = j
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, 16))
    zeros = np.tile(np.arange(16, dtype=np.uint8), (N, 1))
    scales = np.repeat(s[:, None], 16, 1)
    W = oracle.dequant(oracle.pack(codes), scales, oracle.pack(zeros), K, g, False)
    q = np.tile(np.arange(16), 16).astype(np.float64)
    z = np.repeat(np.arange(16), 16).astype(np.float64)
    with np.errstate(over="ignore"):   # products past 65504 round to inf
        want = ((q - z)[None, :] * s.astype(np.float64)[:, None]).astype(np.float16)
    assert np.array_equal(W.view(np.uint16), want.view(np.uint16))


# --------------------------------------------------------------------------
# device layout: definition by worked addresses, inverse, bijection
# --------------------------------------------------------------------------

def test_repack_worked_addresses():
    # N = 20 (two row tiles, the second ragged), K = 136 (two k tiles, ragged)
    N, K, g = 20, 136, 32
    codes = np.zeros((N, K), np.uint8)
    # (n, k) = (0, 0): tile (0, 0), lane 0, word 0, element 0 -> nibble 0
    codes[0, 0] = 0x1
    # (n, k) = (0, 1): element 1 -> nibble 4 of the same word
    codes[0, 1] = 0x2
    # (n, k) = (5, 32*1 + 8*2 + 6): lane 5 + 16*2 = 37, word 1, element 6 -> nibble 3
    codes[5, 54] = 0x3
    # (n, k) = (17, 128 + 7): tile (1, 1), lane 1, word 0, element 7 -> nibble 7
    codes[17, 135] = 0x4
    G = -(-K // g)
    scales = (np.arange(N * G).reshape(N, G) + 1).astype(np.float16)
    zeros = (np.arange(N * G).reshape(N, G) % 16).astype(np.uint8)
    qd, sd, zd = oracle.repack(oracle.pack(codes), scales, oracle.pack(zeros), K, g, False)
    KT = 2
    assert qd.size == 2 * KT * 256
    nz = np.flatnonzero(qd)
    assert list(nz) == [0, 37 * 4 + 1, ((1 * KT + 1) * 64 + 1) * 4 + 0]
    assert qd[0] == 0x00020001
    assert qd[37 * 4 + 1] == 0x3 << 12
    assert qd[((1 * KT + 1) * 64 + 1) * 4] == 0x4 << 28
    # scales [NT][G][16]: (n=17, group 3) -> [1][3][1]; padded rows are 0
    assert sd.reshape(2, G, 16)[1, 3, 1] == scales[17, 3]
    assert np.all(sd.reshape(2, G, 16)[1, :, 4:] == 0)
    # zeros [NT][GW][16] canonical words; GW = 1 here
    assert zd.reshape(2, 1, 16)[1, 0, 1] == oracle.pack(zeros)[17, 0]


@pytest.mark.parametrize("N,K,g", [(16, 128, 128), (48, 4096 // 8, 64), (288, 288, 256), (33, 200, 32)])
def test_repack_inverse_and_bijection(N, K, g):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
    G = -(-K // g)
    qp = oracle.pack(codes)
    zeros = rng.integers(0, 16, (N, G), dtype=np.uint8)
    scales = rng.uniform(0.002, 0.02, (N, G)).astype(np.float16)
    qd, sd, zd = oracle.repack(qp, scales, oracle.pack(zeros), K, g, False)
    assert np.array_equal(oracle.unrepack_q(qd, N, K), qp)
    # the nibble histogram is preserved (padding adds only zeros)
    nib = oracle.np_unpack(qd.reshape(1, -1), qd.size * 8)[0]
    h = np.bincount(nib, minlength=16)
    h0 = np.bincount(codes.reshape(-1), minlength=16)
    assert np.array_equal(h[1:], h0[1:]) and h[0] >= h0[0]
    qd2, sd2, zd2 = oracle.repack(qp, scales, None, K, g, True)
    assert zd2 is None and np.array_equal(qd2, qd) and np.array_equal(sd2, sd)


# --------------------------------------------------------------------------
# the error bound
# --------------------------------------------------------------------------

def test_ulp16_hand_values():
    v = np.array([1.0, 1.5, 2.0, 65504.0, 2.0 ** -14, 2.0 ** -15, 0.0, -3.0, 1000.0])
    want = np.array([2 ** -10, 2 ** -10, 2 ** -9, 32.0, 2 ** -24, 2 ** -24, 2 ** -24,
                     2 ** -9, 0.5])
    assert np.array_equal(oracle.ulp16(v), want)
    # equals the gap to the next fp16 value above |v| for normal fp16 values
    x = np.array([1.0, 3.0, 1000.0, 0.125], np.float16)
    gap = np.nextafter(x, np.float16(np.inf)).astype(np.float64) - x.astype(np.float64)
    assert np.array_equal(oracle.ulp16(x.astype(np.float64)), gap)


def test_check_y_accepts_bound_and_rejects_beyond():
    X = np.array([[3.0, 4.0]], np.float16)          # ||x|| = 5
    y_ref = np.array([[1.0]])
    wn2 = np.array([4.0])                            # ||w|| = 2
    b = 2e-3 * 5 * 2 + 2 ** -10
    ok, _ = oracle.check_y(np.array([[1.0]], np.float16), X, y_ref, wn2)
    assert ok
    inside = np.float16(1.0 + 0.0205)                # 1.0205078 -> err 0.0205 < b
    assert abs(float(inside) - 1.0) <= b
    assert oracle.check_y(np.array([[inside]]), X, y_ref, wn2)[0]
    outside = np.float16(1.0 + 0.03)
    assert abs(float(outside) - 1.0) > b
    assert not oracle.check_y(np.array([[outside]]), X, y_ref, wn2)[0]


# --------------------------------------------------------------------------
# F1: the round-to-nearest group quantizer (o_quantize)
# --------------------------------------------------------------------------

def test_f1_worked_examples():
    gold = _golden("f1_rtn_worked.txt")
    for case, sym in (("A", False), ("B", False), ("C", True), ("D", False),
                      ("E", False), ("F", False), ("G", True), ("H", False)):
        w = np.zeros((1, 32), np.float16)
        vals = [float(v) for v in gold[f"{case}_w"]]
        w[0, :len(vals)] = vals
        codes, s, z = oracle.quantize(w, 32, sym)
        assert int(s.view(np.uint16)[0, 0]) == int(gold[f"{case}_s"][0], 16), case
        assert int(z[0, 0]) == int(gold[f"{case}_z"][0]), case
        q = [int(v) for v in gold[f"{case}_q"]]
        assert codes[0, :len(q)].tolist() == q, case
        # the unlisted columns are 0 and take the code of 0
        assert np.all(codes[0, len(vals):] == (8 if sym else int(gold[f"{case}_z"][0])))


def _reciprocal_form_quantize(w, g, sym):
    """A plausible mistake, planted on the CPU: the quantizer rule with each
    division by s replaced by a product with fp32(1 / s)."""
    f = np.float32
    wf = np.zeros(g, np.float16)
    wf[:len(w)] = w
    wf = wf.astype(f)

    def s_up(t):
        h = np.float16(t)
        return np.nextafter(h, np.float16(np.inf)) if f(h) < t else h
    if sym:
        a = np.abs(wf).max()
        s, z = s_up(f(1) if a == 0 else a / f(7)), 8
    else:
        lo, hi = min(f(0), wf.min()), max(f(0), wf.max())
        s = s_up((hi - lo) / f(15))
        z = int(min(max(np.rint(-lo * (f(1) / f(s))), 0), 15))
    q = np.clip(np.rint(wf * (f(1) / f(s))).astype(int) + z, 0, 15)
    return z, q[:len(w)].tolist()


def test_f1_tie_goldens_reject_the_reciprocal_form():
    """Cases E..H hold exact ties whose scales have inexact fp32 reciprocals:
    the reciprocal form misses each of them, so the goldens pin division."""
    gold = _golden("f1_rtn_worked.txt")
    for case, sym in (("E", False), ("F", False), ("G", True), ("H", False)):
        w = [float(v) for v in gold[f"{case}_w"]]
        z, q = _reciprocal_form_quantize(w, 32, sym)
        want = (int(gold[f"{case}_z"][0]), [int(v) for v in gold[f"{case}_q"]])
        assert (z, q) != want, case
        codes, _, zz = oracle.quantize(np.array([w + [0.0] * (32 - len(w))], np.float16), 32, sym)
        assert (int(zz[0, 0]), codes[0, :len(w)].tolist()) == want, case


def _nearest_even(num, den):
    """Nearest integer to num / den (integers, den > 0), exact ties to even."""
    q, r = divmod(num, den)
    if 2 * r > den or (2 * r == den and q % 2 == 1):
        q += 1
    return q


def _mul_frac(a, b):
    """a / b for exact rationals a = (n, d), b = (n, d): (numerator, denominator)."""
    return a[0] * b[1], a[1] * b[0]


def _f16_exact(v):
    """fp16 value as an exact rational (numerator, power-of-two denominator)."""
    m, e = np.frexp(np.float64(v))
    num = int(np.ldexp(m, 53))
    e = int(e) - 53
    return (num << e, 1) if e >= 0 else (num, 1 << -e)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("sbits", [0x1700, 0x16AC, 0x2C45, 0x3400, 0x0203, 0x1E6B, 0x2A9D, 0x3BFF])
def test_f1_codes_are_exact_nearest_over_every_fp16_weight(sbits, sym):
    """For a fixed scale s, every fp16 w that a group with that scale can
    hold is coded as the nearest integer to the exact w / s (exact ties to
    even) plus z -- checked against integer arithmetic on the exact values,
    and against numpy's correctly rounded float32 division."""
    s = np.array([sbits], np.uint16).view(np.float16)[0]
    sf = float(s)
    f = np.float32

    def down16(v):   # largest fp16 <= v (v > 0)
        h = np.float16(v)
        return np.nextafter(h, np.float16(0)) if float(h) > v else h

    def scale_of(lo, hi):   # the rule's scale for a group of range [lo, hi]
        t = (f(hi) - f(lo)) / f(15) if not sym else f(max(-lo, hi)) / f(7)
        h = np.float16(t)
        return np.nextafter(h, np.float16(np.inf)) if f(h) < t else h
    # a group whose range fixes the scale at exactly s: lo = -a with a the
    # largest fp16 <= 7 s, and hi the largest fp16 whose range still gives s
    lo = -float(down16(7 * sf))
    hi = float(down16(8 * sf)) if not sym else -lo
    while scale_of(lo, hi) != s:
        hi = float(np.nextafter(np.float16(hi), np.float16(0)))
        assert hi > 0
    allw = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allw = allw[np.isfinite(allw)]
    ws = np.unique(allw[(allw >= lo) & (allw <= hi)])
    g = 256
    per = g - 2
    nrow = -(-len(ws) // per)
    W = np.zeros((nrow, g), np.float16)
    W[:, 0], W[:, 1] = lo, hi
    flat = np.zeros(nrow * per, np.float16)
    flat[:len(ws)] = ws
    W[:, 2:] = flat.reshape(nrow, per)
    codes, sc, zz = oracle.quantize(W, g, sym)
    assert np.all(sc.view(np.uint16) == sbits)
    z = 8 if sym else _nearest_even(*_mul_frac(_f16_exact(-lo), _f16_exact(s)))
    assert np.all(zz == z)
    got = codes[:, 2:].reshape(-1)[:len(ws)].astype(np.int64)
    sn, sd = _f16_exact(s)
    exact = []
    for w in ws:
        wn, wd = _f16_exact(w)
        exact.append(min(max(_nearest_even(wn * sd, wd * sn) + z, 0), 15))
    assert got.tolist() == exact
    npdiv = np.clip(np.rint(ws.astype(np.float32) / np.float32(s)).astype(np.int64) + z, 0, 15)
    assert np.array_equal(got, npdiv)
    # ties are present in the sweep, so the rule for them is exercised (a
    # subnormal scale with an odd significand has no fp16 half-multiples)
    ties = sum(2 * ((_f16_exact(w)[0] * sd) % (_f16_exact(w)[1] * sn)) == _f16_exact(w)[1] * sn
               for w in ws)
    assert ties > 0 or (sbits < 0x0400 and sbits % 2 == 1)


def _grid_weight(rng, N, K, g, sym):
    """W = (q - z) * 2^e exactly in fp16, every group spanning the full code
    range (asymmetric: codes 0 and 15 present; symmetric: |q - 8| = 7)."""
    G = -(-K // g)
    q = rng.integers(0, 16, (N, K)).astype(np.int64)
    e = rng.integers(-14, -1, (N, G))
    z = np.full((N, G), 8) if sym else rng.integers(0, 16, (N, G))
    for j in range(G):
        k0, k1 = j * g, min(K, (j + 1) * g)
        cols = rng.permutation(np.arange(k0, k1))[:2]
        if sym:
            q[:, k0:k1] = np.clip(q[:, k0:k1], 1, 15)
            q[:, cols[0]] = 15
        else:
            q[:, cols[0]], q[:, cols[1]] = 0, 15
    gi = np.arange(K) // g
    W = ((q - z[:, gi]) * np.ldexp(1.0, e[:, gi])).astype(np.float16)
    assert np.array_equal(W.astype(np.float64), (q - z[:, gi]) * np.ldexp(1.0, e[:, gi]))
    return W, q.astype(np.uint8), np.ldexp(1.0, e).astype(np.float16), z.astype(np.uint8)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("N,K,g", [(3, 64, 32), (5, 288, 256), (4, 520, 128), (2, 96, 64)])
def test_f1_recovers_grid_weights_exactly(N, K, g, sym):
    """A weight that already lies on a 4-bit grid with a power-of-two scale
    and uses its whole code range is quantized back to exactly that grid."""
    rng = np.random.default_rng(N * 1000 + K + sym)
    W, q, s, z = _grid_weight(rng, N, K, g, sym)
    codes, s2, z2 = oracle.quantize(W, g, sym)
    assert np.array_equal(codes, q)
    assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))
    assert np.array_equal(z2, z)


def _f1_inputs(rng, N, K, kind):
    if kind == "normal":
        return (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    if kind == "outliers":
        W = rng.standard_normal((N, K)) * 0.02
        W[rng.random((N, K)) < 0.01] *= 300
        return W.astype(np.float16)
    if kind == "extremes":
        return (rng.choice([-1, 1], (N, K)) * np.ldexp(1.0, rng.integers(-24, 16, (N, K)))
                * rng.uniform(1, 1.99, (N, K))).astype(np.float16)
    if kind == "positive":
        return np.abs(rng.standard_normal((N, K))).astype(np.float16) + np.float16(1)
    if kind == "sparse":
        W = rng.standard_normal((N, K)).astype(np.float16)
        W[rng.random((N, K)) < 0.9] = 0
        return W
    raise ValueError(kind)


KINDS = ["normal", "outliers", "extremes", "positive", "sparse"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_f1_error_at_most_half_a_step(kind, sym, g):
    """|(q - z) s - W| <= s/2 per element (closed form of rounding to the
    nearest grid point), every code is a nearest one, and exact ties take the
    even offset; the fp16 dequantized value adds at most half an fp16 ulp."""
    rng = np.random.default_rng(zlib.crc32(f"f1/{kind}/{sym}/{g}".encode()))
    N, K = 6, 2 * g + 40          # a partial last group
    W = _f1_inputs(rng, N, K, kind)
    codes, s, z = oracle.quantize(W, g, sym)
    assert codes.max() <= 15 and z.max() <= 15
    gi = np.arange(K) // g
    sd = s.astype(np.float64)[:, gi]
    zd = z.astype(np.float64)[:, gi]
    w = W.astype(np.float64)
    exact = (codes - zd) * sd
    err = np.abs(exact - w)
    assert np.all(err <= sd * 0.5)
    cand = (np.arange(16)[None, None, :] - zd[..., None]) * sd[..., None]
    best = np.abs(cand - w[..., None]).min(-1)
    assert np.all(err == best)
    # an exact tie takes the even offset q - z, unless the even neighbour
    # lies outside the code range 0..15
    tie = err == sd * 0.5
    off = codes - zd
    alt = off + np.where(exact < w, 1, -1)
    alt_in = (alt + zd >= 0) & (alt + zd <= 15)
    assert np.all((off[tie] % 2 == 0) | ~alt_in[tie])
    deq = oracle.dequant(oracle.pack(codes), s, None if sym else oracle.pack(z), K, g, sym)
    ulp = oracle.ulp16(np.abs(w) + sd)
    # the fp16 dequantized value overflows only where the grid point itself
    # lies past the fp16 range (a group reaching within s/2 of 65504)
    fin = np.abs(exact) < 65520
    assert np.all(np.isinf(deq[~fin])) and np.all(np.abs(w[~fin]) > 65504 - sd[~fin] / 2)
    assert np.all(np.abs(deq.astype(np.float64) - w)[fin] <= (sd * (0.5 + 2.0 ** -18) + ulp / 2)[fin])
    # zeros dequantize to exactly zero
    assert np.all(deq[W == 0] == 0)
    if sym:
        assert np.all(z == 8)


def test_f1_partial_group_equals_zero_padding():
    """The torchchat 288 x 288 case with g = 256: quantizing with a 32-wide
    last group gives the codes, scales and zeros of quantizing the weight
    padded with zero columns to 512."""
    rng = np.random.default_rng(288)
    W = (rng.standard_normal((288, 288)) * 0.05).astype(np.float16)
    Wp = np.zeros((288, 512), np.float16)
    Wp[:, :288] = W
    for sym in (False, True):
        c1, s1, z1 = oracle.quantize(W, 256, sym)
        c2, s2, z2 = oracle.quantize(Wp, 256, sym)
        assert np.array_equal(c1, c2[:, :288])
        assert np.array_equal(s1.view(np.uint16), s2.view(np.uint16))
        assert np.array_equal(z1, z2)


# --------------------------------------------------------------------------
# bfloat16 variant: format, dequantization, GEMM
# --------------------------------------------------------------------------

def _bf16_table():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        return bits, (bits << 16).view(np.float32).astype(np.float64)


def test_bf16_decode_all_patterns():
    bits, want = _bf16_table()
    got = np.array([oracle.bf16_bits_to_f64(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_round_values_midpoints_and_specials():
    """Every finite bfloat16 value rounds to itself; the midpoint of two
    neighbours rounds to the one with an even pattern; a hair either side of
    it rounds to the nearer one (brute force over all positive finite
    patterns, checked in fp64 where all of these are exact)."""
    bits, vals = _bf16_table()
    fin = np.isfinite(vals) & (vals >= 0)
    pos = bits[fin][:-1]
    lo, hi = vals[pos], vals[pos + 1]
    f = oracle.f64_to_bf16_bits
    for b, v in zip(pos[::7], lo[::7]):
        assert f(float(v)) == b
    idx = np.arange(0, pos.size, 5)
    for k in idx:
        a, b = lo[k], hi[k]
        mid = (a + b) / 2
        even = int(pos[k]) if pos[k] % 2 == 0 else int(pos[k]) + 1
        assert f(float(mid)) == even, (a, b)
        assert f(float(np.nextafter(mid, -np.inf))) == int(pos[k])
        assert f(float(np.nextafter(mid, np.inf))) == int(pos[k]) + 1
    # overflow: from the midpoint between the largest finite value and 2^128 on
    big = 2.0 ** 127 * (2 - 2 ** -7)
    assert f(big) == 0x7F7F
    assert f(2.0 ** 127 * (2 - 2 ** -8)) == 0x7F80
    assert f(float(np.nextafter(2.0 ** 127 * (2 - 2 ** -8), 0))) == 0x7F7F
    assert f(-np.inf) == 0xFF80 and f(0.0) == 0 and f(-0.0) == 0x8000
    assert f(2.0 ** -134) == 0 and f(float(np.nextafter(2.0 ** -134, 1))) == 1
    assert f(3 * 2.0 ** -134) == 2     # tie between 1 and 2 quanta -> even


def _bf16_rne_of_exact_f32(x):
    """Textbook nearest-even float32 -> bfloat16 (exact float32 inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_dequant_exhaustive_against_textbook_rounding():
    """RNE_bf16((q - z) * s) for every finite bf16 scale and every (q, z):
    the product has at most 13 significant bits, so it is exact in float32
    and the textbook float32 -> bfloat16 rounding gives the reference.
    Layout: row n has zero z = n in every group, column k has code
    q = k % 16, group j (32 columns) has the j-th finite scale."""
    bits, vals = _bf16_table()
    fin = np.isfinite(vals)
    sb = bits[fin].astype(np.uint16)
    G = sb.size
    assert G == 65536 - 2 * 128
    N, g = 16, 32
    K = G * g
    codes = np.tile((np.arange(K) % 16).astype(np.uint8), (N, 1))
    zeros = np.repeat(np.arange(N, dtype=np.uint8)[:, None], G, 1)
    scales = np.tile(sb, (N, 1))
    W = oracle.dequant_bf16(oracle.pack(codes), scales, oracle.pack(zeros), K, g, False)
    qz = (np.arange(K) % 16)[None, :] - np.arange(N)[:, None]            # [N, K]
    with np.errstate(over="ignore"):
        prod = qz.astype(np.float32) * np.repeat(vals[fin].astype(np.float32), g)[None, :]
    assert np.array_equal(W, _bf16_rne_of_exact_f32(prod))


@pytest.mark.parametrize("M,N,K,g,sym", [(4, 32, 512, 128, False), (3, 16, 288, 256, False),
                                         (2, 20, 256, 32, True)])
def test_bf16_exact_family_against_int64(M, N, K, g, sym):
    c = workloads.exact_family_bf16(M, N, K, g, sym, seed=K + N)
    x = oracle.bf16_bits_to_f64_array(c.X)
    s = oracle.bf16_bits_to_f64_array(c.scales)
    e = -np.log2(s)
    assert np.all(e == np.round(e)) and np.all(x == np.round(x))
    gi = np.arange(K) // g
    zeros = np.full((N, -(-K // g)), 8, np.int64) if sym else c.zeros.astype(np.int64)
    w7 = (c.codes.astype(np.int64) - zeros[:, gi]) * (2 ** (7 - e.astype(np.int64)))[:, gi]
    want = (x.astype(np.int64) @ w7.T).astype(np.float64) / 128.0
    y, _ = oracle.gemm_rows_bf16(c.X, oracle.pack(c.codes), c.scales,
                                 None if sym else oracle.pack(c.zeros), K, g, sym)
    assert np.array_equal(y, want)


def test_bf16_brute_force_tiny():
    rng = np.random.default_rng(15)
    for M in (1, 3):
        for K in (8, 40, 96):
            for g in (32, 64):
                N = int(rng.integers(1, 30))
                c = workloads.draw_bf16(M, N, K, g, False, seed=int(rng.integers(1 << 30)))
                qp, zp = oracle.pack(c.codes), oracle.pack(c.zeros)
                W = oracle.bf16_bits_to_f64_array(oracle.dequant_bf16(qp, c.scales, zp, K, g, False))
                y, wn = oracle.gemm_rows_bf16(c.X, qp, c.scales, zp, K, g, False)
                x = oracle.bf16_bits_to_f64_array(c.X)
                ref = x @ W.T
                assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(x) @ np.abs(W).T) + 1e-300)
                assert np.allclose(wn, (W ** 2).sum(1), rtol=1e-14)


def test_bf16_bound_hand_values():
    assert oracle.ulp_bf16(np.array([1.0]))[0] == 2.0 ** -7
    assert oracle.ulp_bf16(np.array([3.0]))[0] == 2.0 ** -6
    assert oracle.ulp_bf16(np.array([2.0 ** -130]))[0] == 2.0 ** -133
    X = workloads.f32_to_bf16_bits(np.array([[3.0, 4.0]], np.float32))  # ||x|| = 5
    b = oracle.y_bound_bf16(X, np.array([[1.0]]), np.array([4.0]))     # ||w|| = 2
    assert b[0, 0] == 2.0 ** -7 * 10 + 2.0 ** -7
