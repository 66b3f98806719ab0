"""Seeded random shapes through every path of the plan: M from 1 to 600 (small
and large kernels, K split or not, LDS-staged or not), ragged N and K, partial
last groups, every group size, symmetric or not, fp16 and bf16, the path left
to the library or forced.  Exact-family inputs, so the GPU result must equal
the rounded exact product bit for bit; random (non-exact) inputs on a subset,
within the error bound."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import weight_only_int4_02_amd as w4
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def draw_config(i):
    rng = np.random.default_rng(zlib.crc32(f"w4a16/fuzz/{i}".encode()))
    while True:
        M = int(np.exp(rng.uniform(0, np.log(600))))
        N = int(rng.integers(1, 3000))
        K = 8 * int(rng.integers(1, 750))
        if M * N * K <= 2e8:
            break
    g = int(rng.choice([32, 64, 128, 256]))
    sym = bool(rng.integers(0, 2))
    dtype = "bf16" if rng.uniform() < 0.35 else "f16"
    path = [None, "small_m", "large_m"][int(rng.integers(0, 3))]
    return M, N, K, g, sym, dtype, path


CONFIGS = [draw_config(i) for i in range(80)]


def ids(c):
    M, N, K, g, sym, dtype, path = c
    return f"M{M}-N{N}-K{K}-g{g}-{'sym' if sym else 'asym'}-{dtype}-{path or 'auto'}"


def to_dev_bits(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


@pytest.mark.parametrize("cfg", CONFIGS, ids=ids)
def test_fuzz_exact_family(cfg):
    M, N, K, g, sym, dtype, path = cfg
    seed = zlib.crc32(ids(cfg).encode())
    if dtype == "bf16":
        c = workloads.exact_family_bf16(M, N, K, g, sym, seed=seed)
        X, scales = to_dev_bits(c.X, dtype), to_dev_bits(c.scales, dtype)
    else:
        c = workloads.exact_family(M, N, K, g, sym, seed=seed)
        X, scales = torch.from_numpy(c.X).cuda(), torch.from_numpy(c.scales).cuda()
    w = w4.quantized_weight(torch.from_numpy(c.codes).cuda(), scales,
                            None if sym else torch.from_numpy(c.zeros).cuda(), g,
                            partial=K % g != 0)
    y = w4.gemm(X, w, path=path).cpu().view(torch.int16).numpy().view(np.uint16)
    qp, zp = oracle.pack(c.codes), None if sym else oracle.pack(c.zeros)
    if dtype == "bf16":
        y_exact, _ = oracle.gemm_rows_bf16(c.X, qp, c.scales, zp, K, g, sym)
        want = np.array([oracle.f64_to_bf16_bits(float(v)) for v in y_exact.ravel()],
                        np.uint16).reshape(y_exact.shape)
    else:
        y_exact, _ = oracle.gemm_rows(c.X, qp, c.scales, zp, K, g, sym)
        want = y_exact.astype(np.float16).view(np.uint16)
    assert np.array_equal(y, want), f"{ids(cfg)}: {np.count_nonzero(y != want)} outputs differ"


@pytest.mark.parametrize("cfg", CONFIGS[::3], ids=ids)
def test_fuzz_random_within_bound(cfg):
    M, N, K, g, sym, dtype, path = cfg
    seed = zlib.crc32(("r" + ids(cfg)).encode())
    if dtype == "bf16":
        c = workloads.draw_bf16(M, N, K, g, sym, seed=seed)
        X, scales = to_dev_bits(c.X, dtype), to_dev_bits(c.scales, dtype)
    else:
        c = workloads.draw(M, N, K, g, sym, seed=seed)
        X, scales = torch.from_numpy(c.X).cuda(), torch.from_numpy(c.scales).cuda()
    w = w4.quantized_weight(torch.from_numpy(c.codes).cuda(), scales,
                            None if sym else torch.from_numpy(c.zeros).cuda(), g,
                            partial=K % g != 0)
    y = w4.gemm(X, w, path=path).cpu().view(torch.int16).numpy().view(np.uint16)
    qp, zp = oracle.pack(c.codes), None if sym else oracle.pack(c.zeros)
    if dtype == "bf16":
        y_ref, wn2 = oracle.gemm_rows_bf16(c.X, qp, c.scales, zp, K, g, sym)
        ok, worst = oracle.check_y_bf16(y, c.X, y_ref, wn2)
    else:
        y_ref, wn2 = oracle.gemm_rows(c.X, qp, c.scales, zp, K, g, sym)
        ok, worst = oracle.check_y(y.view(np.float16), c.X, y_ref, wn2)
    assert ok, f"{ids(cfg)}: worst |err|/bound = {worst:.3f}"
