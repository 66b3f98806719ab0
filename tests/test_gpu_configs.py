"""Every benchmark configuration as a parity case: each (shape, M) of the
decode and prefill sweeps at the Llama-2-7B shapes, of the 70B-class GQA
shapes, and of the group-size / edge variants, through the library's own
path choice, on sampled weight rows (at these sizes the oracle computes rows
one by one).  Inputs as the configurations describe them: X N(0,1) (prefill:
1 % of the columns x20), codes and zeros uniform 0..15, scales U[0.002,
0.02]; one seeded weight per shape, X drawn at the largest M and each M
taking its first rows."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_int4_02_amd as w4
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

def run_sweep(family, N, K, g, sym, ms, outliers=False, n_rows=24):
    c = workloads.draw(max(ms), N, K, g, sym, seed=workloads.shape_seed(family, N, K, g, sym),
                       outliers=outliers)
    w = w4.quantized_weight(torch.from_numpy(c.codes).cuda(), torch.from_numpy(c.scales).cuda(),
                            None if sym else torch.from_numpy(c.zeros).cuda(), g,
                            partial=K % g != 0)
    rng = np.random.default_rng(N * 7 + K)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, n_rows), replace=False)]))
    qp, zp = oracle.pack(c.codes), None if sym else oracle.pack(c.zeros)
    Xd = torch.from_numpy(c.X).cuda()
    y_all, wn2 = oracle.gemm_rows(c.X, qp, c.scales, zp, K, g, sym, rows=rows)
    for M in ms:
        y = w4.gemm(Xd[:M], w).cpu().numpy()[:, rows]
        ok, worst = oracle.check_y(y, c.X[:M], y_all[:M], wn2)
        assert ok, f"{family} N{N} K{K} g{g} sym{sym} M{M}: worst |err|/bound = {worst:.3f}"
        assert np.all(np.isfinite(y.astype(np.float32)))


@pytest.mark.parametrize("shape", list(workloads.LLAMA7B_SHAPES))
def test_decode_sweep(shape):
    N, K = workloads.LLAMA7B_SHAPES[shape]
    run_sweep("cfg1", N, K, 128, False, workloads.DECODE_M)


@pytest.mark.parametrize("shape", list(workloads.LLAMA7B_SHAPES))
def test_prefill_sweep(shape):
    N, K = workloads.LLAMA7B_SHAPES[shape]
    run_sweep("cfg2", N, K, 128, False, workloads.PREFILL_M, outliers=True)


@pytest.mark.parametrize("shape", list(workloads.LLAMA70B_SHAPES))
def test_gqa70b_sweep(shape):
    N, K = workloads.LLAMA70B_SHAPES[shape]
    run_sweep("cfg3", N, K, 128, False, workloads.L70B_M)


@pytest.mark.parametrize("sym", (False, True))
@pytest.mark.parametrize("g", workloads.EDGE_G)
def test_group_size_variants(g, sym):
    run_sweep("cfg4", 4096, 4096, g, sym, workloads.EDGE_M)


@pytest.mark.parametrize("sym", (False, True))
def test_partial_last_group_and_odd_group_count(sym):
    # K = N = 288 with g = 256: a last group 32 wide; K = 11008 with g = 256:
    # 43 groups, no partial group
    run_sweep("cfg4", 288, 288, 256, sym, workloads.EDGE_M, n_rows=288)
    run_sweep("cfg4", 4096, 11008, 256, sym, workloads.EDGE_M)
