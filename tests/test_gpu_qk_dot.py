"""GPU integer dots D_ij = <sign q_i, sign k_j> (ba_qk_int_dot) against the
oracle, bit-exact, for the three routes (fp4 MFMA, int8 MFMA, VALU
xor/popcount), as all pairs and as row sums.  The fp4-MFMA route runs the
device code of the fused kernel's QK step."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import announce, bits_u32, np32

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")


ROUTES = [bq.ROUTE_MFMA_FP4, bq.ROUTE_VALU_POPCOUNT, bq.ROUTE_MFMA_INT8]
SHAPES = [(1, 1, 1, 8), (1, 2, 33, 32), (2, 1, 65, 64), (1, 2, 196, 64), (1, 1, 100, 72), (1, 1, 64, 96),
          (1, 2, 97, 128), (1, 1, 40, 200), (1, 1, 70, 256)]


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("B,H,N,d", SHAPES)
def test_qk_dot_bit_exact(route, B, H, N, d):
    announce("qk_dot", route, B, H, N, d)
    inp = workloads.make_inputs(B, H, N, d, seed=200 + N + d, bias=False)
    qf, kf = np32(inp["q"]), np32(inp["k"])
    qb, _ = bq.pack_signs(inp["q"].cuda())
    kb, _ = bq.pack_signs(inp["k"].cuda())
    dots = bq.qk_int_dot(qb, kb, d, route).cpu().numpy().astype(np.int64)
    want = oracle.sign_dots(qf, kf)
    assert np.array_equal(dots, want)
    assert np.array_equal(dots, oracle.sign_dots_from_bits(bits_u32(qb), bits_u32(kb), d))


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("B,H,N,d", SHAPES + [(1, 1, 300, 64), (1, 1, 129, 128)])
def test_qk_rowsum_bit_exact(route, B, H, N, d):
    """Row sums sum_j D_ij, including ragged key tiles (keys past N must add
    nothing) and query tiles."""
    announce("qk_rowsum", route, B, H, N, d)
    inp = workloads.make_inputs(B, H, N, d, seed=400 + N + d, bias=False)
    qb, _ = bq.pack_signs(inp["q"].cuda())
    kb, _ = bq.pack_signs(inp["k"].cuda())
    sums = bq.qk_int_dot(qb, kb, d, route, rowsum=True).cpu().numpy().astype(np.int64)
    want = oracle.sign_dots(np32(inp["q"]), np32(inp["k"])).sum(axis=-1)
    assert np.array_equal(sums, want)


def test_qk_dot_extremes():
    """D = d on identical rows and -d on negated rows (d = 72: padded bits)."""
    announce("qk_dot extremes")
    d = 72
    inp = workloads.make_inputs(1, 1, 40, d, seed=7, bias=False)
    q = inp["q"].clone()
    q[q == 0] = 1.0
    k = q.clone()
    k[0, 0, 20:] = -q[0, 0, 20:]
    qb, _ = bq.pack_signs(q.cuda())
    kb, _ = bq.pack_signs(k.cuda())
    dots = bq.qk_int_dot(qb, kb, d).cpu().numpy()[0, 0]
    assert np.all(np.diag(dots)[:20] == d)
    assert np.all(np.diag(dots)[20:] == -d)
    assert np.array_equal(dots, oracle.sign_dots(np32(q), np32(k))[0, 0])


def test_qk_dot_workload_detection_sampled():
    """Full detection-backbone shape (N=4096), checked on 8 seeded rows/head."""
    w = workloads.WORKLOADS["detection_64x64"]
    announce("qk_dot workload", w.name)
    inp = workloads.workload_inputs(w)
    qb, _ = bq.pack_signs(inp["q"].cuda())
    kb, _ = bq.pack_signs(inp["k"].cuda())
    dots = bq.qk_int_dot(qb, kb, w.d)
    rows = np.random.default_rng(4).choice(w.N, 8, replace=False)
    got = dots[:, :, rows, :].cpu().numpy()
    want = oracle.sign_dots(np32(inp["q"])[:, :, rows, :], np32(inp["k"]))
    assert np.array_equal(got, want)
