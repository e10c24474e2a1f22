"""GPU parity of the sign/scale pack (ba_pack_signs) against the oracle:
bits bit-exact, alpha within 1e-6 relative (fixed-order fp32 sum over at
most 256 channels: pairwise depth <= 8, so the error is below 8 ulp(1) ~
5e-7 of the sum, plus one rounding for the division by d)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_cases import announce, bits_u32, np32

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 1, 8), (1, 2, 63, 32), (2, 3, 65, 64),
                                     (1, 3, 196, 72), (2, 1, 100, 96), (1, 2, 77, 128),
                                     (1, 1, 130, 200), (1, 2, 64, 256)])
def test_pack_matches_oracle(B, H, N, d):
    announce("pack", B, H, N, d)
    x = workloads.make_inputs(B, H, N, d, seed=100 + d, bias=False)["q"]
    x[0, 0, 0, : d // 2] = 0.0
    x[0, 0, min(1, N - 1), : d // 2] = -0.0
    bits, alpha = bq.pack_signs(x.cuda())
    torch.cuda.synchronize()
    xf = np32(x)
    want_bits = oracle.pack_sign_bits(xf)
    assert np.array_equal(bits_u32(bits), want_bits)
    want_alpha = oracle.token_scale(xf)
    got = alpha.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want_alpha) <= 1e-6 * want_alpha + 1e-30)


def test_pack_special_values():
    announce("pack special")
    d = 72
    x = torch.zeros((1, 1, 4, d), dtype=torch.bfloat16)
    x[0, 0, 1] = -0.0
    x[0, 0, 2] = -1.5
    x[0, 0, 3, ::2] = -2.0
    x[0, 0, 3, 1::2] = 2.0
    bits, alpha = bq.pack_signs(x.cuda())
    b = bits_u32(bits)[0, 0]
    assert b[0].tolist() == [0, 0, 0] and b[1].tolist() == [0, 0, 0]
    assert b[2].tolist() == [0xFFFFFFFF, 0xFFFFFFFF, 0xFF]
    assert b[3].tolist() == [0x55555555, 0x55555555, 0x55]
    assert alpha.cpu().tolist()[0][0] == [0.0, 0.0, 1.5, 2.0]


def test_pack_workload_shapes():
    for name in ("tiny_vit_14x14", "dit512_32x32_d72", "detection_64x64"):
        w = workloads.WORKLOADS[name]
        announce("pack workload", name)
        inp = workloads.workload_inputs(w)
        bits, alpha = bq.pack_signs(inp["k"].cuda())
        xf = np32(inp["k"])
        assert np.array_equal(bits_u32(bits), oracle.pack_sign_bits(xf))
        want = oracle.token_scale(xf)
        assert np.all(np.abs(alpha.cpu().numpy() - want) <= 1e-6 * want)
