"""GPU check of ba_attention_fwd_static, the forward for callers that cannot
allocate: through the C ABI, its output must equal ba_attention_fwd's on
the same inputs (bit for bit: the same kernels on the library's own scratch
instead of a caller's workspace), and meet the oracle's bar on sampled rows.
Two calls run in a row, the second on a smaller problem, so the second
reads a scratch the first left full; a too-large problem is refused before
anything runs."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_cases import announce, device, o_error, oracle_rows, sample_rows, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = 1e-2


def fwd_with_workspace(lib, dev, inp, B, H, N, d):
    gh, gw = inp["gh"], inp["gw"]
    tp = dev["table"].data_ptr() if dev["table"] is not None else None
    nb = lib.ba_workspace_bytes(B, H, N, d, gh, gw)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=device())
    wp = (ws.data_ptr() + 255) // 256 * 256
    out = torch.empty_like(dev["q"])
    bq.check(lib, lib.ba_attention_fwd(dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(), tp, gh, gw,
                                       B, H, N, d, d ** -0.5, out.data_ptr(), wp, nb,
                                       torch.cuda.current_stream().cuda_stream))
    return out


def fwd_static(lib, dev, inp, B, H, N, d):
    gh, gw = inp["gh"], inp["gw"]
    tp = dev["table"].data_ptr() if dev["table"] is not None else None
    out = torch.empty_like(dev["q"])
    bq.check(lib, lib.ba_attention_fwd_static(dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(), tp,
                                              gh, gw, B, H, N, d, d ** -0.5, out.data_ptr(),
                                              torch.cuda.current_stream().cuda_stream))
    return out


def test_static_forward_matches_workspace_forward():
    lib = bq._lib.load()
    cases = [
        (2, 12, 64, 64, 64, 4),   # the 64x64 grid: table rows, pipelined kernel
        (1, 3, 32, 32, 64, 5),    # smaller, on the scratch the first call filled
    ]
    for (B, H, gh, gw, d, seed) in cases:
        N = gh * gw
        announce("static forward", B, H, gh, gw, d)
        inp = workloads.make_inputs(B, H, N, d, seed=9000 + seed, grid=(gh, gw), table_sigma=1.0)
        dev = to_dev(inp)
        o_static = fwd_static(lib, dev, inp, B, H, N, d)
        o_ws = fwd_with_workspace(lib, dev, inp, B, H, N, d)
        torch.cuda.synchronize()
        assert torch.equal(o_static, o_ws)
        rows = sample_rows(N, 24, seed)
        err = o_error(o_static, oracle_rows(inp, rows), inp["v"], rows)
        print("max err / max|V| =", err)
        assert err <= TOL, err


def test_static_forward_refuses_too_large():
    """A problem whose scratch exceeds the library's array is refused before
    any launch (the pointers are never read)."""
    lib = bq._lib.load()
    fake = 1 << 40
    st = lib.ba_attention_fwd_static(fake, fake + (1 << 38), fake + (2 << 38), None, 0, 0, 64, 16, 16384, 128,
                                     0.1, fake + (3 << 38), None)
    assert st == 5
    assert b"scratch" in lib.ba_last_error()
