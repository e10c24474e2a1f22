"""GPU parity on bias grids that neither the table rows staged per key tile
(width a multiple of 32, small window) nor the whole table in LDS (at most
48 KiB) can take: the prologue writes the table out as a dense bias per head
and the dense-bias kernel reads it (es page, section 2, "Mejora mediante
Sesgo"; ko page, section 2 (b).2 and section 4 (a), 16K/32K-token grids).

The tables are N(0, 9) or one-hot (over thousands of keys a narrower table
averages out), so that, as each case first shows on the host, a dropped,
negated or mirrored bias would miss the 1e-2 max|V| bar by at least five
times; then the GPU result must meet the bar against the
oracle on seeded rows (every row a query of the full problem)."""

import numpy as np
import pytest
import torch

import bias_cases as bc
import workloads
from gpu_cases import announce, o_error, sample_rows, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = bc.TOL


def run(inp):
    dev = to_dev(inp)
    o = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"], inp["gh"], inp["gw"])
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("B,H,gh,gw,d,sigma,nrows", [
    (1, 2, 100, 100, 64, 3.0, 24),   # 10000 tokens, width 100
    (1, 1, 128, 256, 64, 3.0, 16),   # 32768 tokens: its 2112-float row window is too big for the tiles
    (2, 1, 80, 81, 72, 3.0, 16),     # 6480 tokens, odd width, d = 72
    (1, 1, 75, 90, 128, 3.0, 16),    # 6750 tokens, d = 128
])
def test_fwd_expanded_table(B, H, gh, gw, d, sigma, nrows):
    n = gh * gw
    announce("fwd expanded table", B, H, gh, gw, d, sigma)
    inp = workloads.make_inputs(B, H, n, d, seed=7000 + n + d, grid=(gh, gw), table_sigma=sigma)
    rows = sample_rows(n, nrows, 7001 + n)
    ref = bc.oracle_o(inp, rows)
    print("mutations:", bc.assert_discriminates(inp, ref, rows))
    o = run(inp)
    err = o_error(o, ref, inp["v"], rows)
    print("max err / max|V| =", err)
    assert err <= TOL, err


def test_fwd_expanded_table_one_hot():
    """Q = 0 and a one-hot table on a 100 x 100 grid: each query returns the
    value row at the entry's grid offset (the column mean where none)."""
    gh = gw = 100
    announce("fwd expanded one-hot", gh, gw)
    inp = bc.one_hot_inputs(1, 1, gh, gw, 64, 7100, 7, -11, 20.0)
    rows = sample_rows(gh * gw, 32, 7101)
    ref = bc.oracle_o(inp, rows)
    assert bc.rel_err(ref, bc.one_hot_expected(inp, 7, -11)[:, :, rows], inp["v"]) < 1e-4
    o = run(inp)
    err = o_error(o, ref, inp["v"], rows)
    print("max err / max|V| =", err)
    assert err <= TOL, err


def test_fwd_expanded_prepared_equals_whole():
    """ba_attention_prepare + ba_attention_fwd_prepared equal ba_attention_fwd
    bit for bit on an expanded table (the prepared call reads the dense form
    the prepare wrote)."""
    gh, gw, d = 70, 100, 64
    announce("fwd expanded prepared", gh, gw)
    inp = workloads.make_inputs(1, 2, gh * gw, d, seed=7200, grid=(gh, gw), table_sigma=1.0)
    dev = to_dev(inp)
    lib = bq._lib.load()
    B, H, N = 1, 2, gh * gw
    nb = lib.ba_workspace_bytes(B, H, N, d, gh, gw)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device="cuda")
    wp = (ws.data_ptr() + 255) // 256 * 256
    st = torch.cuda.current_stream().cuda_stream
    tp = dev["table"].data_ptr()
    o1 = torch.empty_like(dev["q"])
    o2 = torch.empty_like(dev["q"])
    bq.check(lib, lib.ba_attention_fwd(dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(), tp, gh, gw,
                                       B, H, N, d, d ** -0.5, o1.data_ptr(), wp, nb, st))
    bq.check(lib, lib.ba_attention_prepare(dev["k"].data_ptr(), dev["v"].data_ptr(), tp, gh, gw, B, H, N, d,
                                           wp, nb, st))
    bq.check(lib, lib.ba_attention_fwd_prepared(dev["q"].data_ptr(), tp, gh, gw, B, H, N, d, d ** -0.5,
                                                o2.data_ptr(), wp, nb, st))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
