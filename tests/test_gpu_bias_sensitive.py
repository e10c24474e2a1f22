"""GPU parity on inputs where the bias, the sign rule and the softmax
rescale decide the answer.

Each case first shows on the host that it discriminates: the oracle run with
the bias dropped, negated or mirrored (or with -0.0 read as negative) misses
the 1e-2 max|V| bar by at least five times.  Then the GPU result must meet
the bar against the oracle.

Coverage of the kernel's bias readers (es page, section 2, "Mejora mediante
Sesgo"; ko page, section 2 (b).2):
* the whole table in LDS: grids whose width is not a multiple of 32, in the
  one-launch kernel (N <= 256, d in {32, 64}) and in the two-launch kernel;
* the shifted table rows staged per key tile: widths 32, 64 and 128, with a
  ragged last tile;
* both softmax paths: the offset-free one (logit bound <= 32) and the
  online one (queries scaled up, or Q = 0 with a one-hot entry of 40).
Full-size workload grids are checked on sampled rows."""

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


SMALL = [
    # B, H, gh, gw, d, table sigma, q scale
    (1, 3, 14, 14, 64, 2.0, 1.0),   # one-launch kernel, table in LDS (tiny ViT grid)
    (2, 2, 7, 9, 64, 2.0, 1.0),     # one-launch, ragged N = 63
    (1, 2, 14, 14, 32, 2.0, 1.0),   # one-launch, d = 32
    (1, 2, 14, 14, 64, 1.0, 8.0),   # one-launch, online softmax
    (1, 2, 20, 20, 64, 2.0, 1.0),   # two launches, table in LDS (N = 400)
    (1, 2, 14, 14, 128, 2.0, 1.0),  # two launches, d = 128
    (1, 1, 7, 9, 72, 2.0, 1.0),     # d = 72 (padded to 96), table in LDS
    (1, 2, 20, 20, 64, 1.0, 8.0),   # table in LDS, online softmax
    (1, 2, 3, 32, 64, 2.0, 1.0),    # table rows, ragged last tile (N % 64 == 32)
    (1, 2, 32, 32, 64, 2.0, 1.0),   # table rows, N = 1024
    (1, 1, 8, 64, 128, 2.0, 1.0),   # table rows, width 64, d = 128
    (1, 1, 32, 32, 72, 2.0, 1.0),   # table rows, d = 72
    (1, 2, 32, 32, 64, 1.0, 8.0),   # table rows, online softmax
    (1, 1, 4, 128, 64, 2.0, 1.0),   # table rows, width 128
    (1, 2, 9, 32, 32, 2.0, 1.0),    # table rows, d = 32 (N = 288: inner tile group, then the last tiles)
    (1, 1, 6, 64, 32, 1.0, 8.0),    # table rows, d = 32, online softmax
    (1, 1, 4, 128, 128, 2.0, 1.0),  # table rows, width 128, d = 128 (one window row per tile)
]


@pytest.mark.parametrize("B,H,gh,gw,d,sigma,qs", SMALL)
def test_fwd_wide_table(B, H, gh, gw, d, sigma, qs):
    announce("fwd wide table", B, H, gh, gw, d, sigma, qs)
    inp = workloads.make_inputs(B, H, gh * gw, d, seed=5000 + gh * gw + d, grid=(gh, gw),
                                table_sigma=sigma, q_scale=qs)
    ref = bc.oracle_o(inp)
    print("mutations:", bc.assert_discriminates(inp, ref))
    o = run(inp)
    err = o_error(o, ref, inp["v"])
    print("max err / max|V| =", err)
    assert err <= TOL, err


@pytest.mark.parametrize("name", ["vit_base_b32_14x14", "dit512_32x32_d72", "detection_64x64",
                                  "diffusion_128x128_d128"])
def test_fwd_workload_grid_wide_table(name):
    """The workload shapes at full size (the benchmark's launch) with a
    sigma-2 table; sampled rows."""
    w = workloads.WORKLOADS[name]
    announce("fwd workload wide table", name)
    inp = workloads.workload_inputs(w, table_sigma=2.0)
    rows = sample_rows(w.N, 24, w.seed + 500)
    ref = bc.oracle_o(inp, rows)
    print("mutations:", bc.assert_discriminates(inp, ref, rows))
    o = run(inp)
    err = o_error(o, ref, inp["v"], rows)
    print(name, "max err / max|V| =", err)
    assert err <= TOL, (name, err)


def test_fwd_exact_path_full_headline_shape():
    """B=2 H=12 on the 64x64 grid with Q x 8 (logit bound > 32: the online
    softmax) and a sigma-1 table; sampled rows."""
    w = workloads.WORKLOADS["detection_64x64"]
    announce("fwd exact path 64x64")
    inp = workloads.workload_inputs(w, table_sigma=1.0, q_scale=8.0)
    rows = sample_rows(w.N, 24, 4501)
    ref = bc.oracle_o(inp, rows)
    print("mutations:", bc.assert_discriminates(inp, ref, rows))
    o = run(inp)
    err = o_error(o, ref, inp["v"], rows)
    print("max err / max|V| =", err)
    assert err <= TOL, err


@pytest.mark.parametrize("gh,gw,d,height,dy0,dx0", [
    (14, 14, 64, 20.0, 3, -5),    # one-launch, offset-free path
    (14, 14, 64, 40.0, -6, 2),    # one-launch, online path
    (20, 20, 128, 20.0, 4, 7),    # table in LDS, two launches
    (64, 64, 64, 20.0, -9, 13),   # table rows, the headline grid
    (64, 64, 64, 40.0, 17, -30),  # table rows, online path
    (32, 32, 72, 20.0, 1, -1),    # table rows, d = 72
])
def test_fwd_one_hot_table_picks_offset(gh, gw, d, height, dy0, dx0):
    """Q = 0 and a one-hot table: each query must return the value row at
    the table entry's grid offset (the pages' position-sensitive bias, with
    the sign convention of the oracle's pins)."""
    announce("fwd one-hot", gh, gw, d, height, dy0, dx0)
    inp = bc.one_hot_inputs(1, 2, gh, gw, d, 5200 + gh + d, dy0, dx0, height)
    n = gh * gw
    rows = None if n <= 1024 else sample_rows(n, 64, 5201)
    ref = bc.oracle_o(inp, rows)
    want = bc.one_hot_expected(inp, dy0, dx0)
    want = want if rows is None else want[:, :, rows]
    assert bc.rel_err(ref, want, inp["v"]) < 1e-4
    bc.assert_discriminates(inp, ref, rows)
    o = run(inp)
    err = o_error(o, ref, inp["v"], rows)
    print("max err / max|V| =", err)
    assert err <= TOL, err


@pytest.mark.parametrize("gh,gw", [(64, 64), (14, 14)])
def test_fwd_textbook_reduction_full_grid(gh, gw):
    """Constant-magnitude Q and K rows make BinaryAttention textbook
    attention; checked against torch's float64 scaled_dot_product_attention
    with the bias as an additive mask (B=2 H=12, sigma-1 table)."""
    announce("fwd textbook reduction", gh, gw)
    inp = bc.constant_magnitude_inputs(2, 12, gh, gw, 64, 5300 + gw)
    n = gh * gw
    rows = sample_rows(n, 32, 5301) if n > 256 else np.arange(n)
    want = bc.textbook_rows(inp, rows)
    ref = bc.oracle_o(inp, rows)
    assert bc.rel_err(ref, want, inp["v"]) < 1e-9
    bc.assert_discriminates(inp, ref, rows)
    o = run(inp)
    err = o_error(o, want, inp["v"], rows)
    print("max err / max|V| =", err)
    assert err <= TOL, err


@pytest.mark.parametrize("gh,gw,d", [(14, 14, 64), (32, 32, 64), (7, 9, 72)])
def test_fwd_signed_zeros(gh, gw, d):
    """Half of Q's and K's entries are -0.0, which the sign rule reads as +1;
    a kernel that took the sign bit would miss the bar by far."""
    announce("fwd signed zeros", gh, gw, d)
    inp = bc.signed_zero_inputs(1, 2, gh, gw, d, 5400 + gw)
    assert (np.signbit(bc.np64(inp["q"])) & (bc.np64(inp["q"]) == 0)).mean() > 0.4
    ref = bc.oracle_o(inp)
    wrong = bc.oracle.binary_attention_rows(
        bc.signbit_zero_mutation(inp["q"]), bc.signbit_zero_mutation(inp["k"]), bc.np64(inp["v"]),
        bc.np64(inp["table"]), gh, gw)["O"]
    assert bc.rel_err(wrong, ref, inp["v"]) > bc.SEP_FACTOR * TOL
    o = run(inp)
    err = o_error(o, ref, inp["v"])
    print("max err / max|V| =", err)
    assert err <= TOL, err


@pytest.mark.parametrize("gh,gw", [(32, 32), (64, 64)])
def test_fwd_rescale_late_in_the_keys(gh, gw):
    """Logits that grow along the keys: the online softmax's rescale must
    fire for key blocks past the first 256 keys (shown by replaying the rule
    on the oracle's scores)."""
    announce("fwd late rescale", gh, gw)
    inp = bc.growing_key_inputs(1, 2, gh, gw, 64, 5500 + gw)
    rows = sample_rows(gh * gw, 32, 5501)
    assert bc.late_rescales(inp, rows) > 0
    ref = bc.oracle_o(inp, rows)
    o = run(inp)
    err = o_error(o, ref, inp["v"], rows)
    print("max err / max|V| =", err)
    assert err <= TOL, err


LOCAL = [
    # B, H, gh, gw, d: table rows (pipelined kernel), the whole table in LDS
    # (one-launch and general kernels), d = 72 and d = 128
    (1, 2, 8, 64, 64),
    (1, 1, 4, 32, 72),
    (1, 1, 4, 128, 128),
    (1, 2, 14, 14, 64),
    (1, 2, 20, 20, 64),
]


@pytest.mark.parametrize("B,H,gh,gw,d", LOCAL)
def test_fwd_local_window_table(B, H, gh, gw, d):
    """A table that masks every key more than 1 grid row or 3 columns away
    with -inf (windowed attention through the bias).  The logit bound is
    infinite, so the online softmax runs, and most queries meet whole key
    blocks of -inf logits before their first finite one: those blocks must
    contribute 0, not NaN."""
    announce("fwd local-window table", B, H, gh, gw, d)
    inp = workloads.make_inputs(B, H, gh * gw, d, seed=7100 + gh * gw + d, grid=(gh, gw), table_sigma=1.0)
    t = inp["table"].clone()
    dy = torch.arange(-(gh - 1), gh).abs().view(1, -1, 1)
    dx = torch.arange(-(gw - 1), gw).abs().view(1, 1, -1)
    far = ((dy > 1) | (dx > 3)).expand_as(t)
    t[far] = float("-inf")
    inp["table"] = t
    ref = bc.oracle_o(inp)
    assert np.isfinite(ref).all()
    o = run(inp)
    assert torch.isfinite(o.float()).all()
    err = o_error(o, ref, inp["v"])
    print("max err / max|V| =", err)
    assert err <= TOL, err
