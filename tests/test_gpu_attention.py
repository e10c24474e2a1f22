"""GPU parity of the fused BinaryAttention forward (ba_attention_fwd) with
the float64 oracle.

Bar: max |O_gpu - O_oracle| <= 1e-2 * max |V| (bf16 P.V).  The derivation:
rounding P to bf16 and O to bf16 each cost <= 2^-8 max|V|, and the fp32
scores, exp2 and alpha contribute ~1e-6, so the bound is ~0.008 max|V|.

Small problems are checked on every row.  The workload shapes are run at
full size in the launch configuration the benchmark times, and checked on a
seeded sample of rows (rows are independent, so a row of the full problem is
exactly what the oracle computes for that row)."""

import numpy as np
import pytest
import torch

import workloads
from gpu_cases import announce, device, o_error, oracle_rows, sample_rows, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = 1e-2


def run(inp):
    dev = to_dev(inp)
    o = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"], inp["gh"], inp["gw"])
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("B,H,gh,gw,d", [
    (1, 2, 1, 1, 64),      # N = 1: O = V
    (1, 1, 1, 2, 32),      # N = 2
    (1, 2, 7, 9, 64),      # N = 63, generic table path
    (2, 1, 8, 8, 64),      # N = 64
    (1, 2, 5, 13, 64),     # N = 65
    (1, 3, 14, 14, 64),    # the tiny ViT grid
    (1, 2, 4, 32, 64),     # gw % 32 == 0: table-row path, N = 128
    (1, 1, 3, 32, 72),     # d = 72 (bits padded to 96), N = 96: ragged tile
    (1, 2, 6, 32, 96),
    (1, 1, 5, 64, 128),    # N = 320
    (1, 2, 9, 32, 32),     # d = 32, N = 288: two launches, output rows staged in LDS
    (1, 1, 2, 96, 40),     # gw = 96, d = 40
    (1, 1, 3, 32, 200),
    (1, 1, 7, 9, 80),      # table mode, d = 80: two QK chunks, three output blocks
    (1, 1, 7, 9, 144),     # table mode, d = 144: three QK chunks, five output blocks
    (1, 1, 3, 32, 144),    # table rows, d = 144
    (1, 1, 2, 64, 256),
    (1, 1, 2, 128, 8),
    # table rows with a ragged last tile (N % 64 == 32) and d % 32 == 0, where
    # the row sums come from the vector ALU and padded keys must be masked
    (1, 1, 3, 32, 64),
    (1, 2, 3, 32, 128),
    (2, 1, 5, 96, 32),
])
def test_fwd_small_with_bias(B, H, gh, gw, d):
    announce("fwd bias", B, H, gh, gw, d)
    inp = workloads.make_inputs(B, H, gh * gw, d, seed=300 + gh * gw + d, grid=(gh, gw))
    o = run(inp)
    err = o_error(o, oracle_rows(inp), inp["v"])
    assert err <= TOL, err


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 1, 64), (1, 2, 2, 64), (2, 1, 63, 32), (1, 1, 64, 64),
                                     (1, 2, 65, 72), (1, 1, 129, 128), (1, 1, 300, 16),
                                     (1, 1, 100, 144)])
def test_fwd_small_no_bias(B, H, N, d):
    announce("fwd nobias", B, H, N, d)
    inp = workloads.make_inputs(B, H, N, d, seed=400 + N + d, bias=False)
    o = run(inp)
    err = o_error(o, oracle_rows(inp), inp["v"])
    assert err <= TOL, err


def test_fwd_single_token_is_v():
    announce("fwd N=1")
    inp = workloads.make_inputs(2, 3, 1, 64, seed=5, grid=(1, 1))
    o = run(inp)
    assert torch.equal(o.cpu(), inp["v"])


@pytest.mark.parametrize("scale", [4.0, 16.0])
def test_fwd_large_logits(scale):
    """Large |S| (Q and K scaled up): the running max moves by more than the
    lazy-rescale threshold, so the rescale branch runs."""
    announce("fwd large logits", scale)
    inp = workloads.make_inputs(1, 2, 256, 64, seed=9, grid=(8, 32), q_scale=scale, k_scale=scale)
    o = run(inp)
    err = o_error(o, oracle_rows(inp), inp["v"])
    assert err <= TOL, err


def test_fwd_large_logits_ragged_rows():
    """The exact path on table rows with a ragged last tile (N = 96)."""
    announce("fwd large logits ragged rows")
    inp = workloads.make_inputs(1, 2, 96, 64, seed=19, grid=(3, 32), q_scale=8.0, k_scale=8.0)
    o = run(inp)
    err = o_error(o, oracle_rows(inp), inp["v"])
    assert err <= TOL, err


@pytest.mark.parametrize("N,d,grid", [(100, 64, None), (65, 72, None), (160, 128, None), (96, 64, (3, 32)),
                                      (96, 72, (3, 32)), (480, 32, (5, 96))])
def test_fwd_keys_past_n_never_read(N, d, grid):
    """Keys past N of the last head: V ends where the allocation's NaN-filled
    tail starts, so a tile copy that read rows past N would put NaN into O
    (a masked key has P = 0, and 0 * NaN is NaN)."""
    announce("fwd V at the end of a NaN tail", N, d, grid)
    B, H = 1, 2
    inp = workloads.make_inputs(B, H, N, d, seed=700 + N + d, grid=grid, bias=grid is not None)
    dev = to_dev(inp)
    n = B * H * N * d
    store = torch.full((n + 64 * 1024,), float("nan"), dtype=torch.bfloat16, device=device())
    store[:n] = dev["v"].reshape(-1)
    v = store[:n].view(B, H, N, d)
    gh, gw = grid if grid is not None else (0, 0)
    o = bq.attention_fwd(dev["q"], dev["k"], v, dev["table"], gh, gw)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    err = o_error(o, oracle_rows(inp), inp["v"])
    assert err <= TOL, err


def test_fwd_zero_queries_give_bias_softmax():
    """Q = 0: alpha_q = 0, so S is the bias alone."""
    announce("fwd zero q")
    inp = workloads.make_inputs(1, 2, 128, 64, seed=10, grid=(4, 32))
    inp["q"] = torch.zeros_like(inp["q"])
    o = run(inp)
    err = o_error(o, oracle_rows(inp), inp["v"])
    assert err <= TOL, err


def test_fwd_deterministic():
    announce("fwd determinism")
    inp = workloads.make_inputs(2, 3, 1024, 64, seed=11, grid=(32, 32))
    dev = to_dev(inp)
    o1 = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"], 32, 32)
    o2 = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"], 32, 32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_fwd_workloads(name):
    w = workloads.WORKLOADS[name]
    announce("fwd workload", name)
    inp = workloads.workload_inputs(w)
    o = run(inp)
    assert torch.isfinite(o.float()).all()
    rows = None if w.N * w.B * w.H <= 600 else sample_rows(w.N, 48, w.seed)
    err = o_error(o, oracle_rows(inp, rows), inp["v"], rows)
    assert err <= TOL, (name, err)
