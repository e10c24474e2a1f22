"""GPU parity of ba_attention_fwd_int8pv (the pages' hybrid 8-bit P.V) with
the oracle's binary_attention_int8_pv_rows.

Bar: max |O_gpu - O_oracle| <= 1e-2 * max |V|.  Derivation: the value codes
are decided the same way on both sides (float32, one correctly rounded
division, one product, one rounding) and every product and sum of codes is
exact (int32); a coefficient code can differ by one where 255 * 2^(s - m)
lies within float32 rounding of a half-integer, which moves O_i by at most
2 max|V| / sum_j code_ij <= 2 max|V| / 255 (the row maximum is code 255);
the bf16 output adds 2^-9 |O|.  In practice far fewer codes flip, and the
measured error is printed with each case."""

import numpy as np
import pytest
import torch

import bias_cases as bc
import oracle
import workloads
from gpu_cases import announce, np32, o_error, sample_rows, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = 1e-2


def oracle_int8(inp, rows=None):
    table = inp.get("table")
    return oracle.binary_attention_int8_pv_rows(
        np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), None if table is None else np32(table),
        inp["gh"], inp["gw"], rows=rows)["O"]


def run(inp):
    dev = to_dev(inp)
    o = bq.attention_fwd_int8pv(dev["q"], dev["k"], dev["v"], dev["table"], inp["gh"], inp["gw"])
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("B,H,gh,gw,d", [
    (1, 2, 1, 1, 64),      # N = 1
    (1, 1, 1, 2, 32),
    (1, 2, 7, 9, 64),      # table mode, N = 63 (ragged tile)
    (2, 1, 8, 8, 64),
    (1, 3, 14, 14, 64),    # the tiny ViT grid
    (1, 2, 4, 32, 64),     # table rows (gw % 32 == 0)
    (1, 1, 3, 32, 72),     # d = 72: value codes padded to 96 channels
    (1, 2, 6, 32, 96),
    (1, 1, 5, 64, 128),
    (1, 1, 2, 96, 40),
])
def test_int8_small_with_bias(B, H, gh, gw, d):
    announce("int8 bias", B, H, gh, gw, d)
    inp = workloads.make_inputs(B, H, gh * gw, d, seed=3000 + gh * gw + d, grid=(gh, gw))
    o = run(inp)
    err = o_error(o, oracle_int8(inp), inp["v"])
    print("max err / max|V| =", err)
    assert err <= TOL, err


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 64, 64), (2, 1, 63, 32), (1, 2, 300, 16), (1, 1, 129, 128)])
def test_int8_small_no_bias(B, H, N, d):
    announce("int8 no bias", B, H, N, d)
    inp = workloads.make_inputs(B, H, N, d, seed=3100 + N + d, bias=False)
    o = run(inp)
    err = o_error(o, oracle_int8(inp), inp["v"])
    print("max err / max|V| =", err)
    assert err <= TOL, err


def test_int8_grid_values_and_zero_channel():
    """Q = 0 and no bias: every code is 255, so O is the exact column mean of
    the values' codes times their scales; values on their code grid make that
    the column mean of V, up to the bf16 output.  An all-zero channel has
    scale 0 and gives exactly 0."""
    announce("int8 grid values")
    B, H, N, d = 2, 2, 200, 64
    rng = np.random.default_rng(3201)
    n = rng.integers(-127, 128, size=(B, H, N, d))
    n[:, :, 0, :] = 127
    v = torch.from_numpy((n * 2.0 ** -6).astype(np.float32)).to(torch.bfloat16)
    v[..., 5] = 0.0
    inp = workloads.make_inputs(B, H, N, d, seed=3202, bias=False)
    inp["q"] = torch.zeros_like(inp["q"])
    inp["v"] = v
    o = run(inp).float().cpu().numpy()
    want = np32(v).astype(np.float64).mean(axis=2, keepdims=True)
    assert np.allclose(o, np.broadcast_to(want, o.shape), rtol=2 ** -8, atol=1e-6)
    assert (o[..., 5] == 0).all()


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_int8_workloads(name):
    """The workload shapes at full size, sampled rows against the oracle (the
    value codes use all N keys of each head, as in the full problem)."""
    w = workloads.WORKLOADS[name]
    announce("int8 workload", name)
    inp = workloads.workload_inputs(w)
    o = run(inp)
    assert torch.isfinite(o.float()).all()
    rows = None if w.N * w.B * w.H <= 600 else sample_rows(w.N, 32, w.seed + 50)
    err = o_error(o, oracle_int8(inp, rows), inp["v"], rows)
    print(name, "max err / max|V| =", err)
    assert err <= TOL, (name, err)


def _int8_oracle_table(inp, table, rows=None):
    return oracle.binary_attention_int8_pv_rows(
        np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), table, inp["gh"], inp["gw"], rows=rows)["O"]


@pytest.mark.parametrize("gh,gw,d,dy0,dx0", [
    (14, 14, 64, 2, -3),    # table in LDS
    (7, 9, 32, -1, 4),      # table in LDS, ragged N = 63
    (32, 32, 64, 5, 7),     # table rows
    (64, 64, 64, -11, 20),  # table rows, the 64x64 grid
    (32, 32, 72, 3, -2),    # d = 72: codes padded to 96 channels
])
def test_int8_one_hot_returns_code_grid_row(gh, gw, d, dy0, dx0):
    """Q = 0, values on their code grid and a one-hot table entry of 7: the
    row maximum is the key at the entry's grid offset (code 255), and every
    other coefficient, 255 e^-7 = 0.23, rounds to code 0.  The 8-bit product
    therefore returns exactly that key's value row, while the exact softmax
    (and a bf16 P.V) still gives every other key weight e^-7 each, which
    moves O by 6 % (N = 63) to 80 % (N = 4096) of max|V|, at least five
    times the bar (es page, section 2, "Cuantizacion Hibrida")."""
    announce("int8 one-hot", gh, gw, d, dy0, dx0)
    B, H, n = 1, 2, gh * gw
    rng = np.random.default_rng(3300 + n + d)
    codes = rng.integers(-127, 128, size=(B, H, n, d))
    codes[:, :, 0, :] = 127
    v = torch.from_numpy((codes * 2.0 ** -4).astype(np.float32)).to(torch.bfloat16)
    inp = workloads.make_inputs(B, H, n, d, seed=3301 + n, grid=(gh, gw))
    inp["q"] = torch.zeros_like(inp["q"])
    inp["v"] = v
    t = torch.zeros_like(inp["table"])
    t[:, dy0 + gh - 1, dx0 + gw - 1] = 7.0
    inp["table"] = t
    rows = None if n <= 1024 else sample_rows(n, 64, 3302)
    want = oracle_int8(inp, rows)
    vv = np32(v).astype(np.float64)
    rr = np.arange(n) if rows is None else rows
    for idx, i in enumerate(rr):
        yi, xi = divmod(int(i), gw)
        yj, xj = yi - dy0, xi - dx0
        row = vv[:, :, yj * gw + xj] if (0 <= yj < gh and 0 <= xj < gw) else vv.mean(axis=2)
        assert np.allclose(want[:, :, idx], row, rtol=0, atol=1e-12), i
    exact = bc.oracle_o(inp, rows)
    sep = float(np.abs(exact - want).max()) / float(np.abs(vv).max())
    assert sep > bc.SEP_FACTOR * TOL, sep
    o = run(inp)
    err = o_error(o, want, inp["v"], rows)
    print("max err / max|V| =", err, "exact softmax differs by", sep)
    assert err <= TOL, err


@pytest.mark.parametrize("gh,gw,d", [(14, 14, 64), (32, 32, 64), (7, 9, 72)])
def test_int8_wide_table(gh, gw, d):
    """A sigma-2 table through the 8-bit kernel: dropping, negating or
    mirroring the bias moves the 8-bit oracle's O by more than five times
    the bar."""
    announce("int8 wide table", gh, gw, d)
    inp = workloads.make_inputs(1, 2, gh * gw, d, seed=3400 + gh * gw + d, grid=(gh, gw), table_sigma=2.0)
    want = oracle_int8(inp)
    for name, t in bc.bias_mutations(inp["table"]).items():
        sep = bc.rel_err(_int8_oracle_table(inp, t), want, inp["v"])
        assert sep > bc.SEP_FACTOR * TOL, (name, sep)
    o = run(inp)
    err = o_error(o, want, inp["v"])
    print("max err / max|V| =", err)
    assert err <= TOL, err
