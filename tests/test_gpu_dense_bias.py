"""GPU parity of ba_attention_fwd_dense_bias (a dense bias per query, key
and head) with the float64 oracle's binary_attention_dense_bias_rows.

Bar: max |O_gpu - O_oracle| <= 1e-2 * max |V|, as for the table bias: the
dense mode runs the exact online softmax (P <= 2^8 before bf16 rounding),
whose rounding is the same bf16 P and bf16 O as the offset-free path."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_cases import announce, device, np32, o_error, sample_rows, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = 1e-2


def ld_for(n):
    return (n + 7) // 8 * 8


def oracle_dense(inp, bias, rows=None):
    return oracle.binary_attention_dense_bias_rows(
        np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(bias.contiguous()), rows=rows)["O"]


def run_dense(inp, bias):
    dev = to_dev(inp)
    # keep the padded row stride of `bias` on the device
    if bias.is_contiguous():
        bdev = bias.to(device())
    else:
        n = bias.shape[-1]
        wide = torch.zeros(bias.shape[:-1] + (bias.stride(2),), dtype=torch.bfloat16)
        wide[..., :n] = bias
        bdev = wide.to(device())[..., :n]
    o = bq.attention_fwd_dense_bias(dev["q"], dev["k"], dev["v"], bdev)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("B,H,N,d,Bb", [
    (1, 1, 1, 64, 1),       # N = 1: O = V
    (1, 2, 2, 64, 1),
    (2, 1, 63, 32, 2),      # ragged tile, one bias per batch entry
    (2, 2, 64, 64, 1),      # bias shared by the batch
    (1, 2, 65, 72, 1),      # d = 72: pads to 96
    (2, 1, 130, 128, 2),
    (1, 1, 196, 64, 1),     # the ViT token count (rows padded to 200)
    (1, 1, 300, 16, 1),
    (1, 1, 256, 256, 1),
])
def test_dense_small(B, H, N, d, Bb):
    announce("dense", B, H, N, d, Bb)
    inp = workloads.make_inputs(B, H, N, d, seed=1000 + N + d, bias=False)
    bias = workloads.make_dense_bias(Bb, H, N, seed=2000 + N + d, sigma=1.0, ld=ld_for(N))
    o = run_dense(inp, bias)
    err = o_error(o, oracle_dense(inp, bias), inp["v"])
    assert err <= TOL, err


def test_dense_large_values():
    """Bias values in the tens: the exact path's rescaling at work."""
    announce("dense large")
    inp = workloads.make_inputs(2, 2, 200, 64, seed=1101, bias=False)
    bias = workloads.make_dense_bias(2, 2, 200, seed=1102, sigma=12.0)
    o = run_dense(inp, bias)
    err = o_error(o, oracle_dense(inp, bias), inp["v"])
    assert err <= TOL, err


def test_dense_minus_inf_masks():
    """-inf entries mask keys.  Rows >= 64 mask every key < 64, so their
    whole first tile is -inf (the row max starts at -inf there); rows < 64
    mask keys j > i (a causal pattern)."""
    announce("dense -inf")
    B, H, N, d = 1, 2, 192, 64
    inp = workloads.make_inputs(B, H, N, d, seed=1201, bias=False)
    bias = workloads.make_dense_bias(1, H, N, seed=1202, sigma=0.5).float()
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    mask = ((i >= 64) & (j < 64)) | ((i < 64) & (j > i))
    bias[:, :, mask] = float("-inf")
    bias = bias.to(torch.bfloat16)
    o = run_dense(inp, bias)
    assert torch.isfinite(o.float()).all()
    err = o_error(o, oracle_dense(inp, bias), inp["v"])
    assert err <= TOL, err


def test_dense_equals_table_bias():
    """The relative-position table written out as a dense bias gives the
    table path's answer."""
    announce("dense vs table")
    gh, gw = 8, 32
    inp = workloads.make_inputs(1, 2, gh * gw, 64, seed=1301, grid=(gh, gw))
    dense = oracle.rel_pos_bias(np32(inp["table"]), gh, gw)[None]
    bias = torch.from_numpy(dense.astype(np.float32)).to(torch.bfloat16)
    o_dense = run_dense(inp, bias)
    dev = to_dev(inp)
    o_table = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"], gh, gw)
    torch.cuda.synchronize()
    ref = oracle.binary_attention_rows(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]),
                                       np32(inp["table"]), gh, gw)["O"]
    assert o_error(o_dense, ref, inp["v"]) <= TOL
    assert o_error(o_table, ref, inp["v"]) <= TOL


def test_dense_full_length_sampled():
    """N = 4096 (the 64x64 grid) with a bias shared over the batch, at the
    launch shape of the benchmark; sampled rows against the oracle."""
    B, H, N, d = 2, 2, 4096, 64
    announce("dense full", B, H, N, d)
    inp = workloads.make_inputs(B, H, N, d, seed=1401, bias=False)
    bias = workloads.make_dense_bias(1, H, N, seed=1402, sigma=0.02)
    o = run_dense(inp, bias)
    rows = sample_rows(N, 24, 1403)
    err = o_error(o, oracle_dense(inp, bias, rows), inp["v"], rows)
    assert err <= TOL, err


def test_dense_prepared_split_is_bit_identical():
    """ba_attention_prepare + ba_attention_fwd_dense_bias_prepared gives the
    one-call result bit for bit, and one prepared workspace serves two
    different biases."""
    B, H, N, d = 2, 3, 200, 64
    announce("dense prepared", B, H, N, d)
    inp = workloads.make_inputs(B, H, N, d, seed=1501, bias=False)
    b1 = workloads.make_dense_bias(B, H, N, seed=1502, sigma=1.0)
    b2 = workloads.make_dense_bias(1, H, N, seed=1503, sigma=1.0)
    lib = bq._lib.load()
    dev = to_dev(inp)
    q, k, v = dev["q"], dev["k"], dev["v"]
    nbytes = lib.ba_workspace_bytes(B, H, N, d, 0, 0)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device())
    wsp = (ws.data_ptr() + 255) // 256 * 256
    sp = torch.cuda.current_stream(device()).cuda_stream
    bq.check(lib, lib.ba_attention_prepare(k.data_ptr(), v.data_ptr(), None, 0, 0, B, H, N, d, wsp, nbytes, sp))
    outs = []
    for bias, sb in ((b1.to(device()), H * N * N), (b2.to(device()), 0)):
        o = torch.empty_like(q)
        bq.check(lib, lib.ba_attention_fwd_dense_bias_prepared(
            q.data_ptr(), bias.data_ptr(), sb, N * N, N, B, H, N, d, 1.0 / d ** 0.5, o.data_ptr(),
            wsp, nbytes, sp))
        outs.append(o)
    torch.cuda.synchronize()
    for o, bias in zip(outs, (b1, b2)):
        ref = bq.attention_fwd_dense_bias(q, k, v, bias.to(device()))
        torch.cuda.synchronize()
        assert torch.equal(o, ref)
        assert o_error(o, oracle_dense(inp, bias), inp["v"]) <= TOL
