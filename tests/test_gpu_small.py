"""GPU parity of the one-launch forward for short sequences.

For N <= 256 and d in {32, 64}, with a table or without a bias, the whole
forward (ba_attention_fwd, its strided and training forms) runs as one
kernel that packs each head's keys and values into LDS itself, in the
layouts the prologue writes.  Same arithmetic in the same order, so its
output must equal the two-launch path (ba_attention_prepare +
ba_attention_fwd_prepared, which always runs the prologue) bit for bit; it is
also held to the oracle's bar, max |dO| <= 1e-2 max |V|."""

import pytest
import torch

import workloads
from gpu_cases import announce, device, o_error, oracle_rows, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = 1e-2


def two_launch(dev, inp, B, H, N, d, table):
    lib = bq._lib.load()
    gh, gw = (inp["gh"], inp["gw"]) if table else (0, 0)
    tp = dev["table"].data_ptr() if table else None
    nb = lib.ba_workspace_bytes(B, H, N, d, gh, gw)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=device())
    wp = (ws.data_ptr() + 255) // 256 * 256
    out = torch.empty_like(dev["q"])
    sp = torch.cuda.current_stream().cuda_stream
    bq.check(lib, lib.ba_attention_prepare(dev["k"].data_ptr(), dev["v"].data_ptr(), tp, gh, gw, B, H, N, d,
                                           wp, nb, sp))
    bq.check(lib, lib.ba_attention_fwd_prepared(dev["q"].data_ptr(), tp, gh, gw, B, H, N, d, d ** -0.5,
                                                out.data_ptr(), wp, nb, sp))
    torch.cuda.synchronize()
    return out


CASES = [
    # B, H, gh, gw, d, table, q_scale
    (1, 3, 14, 14, 64, True, 1.0),     # the tiny ViT grid, N = 196
    (2, 2, 14, 14, 32, True, 1.0),     # d = 32
    (2, 2, 16, 16, 64, True, 1.0),     # N = 256: four full tiles
    (2, 1, 1, 256, 64, False, 1.0),    # no bias, N = 256
    (1, 2, 1, 65, 64, False, 1.0),     # ragged: one full tile and one key
    (3, 2, 1, 1, 64, False, 1.0),      # N = 1
    (1, 2, 7, 9, 64, True, 1.0),       # N = 63: one ragged tile
    (1, 3, 14, 14, 64, True, 8.0),     # large logits: the exact path
    (2, 2, 5, 13, 32, False, 8.0),     # exact path without a bias
]


@pytest.mark.parametrize("B,H,gh,gw,d,table,q_scale", CASES)
def test_small_matches_two_launch(B, H, gh, gw, d, table, q_scale):
    announce("small", B, H, gh, gw, d, table, q_scale)
    N = gh * gw
    inp = workloads.make_inputs(B, H, N, d, seed=7000 + N + d, grid=(gh, gw) if table else None, bias=table,
                                q_scale=q_scale, k_scale=q_scale)
    dev = to_dev(inp)
    o = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"] if table else None,
                         inp["gh"] if table else 0, inp["gw"] if table else 0)
    torch.cuda.synchronize()
    ref = two_launch(dev, inp, B, H, N, d, table)
    assert torch.equal(o, ref)
    err = o_error(o, oracle_rows(inp), inp["v"])
    assert err <= TOL, err


def test_small_strided_and_train():
    """The one-launch kernel reads K and V through their strides ([B,N,H,d]
    here), and the training forward takes it too (same O, plus lse)."""
    B, H, gh, gw, d = 2, 3, 14, 14, 64
    announce("small strided/train", B, H, gh, gw, d)
    N = gh * gw
    inp = workloads.make_inputs(B, H, N, d, seed=7100, grid=(gh, gw))
    dev = to_dev(inp)
    ref = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"], gh, gw)
    bnhd = [x.transpose(1, 2).contiguous().transpose(1, 2) for x in (dev["q"], dev["k"], dev["v"])]
    o = bq.attention_fwd(*bnhd, dev["table"], gh, gw)
    o2, lse = bq.attention_fwd_train(dev["q"], dev["k"], dev["v"], dev["table"], gh, gw)
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous(), ref)
    assert torch.equal(o2, ref)
    assert bool(torch.isfinite(lse).all())
