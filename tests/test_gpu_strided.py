"""GPU parity of ba_attention_fwd_strided: the forward on strided views.

Every case runs the same inputs twice, once in contiguous [B,H,N,d] tensors
through ba_attention_fwd and once in another memory layout through the
strided entry.  The layout changes only where rows are read and written, not
the arithmetic, so the two outputs must be equal bit for bit; the strided
output is also held to the oracle's bar, max |dO| <= 1e-2 max |V|."""

import pytest
import torch

import workloads
from gpu_cases import announce, device, o_error, oracle_rows, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = 1e-2


def bnhd(x):
    """The same values stored as [B,N,H,d], seen as a [B,H,N,d] view."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def contiguous_reference(inp, dev):
    o = bq.attention_fwd(dev["q"], dev["k"], dev["v"], dev["table"], inp["gh"], inp["gw"])
    torch.cuda.synchronize()
    return o


def check(inp, dev, q, k, v, out, tag):
    assert not all(t.is_contiguous() for t in (q, k, v, out)), "case must take the strided entry"
    o = bq.attention_fwd(q, k, v, dev["table"], inp["gh"], inp["gw"], out=out)
    torch.cuda.synchronize()
    ref = contiguous_reference(inp, dev)
    assert torch.equal(o.contiguous(), ref), tag
    err = o_error(o.contiguous(), oracle_rows(inp), inp["v"])
    assert err <= TOL, (tag, err)


SHAPES = [
    # B, H, gh, gw, d
    (2, 3, 8, 8, 64),      # table mode, N = 64
    (1, 2, 4, 32, 64),     # row mode, N = 128
    (2, 2, 3, 32, 72),     # d = 72 padded to 96, N = 96 (ragged tile)
    (1, 2, 5, 13, 128),    # N = 65
    (1, 2, 9, 32, 64),     # N = 288: two launches, staged rows into strided o
]


@pytest.mark.parametrize("B,H,gh,gw,d", SHAPES)
def test_bnhd_layout(B, H, gh, gw, d):
    """q, k, v and o all stored as [B,N,H,d]."""
    announce("strided bnhd", B, H, gh, gw, d)
    inp = workloads.make_inputs(B, H, gh * gw, d, seed=700 + gh * gw + d, grid=(gh, gw))
    dev = to_dev(inp)
    out = torch.empty((B, gh * gw, H, d), dtype=torch.bfloat16, device=device()).transpose(1, 2)
    check(inp, dev, bnhd(dev["q"]), bnhd(dev["k"]), bnhd(dev["v"]), out, "bnhd")


@pytest.mark.parametrize("B,H,gh,gw,d", SHAPES)
def test_fused_qkv_slices(B, H, gh, gw, d):
    """q, k and v as the three slices of one [B,N,3,H,d] projection output;
    o contiguous."""
    announce("strided qkv", B, H, gh, gw, d)
    inp = workloads.make_inputs(B, H, gh * gw, d, seed=800 + gh * gw + d, grid=(gh, gw))
    dev = to_dev(inp)
    qkv = torch.stack([dev["q"], dev["k"], dev["v"]], dim=1)     # [B,3,H,N,d]
    qkv = qkv.permute(0, 3, 1, 2, 4).contiguous()                # [B,N,3,H,d]
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    out = torch.empty_like(dev["q"])
    check(inp, dev, q, k, v, out, "qkv")


def test_padded_rows_and_broadcast_kv():
    """Rows padded to d + 64 channels, and K/V shared by the whole batch
    (batch stride 0)."""
    B, H, gh, gw, d = 3, 2, 4, 32, 64
    announce("strided padded/broadcast", B, H, gh, gw, d)
    inp = workloads.make_inputs(B, H, gh * gw, d, seed=901, grid=(gh, gw))
    inp["k"] = inp["k"][:1].expand(B, -1, -1, -1).contiguous()
    inp["v"] = inp["v"][:1].expand(B, -1, -1, -1).contiguous()
    dev = to_dev(inp)
    N = gh * gw
    wide = torch.zeros((B, H, N, d + 64), dtype=torch.bfloat16, device=device())
    wide[..., :d] = dev["q"]
    q = wide[..., :d]
    k = dev["k"][:1].expand(B, -1, -1, -1)
    v = dev["v"][:1].expand(B, -1, -1, -1)
    assert k.stride(0) == 0
    out_wide = torch.full((B, H, N, d + 64), 7.0, dtype=torch.bfloat16, device=device())
    out = out_wide[..., :d]
    check(inp, dev, q, k, v, out, "padded")
    # the channels past d of the padded output rows are untouched
    assert bool((out_wide[..., d:] == 7.0).all())
