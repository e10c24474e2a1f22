"""GPU parity of ba_attention_bwd with the oracle's binary_attention_backward.

Bar, per gradient tensor G: max |G_gpu - G_oracle| <= 1e-2 * max |G_oracle|.
Derivation: the kernels round P, dS * alpha and the value / output rows to
bf16 (relative 2^-9 each) before the matrix products, accumulate in fp32,
and rebuild P from the forward's row sums of bf16 P (the forward's own
normalisation, R3); the +/-1 sign operands and the straight-through
decision |x| <= 1 are exact (bf16 inputs on both sides).  Each gradient
entry is a sum of such rounded terms, so its error is a few 2^-9 of the
sum of the magnitudes of its terms, which on these inputs stays below 0.5 %
of the largest entry (measured 0.1-0.3 %); the table gradient sums dS over
many pairs and lands lower (measured < 0.05 %)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_cases import announce, device, np32, to_dev

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_qk_quantisation_amd")

TOL = 1e-2


def run_case(B, H, gh, gw, d, seed, bias=True, q_scale=1.0, table_sigma=0.02, discriminate=False, table_fn=None):
    N = gh * gw
    inp = workloads.make_inputs(B, H, N, d, seed=seed, grid=(gh, gw) if bias else None, bias=bias,
                                q_scale=q_scale, table_sigma=table_sigma)
    if table_fn is not None:
        inp["table"] = table_fn(inp["table"])
    rng = np.random.default_rng(seed + 1)
    do = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(torch.bfloat16)
    dev = to_dev(inp)
    got = bq.attention_bwd(dev["q"], dev["k"], dev["v"], do.to(device()), dev["table"], inp["gh"], inp["gw"])
    torch.cuda.synchronize()
    ref = oracle.binary_attention_backward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(do),
                                           np32(inp["table"]) if bias else None, inp["gh"], inp["gw"])
    if discriminate:
        # the same gradients with the bias dropped or mirrored miss the bar
        # by five times or more in dq, dk and dv
        t = np32(inp["table"])
        for name, tm in (("dropped", None), ("negated", -t), ("dx mirrored", t[:, :, ::-1].copy())):
            alt = oracle.binary_attention_backward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(do),
                                                   tm, inp["gh"], inp["gw"])
            for g in ("dq", "dk", "dv"):
                sep = float(np.abs(alt[g] - ref[g]).max() / np.abs(ref[g]).max())
                assert sep > 5 * TOL, (name, g, sep)
    errs = {}
    for name, g in zip(("dq", "dk", "dv", "dtable"), got):
        if g is None:
            assert ref[name] is None
            continue
        gg = g.cpu().numpy().astype(np.float64)
        assert np.isfinite(gg).all(), name
        errs[name] = float(np.abs(gg - ref[name]).max() / np.abs(ref[name]).max())
    print("relative max errors:", errs)
    for name, e in errs.items():
        assert e <= TOL, (name, e)


@pytest.mark.parametrize("B,H,gh,gw,d", [
    (1, 1, 8, 8, 64),      # table mode
    (2, 2, 7, 9, 32),      # table mode, N = 63 (ragged tile)
    (1, 3, 14, 14, 64),    # the tiny ViT grid
    (1, 2, 4, 32, 64),     # table rows
    (2, 1, 3, 32, 32),     # table rows, N = 96: ragged tile, padded block skipped
    (1, 1, 5, 13, 128),
    (1, 1, 2, 64, 128),    # table rows, d = 128
    (2, 2, 16, 64, 64),
])
def test_bwd_with_bias(B, H, gh, gw, d):
    announce("bwd", B, H, gh, gw, d)
    run_case(B, H, gh, gw, d, seed=6000 + gh * gw + d)


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 64, 64), (2, 1, 100, 32), (1, 2, 130, 128)])
def test_bwd_no_bias(B, H, N, d):
    announce("bwd no bias", B, H, N, d)
    run_case(B, H, 1, N, d, seed=6100 + N + d, bias=False)


@pytest.mark.parametrize("B,H,gh,gw,d", [
    (1, 2, 14, 14, 64),    # table in LDS
    (1, 2, 4, 32, 64),     # table rows
    (1, 1, 2, 64, 128),    # table rows, d = 128
])
def test_bwd_wide_table(B, H, gh, gw, d):
    """A sigma-2 table: the bias shapes P, so the gradients see how it is
    read (shown on the host with the bias dropped, negated and mirrored)."""
    announce("bwd wide table", B, H, gh, gw, d)
    run_case(B, H, gh, gw, d, seed=6300 + gh * gw + d, table_sigma=2.0, discriminate=True)


def test_bwd_large_logits():
    """Queries scaled up: the forward takes its exact path, whose row maximum
    enters the saved log2-sum-exp2."""
    announce("bwd large logits")
    run_case(1, 2, 4, 32, 64, seed=6201, q_scale=8.0)


def test_bwd_full_length_64x64():
    """N = 4096 on the 64x64 grid (the detection shape's sequence), one head."""
    announce("bwd 64x64")
    run_case(1, 1, 64, 64, 64, seed=6301)


@pytest.mark.parametrize("gh,gw", [(14, 14), (7, 9)])
def test_bwd_table_gradient_scales_exactly(gh, gw):
    """Table mode sums the table gradient as integers round(dS 2^k), with k
    chosen per workgroup from a bound that is linear in dO.  Every step of
    the backward is linear in dO, so scaling dO by 2^10 or 2^-10 must scale
    the table gradient by exactly that power of two (the same integers are
    summed at a shifted scale), and the result stays within the bar of the
    oracle at both scales."""
    announce("bwd table gradient scaling", gh, gw)
    B, H, d = 2, 2, 64
    N = gh * gw
    inp = workloads.make_inputs(B, H, N, d, seed=6300 + N, grid=(gh, gw))
    rng = np.random.default_rng(6301 + N)
    do = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(torch.bfloat16)
    dev = to_dev(inp)
    tabs = {}
    for e in (0, 10, -10):
        dos = (do.float() * 2.0 ** e).to(torch.bfloat16)  # exact: a power of two
        got = bq.attention_bwd(dev["q"], dev["k"], dev["v"], dos.to(device()), dev["table"], gh, gw)
        torch.cuda.synchronize()
        tabs[e] = got[3].cpu().numpy().astype(np.float64)
        assert np.isfinite(tabs[e]).all()
    for e in (10, -10):
        assert np.array_equal(tabs[e], tabs[0] * 2.0 ** e), e
    ref = oracle.binary_attention_backward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(do),
                                           np32(inp["table"]), gh, gw)["dtable"]
    assert float(np.abs(tabs[0] - ref).max() / np.abs(ref).max()) <= TOL


TRAIN_CASES = [
    # B, H, gh, gw, d, bias, q_scale
    (2, 2, 8, 8, 64, True, 1.0),      # table mode
    (1, 2, 4, 32, 64, True, 1.0),     # table rows
    (1, 2, 4, 32, 64, True, 8.0),     # table rows, exact path (large logits)
    (2, 1, 1, 100, 32, False, 1.0),   # no bias, ragged tile
    (1, 2, 16, 64, 64, True, 1.0),    # table rows, N = 1024: the key role on the side stream
]


@pytest.mark.parametrize("B,H,gh,gw,d,bias,q_scale", TRAIN_CASES)
def test_fwd_train_and_saved_bwd(B, H, gh, gw, d, bias, q_scale):
    """attention_fwd_train gives attention_fwd's O bit for bit and each row's
    ln sum_j exp(S_ij); attention_bwd with that O and lse gives the
    gradients of the recomputing backward.

    lse bar: the kernel forms the row sum l from the bf16 P it multiplies V
    with (relative rounding at most 2^-9 per term, so at most 2^-9 for the
    sum), and m + log2 l in fp32, so |lse - lse_oracle| <= 2^-9 + a few ulps:
    4e-3 here.  The two backwards differ only by lse's change of units
    (natural log and back, two fp32 roundings), which can flip a bf16 rounding
    of P or dS now and then: 1e-3 of each gradient's largest entry."""
    announce("fwd train / saved bwd", B, H, gh, gw, d, bias, q_scale)
    N = gh * gw
    inp = workloads.make_inputs(B, H, N, d, seed=6400 + N + d, grid=(gh, gw) if bias else None, bias=bias,
                                q_scale=q_scale)
    dev = to_dev(inp)
    tg, tgh, tgw = (dev["table"], inp["gh"], inp["gw"]) if bias else (None, 0, 0)
    o_ref = bq.attention_fwd(dev["q"], dev["k"], dev["v"], tg, tgh, tgw)
    o, lse = bq.attention_fwd_train(dev["q"], dev["k"], dev["v"], tg, tgh, tgw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    ref = oracle.binary_attention_rows(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]),
                                       np32(inp["table"]) if bias else None, inp["gh"], inp["gw"], keep=True)
    s = ref["S"]
    smax = s.max(axis=-1, keepdims=True)
    lse_ref = (smax + np.log(np.exp(s - smax).sum(axis=-1, keepdims=True)))[..., 0]
    err = float(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref).max())
    print("lse max abs error", err)
    assert err <= 4e-3

    rng = np.random.default_rng(6401 + N)
    do = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(torch.bfloat16).to(device())
    g_re = bq.attention_bwd(dev["q"], dev["k"], dev["v"], do, tg, tgh, tgw)
    g_sv = bq.attention_bwd(dev["q"], dev["k"], dev["v"], do, tg, tgh, tgw, o=o, lse=lse)
    torch.cuda.synchronize()
    gref = oracle.binary_attention_backward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(do.cpu()),
                                            np32(inp["table"]) if bias else None, inp["gh"], inp["gw"])
    for name, a, b in zip(("dq", "dk", "dv", "dtable"), g_re, g_sv):
        if a is None:
            assert b is None
            continue
        a64, b64 = a.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64)
        scale = np.abs(a64).max()
        assert float(np.abs(a64 - b64).max()) <= 1e-3 * scale, name
        assert float(np.abs(b64 - gref[name]).max() / np.abs(gref[name]).max()) <= TOL, name


def local_window(table):
    """-inf for every offset more than one grid row or three columns away."""
    H, r, c = table.shape
    gh, gw = (r + 1) // 2, (c + 1) // 2
    dy = torch.arange(-(gh - 1), gh).abs().view(1, -1, 1)
    dx = torch.arange(-(gw - 1), gw).abs().view(1, 1, -1)
    t = table.clone()
    t[((dy > 1) | (dx > 3)).expand_as(t)] = float("-inf")
    return t


@pytest.mark.parametrize("B,H,gh,gw,d", [(1, 2, 8, 8, 64), (1, 1, 8, 64, 64), (1, 1, 4, 32, 128)])
def test_bwd_local_window_table(B, H, gh, gw, d):
    """Gradients through a table that masks far keys with -inf: the masked
    pairs contribute nothing to dq, dk, dv, and their table entries get a
    zero gradient (table mode, table rows, d = 128)."""
    announce("bwd local-window table", B, H, gh, gw, d)
    run_case(B, H, gh, gw, d, seed=7300 + gh * gw + d, table_sigma=1.0, table_fn=local_window)
