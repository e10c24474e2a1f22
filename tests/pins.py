"""Pins that tie the CPU oracle to what the BinaryAttention pages and plain
mathematics fix, without trusting the oracle itself.

Each pin takes the oracle module (``oracle.dense_fp64``) as ``ob`` and
raises AssertionError on a mismatch.  The same pins run against deliberately
broken copies of the oracle in test_oracle_mutations.py, where at least one
of them must fail for every planted mistake.

What each pin compares against:
* golden_hand_example: a worked example derived by hand (tests/golden/);
* bits_*: the per-element definition of the sign bit, popcounts, +/-0;
* alpha_*: closed forms (x = a * (+/-1 pattern) gives mu = |a|);
* dots_*: the +/-1 dot product against d - 2*Hamming, parity and extremes;
* textbook_reduction: when every Q/K token has entries of one magnitude,
  BinaryAttention is exactly softmax(scale Q K^T + B) V, which torch's
  scaled_dot_product_attention computes (an independent library routine);
* bias_*: which key a single large table entry points at, on a non-square
  grid, and the closed form O = mean(V) when Q = 0 without bias;
* brute_force_tiny: a triple loop in Python ints and math.fsum;
* sheppard: E[sign(q) sign(k)] = (2/pi) asin(rho) for correlated normals.
"""

from __future__ import annotations

import math
import pathlib

import numpy as np
import torch

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_values(rng, shape, scale=1.0):
    """Random float64 values that are exactly representable in bf16."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


# --------------------------------------------------------------------------
# golden
# --------------------------------------------------------------------------

def load_hand_example():
    rec: dict = {}
    for line in (GOLDEN / "hand_example_d4.txt").read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        rec.setdefault(key, []).append(vals)
    grid = tuple(int(x) for x in rec["grid"][0])
    d = int(rec["d"][0][0])

    def arr(key, dtype=float):
        return np.array([[dtype(x) for x in row] for row in rec[key]])

    return {
        "gh": grid[0], "gw": grid[1], "d": d,
        "q": arr("q")[None, None], "k": arr("k")[None, None],
        "v": arr("v")[None, None], "table": arr("table")[None],
        "qbits": arr("qbits", int)[:, 0], "kbits": arr("kbits", int)[:, 0],
        "alpha_q": arr("alpha_q")[0], "alpha_k": arr("alpha_k")[0],
        "D": arr("D", int), "S": arr("S"),
    }


def golden_hand_example(ob):
    g = load_hand_example()
    assert np.array_equal(ob.pack_sign_bits(g["q"])[0, 0, :, 0], g["qbits"])
    assert np.array_equal(ob.pack_sign_bits(g["k"])[0, 0, :, 0], g["kbits"])
    assert np.array_equal(ob.token_scale(g["q"])[0, 0], g["alpha_q"])
    assert np.array_equal(ob.token_scale(g["k"])[0, 0], g["alpha_k"])
    assert np.array_equal(ob.sign_dots(g["q"], g["k"])[0, 0], g["D"])
    res = ob.binary_attention_rows(g["q"], g["k"], g["v"], g["table"],
                                   g["gh"], g["gw"], keep=True)
    assert np.allclose(res["S"][0, 0], g["S"], rtol=0, atol=1e-15)
    v = g["v"][0, 0]
    for i in range(2):
        w = [math.exp(s) for s in g["S"][i]]
        tot = math.fsum(w)
        expect = [math.fsum(w[j] * v[j, c] for j in range(2)) / tot
                  for c in range(g["d"])]
        assert np.allclose(res["O"][0, 0, i], expect, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# bits
# --------------------------------------------------------------------------

def bits_definition(ob):
    rng = _rng(11)
    for d in (1, 7, 31, 32, 33, 64, 72, 96, 128, 200):
        x = _bf16_values(rng, (3, d))
        x[0, : d // 3] = 0.0
        x[1, : d // 3] = -0.0
        bits = ob.pack_sign_bits(x)
        w = (d + 31) // 32
        assert bits.shape == (3, w) and bits.dtype == np.uint32
        for t in range(3):
            for c in range(32 * w):
                got = (int(bits[t, c // 32]) >> (c % 32)) & 1
                want = int(c < d and x[t, c] < 0)
                assert got == want, (d, t, c)
            assert sum(bin(int(b)).count("1") for b in bits[t]) == \
                int(np.sum(x[t] < 0))
        assert np.array_equal(ob.unpack_sign_bits(bits, d),
                              np.where(x < 0, -1.0, 1.0))


def bits_special_values(ob):
    for d in (5, 32, 40, 64, 72):
        zeros = np.zeros((1, d))
        negz = -np.zeros((1, d))
        assert np.signbit(negz).all()
        assert not ob.pack_sign_bits(zeros).any()
        assert not ob.pack_sign_bits(negz).any()
        allneg = -np.ones((1, d))
        bits = ob.pack_sign_bits(allneg)[0]
        for w, word in enumerate(bits):
            nvalid = min(32, d - 32 * w)
            assert int(word) == (1 << nvalid) - 1
        assert np.array_equal(ob.sign_pm1(np.array([0.0, -0.0, -1e-30, 1e-30])),
                              [1.0, 1.0, -1.0, 1.0])


# --------------------------------------------------------------------------
# alpha
# --------------------------------------------------------------------------

def alpha_closed_form(ob):
    rng = _rng(12)
    for d in (1, 3, 64, 72, 128):
        a = np.array([0.75, -1.5, 2.0 ** -7, 3.0, 0.0])
        pattern = np.where(rng.random((5, d)) < 0.5, -1.0, 1.0)
        x = a[:, None] * pattern
        mu = ob.token_scale(x)
        assert np.array_equal(mu, np.abs(a)), (d, mu)
        assert np.array_equal(mu[:, None] * ob.sign_pm1(x)[:, :], x + 0.0)
    assert ob.token_scale(np.array([[3.0, -1.0]]))[0] == 2.0
    assert ob.token_scale(np.array([[-2.0, -2.0, -2.0, 6.0]]))[0] == 3.0


# --------------------------------------------------------------------------
# integer dots
# --------------------------------------------------------------------------

def dots_two_formulas(ob):
    rng = _rng(13)
    for d in (1, 7, 31, 32, 33, 64, 72, 96, 128, 256):
        q = _bf16_values(rng, (2, 1, 9, d))
        k = _bf16_values(rng, (2, 1, 7, d))
        q[0, 0, 0, :3] = -0.0
        dd = ob.sign_dots(q, k)
        hd = ob.sign_dots_from_bits(ob.pack_sign_bits(q),
                                    ob.pack_sign_bits(k), d)
        assert np.array_equal(dd, hd), d
        assert np.all((dd - d) % 2 == 0)
        assert np.all(np.abs(dd) <= d)
        # brute force with Python ints
        for b in range(2):
            for i in range(9):
                for j in range(7):
                    s = sum((-1 if q[b, 0, i, c] < 0 else 1) *
                            (-1 if k[b, 0, j, c] < 0 else 1) for c in range(d))
                    assert int(dd[b, 0, i, j]) == s


def dots_extremes(ob):
    rng = _rng(14)
    for d in (1, 33, 64, 72):
        q = _bf16_values(rng, (1, 1, 4, d))
        q[q == 0] = 1.0
        both = np.concatenate([q, -q], axis=2)
        dd = ob.sign_dots(q, both)[0, 0]
        assert np.all(np.diag(dd[:, :4]) == d)
        assert np.all(np.diag(dd[:, 4:]) == -d)


# --------------------------------------------------------------------------
# softmax / whole pipeline
# --------------------------------------------------------------------------

def softmax_rows_normalised(ob):
    rng = _rng(15)
    q = _bf16_values(rng, (2, 2, 12, 40), 3.0)
    k = _bf16_values(rng, (2, 2, 12, 40), 3.0)
    v = _bf16_values(rng, (2, 2, 12, 40))
    t = _bf16_values(rng, (2, 5, 7), 0.5)
    res = ob.binary_attention_rows(q, k, v, t, 3, 4, keep=True)
    p = res["P"]
    assert p.shape == (2, 2, 12, 12)
    assert np.all(p > 0)
    assert np.allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)


def _dense_bias_loops(table, gh, gw):
    """Dense [H, N, N] bias from explicit (y, x) coordinates."""
    h = table.shape[0]
    n = gh * gw
    out = np.zeros((h, n, n))
    for i in range(n):
        for j in range(n):
            yi, xi = divmod(i, gw)
            yj, xj = divmod(j, gw)
            out[:, i, j] = table[:, (yi - yj) + gh - 1, (xi - xj) + gw - 1]
    return out


def textbook_reduction(ob):
    """Constant-magnitude rows: alpha * sign(x) == x exactly, so the method
    must equal textbook attention softmax(scale Q K^T + B) V."""
    rng = _rng(16)
    for (b, h, gh, gw, d) in ((1, 2, 3, 4, 8), (2, 1, 2, 5, 33), (1, 1, 4, 4, 64)):
        n = gh * gw
        mag_q = np.abs(_bf16_values(rng, (b, h, n, 1))) + 0.25
        mag_k = np.abs(_bf16_values(rng, (b, h, n, 1))) + 0.25
        q = mag_q * np.where(rng.random((b, h, n, d)) < 0.5, -1.0, 1.0)
        k = mag_k * np.where(rng.random((b, h, n, d)) < 0.5, -1.0, 1.0)
        v = _bf16_values(rng, (b, h, n, d))
        t = _bf16_values(rng, (h, 2 * gh - 1, 2 * gw - 1), 0.7)
        scale = 1.0 / math.sqrt(d)
        mask = torch.from_numpy(_dense_bias_loops(t, gh, gw))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=mask, scale=scale).numpy()
        got = ob.binary_attention(q, k, v, t, gh, gw)["O"]
        assert np.allclose(got, ref, rtol=0, atol=1e-12), np.abs(got - ref).max()
        ref_nb = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            scale=scale).numpy()
        got_nb = ob.binary_attention(q, k, v)["O"]
        assert np.allclose(got_nb, ref_nb, rtol=0, atol=1e-12)


def bias_points_at_offset(ob):
    """With Q = 0 the scores are the bias alone.  One large entry at table
    index (dy0 + gh - 1, dx0 + gw - 1) must send each query i almost all of
    its mass to the key j with yi - yj = dy0 and xi - xj = dx0."""
    gh, gw, d = 3, 5, 4
    n = gh * gw
    for dy0, dx0 in ((1, -2), (-2, 3), (0, 1), (2, 0)):
        table = np.zeros((1, 2 * gh - 1, 2 * gw - 1))
        table[0, dy0 + gh - 1, dx0 + gw - 1] = 40.0
        q = np.zeros((1, 1, n, d))
        k = _bf16_values(_rng(17), (1, 1, n, d))
        v = np.eye(n)[None, None][..., :n]
        res = ob.binary_attention_rows(q, k, v, table, gh, gw, keep=True)
        p = res["P"][0, 0]
        for i in range(n):
            yi, xi = divmod(i, gw)
            yj, xj = yi - dy0, xi - dx0
            if 0 <= yj < gh and 0 <= xj < gw:
                assert p[i, yj * gw + xj] > 0.999, (dy0, dx0, i)
            else:
                assert np.allclose(p[i], 1.0 / n, atol=1e-12)


def zero_query_mean(ob):
    rng = _rng(18)
    q = np.zeros((2, 3, 10, 16))
    k = _bf16_values(rng, (2, 3, 10, 16))
    v = _bf16_values(rng, (2, 3, 10, 16))
    o = ob.binary_attention(q, k, v)["O"]
    assert np.allclose(o, v.mean(axis=2, keepdims=True), rtol=0, atol=1e-14)


def single_token(ob):
    rng = _rng(19)
    q = _bf16_values(rng, (2, 2, 1, 24))
    k = _bf16_values(rng, (2, 2, 1, 24))
    v = _bf16_values(rng, (2, 2, 1, 24))
    t = _bf16_values(rng, (2, 1, 1))
    assert np.allclose(ob.binary_attention(q, k, v, t, 1, 1)["O"], v,
                       rtol=0, atol=1e-15)


def brute_force_tiny(ob):
    """Naive loops: Python ints for D, math.fsum/math.exp for the rest."""
    rng = _rng(20)
    for (gh, gw, d) in ((3, 3, 1), (2, 3, 7), (3, 3, 31), (1, 4, 32),
                        (3, 2, 33), (2, 2, 40), (3, 3, 72)):
        n = gh * gw
        q = _bf16_values(rng, (1, 2, n, d))
        k = _bf16_values(rng, (1, 2, n, d))
        v = _bf16_values(rng, (1, 2, n, d))
        t = _bf16_values(rng, (2, 2 * gh - 1, 2 * gw - 1), 0.3)
        q[0, 0, 0, 0] = -0.0
        got = ob.binary_attention(q, k, v, t, gh, gw)["O"]
        for h in range(2):
            mq = [math.fsum(abs(float(z)) for z in q[0, h, i]) / d for i in range(n)]
            mk = [math.fsum(abs(float(z)) for z in k[0, h, j]) / d for j in range(n)]
            for i in range(n):
                srow = []
                for j in range(n):
                    dot = 0
                    for c in range(d):
                        a = -1 if q[0, h, i, c] < 0 else 1
                        b = -1 if k[0, h, j, c] < 0 else 1
                        dot += a * b
                    yi, xi = divmod(i, gw)
                    yj, xj = divmod(j, gw)
                    bias = float(t[h, yi - yj + gh - 1, xi - xj + gw - 1])
                    srow.append(mq[i] * mk[j] * dot / math.sqrt(d) + bias)
                m = max(srow)
                e = [math.exp(s - m) for s in srow]
                tot = math.fsum(e)
                for c in range(d):
                    o = math.fsum(e[j] * float(v[0, h, j, c]) for j in range(n)) / tot
                    assert abs(o - got[0, h, i, c]) <= 1e-12, (gh, gw, d, h, i, c)


def sheppard(ob):
    """For correlated standard normals, E[sign q sign k] = (2/pi) asin(rho)
    (Sheppard's formula): the flavour of the pages' Theorem 1 that sign
    vectors keep the covariance structure."""
    rng = _rng(21)
    n = 400_000
    for rho in (-0.6, 0.0, 0.3, 0.9):
        z1 = rng.standard_normal(n)
        z2 = rho * z1 + math.sqrt(1 - rho * rho) * rng.standard_normal(n)
        dot = ob.sign_dots(z1[None, None, None, :], z2[None, None, None, :])
        est = dot[0, 0, 0, 0] / n
        want = 2.0 / math.pi * math.asin(rho)
        assert abs(est - want) < 5.0 / math.sqrt(n), (rho, est, want)


def dense_bias_matches_table(ob):
    """A dense bias written out from a relative-position table gives the
    table path's O (the table path is pinned on its own above); the table's
    bias is not symmetric in (i, j), so this also fixes which index is the
    query."""
    rng = _rng(22)
    for (b, h, gh, gw, d) in ((2, 2, 3, 4, 16), (1, 3, 2, 5, 40)):
        n = gh * gw
        q = _bf16_values(rng, (b, h, n, d))
        k = _bf16_values(rng, (b, h, n, d))
        v = _bf16_values(rng, (b, h, n, d))
        t = _bf16_values(rng, (h, 2 * gh - 1, 2 * gw - 1), 0.8)
        dense = _dense_bias_loops(t, gh, gw)[None]
        got = ob.binary_attention_dense_bias_rows(q, k, v, dense)["O"]
        ref = ob.binary_attention(q, k, v, t, gh, gw)["O"]
        assert np.allclose(got, ref, rtol=0, atol=1e-13), np.abs(got - ref).max()


def dense_bias_one_hot(ob):
    """With Q = 0 the scores are the bias alone.  A bias of 40 at (i, pi(i))
    for a per-batch permutation pi sends query i almost all of its mass to
    key pi(i): O_i = V_pi(i) up to e^-40."""
    rng = _rng(23)
    b, h, n, d = 2, 2, 7, 5
    q = np.zeros((b, h, n, d))
    k = _bf16_values(rng, (b, h, n, d))
    v = _bf16_values(rng, (b, h, n, d))
    bias = np.zeros((b, h, n, n))
    perm = [[rng.permutation(n) for _ in range(h)] for _ in range(b)]
    for bi in range(b):
        for hi in range(h):
            bias[bi, hi, np.arange(n), perm[bi][hi]] = 40.0
    o = ob.binary_attention_dense_bias_rows(q, k, v, bias)["O"]
    for bi in range(b):
        for hi in range(h):
            want = v[bi, hi, perm[bi][hi]]
            assert np.allclose(o[bi, hi], want, rtol=0, atol=1e-14), (bi, hi)


def dense_bias_row_shift_and_broadcast(ob):
    """Adding c_i to a whole bias row changes nothing (softmax ignores a
    per-row shift), a zero bias is no bias, and a [1, H, N, N] bias acts
    like the same bias repeated for every batch entry."""
    rng = _rng(24)
    b, h, n, d = 3, 2, 6, 24
    q = _bf16_values(rng, (b, h, n, d))
    k = _bf16_values(rng, (b, h, n, d))
    v = _bf16_values(rng, (b, h, n, d))
    base = ob.binary_attention(q, k, v)["O"]
    zero = ob.binary_attention_dense_bias_rows(q, k, v, np.zeros((1, h, n, n)))["O"]
    assert np.allclose(zero, base, rtol=0, atol=1e-15)
    shift = np.broadcast_to(rng.normal(size=(b, h, n, 1)) * 5.0, (b, h, n, n))
    got = ob.binary_attention_dense_bias_rows(q, k, v, shift)["O"]
    assert np.allclose(got, base, rtol=0, atol=1e-13)
    one = rng.normal(size=(1, h, n, n))
    a1 = ob.binary_attention_dense_bias_rows(q, k, v, one)["O"]
    a2 = ob.binary_attention_dense_bias_rows(q, k, v, np.repeat(one, b, axis=0))["O"]
    assert np.array_equal(a1, a2)
    rows = np.array([5, 0, 3])
    part = ob.binary_attention_dense_bias_rows(q, k, v, one, rows=rows)["O"]
    assert np.allclose(part, a1[:, :, rows, :], rtol=0, atol=1e-15)


def _grid_values(rng, shape, step):
    """Values step * n with integer n in [-127, 127] and |n| = 127 reached in
    every channel of every (b, h): exactly what per-channel 8-bit codes with
    scale `step` represent."""
    n = rng.integers(-127, 128, size=shape)
    n[..., 0, :] = np.where(rng.random(shape[:-2] + (shape[-1],)) < 0.5, -127, 127)
    return step * n.astype(np.float64), n


def int8_quantizers(ob):
    """Per-channel value codes: v = s*n + e with |e| < s/2 must give code n
    (round to nearest) and scale s when |n| reaches 127; an all-zero channel
    gives scale 0 and codes 0.  Coefficient codes: every row's maximum maps
    to 255, all codes lie in [0, 255], and a score ln(2)·k below the
    maximum gives round(255 / 2^k)."""
    rng = _rng(25)
    step = 2.0 ** -5
    v, n = _grid_values(rng, (2, 3, 40, 16), step)
    e = rng.uniform(-0.45, 0.45, size=v.shape) * step
    e[np.abs(n) == 127] = 0.0   # keep max |v| of each channel at exactly 127 steps
    v = v + e
    v[..., 7] = 0.0
    n[..., 7] = 0
    res = ob.quantize_values_int8(v)
    assert np.array_equal(res["codes"], n)
    want = np.full((2, 3, 16), step)
    want[..., 7] = 0.0
    assert np.allclose(res["scale"], want, rtol=0, atol=1e-15)
    s = rng.normal(size=(3, 5, 30)) * 4.0
    pq = ob.quantize_probs_u8(s)
    assert pq.min() >= 0 and pq.max() <= 255
    assert np.array_equal(pq.max(axis=-1), np.full((3, 5), 255))
    assert np.array_equal(np.argmax(s, axis=-1), np.argmax(pq, axis=-1))
    ladder = -math.log(2.0) * np.arange(9.0)
    assert np.array_equal(ob.quantize_probs_u8(ladder[None]),
                          np.array([[255, 128, 64, 32, 16, 8, 4, 2, 1]]))


def int8_closed_forms(ob):
    """Hybrid 8-bit attention on values that lie on their code grid: with
    Q = 0 and no bias every coefficient code is 255 and O is the exact column
    mean of V; with a one-hot table entry of 20 (other codes round to 0) each
    query gets exactly the value row of the key at that grid offset."""
    rng = _rng(26)
    step = 2.0 ** -4
    b, h, gh, gw, d = 2, 2, 3, 4, 8
    n = gh * gw
    v, _ = _grid_values(rng, (b, h, n, d), step)
    k = _bf16_values(rng, (b, h, n, d))
    q = np.zeros((b, h, n, d))
    o = ob.binary_attention_int8_pv_rows(q, k, v)["O"]
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), rtol=0, atol=1e-15)
    dy0, dx0 = 1, -2
    table = np.zeros((h, 2 * gh - 1, 2 * gw - 1))
    table[:, dy0 + gh - 1, dx0 + gw - 1] = 20.0
    o = ob.binary_attention_int8_pv_rows(q, k, v, table, gh, gw)["O"]
    for i in range(n):
        yi, xi = divmod(i, gw)
        yj, xj = yi - dy0, xi - dx0
        if 0 <= yj < gh and 0 <= xj < gw:
            assert np.allclose(o[:, :, i], v[:, :, yj * gw + xj], rtol=0, atol=1e-15), i
        else:
            assert np.allclose(o[:, :, i], v.mean(axis=2), rtol=0, atol=1e-15), i


def int8_error_bound(ob):
    """Against the exact attention (itself pinned above): rounding V costs at
    most s_c / 2, and rounding each coefficient by at most 1/2 of a code
    moves the normalised weights by at most N / sum_j Pq_ij in total, so
    |O8 - O| <= s_c / 2 + max_j |v_jc| * N / sum_j Pq_ij, element by element."""
    rng = _rng(27)
    for (b, h, gh, gw, d, spread) in ((1, 2, 4, 4, 16, 1.0), (2, 1, 3, 7, 33, 3.0), (1, 1, 8, 8, 64, 0.3)):
        n = gh * gw
        q = _bf16_values(rng, (b, h, n, d), spread)
        k = _bf16_values(rng, (b, h, n, d), spread)
        v = _bf16_values(rng, (b, h, n, d))
        t = _bf16_values(rng, (h, 2 * gh - 1, 2 * gw - 1), 0.5)
        r8 = ob.binary_attention_int8_pv_rows(q, k, v, t, gh, gw, keep=True)
        ref = ob.binary_attention(q, k, v, t, gh, gw)["O"]
        den = r8["Pq"].sum(axis=-1, keepdims=True)
        vmax = np.abs(v).max(axis=2, keepdims=True)
        bound = r8["v_scale"][:, :, None, :] / 2 + vmax * n / den + 1e-12
        assert (np.abs(r8["O"] - ref) <= bound).all(), float((np.abs(r8["O"] - ref) - bound).max())


def _loss_fd(fn, x, dof, eps=1e-6):
    """Central differences of L = sum(dO * O(x)) for every entry of x."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        lp = float((dof * fn(x)).sum())
        x[i] = old - eps
        lm = float((dof * fn(x)).sum())
        x[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


def backward_values_and_table(ob):
    """dV and the table gradient are exact derivatives (the forward is smooth
    in V and in the table): central differences of L = sum(dO * O) agree,
    and the invariants sum_j dV_j = sum_i dO_i and sum(dtable) = 0 (each
    row of dS sums to 0) hold."""
    rng = _rng(28)
    b, h, gh, gw, d = 2, 2, 2, 3, 5
    n = gh * gw
    q = _bf16_values(rng, (b, h, n, d))
    k = _bf16_values(rng, (b, h, n, d))
    v = _bf16_values(rng, (b, h, n, d))
    t = _bf16_values(rng, (h, 2 * gh - 1, 2 * gw - 1), 0.7)
    do = rng.normal(size=(b, h, n, d))
    g = ob.binary_attention_backward(q, k, v, do, t, gh, gw)
    fd_v = _loss_fd(lambda x: ob.binary_attention(q, k, x, t, gh, gw)["O"], v.copy(), do)
    assert np.allclose(g["dv"], fd_v, rtol=0, atol=1e-7), np.abs(g["dv"] - fd_v).max()
    fd_t = _loss_fd(lambda x: ob.binary_attention(q, k, v, x, gh, gw)["O"], t.copy(), do)
    assert np.allclose(g["dtable"], fd_t, rtol=0, atol=1e-7), np.abs(g["dtable"] - fd_t).max()
    assert np.allclose(g["dv"].sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-12)
    assert abs(g["dtable"].sum()) < 1e-12


def backward_queries_keys_alpha_path(ob):
    """With every |x| > 1 the straight-through term vanishes and sign is
    constant near x, so dq and dk are the exact derivatives (through alpha
    = mean |x| only): central differences of L agree."""
    rng = _rng(29)
    b, h, gh, gw, d = 1, 2, 2, 3, 6
    n = gh * gw

    def far(shape):
        return np.where(rng.random(shape) < 0.5, -1.0, 1.0) * (1.25 + np.abs(rng.normal(size=shape)))
    q, k = far((b, h, n, d)), far((b, h, n, d))
    v = _bf16_values(rng, (b, h, n, d))
    t = _bf16_values(rng, (h, 2 * gh - 1, 2 * gw - 1), 0.7)
    do = rng.normal(size=(b, h, n, d))
    g = ob.binary_attention_backward(q, k, v, do, t, gh, gw)
    fd_q = _loss_fd(lambda x: ob.binary_attention(x, k, v, t, gh, gw)["O"], q.copy(), do)
    fd_k = _loss_fd(lambda x: ob.binary_attention(q, x, v, t, gh, gw)["O"], k.copy(), do)
    assert np.allclose(g["dq"], fd_q, rtol=0, atol=1e-7), np.abs(g["dq"] - fd_q).max()
    assert np.allclose(g["dk"], fd_k, rtol=0, atol=1e-7), np.abs(g["dk"] - fd_k).max()


def binarize_backward_surrogate(ob):
    """The reading of the sign gradient, checked on its own: at x0 the
    gradient equals the transposed Jacobian of the surrogate
    F(x) = alpha(x) sign(x0) + alpha(x0) (clip(x, -1, 1) - clip(x0, -1, 1)),
    which has the same value as alpha(x) sign(x) at x0 and the clipped
    straight-through derivative; the Jacobian comes from central
    differences."""
    rng = _rng(30)
    d = 9
    for _ in range(4):
        x0 = rng.normal(size=d) * 1.2
        x0[np.abs(np.abs(x0) - 1.0) < 1e-3] += 0.01  # stay off the clip corners
        g = rng.normal(size=d)
        s0 = np.where(x0 < 0, -1.0, 1.0)
        a0 = np.abs(x0).mean()

        def f(x):
            return np.abs(x).mean() * s0 + a0 * (np.clip(x, -1, 1) - np.clip(x0, -1, 1))
        jac = np.zeros((d, d))
        for c in range(d):
            e = np.zeros(d)
            e[c] = 1e-6
            jac[:, c] = (f(x0 + e) - f(x0 - e)) / 2e-6
        got = ob.binarize_backward(x0[None], g[None])[0]
        assert np.allclose(got, jac.T @ g, rtol=0, atol=1e-8), np.abs(got - jac.T @ g).max()


ALL_PINS = [
    golden_hand_example,
    bits_definition,
    bits_special_values,
    alpha_closed_form,
    dots_two_formulas,
    dots_extremes,
    softmax_rows_normalised,
    textbook_reduction,
    bias_points_at_offset,
    zero_query_mean,
    single_token,
    brute_force_tiny,
    sheppard,
    dense_bias_matches_table,
    dense_bias_one_hot,
    dense_bias_row_shift_and_broadcast,
    int8_quantizers,
    int8_closed_forms,
    int8_error_bound,
    backward_values_and_table,
    backward_queries_keys_alpha_path,
    binarize_backward_surrogate,
]
