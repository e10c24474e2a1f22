"""CPU oracle for the BinaryAttention forward pass (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code, table or helper with the HIP library.

Sources (the two gist.science summaries of "BinaryAttention: One-Bit
QK-Attention for Vision and Diffusion Transformers"):

* es page, technical summary, section 2 "Metodologia", item "Representaciones
  Binarias Escaladas": queries and keys become s_i = mu_q * sign(q_i) and
  t_j = mu_k * sign(k_j), and their similarity is taken with XNOR + popcount.
* es page, section 2, item "Mejora mediante Sesgo": a learnable bias b_ij is
  added to the scores; one of its forms is position-sensitive.
* es page, section 2, item "Implementacion en Hardware" and ko page, section
  2 (c) "hardware-aware implementation": the kernel follows FlashAttention2,
  i.e. it computes exactly softmax(S) V; tiling changes the order, not the
  result.
* ko page, section 2 (b).1: the scale is a mean taken over the token's
  channels.

Readings where the pages are silent (each one is listed with its reason in
the design notes that accompany the repository):

* the per-token scale is alpha = mean over the d channels of |x|;
* sign(x) = -1 if x < 0 else +1, so +0.0 and -0.0 both give +1 (bit 0);
* packed bits: channel c goes to word c // 32, bit c % 32 (LSB first);
  bit = 1 means negative; bits for channels >= d are 0;
* <sign q, sign k> = d - 2 * popcount(qbits XOR kbits) (XOR with zero pad
  bits, equal to the XNOR-popcount form over the d real channels);
* S_ij = scale * alpha_q,i * alpha_k,j * D_ij + T[h, yi - yj + gh - 1,
  xi - xj + gw - 1] with tokens in row-major (y, x) order on a gh x gw grid,
  the table shared over the batch, and scale = 1/sqrt(d) by default;
* no masking: vision/diffusion attention is bidirectional.

Every value is computed in float64 from the exact widening of the bf16
inputs; integer quantities (bits, D) are returned as integers.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "sign_pm1",
    "token_scale",
    "pack_words",
    "pack_sign_bits",
    "unpack_sign_bits",
    "sign_dots",
    "sign_dots_from_bits",
    "rel_pos_bias",
    "binary_scores",
    "softmax_rows",
    "binary_attention",
    "binary_attention_rows",
]


def _f64(x) -> np.ndarray:
    """Widen an array-like (float32 holding bf16 values, or float64) to float64."""
    a = np.asarray(x)
    if a.dtype.kind != "f":
        raise TypeError(f"expected a floating-point array, got {a.dtype}")
    return a.astype(np.float64, copy=False)


def pack_words(d: int) -> int:
    """Number of 32-bit sign words per token: ceil(d / 32)."""
    if d < 1:
        raise ValueError("d must be >= 1")
    return (d + 31) // 32


def sign_pm1(x) -> np.ndarray:
    """sign() of the scaled binary representation (es page, section 2,
    "Representaciones Binarias Escaladas"), with sign(0) = +1.

    Uses an IEEE compare, so -0.0 < 0 is False and -0.0 maps to +1.
    """
    a = _f64(x)
    return np.where(a < 0.0, -1.0, 1.0)


def token_scale(x) -> np.ndarray:
    """Per-token scale mu (alpha): the mean of |x| over the last axis (the d
    channels of one token).  es page section 2 "Representaciones Binarias
    Escaladas" (mu is a mean of the queries/keys); ko page section 2 (b).1
    (mean over the channel axis)."""
    a = _f64(x)
    return np.abs(a).sum(axis=-1) / a.shape[-1]


def pack_sign_bits(x) -> np.ndarray:
    """Pack the signs of x[..., d] into uint32 words [..., ceil(d/32)].

    Channel c -> word c // 32, bit c % 32; bit = 1 iff x_c < 0; pad bits 0.
    The packing is what lets the similarity be taken with XOR/XNOR and
    popcount (es page, section 2, "Representaciones Binarias Escaladas").
    """
    a = _f64(x)
    d = a.shape[-1]
    w = pack_words(d)
    neg = a < 0.0
    pad = np.zeros(a.shape[:-1] + (32 * w - d,), dtype=bool)
    neg = np.concatenate([neg, pad], axis=-1).reshape(a.shape[:-1] + (w, 32))
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    words = (neg.astype(np.uint64) * weights).sum(axis=-1)
    return words.astype(np.uint32)


def unpack_sign_bits(bits, d: int) -> np.ndarray:
    """Inverse of pack_sign_bits: +/-1 float64 array [..., d]."""
    b = np.asarray(bits, dtype=np.uint32)
    w = b.shape[-1]
    if w != pack_words(d):
        raise ValueError("word count does not match d")
    shifts = np.arange(32, dtype=np.uint32)
    flags = (b[..., :, None] >> shifts) & np.uint32(1)
    flags = flags.reshape(b.shape[:-1] + (32 * w,))[..., :d]
    return np.where(flags == 1, -1.0, 1.0)


def sign_dots(q, k) -> np.ndarray:
    """D = sign(Q) sign(K)^T per leading index, as int64.

    A float64 matmul of +/-1 entries is exact (|D| <= d << 2**53)."""
    sq = sign_pm1(q)
    sk = sign_pm1(k)
    dots = np.matmul(sq, np.swapaxes(sk, -1, -2))
    return np.rint(dots).astype(np.int64)


def sign_dots_from_bits(qbits, kbits, d: int) -> np.ndarray:
    """D = d - 2 * popcount(qbits XOR kbits), the XNOR/popcount similarity
    of the es page (section 2, "Representaciones Binarias Escaladas")
    written with XOR over zero-padded words.

    qbits [..., Nq, W], kbits [..., Nk, W] -> int64 [..., Nq, Nk]."""
    qb = np.asarray(qbits, dtype=np.uint32)
    kb = np.asarray(kbits, dtype=np.uint32)
    x = np.bitwise_xor(qb[..., :, None, :], kb[..., None, :, :])
    ham = np.bitwise_count(x).astype(np.int64).sum(axis=-1)
    return d - 2 * ham


def rel_pos_bias(table, gh: int, gw: int) -> np.ndarray:
    """Dense position-sensitive bias b_ij (es page, section 2, "Mejora
    mediante Sesgo") from a per-head 2-D relative-position table.

    table: [H, 2*gh-1, 2*gw-1]; tokens are row-major on a gh x gw grid,
    token i at (yi, xi) = (i // gw, i % gw).
    Returns [H, N, N] with B[h, i, j] = table[h, yi-yj+gh-1, xi-xj+gw-1].
    """
    t = _f64(table)
    if t.ndim != 3 or t.shape[1] != 2 * gh - 1 or t.shape[2] != 2 * gw - 1:
        raise ValueError("table must be [H, 2*gh-1, 2*gw-1]")
    n = gh * gw
    idx = np.arange(n)
    y, x = idx // gw, idx % gw
    dy = y[:, None] - y[None, :] + gh - 1
    dx = x[:, None] - x[None, :] + gw - 1
    return t[:, dy, dx]


def binary_scores(q, k, table=None, gh: int = 0, gw: int = 0, scale=None,
                  rows=None) -> dict:
    """Scores S = scale * alpha_q alpha_k^T * D + b for q, k [B, H, N, d].

    rows: optional 1-D array of query indices; then only those rows of S
    are formed (keys are always all N).  Returns the intermediates.
    """
    qf = _f64(q)
    kf = _f64(k)
    if qf.shape != kf.shape or qf.ndim != 4:
        raise ValueError("q and k must both be [B, H, N, d]")
    n, d = qf.shape[2], qf.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    aq = token_scale(qf)
    ak = token_scale(kf)
    dots = sign_dots(qf[:, :, r, :], kf)
    s = float(scale) * aq[:, :, r, None] * ak[:, :, None, :] * dots
    if table is not None:
        if gh * gw != n:
            raise ValueError("N must equal gh * gw when a bias table is given")
        t = _f64(table)
        idx = np.arange(n)
        y, x = idx // gw, idx % gw
        dy = y[r][:, None] - y[None, :] + gh - 1
        dx = x[r][:, None] - x[None, :] + gw - 1
        s = s + t[:, dy, dx][None, :, :, :]
    return {"alpha_q": aq, "alpha_k": ak, "D": dots, "S": s, "rows": r}


def softmax_rows(s) -> np.ndarray:
    """Row softmax over the last axis, in float64 (max-shifted for range)."""
    a = _f64(s)
    m = a.max(axis=-1, keepdims=True)
    e = np.exp(a - m)
    return e / e.sum(axis=-1, keepdims=True)


def binary_attention_rows(q, k, v, table=None, gh: int = 0, gw: int = 0,
                          scale=None, rows=None, keep=False) -> dict:
    """O = softmax(S) V for a subset of query rows (all rows if rows=None).

    Rows of attention are independent, so a subset of rows is computed
    exactly as in the full problem.  keep=True also returns S and P.
    """
    vf = _f64(v)
    sc = binary_scores(q, k, table, gh, gw, scale, rows)
    p = softmax_rows(sc["S"])
    o = np.matmul(p, vf)
    out = {"O": o, "alpha_q": sc["alpha_q"], "alpha_k": sc["alpha_k"],
           "rows": sc["rows"]}
    if keep:
        out.update(S=sc["S"], P=p, D=sc["D"])
    return out


def binary_attention(q, k, v, table=None, gh: int = 0, gw: int = 0,
                     scale=None, block_rows: int = 1024) -> dict:
    """Full BinaryAttention forward in float64.

    q, k, v: [B, H, N, d] float arrays holding the (bf16) inputs.
    table:   [H, 2*gh-1, 2*gw-1] or None (no bias).
    Returns bits (uint32 [B,H,N,W]) for q and k, alpha (float64 [B,H,N]) for
    q and k, and O (float64 [B,H,N,d]).  Rows are processed in blocks only to
    bound memory; the result does not depend on block_rows.
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    b, h, n, d = qf.shape
    o = np.empty((b, h, n, d), dtype=np.float64)
    for r0 in range(0, n, block_rows):
        rows = np.arange(r0, min(n, r0 + block_rows))
        o[:, :, rows, :] = binary_attention_rows(
            qf, kf, vf, table, gh, gw, scale, rows)["O"]
    return {
        "q_bits": pack_sign_bits(qf),
        "k_bits": pack_sign_bits(kf),
        "alpha_q": token_scale(qf),
        "alpha_k": token_scale(kf),
        "O": o,
    }


def binary_attention_dense_bias_rows(q, k, v, bias, scale=None, rows=None,
                                     keep=False) -> dict:
    """O = softmax(S) V with a dense bias, for a subset of query rows.

    The bias term b_ij of es page, section 2, item "Mejora mediante Sesgo"
    (ko page, section 2 (b).2) may be dense: one learnable value per query,
    key and head.  Here it is given in full:

    bias: [Bb, H, N, N] with Bb = 1 (one bias for the whole batch) or Bb = B;
    S[b, h, i, j] = scale * alpha_q,i * alpha_k,j * D_ij + bias[b', h, i, j]
    with b' = b when Bb = B and b' = 0 when Bb = 1.
    """
    vf = _f64(v)
    sc = binary_scores(q, k, None, 0, 0, scale, rows)
    bf = _f64(bias)
    bq, hq, n = vf.shape[0], vf.shape[1], vf.shape[2]
    if bf.ndim != 4 or bf.shape[1:] != (hq, n, n) or bf.shape[0] not in (1, bq):
        raise ValueError("bias must be [1 or B, H, N, N]")
    s = sc["S"] + bf[:, :, sc["rows"], :]
    p = softmax_rows(s)
    o = np.matmul(p, vf)
    out = {"O": o, "alpha_q": sc["alpha_q"], "alpha_k": sc["alpha_k"],
           "rows": sc["rows"]}
    if keep:
        out.update(S=s, P=p, D=sc["D"])
    return out


def quantize_values_int8(v) -> dict:
    """Per-channel signed 8-bit values (es page, section 2, item
    "Cuantizacion Hibrida": the values are quantized to 8 bits per channel;
    ko page, section 2 (b).3).

    For each leading index and channel c: amax_c = max_j |v_jc|, the scale
    s_c = amax_c / 127 and the code vq_jc = round-half-even(v_jc * (127 /
    amax_c)) in [-127, 127]; a channel that is all zero gets scale 0 and
    codes 0.  The codes are decided in float32 (127 / amax_c correctly
    rounded, then the product, then the rounding), the precision a kernel
    decides them in.  Returns float64 scale [..., d] and int64 codes
    [..., N, d]."""
    vf = np.asarray(_f64(v), dtype=np.float32)
    amax = np.abs(vf).max(axis=-2)
    safe = np.where(amax > 0, amax, np.float32(1.0))
    inv = np.where(amax > 0, np.float32(127.0) / safe, np.float32(0.0)).astype(np.float32)
    codes = np.rint(vf * inv[..., None, :]).astype(np.int64)
    return {"scale": amax.astype(np.float64) / 127.0, "codes": codes}


def quantize_probs_u8(s) -> np.ndarray:
    """Static unsigned 8-bit attention coefficients (es page, section 2,
    item "Cuantizacion Hibrida": coefficients in [0, 1] take a static
    unsigned 8-bit quantization).

    Over the last axis, p = exp(s - max s) lies in [0, 1] (1 at the row
    maximum), and the code is round-half-even(255 p) in [0, 255], decided in
    float32.  Returns int64 codes."""
    a = _f64(s)
    m = a.max(axis=-1, keepdims=True)
    p = np.exp(a - m).astype(np.float32)
    return np.rint(np.float32(255.0) * p).astype(np.int64)


def binary_attention_int8_pv_rows(q, k, v, table=None, gh: int = 0, gw: int = 0,
                                  scale=None, rows=None, keep=False) -> dict:
    """BinaryAttention with the pages' hybrid 8-bit P.V (es page, section 2,
    item "Cuantizacion Hibrida"; ko page, section 2 (b).3: 1-bit Q/K, 8-bit
    attention coefficients and values), for a subset of query rows.

    S as in binary_scores; Pq = quantize_probs_u8(S) (row maximum -> 255);
    (s_c, Vq) = quantize_values_int8(V) over all N keys of each (b, h);
    O_ic = s_c * sum_j Pq_ij Vq_jc / sum_j Pq_ij.
    The row sum is taken over the same codes that multiply V, so the 1/255
    of the static scale cancels."""
    sc = binary_scores(q, k, table, gh, gw, scale, rows)
    pq = quantize_probs_u8(sc["S"])
    vq = quantize_values_int8(v)
    num = np.matmul(pq, vq["codes"]).astype(np.float64)
    den = pq.sum(axis=-1, keepdims=True).astype(np.float64)
    o = vq["scale"][..., None, :] * num / den
    out = {"O": o, "alpha_q": sc["alpha_q"], "alpha_k": sc["alpha_k"], "rows": sc["rows"]}
    if keep:
        out.update(S=sc["S"], Pq=pq, Vq=vq["codes"], v_scale=vq["scale"])
    return out


def binarize_backward(x, g) -> np.ndarray:
    """Gradient through the scaled binary representation x~ = alpha(x) sign(x)
    of es page, section 2, item "Representaciones Binarias Escaladas".

    The pages train with quantization-aware training and self-distillation
    (es section 2, item "Entrenamiento y Optimizacion"; ko section 2 (c))
    but give no gradient for sign.  Reading: alpha = mean |x| takes its exact
    derivative sign(x_c) / d, and sign takes the clipped straight-through
    estimator, derivative 1 where |x| <= 1 and 0 elsewhere.  So for the
    gradient g of x~ (one token, last axis = channels):
        dx = sign(x) * <sign(x), g> / d + alpha * 1{|x| <= 1} * g."""
    xf = _f64(x)
    gf = _f64(g)
    d = xf.shape[-1]
    s = sign_pm1(xf)
    a = token_scale(xf)[..., None]
    return s * (s * gf).sum(axis=-1, keepdims=True) / d + a * (np.abs(xf) <= 1.0) * gf


def binary_attention_backward(q, k, v, do, table=None, gh: int = 0, gw: int = 0,
                              scale=None) -> dict:
    """Gradients of the BinaryAttention forward for the output gradient dO
    (the loss L with dL/dO = dO), in float64.

    With q~ = alpha_q sign(q), k~ = alpha_k sign(k) and
    S = scale q~ k~^T + b, P = softmax_rows(S), O = P V:
        dV = P^T dO
        dS = P * (dO V^T - rowsum(dO * O))
        dq~ = scale dS k~,   dk~ = scale dS^T q~
        dq, dk = binarize_backward(q, dq~), binarize_backward(k, dk~)
        dtable[h, dy, dx] = sum over b and all (i, j) at grid offset
                            (yi - yj, xi - xj) = (dy - gh + 1, dx - gw + 1) of dS_ij
    (the table is shared over the batch).  Returns dq, dk, dv [B,H,N,d],
    dtable [H, 2gh-1, 2gw-1] (or None), and O."""
    qf, kf, vf, gf = _f64(q), _f64(k), _f64(v), _f64(do)
    b, h, n, d = qf.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qt = token_scale(qf)[..., None] * sign_pm1(qf)
    kt = token_scale(kf)[..., None] * sign_pm1(kf)
    s = float(scale) * np.matmul(qt, np.swapaxes(kt, -1, -2))
    if table is not None:
        s = s + rel_pos_bias(table, gh, gw)[None]
    p = softmax_rows(s)
    o = np.matmul(p, vf)
    dv = np.matmul(np.swapaxes(p, -1, -2), gf)
    delta = (gf * o).sum(axis=-1, keepdims=True)
    ds = p * (np.matmul(gf, np.swapaxes(vf, -1, -2)) - delta)
    dqt = float(scale) * np.matmul(ds, kt)
    dkt = float(scale) * np.matmul(np.swapaxes(ds, -1, -2), qt)
    dtable = None
    if table is not None:
        t = _f64(table)
        dtable = np.zeros_like(t)
        idx = np.arange(n)
        y, x = idx // gw, idx % gw
        dy = (y[:, None] - y[None, :] + gh - 1).ravel()
        dx = (x[:, None] - x[None, :] + gw - 1).ravel()
        dsum = ds.sum(axis=0)  # over the batch
        for hh in range(h):
            np.add.at(dtable[hh], (dy, dx), dsum[hh].ravel())
    return {"dq": binarize_backward(qf, dqt), "dk": binarize_backward(kf, dkt), "dv": dv,
            "dtable": dtable, "O": o}
