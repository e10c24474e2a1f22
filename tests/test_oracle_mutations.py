"""Plant plausible mistakes in the CPU oracle and check that the pins catch
each one.  Every mutation below patches one function of oracle.dense_fp64
for the duration of a test; the pins call through the module, so the
patched function is the one the rest of the oracle uses.
"""

import math

import numpy as np
import pytest

import oracle.dense_fp64 as ob
import pins

_orig = {name: getattr(ob, name) for name in (
    "sign_pm1", "token_scale", "pack_sign_bits", "sign_dots",
    "sign_dots_from_bits", "binary_scores", "softmax_rows",
    "binary_attention_rows")}


def _sign_zero_negative(x):
    a = ob._f64(x)
    return np.where(a <= 0.0, -1.0, 1.0)


def _sign_from_signbit(x):
    a = ob._f64(x)
    return np.where(np.signbit(a), -1.0, 1.0)


def _scale_signed_mean(x):
    a = ob._f64(x)
    return a.sum(axis=-1) / a.shape[-1]


def _scale_rms(x):
    a = ob._f64(x)
    return np.sqrt((a * a).sum(axis=-1) / a.shape[-1])


def _bits_msb_first(x):
    b = _orig["pack_sign_bits"](x)
    out = np.zeros_like(b)
    for i in range(32):
        out |= ((b >> np.uint32(i)) & np.uint32(1)) << np.uint32(31 - i)
    return out


def _bits_signbit(x):
    a = ob._f64(x)
    return _orig["pack_sign_bits"](np.where(np.signbit(a), -1.0, 1.0))


def _hamming_xnor_pads(qbits, kbits, d):
    qb = np.asarray(qbits, dtype=np.uint32)
    kb = np.asarray(kbits, dtype=np.uint32)
    x = ~np.bitwise_xor(qb[..., :, None, :], kb[..., None, :, :])
    agree = np.bitwise_count(x).astype(np.int64).sum(axis=-1)
    return 2 * agree - d


def _scores_factory(**kw):
    """A copy of binary_scores with one planted mistake selected by kw."""
    def scores(q, k, table=None, gh=0, gw=0, scale=None, rows=None):
        qf, kf = ob._f64(q), ob._f64(k)
        n, d = qf.shape[2], qf.shape[3]
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if kw.get("no_scale"):
            scale = 1.0
        if kw.get("scale_1_over_d"):
            scale = 1.0 / d
        r = np.arange(n) if rows is None else np.asarray(rows)
        aq, ak = ob.token_scale(qf), ob.token_scale(kf)
        if kw.get("drop_alpha_k"):
            ak = np.ones_like(ak)
        dots = ob.sign_dots(qf[:, :, r, :], kf)
        s = scale * aq[:, :, r, None] * ak[:, :, None, :] * dots
        if kw.get("transpose_dots"):
            s = np.swapaxes(s, -1, -2)
        if table is not None:
            t = ob._f64(table)
            idx = np.arange(n)
            y, x = idx // gw, idx % gw
            dy = y[r][:, None] - y[None, :] + gh - 1
            dx = x[r][:, None] - x[None, :] + gw - 1
            if kw.get("bias_sign"):
                dy = y[None, :] - y[r][:, None] + gh - 1
                dx = x[None, :] - x[r][:, None] + gw - 1
            if kw.get("bias_dx_sign"):
                dx = x[None, :] - x[r][:, None] + gw - 1
            if kw.get("bias_swap_axes"):
                s = s + t[:, dx % t.shape[1], dy % t.shape[2]][None]
            elif kw.get("drop_bias"):
                pass
            else:
                s = s + t[:, dy, dx][None]
        return {"alpha_q": aq, "alpha_k": ak, "D": dots, "S": s, "rows": r}
    return scores


def _softmax_columns(s):
    a = ob._f64(s)
    m = a.max(axis=-2, keepdims=True)
    e = np.exp(a - m)
    return e / e.sum(axis=-2, keepdims=True)


def _softmax_no_normalise(s):
    a = ob._f64(s)
    return np.exp(a - a.max(axis=-1, keepdims=True))


def _attention_v_transposed(q, k, v, table=None, gh=0, gw=0, scale=None,
                            rows=None, keep=False):
    out = _orig["binary_attention_rows"](q, k, v, table, gh, gw, scale,
                                         rows, keep=True)
    p = out["P"]
    vf = ob._f64(v)
    out["O"] = np.matmul(np.swapaxes(p, -1, -2), vf) if p.shape[-1] == p.shape[-2] \
        else out["O"] * 1.01
    return out



def _dense_factory(**kw):
    """A copy of binary_attention_dense_bias_rows with one planted mistake."""
    def dense(q, k, v, bias, scale=None, rows=None, keep=False):
        vf = ob._f64(v)
        sc = ob.binary_scores(q, k, None, 0, 0, scale, rows)
        bf = ob._f64(bias)
        if kw.get("transposed"):
            bf = np.swapaxes(bf, -1, -2)
        if kw.get("first_batch_only"):
            bf = bf[:1]
        s = sc["S"] if kw.get("dropped") else sc["S"] + bf[:, :, sc["rows"], :]
        p = ob.softmax_rows(s)
        return {"O": np.matmul(p, vf), "alpha_q": sc["alpha_q"], "alpha_k": sc["alpha_k"],
                "rows": sc["rows"]}
    return dense



def _qv_per_token(v):
    vf = np.asarray(ob._f64(v), dtype=np.float32)
    amax = np.abs(vf).max(axis=-1, keepdims=True)
    inv = (np.float32(127.0) / np.where(amax > 0, amax, np.float32(1.0))).astype(np.float32)
    return {"scale": np.broadcast_to(amax.max(axis=-2), vf.shape[:-2] + vf.shape[-1:]).astype(np.float64) / 127.0,
            "codes": np.rint(vf * inv).astype(np.int64)}


def _qv_floor(v):
    vf = np.asarray(ob._f64(v), dtype=np.float32)
    amax = np.abs(vf).max(axis=-2)
    inv = np.where(amax > 0, np.float32(127.0) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    return {"scale": amax.astype(np.float64) / 127.0, "codes": np.floor(vf * inv[..., None, :]).astype(np.int64)}


def _qp_not_shifted(s):
    a = ob._f64(s)
    return np.rint(np.float32(255.0) * np.minimum(np.exp(a), 1.0).astype(np.float32)).astype(np.int64)


def _qp_127(s):
    a = ob._f64(s)
    p = np.exp(a - a.max(axis=-1, keepdims=True)).astype(np.float32)
    return np.rint(np.float32(127.0) * p).astype(np.int64)


def _int8_factory(**kw):
    def f(q, k, v, table=None, gh=0, gw=0, scale=None, rows=None, keep=False):
        sc = ob.binary_scores(q, k, table, gh, gw, scale, rows)
        pq = ob.quantize_probs_u8(sc["S"])
        vq = ob.quantize_values_int8(v)
        num = np.matmul(pq, vq["codes"]).astype(np.float64)
        if kw.get("den_float"):
            a = sc["S"]
            den = 255.0 * np.exp(a - a.max(axis=-1, keepdims=True)).sum(axis=-1, keepdims=True)
        else:
            den = pq.sum(axis=-1, keepdims=True).astype(np.float64)
        sv = 1.0 if kw.get("no_scale") else vq["scale"][..., None, :]
        out = {"O": sv * num / den, "alpha_q": sc["alpha_q"], "alpha_k": sc["alpha_k"], "rows": sc["rows"]}
        if keep:
            out.update(S=sc["S"], Pq=pq, Vq=vq["codes"], v_scale=vq["scale"])
        return out
    return f



def _bwd_factory(**kw):
    """A copy of binary_attention_backward with one planted mistake."""
    def bwd(q, k, v, do, table=None, gh=0, gw=0, scale=None):
        qf, kf, vf, gf = ob._f64(q), ob._f64(k), ob._f64(v), ob._f64(do)
        b, h, n, d = qf.shape
        sc = 1.0 / math.sqrt(d) if scale is None else scale
        qt = ob.token_scale(qf)[..., None] * ob.sign_pm1(qf)
        kt = ob.token_scale(kf)[..., None] * ob.sign_pm1(kf)
        s = sc * np.matmul(qt, np.swapaxes(kt, -1, -2))
        if table is not None:
            s = s + ob.rel_pos_bias(table, gh, gw)[None]
        p = ob.softmax_rows(s)
        o = np.matmul(p, vf)
        dv = np.matmul(p if kw.get("dv_untransposed") else np.swapaxes(p, -1, -2), gf)
        delta = 0.0 if kw.get("no_delta") else (gf * o).sum(axis=-1, keepdims=True)
        ds = p * (np.matmul(gf, np.swapaxes(vf, -1, -2)) - delta)
        dqt = sc * np.matmul(ds, kt)
        dkt = sc * np.matmul(ds if kw.get("dk_untransposed") else np.swapaxes(ds, -1, -2), qt)
        dtable = None
        if table is not None:
            t = ob._f64(table)
            dtable = np.zeros_like(t)
            idx = np.arange(n)
            y, x = idx // gw, idx % gw
            sgn = -1 if kw.get("dtable_mirrored") else 1
            dy = (sgn * (y[:, None] - y[None, :]) + gh - 1).ravel()
            dx = (sgn * (x[:, None] - x[None, :]) + gw - 1).ravel()
            dsum = ds.sum(axis=0)
            for hh in range(h):
                np.add.at(dtable[hh], (dy, dx), dsum[hh].ravel())
        return {"dq": ob.binarize_backward(qf, dqt), "dk": ob.binarize_backward(kf, dkt), "dv": dv,
                "dtable": dtable, "O": o}
    return bwd


def _binb_unclipped(x, g):
    xf, gf = ob._f64(x), ob._f64(g)
    d = xf.shape[-1]
    s = ob.sign_pm1(xf)
    return s * (s * gf).sum(axis=-1, keepdims=True) / d + ob.token_scale(xf)[..., None] * gf


def _binb_no_alpha_path(x, g):
    xf, gf = ob._f64(x), ob._f64(g)
    return ob.token_scale(xf)[..., None] * (np.abs(xf) <= 1.0) * gf


MUTATIONS = {
    "sign_zero_is_negative": ("sign_pm1", _sign_zero_negative),
    "sign_from_signbit": ("sign_pm1", _sign_from_signbit),
    "scale_signed_mean": ("token_scale", _scale_signed_mean),
    "scale_rms": ("token_scale", _scale_rms),
    "bits_msb_first": ("pack_sign_bits", _bits_msb_first),
    "bits_from_signbit": ("pack_sign_bits", _bits_signbit),
    "xnor_counts_pad_bits": ("sign_dots_from_bits", _hamming_xnor_pads),
    "no_softmax_scale": ("binary_scores", _scores_factory(no_scale=True)),
    "scale_one_over_d": ("binary_scores", _scores_factory(scale_1_over_d=True)),
    "alpha_k_dropped": ("binary_scores", _scores_factory(drop_alpha_k=True)),
    "dots_transposed": ("binary_scores", _scores_factory(transpose_dots=True)),
    "bias_sign_flipped": ("binary_scores", _scores_factory(bias_sign=True)),
    "bias_dx_sign_flipped": ("binary_scores", _scores_factory(bias_dx_sign=True)),
    "bias_axes_swapped": ("binary_scores", _scores_factory(bias_swap_axes=True)),
    "bias_dropped": ("binary_scores", _scores_factory(drop_bias=True)),
    "softmax_over_columns": ("softmax_rows", _softmax_columns),
    "softmax_not_normalised": ("softmax_rows", _softmax_no_normalise),
    "pv_transposed": ("binary_attention_rows", _attention_v_transposed),
    "dense_bias_transposed": ("binary_attention_dense_bias_rows", _dense_factory(transposed=True)),
    "dense_bias_dropped": ("binary_attention_dense_bias_rows", _dense_factory(dropped=True)),
    "dense_bias_first_batch_only": ("binary_attention_dense_bias_rows",
                                    _dense_factory(first_batch_only=True)),
    "int8_v_scale_per_token": ("quantize_values_int8", _qv_per_token),
    "int8_v_codes_floor": ("quantize_values_int8", _qv_floor),
    "int8_p_not_shifted_by_row_max": ("quantize_probs_u8", _qp_not_shifted),
    "int8_p_scale_127": ("quantize_probs_u8", _qp_127),
    "int8_row_sum_unquantized": ("binary_attention_int8_pv_rows", _int8_factory(den_float=True)),
    "int8_value_scale_dropped": ("binary_attention_int8_pv_rows", _int8_factory(no_scale=True)),
    "bwd_dv_untransposed": ("binary_attention_backward", _bwd_factory(dv_untransposed=True)),
    "bwd_no_delta": ("binary_attention_backward", _bwd_factory(no_delta=True)),
    "bwd_dk_untransposed": ("binary_attention_backward", _bwd_factory(dk_untransposed=True)),
    "bwd_dtable_mirrored": ("binary_attention_backward", _bwd_factory(dtable_mirrored=True)),
    "bwd_ste_unclipped": ("binarize_backward", _binb_unclipped),
    "bwd_alpha_path_dropped": ("binarize_backward", _binb_no_alpha_path),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ob, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(ob)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"
