"""The C ABI without a GPU: the library loads, exports every symbol that
include/binattn.h declares, and rejects bad arguments synchronously, before
any HIP call (no compute happens in these tests)."""

import ctypes
import pathlib
import re

import pytest

from bit_qk_quantisation_amd import _lib

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "binattn.h"

pytestmark = pytest.mark.skipif(not _lib.LIB_PATH.exists(),
                                reason="libbinattn.so not built")


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ba_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_matches_binding_list():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.ba_version() == 1
    for code, name in _lib.STATUS.items():
        assert lib.ba_status_string(code).decode() == name
    assert lib.ba_status_string(99).decode() == "BA_ERR_UNKNOWN"


@pytest.mark.parametrize("d,w", [(0, 0), (1, 1), (8, 1), (32, 1), (33, 2), (64, 2),
                                 (72, 3), (128, 4), (256, 8)])
def test_pack_words(lib, d, w):
    assert lib.ba_pack_words(d) == w


def _round(x, m):
    return (x + m - 1) // m * m


def expected_workspace(B, H, N, d, gh=0, gw=0, int8pv=False):
    """Workspace sections as the header describes them: the K signs as fp4
    MFMA operands (32 bytes per 64 channels), the K scales, their maxima per
    64 tokens and V^T, per head
    padded to a multiple of 128 tokens, each section 256-byte aligned; plus,
    for a grid width that is a multiple of 32 and a key tile's window of at
    most 8 rows and 2048 floats, the float32 bias rows (4 shifted copies per
    row, each padded to 16 mod 64 floats, 8 padding rows on each side) and
    their maxima; for other grids whose table exceeds 48 KiB of float32, the
    table written out as a dense bias."""
    npad = _round(N, 128)
    W = (d + 31) // 32
    dpad = 32 * W
    secs = [B * H * npad * ((W + 1) // 2) * 32, B * H * npad * 4, B * H * (npad // 64) * 4]
    if int8pv:
        # int8 value codes, per-tile channel maxima, channel scales, code column sums
        secs += [B * H * dpad * npad, B * H * (npad // 64) * dpad * 4, B * H * dpad * 4, B * H * dpad * 4]
    else:
        secs.append(B * H * dpad * npad * 2)
    lpad = 0
    if gh and gw % 32 == 0:
        lpad = _round(2 * gw - 1 + 3, 4)
        while lpad % 64 != 16:
            lpad += 4
    # table rows: a window of at most 8 rows and 2048 floats per key tile
    rows = bool(gh) and gw % 32 == 0 and _window_rows(N, gw) <= 8 and _window_rows(N, gw) * 4 * lpad <= 2048 \
        and lpad <= 64 * 5
    if rows:
        secs.append(H * (2 * gh - 1 + 16) * 4 * lpad * 4)
        secs.append(H * (2 * gh - 1) * 4)
    if not int8pv and _prepared_pipelined(N, d, gh, gw, rows, lpad):
        # the values' natural rows, for the prepared forward's pipelined kernel
        secs.append(B * H * npad * d * 2)
    if not int8pv and _pipelined_shape(N, d, gh, gw, rows, lpad):
        # the key scales as the pipelined kernel's matrix operands
        secs.append(B * H * npad * 12)
    if gh and not rows and (2 * gh - 1) * (2 * gw - 1) * 4 > 48 * 1024:
        # any other grid: the table written out as a dense bf16 bias per head
        secs.append(H * npad * npad * 2)
    return sum(_round(s, 256) for s in secs)


def _window_rows(N, gw):
    qspan = max(((q0 + 127) // gw - q0 // gw) for q0 in range(0, _round(N, 128), 128))
    kspan = max(((k0 + 63) // gw - k0 // gw) for k0 in range(0, N, 64))
    return qspan + kspan + 1


def _pipelined_shape(N, d, gh, gw, rows, lpad):
    """The pipelined kernel takes d in {32, 64, 72, 128} with table rows whose
    window fits its buffers, or without a bias."""
    if d not in (32, 64, 72, 128) or (gh and not rows):
        return False
    return not rows or _window_rows(N, gw) * 4 * lpad <= (1664 if d <= 72 else 1152)


def _prepared_pipelined(N, d, gh, gw, rows, lpad):
    """The prepared forward runs the pipelined kernel (and the workspace holds
    a natural copy of V) for d in {32, 64, 72, 128} with table rows whose window
    fits its buffers, or without a bias, unless the whole forward would run
    as one launch (N <= 256, d in {32, 64}, no table rows)."""
    if d not in (32, 64, 72, 128) or (gh and not rows):
        return False
    if N <= 256 and d in (32, 64) and not rows:
        return False
    return not rows or _window_rows(N, gw) * 4 * lpad <= (1664 if d <= 72 else 1152)


@pytest.mark.parametrize("shape", [(1, 3, 196, 64, 14, 14), (32, 12, 196, 64, 14, 14),
                                   (8, 16, 1024, 72, 32, 32), (2, 12, 4096, 64, 64, 64),
                                   (1, 16, 16384, 128, 128, 128), (2, 2, 100, 40, 0, 0),
                                   (1, 2, 10000, 64, 100, 100), (1, 1, 32768, 64, 128, 256)])
def test_workspace_bytes(lib, shape):
    B, H, N, d, gh, gw = shape
    assert lib.ba_workspace_bytes(B, H, N, d, gh, gw) == expected_workspace(*shape)


@pytest.mark.parametrize("args", [(1, 1, 10, 7, 0, 0), (1, 1, 10, 264, 0, 0), (0, 1, 10, 64, 0, 0),
                                  (1, 1, 0, 64, 0, 0), (1, 1, 12, 64, 3, 5), (1, 1, 12, 64, 0, 12)])
def test_workspace_bytes_rejects(lib, args):
    assert lib.ba_workspace_bytes(*args) == 0


# Fake, never-dereferenced device addresses: validation must fail before use.
A = 0x100000
GB = 1 << 30


def fwd(lib, q=A, k=A + GB, v=A + 2 * GB, bias=None, gh=0, gw=0, B=1, H=2, N=64, d=64,
        scale=0.125, o=A + 3 * GB, ws=A + 4 * GB, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.ba_attention_fwd(q, k, v, bias, gh, gw, B, H, N, d, scale, o, ws, ws_bytes, None)


def test_fwd_null_pointers(lib):
    assert fwd(lib, q=None) == 1
    assert fwd(lib, v=None) == 1
    assert fwd(lib, o=None) == 1
    assert b"non-NULL" in lib.ba_last_error()


def test_fwd_shapes(lib):
    assert fwd(lib, N=0) == 2
    assert fwd(lib, B=-1) == 2
    assert fwd(lib, bias=A + 5 * GB, gh=4, gw=15, N=64) == 2      # gh*gw != N
    assert fwd(lib, scale=float("nan")) == 2
    assert fwd(lib, scale=-1.0) == 2
    assert fwd(lib, o=A + 16) == 2                                 # o overlaps q
    assert fwd(lib, B=1 << 20, H=1 << 10, N=1 << 12) == 2           # > 2^31 tokens


@pytest.mark.parametrize("d", [0, 4, 12, 100, 264, 512])
def test_fwd_unsupported_d(lib, d):
    assert fwd(lib, d=d) == 3


def test_fwd_unsupported_bias_table(lib):
    # gw not a multiple of 32, a table bigger than 48 KiB of float32, and a
    # dense form of 4 GiB or more per head (N = 50000)
    assert fwd(lib, bias=A + 5 * GB, gh=200, gw=250, N=50000) == 3
    assert lib.ba_workspace_bytes(1, 2, 50000, 64, 200, 250) == 0


def test_expanded_table_limits(lib):
    """Grids that only the dense expansion takes: the forward accepts them
    (it gets as far as the launch here, without a GPU), the 8-bit P.V forward
    and the backward refuse them."""
    tab = dict(bias=A + 5 * GB, gh=100, gw=70, N=7000)
    assert fwd(lib, **tab) == 6
    assert lib.ba_workspace_bytes_int8pv(1, 2, 7000, 64, 100, 70) == 0
    assert lib.ba_workspace_bytes_bwd(1, 2, 7000, 64, 100, 70) == 0
    assert lib.ba_attention_fwd_int8pv(A, A + GB, A + 2 * GB, A + 5 * GB, 100, 70, 1, 2, 7000, 64, 0.125,
                                       A + 3 * GB, A + 4 * GB, 1 << 40, None) == 3
    big = 1 << 40
    assert lib.ba_attention_bwd(A, A + GB, A + 2 * GB, A + 5 * GB, 100, 70, 1, 2, 7000, 64, 0.125, A + 6 * GB,
                                A + 7 * GB, A + 8 * GB, A + 9 * GB, None, A + 4 * GB, big, None) == 3


def test_fwd_alignment(lib):
    assert fwd(lib, q=A + 8) == 4
    assert fwd(lib, bias=A + 5 * GB + 2, gh=8, gw=8) == 4
    assert fwd(lib, ws=A + 4 * GB + 16) == 4                       # needs 256


def test_fwd_workspace(lib):
    assert fwd(lib, ws=None) == 5
    need = lib.ba_workspace_bytes(1, 2, 64, 64, 0, 0)
    assert fwd(lib, ws_bytes=need - 1) == 5
    assert b"too small" in lib.ba_last_error()
    assert fwd(lib, bias=A + 4 * GB + 256, gh=8, gw=8) == 5       # the table inside the workspace


def test_pack_validation(lib):
    assert lib.ba_pack_signs(None, 1, 1, 8, 64, A, A + GB, None) == 1
    assert lib.ba_pack_signs(A, 1, 1, 8, 63, A + GB, A + 2 * GB, None) == 3
    assert lib.ba_pack_signs(A, 1, 1, 0, 64, A + GB, A + 2 * GB, None) == 2
    assert lib.ba_pack_signs(A + 4, 1, 1, 8, 64, A + GB, A + 2 * GB, None) == 4


def test_qk_dot_validation(lib):
    assert lib.ba_qk_int_dot(None, A, 1, 1, 8, 64, 0, A + GB, None) == 1
    assert lib.ba_qk_int_dot(A, A + GB, 1, 1, 8, 64, 7, A + 2 * GB, None) == 3
    assert lib.ba_qk_int_dot(A, A + GB, 1, 1, 70000, 64, 0, A + 2 * GB, None) == 2
    assert lib.ba_qk_int_dot(A, A + GB, 1, 1, 8, 64, 0, A + 2 * GB + 4, None) == 4
    assert lib.ba_qk_int_dot(A, A + GB, 1, 1, 8, 64, 3 | 0x100, A + 2 * GB, None) == 3   # unknown route
    assert lib.ba_qk_int_dot(A, A + GB, 1, 1, 8, 72, 0x200, A + 2 * GB, None) == 3       # unknown flag
    # the row sums write B*H*N values, so the 2^40 bound on N*N does not apply
    assert lib.ba_qk_int_dot(A, A + GB, 65535, 1, 65535, 64, 0, A + 2 * GB, None) == 2
    assert lib.ba_qk_int_dot(A, A + GB, 1, 1, 65535, 64, 0x100 | 2, A + 2 * GB + 4, None) == 4


def test_last_error_is_thread_local(lib):
    import threading
    assert fwd(lib, d=12) == 3
    seen = []

    def other():
        seen.append(lib.ba_last_error())
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == [b""]
    assert b"d=12" in lib.ba_last_error()


def test_split_entry_validation(lib):
    """ba_attention_prepare takes k and v, ba_attention_fwd_prepared takes q
    and o; each validates only what it reads or writes."""
    ws = A + 4 * GB
    assert lib.ba_attention_prepare(None, A + 2 * GB, None, 0, 0, 1, 2, 64, 64, ws, 1 << 40, None) == 1
    assert lib.ba_attention_prepare(A + GB + 8, A + 2 * GB, None, 0, 0, 1, 2, 64, 64, ws, 1 << 40, None) == 4
    assert lib.ba_attention_prepare(A + GB, A + 2 * GB, None, 0, 0, 1, 2, 64, 64, ws, 16, None) == 5
    assert lib.ba_attention_fwd_prepared(None, None, 0, 0, 1, 2, 64, 64, 0.125, A + 3 * GB, ws, 1 << 40, None) == 1
    assert lib.ba_attention_fwd_prepared(A, None, 0, 0, 1, 2, 64, 64, 0.125, None, ws, 1 << 40, None) == 1
    assert lib.ba_attention_fwd_prepared(A, None, 0, 0, 1, 2, 64, 64, float("inf"), A + 3 * GB, ws, 1 << 40,
                                         None) == 2
    assert lib.ba_attention_fwd_prepared(A, None, 0, 0, 1, 2, 64, 64, 0.125, A + 16, ws, 1 << 40, None) == 2


def fwd_strided(lib, strides, q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, B=1, H=2, N=64, d=64,
                ws_bytes=1 << 40):
    arr = None if strides is None else (ctypes.c_int64 * 12)(*strides)
    return lib.ba_attention_fwd_strided(q, k, v, None, 0, 0, B, H, N, d, 0.125, o, arr,
                                        A + 4 * GB, ws_bytes, None)


# Stride checks come before the workspace size check, so a call with valid
# strides and a 16-byte workspace stops with BA_ERR_WORKSPACE: nothing is
# launched on the fake addresses these tests use.
WS_TOO_SMALL = 5


def bnhd(B, H, N, d):
    """(batch, head, token) strides of a [B,N,H,d] tensor viewed as [B,H,N,d]."""
    return (N * H * d, d, H * d)


def test_strided_validation(lib):
    """Checks the strided entry makes before it launches anything."""
    s = bnhd(1, 2, 64, 64) * 4
    assert fwd_strided(lib, None) == 1
    assert b"strides" in lib.ba_last_error()
    bad = list(s)
    bad[2] = 68                                    # q token stride not a multiple of 8
    assert fwd_strided(lib, bad) == 2
    bad = list(s)
    bad[4] = -8                                    # negative k head stride
    assert fwd_strided(lib, bad) == 2
    bad = list(s)
    bad[9:12] = [0, 64, 64]                        # o: heads 0 and 1 share rows 1.. of head 0
    assert fwd_strided(lib, bad) == 2
    assert b"overlap" in lib.ba_last_error()
    bad = list(s)
    bad[9:12] = [8192, 64, 32]                     # o rows 32 channels apart, d = 64
    assert fwd_strided(lib, bad) == 2
    # q, k and v as slices of one [B,N,3,H,d] tensor; o written over it
    qkv = (64 * 3 * 2 * 64, 64, 3 * 2 * 64)
    assert fwd_strided(lib, list(qkv) * 3 + list(bnhd(1, 2, 64, 64)),
                       q=A, k=A + 256, v=A + 512, o=A + 1024) == 2
    assert b"o must not overlap" in lib.ba_last_error()
    # broadcast inputs (stride 0) are fine for reads
    assert fwd_strided(lib, [0, 0, 64] * 3 + [2 * 64 * 64, 64 * 64, 64], o=A + 8 * GB,
                       ws_bytes=16) == WS_TOO_SMALL


def test_rows_disjoint_rule(lib):
    """The output-layout rule on a few permutations: every dense layout of
    [B,H,N,d] passes, a padded one passes, and a folded one fails."""
    B, H, N, d = 2, 3, 16, 64
    ok = [(H * N * d, N * d, d), bnhd(B, H, N, d), (d, B * N * d, B * d),
          (H * N * (d + 64), N * (d + 64), d + 64)]
    for o in ok:
        st = fwd_strided(lib, list(bnhd(B, H, N, d)) * 3 + list(o), o=A + 8 * GB, B=B, H=H, N=N,
                         ws_bytes=16)
        assert st == WS_TOO_SMALL, (o, lib.ba_last_error())
    assert fwd_strided(lib, list(bnhd(B, H, N, d)) * 3 + [N * d, N * d, d], o=A + 8 * GB,
                       B=B, H=H, N=N) == 2


def fwd_dense(lib, bias=A + 5 * GB, sb=0, sh=64 * 64, ld=64, B=1, H=2, N=64, d=64, o=A + 3 * GB,
              strides=None, ws_bytes=1 << 40):
    arr = None if strides is None else (ctypes.c_int64 * 12)(*strides)
    return lib.ba_attention_fwd_dense_bias(A, A + GB, A + 2 * GB, bias, sb, sh, ld, B, H, N, d, 0.125, o,
                                           arr, A + 4 * GB, ws_bytes, None)


def test_dense_bias_validation(lib):
    """Checks of the dense-bias entry, all before any launch (the valid
    cases stop at the 16-byte workspace)."""
    assert fwd_dense(lib, bias=None) == 1
    assert fwd_dense(lib, bias=A + 5 * GB + 8) == 4
    assert fwd_dense(lib, ld=60) == 2                       # row stride not a multiple of 8
    assert fwd_dense(lib, sh=-8) == 2
    assert fwd_dense(lib, o=A + 5 * GB + 64) == 2           # o overlaps the bias
    assert b"bias" in lib.ba_last_error()
    # one head's bias must stay below 4 GiB of offsets
    assert fwd_dense(lib, N=40000, ld=60000, sh=0, ws_bytes=16) == 3
    assert fwd_dense(lib, ws_bytes=16) == WS_TOO_SMALL
    assert fwd_dense(lib, sb=2 * 64 * 64, B=2, ws_bytes=16) == WS_TOO_SMALL
    assert fwd_dense(lib, strides=list(bnhd(1, 2, 64, 64)) * 4, ws_bytes=16) == WS_TOO_SMALL
    # the workspace is the one without a table
    need = lib.ba_workspace_bytes(1, 2, 64, 64, 0, 0)
    assert fwd_dense(lib, ws_bytes=need - 1) == 5


@pytest.mark.parametrize("shape", [(1, 3, 196, 64, 14, 14), (8, 16, 1024, 72, 32, 32), (2, 12, 4096, 64, 64, 64),
                                   (1, 16, 16384, 128, 128, 128), (2, 2, 100, 40, 0, 0)])
def test_workspace_bytes_int8pv(lib, shape):
    assert lib.ba_workspace_bytes_int8pv(*shape) == expected_workspace(*shape, int8pv=True)


def test_int8pv_validation(lib):
    """The 8-bit P.V entry: d <= 128 and N <= 65536 (exact int32 sums),
    otherwise the checks of ba_attention_fwd; nothing is launched."""
    assert lib.ba_workspace_bytes_int8pv(1, 1, 64, 136, 0, 0) == 0
    assert lib.ba_workspace_bytes_int8pv(1, 1, 65537, 64, 0, 0) == 0

    def call(**kw):
        a = dict(q=A, k=A + GB, v=A + 2 * GB, bias=None, gh=0, gw=0, B=1, H=2, N=64, d=64, scale=0.125,
                 o=A + 3 * GB, ws=A + 4 * GB, ws_bytes=1 << 40)
        a.update(kw)
        return lib.ba_attention_fwd_int8pv(a["q"], a["k"], a["v"], a["bias"], a["gh"], a["gw"], a["B"], a["H"],
                                           a["N"], a["d"], a["scale"], a["o"], a["ws"], a["ws_bytes"], None)
    assert call(d=136) == 3
    assert call(N=65537) == 3
    assert call(q=None) == 1
    assert call(o=A + 16) == 2
    need = lib.ba_workspace_bytes_int8pv(1, 2, 64, 64, 0, 0)
    assert need > lib.ba_workspace_bytes(1, 2, 64, 64, 0, 0) - 2 * 64 * 128 * 2
    assert call(ws_bytes=need - 1) == 5


def test_bwd_validation(lib):
    """ba_attention_bwd checks (nothing is launched)."""
    assert lib.ba_workspace_bytes_bwd(1, 2, 64, 72, 0, 0) == 0           # d must be 32, 64 or 128
    need = lib.ba_workspace_bytes_bwd(1, 2, 64, 64, 8, 8)
    assert need > lib.ba_workspace_bytes(1, 2, 64, 64, 8, 8)

    def call(**kw):
        a = dict(q=A, k=A + GB, v=A + 2 * GB, bias=None, gh=0, gw=0, B=1, H=2, N=64, d=64, scale=0.125,
                 do=A + 3 * GB, dq=A + 5 * GB, dk=A + 6 * GB, dv=A + 7 * GB, dt=None, ws=A + 4 * GB, wsb=16)
        a.update(kw)
        return lib.ba_attention_bwd(a["q"], a["k"], a["v"], a["bias"], a["gh"], a["gw"], a["B"], a["H"], a["N"],
                                    a["d"], a["scale"], a["do"], a["dq"], a["dk"], a["dv"], a["dt"], a["ws"],
                                    a["wsb"], None)
    assert call(d=72) == 3
    assert call(do=None) == 1
    assert call(dq=A + 5 * GB + 4) == 4
    assert call(scale=float("nan")) == 2
    assert call() == 5                                                     # workspace too small
    big = 1 << 40
    assert call(dt=A + 8 * GB, wsb=big) == 2                               # dtable without a table
    assert call(dk=A + 5 * GB + 64, wsb=big) == 2                          # dq and dk overlap
    tab = dict(bias=A + 9 * GB, gh=8, gw=8, wsb=big)
    assert call(dt=A + 6 * GB + 64, **tab) == 2                            # dtable inside dk
    assert call(dt=A + GB + 64, **tab) == 2                                # dtable inside k
    assert call(dt=A + 9 * GB + 16, **tab) == 2                            # dtable overlaps the table
    # inputs inside the workspace, also in its part past the forward's sections
    fwd = lib.ba_workspace_bytes(1, 2, 64, 64, 0, 0)
    full = lib.ba_workspace_bytes_bwd(1, 2, 64, 64, 0, 0)
    assert full > fwd + 4096
    assert call(q=A + 4 * GB + 256, wsb=big) == 5
    assert call(do=A + 4 * GB + fwd + 256, wsb=big) == 5
    assert call(k=A + 4 * GB + full - 4096, wsb=big) == 5
    assert call(v=A + 4 * GB - 4096, wsb=big) == 5                        # v's rows run into it
    full_t = lib.ba_workspace_bytes_bwd(1, 2, 64, 64, 8, 8)
    assert call(bias=A + 4 * GB + full_t - 512, gh=8, gw=8, wsb=big) == 5  # the table inside it


def test_fwd_train_validation(lib):
    """ba_attention_fwd_train checks lse after the forward's own checks
    (nothing is launched: every case below fails)."""
    def call(**kw):
        a = dict(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 5 * GB, ws=A + 4 * GB, wsb=1 << 40)
        a.update(kw)
        return lib.ba_attention_fwd_train(a["q"], a["k"], a["v"], None, 0, 0, 1, 2, 64, 64, 0.125, a["o"],
                                          a["lse"], a["ws"], a["wsb"], None)
    assert call(lse=None) == 1
    assert call(lse=A + 5 * GB + 2) == 4                                    # not 4-byte aligned
    assert call(lse=A + GB + 64) == 2                                       # inside k
    assert call(lse=A + 4 * GB + 256) == 5                                  # inside the workspace
    assert call(wsb=16) == 5                                                # the forward's own check


def test_bwd_saved_validation(lib):
    """ba_attention_bwd_saved checks o and lse (nothing is launched)."""
    def call(**kw):
        a = dict(q=A, k=A + GB, v=A + 2 * GB, o=A + 9 * GB, lse=A + 10 * GB, do=A + 3 * GB, dq=A + 5 * GB,
                 dk=A + 6 * GB, dv=A + 7 * GB, ws=A + 4 * GB, wsb=1 << 40)
        a.update(kw)
        return lib.ba_attention_bwd_saved(a["q"], a["k"], a["v"], None, 0, 0, 1, 2, 64, 64, 0.125, a["o"],
                                          a["lse"], a["do"], a["dq"], a["dk"], a["dv"], None, a["ws"], a["wsb"],
                                          None)
    assert call(o=None) == 1
    assert call(lse=None) == 1
    assert call(o=A + 9 * GB + 8) == 4                                      # o not 16-byte aligned
    assert call(lse=A + 10 * GB + 2) == 4                                   # lse not 4-byte aligned
    assert call(o=A + 5 * GB) == 2                                          # o overlaps dq
    assert call(lse=A + 6 * GB + 4) == 2                                    # lse overlaps dk
    assert call(lse=A + 4 * GB + 256) == 5                                  # lse inside the workspace
    assert call(wsb=16) == 5


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 exits with a message, before
    it touches a GPU."""
    import subprocess
    import sys
    root = pathlib.Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=root, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_default_workspace_per_stream():
    """The binding's workspace cache gives each (device, stream) its own
    buffer, so calls on two streams cannot race on one, and grows a buffer
    in place of the old one only for its own stream."""
    import torch
    from bit_qk_quantisation_amd import Workspace
    ws = Workspace()
    cpu = torch.device("cpu")
    a = ws.get(cpu, 1000, stream=111)
    b = ws.get(cpu, 1000, stream=222)
    assert a.data_ptr() != b.data_ptr()
    assert ws.get(cpu, 900, stream=111).data_ptr() == a.data_ptr()
    c = ws.get(cpu, 5000, stream=111)
    assert c.numel() >= 5000 and ws.get(cpu, 1000, stream=222).data_ptr() == b.data_ptr()


def test_static_forward_validation(lib):
    """ba_attention_fwd_static refuses, before any HIP call, what
    ba_attention_fwd refuses, and problems beyond its scratch array."""
    def call(**kw):
        a = dict(q=A, k=A + GB, v=A + 2 * GB, bias=None, gh=0, gw=0, B=1, H=2, N=64, d=64, scale=0.125,
                 o=A + 3 * GB)
        a.update(kw)
        return lib.ba_attention_fwd_static(a["q"], a["k"], a["v"], a["bias"], a["gh"], a["gw"], a["B"], a["H"],
                                           a["N"], a["d"], a["scale"], a["o"], None)
    assert call(d=72 + 4) == 3
    assert call(N=0) == 2
    assert call(bias=A + 5 * GB, gh=4, gw=15) == 2
    assert call(B=64, H=16, N=16384, d=128) == 5          # needs more than BA_STATIC_SCRATCH_MIB
    assert b"scratch" in lib.ba_last_error()
    assert call(bias=A + 5 * GB, gh=100, gw=70, N=7000) == 5             # its dense bias exceeds the scratch
