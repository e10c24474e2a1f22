#!/usr/bin/env python3
"""Benchmark of the BinaryAttention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--layout bhnd|bnhd|qkv] [--bias table|dense|dense-batch] [--pv bf16|int8] [--bwd]

One step is one full forward, one ba_attention_fwd call, over the resident
bf16 inputs of the chosen workload (default: the 64x64-grid detection
backbone, B=2 H=12 N=4096 d=64).  W untimed steps run first, then exactly K
steps are timed between two device synchronisations.  A second pass of K
steps brackets each call with HIP events on the launch stream, followed by
the fused kernel alone (ba_attention_fwd_prepared on a workspace that
ba_attention_prepare filled once, outside both passes): that gives the fused
kernel's average duration, and the rest of the call is the prologue.  Shapes
the pipelined kernel does not take run ba_attention_prepare +
ba_attention_fwd_prepared per step (exactly what ba_attention_fwd runs).

--layout bnhd stores q, k, v and o as [B,N,H,d]; --layout qkv takes q, k and
v as the slices of one [B,N,3,H,d] tensor and writes a [B,N,H,d] o.  Both go
through ba_attention_fwd_strided, one call per step, so only the whole step
is timed and the roofline figure is taken over the step.

--bias dense replaces the workload's relative-position table by a dense bf16
bias [H,N,N] shared by the batch (dense-batch: [B,H,N,N]), drawn N(0, 0.02);
the step is then ba_attention_prepare + ba_attention_fwd_dense_bias_prepared,
and the roofline object names whichever bound (matrix cores or HBM) the fused
kernel is closer to.

--qk-routes times ba_qk_int_dot's row-sum form for the three ways of taking
the integer dots (fp4 MFMA, the fused kernel's route; int8 MFMA; VALU
xor/popcount) on the workload's packed Q and K, and prints their times
instead of the forward's line.

--pv int8 runs the pages' hybrid 8-bit P.V (ba_attention_fwd_int8pv: three
kernels in one call), so only the whole step is timed; its roofline takes the
fp4 QK + int8 P.V matrix-core bound.

--bwd times the backward instead (ba_attention_bwd: six kernels in one call
with the table gradient, the forward recomputed inside; with --saved,
ba_attention_bwd_saved on the O and log-sum-exp of one earlier
ba_attention_fwd_train call, five kernels, as a training step runs it),
counted as 10*B*H*N^2*d FLOP-eq per step (the
products S, dP, dV, dQ and dK of a flash-attention backward); its roofline
takes the fp4 + bf16 matrix-core bound of those products (S on fp4, the
other four on bf16).

Printed: one JSON line on stdout with the throughput in TFLOP-eq/s
(4*B*H*N^2*d per step, the FLOPs of dense QK^T and P.V), the fused kernel's
roofline position and the CPU oracle's own throughput on a bounded sample of
the same workload (the oracle runs on the host cores; it is a baseline, not
the target).  Every mode times its own oracle: the bf16, 8-bit P.V or
dense-bias forward, or the backward; the sample's parity against the GPU
result rides along.  Diagnostics go to stderr.

Only one GPU is used: --gpus above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = ("binary-QK attention fwd TFLOP-eq/s (4·B·H·N²·d) "
          "+ % roofline, N=4096 d=64")

# MI355X dense peaks (published): fp4 MFMA 10.1 PFLOP/s, bf16 MFMA 2.5
# PFLOP/s, int8 MFMA 5.0 POP/s; HBM3E 8 TB/s.
PEAK_FP4 = 10100.0
PEAK_BF16 = 2500.0
PEAK_INT8 = 5000.0
PEAK_HBM_GBS = 8000.0
# Vector ALU: 256 CUs x 4 SIMDs x 16 lanes issue 16 lane-operations per SIMD
# per cycle at 2.4 GHz (a wave64 FMA takes 4 cycles), 39.3 T lane-cycles/s.
# The pipelined kernel's vector work per score is one exp2 (a transcendental,
# which takes a SIMD twice as long as an FMA: 8 cycles per wave64
# instruction, measured), one FMA and half a bf16 pack: 3.5 lane-cycles.
PEAK_VALU_TLC = 256 * 4 * 16 * 2.4e9 / 1e12
VALU_LC_PER_SCORE = 3.5
# The fused kernel runs QK (2d flops-eq per score) on the fp4 unit and P.V
# (2d flops per score) on the bf16 unit; with both at their peaks, one after
# the other, the matrix-core bound of 4d flops-eq per score is:
PEAK_MFMA_COMPOSITE = 4.0 / (2.0 / PEAK_FP4 + 2.0 / PEAK_BF16)
PEAK_MFMA_INT8_BF16 = 4.0 / (2.0 / PEAK_INT8 + 2.0 / PEAK_BF16)
# 8-bit P.V: QK on the fp4 unit, P.V on the int8 unit.
PEAK_MFMA_FP4_INT8 = 4.0 / (2.0 / PEAK_FP4 + 2.0 / PEAK_INT8)

PROFILES = ROOT / "profiles"
FUSED_SOURCES = ("bit_qk_quantisation_amd/csrc/flash.hip",
                 "bit_qk_quantisation_amd/csrc/ba_device.h",
                 "bit_qk_quantisation_amd/csrc/ba_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update((ROOT / p).read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per fused-kernel launch from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source changed since."""
    f = PROFILES / f"fused_attention_{workload}_traffic.json"
    if not f.exists():
        return None
    rec = json.loads(f.read_text())
    if rec.get("source_hash") != source_hash(FUSED_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def _lpad(gw):
    lpad = (2 * gw - 1 + 3 + 3) // 4 * 4
    while lpad % 64 != 16:
        lpad += 4
    return lpad


def _window_rows(N, gw):
    qspan = max(((q0 + 127) // gw - q0 // gw) for q0 in range(0, (N + 127) // 128 * 128, 128))
    kspan = max(((k0 + 63) // gw - k0 // gw) for k0 in range(0, N, 64))
    return qspan + kspan + 1


def pipelined(w, table=True):
    """Whether ba_attention_fwd runs the pipelined kernel (natural V, no V^T
    from the prologue) on this workload: d in {32, 64, 72, 128}, and table rows
    whose per-tile window fits its buffers or no bias; shorter sequences with
    a table or no bias (N <= 256, d in {32, 64}) take the one-launch kernel."""
    rows = table and w.gw % 32 == 0
    if w.d not in (32, 64, 72, 128) or (table and not rows):
        return False
    if w.N <= 256 and w.d in (32, 64) and not rows:
        return False
    return not rows or _window_rows(w.N, w.gw) * 4 * _lpad(w.gw) <= (1664 if w.d <= 72 else 1152)


def algorithmic_bytes(w, npad, dense_bytes=None):
    """Compulsory HBM bytes of the two kernels of one step.  Pipelined
    kernel: the prologue reads K and writes the fp4 key operands and the key
    scales as matrix operands (and the scales' maxima per 64 tokens), plus the
    bias rows from the table; the fused kernel reads Q, those, V and the bias
    rows and writes O.
    Otherwise the prologue also reads V and writes V^T, which the fused kernel
    reads instead of V."""
    W = (w.d + 31) // 32
    nch = (W + 1) // 2
    dpad = 32 * W
    bh = w.B * w.H
    tok = bh * w.N
    keys = bh * npad * (32 * nch + 4) + bh * (npad // 64) * 4
    # the pipelined kernel takes the key scales as matrix operands (12 bytes
    # per key) instead of floats
    keys_p = bh * npad * (32 * nch + 12) + bh * (npad // 64) * 4
    vt = bh * dpad * npad * 2
    rows = 0
    if w.gw % 32 == 0:
        rows = w.H * (2 * w.gh - 1 + 16) * 4 * _lpad(w.gw) * 4
    table = w.H * (2 * w.gh - 1) * (2 * w.gw - 1) * 2
    if dense_bytes is not None:  # no table: the fused kernel reads the dense bias once
        return 2 * tok * w.d * 2 + keys + vt, tok * w.d * 2 + keys + vt + dense_bytes + tok * w.d * 2
    if pipelined(w):
        prologue = tok * w.d * 2 + keys_p + ((table + rows) if rows else 0)
        fused = tok * w.d * 2 + keys_p + tok * w.d * 2 + (rows if rows else table) + tok * w.d * 2
        return prologue, fused
    prologue = 2 * tok * w.d * 2 + keys + vt + ((table + rows) if rows else 0)
    fused = tok * w.d * 2 + keys + vt + (rows if rows else table) + tok * w.d * 2
    return prologue, fused


def _host_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads") or 1 for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - informational only
        return os.cpu_count() or 1


def cpu_baseline(w, inp, o_gpu, seconds: float, pv: str = "bf16", dense=None):
    """The float64 oracle on whole (b, h) heads of the same inputs, for about
    `seconds` of host time; also returns the parity of those rows.  pv="int8"
    times the 8-bit P.V oracle; `dense` (the GPU's [Bb,H,N,N] bias) the
    dense-bias oracle, one head's bias copied to the host at a time."""
    import numpy as np

    import oracle
    import workloads
    q = workloads.as_f32(inp["q"])
    k = workloads.as_f32(inp["k"])
    v = workloads.as_f32(inp["v"])
    t = workloads.as_f32(inp["table"])
    og = o_gpu.float().cpu().numpy()
    vmax = float(np.abs(v).max())
    heads, worst = 0, 0.0
    rows_per = min(w.N, 1024)
    t0 = time.perf_counter()
    elapsed = 0.0
    for b in range(w.B):
        for h in range(w.H):
            qs, ks, vs = q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1]
            if dense is not None:
                bias = dense[b if dense.shape[0] > 1 else 0, h].float().cpu().numpy()[None, None]
            for r0 in range(0, w.N, rows_per):
                rows = np.arange(r0, min(w.N, r0 + rows_per))
                if dense is not None:
                    res = oracle.binary_attention_dense_bias_rows(qs, ks, vs, bias, rows=rows)
                elif pv == "int8":
                    res = oracle.binary_attention_int8_pv_rows(qs, ks, vs, None if t is None else t[h:h + 1],
                                                               inp["gh"], inp["gw"], rows=rows)
                else:
                    res = oracle.binary_attention_rows(qs, ks, vs, None if t is None else t[h:h + 1],
                                                       inp["gh"], inp["gw"], rows=rows)
                err = float(np.abs(res["O"][0, 0] - og[b, h, rows]).max()) / vmax
                worst = max(worst, err)
            heads += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= seconds:
                break
        if elapsed >= seconds:
            break
    flop = 4.0 * heads * w.N * w.N * w.d
    what = ("binary_attention_dense_bias_rows" if dense is not None else
            "binary_attention_int8_pv_rows" if pv == "int8" else "binary_attention_rows")
    return {
        "value": flop / elapsed / 1e12,
        "unit": "TFLOP-eq/s",
        "cores": int(_host_threads()),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} (b,h) heads, all {w.N} query rows each, "
                  f"float64 numpy on the host, oracle.{what} ({elapsed:.1f} s)",
        "parity_max_err_over_max_v": worst,
    }


def cpu_baseline_bwd(w, inp, dout, grads, seconds: float):
    """The float64 backward oracle on the whole batch of one head at a time
    (the table gradient sums over the batch), for about `seconds` of host
    time, counted as 10 N^2 d FLOP-eq per (b, h).  Parity: per gradient,
    max |GPU - oracle| over max |oracle| on the heads done."""
    import numpy as np

    import oracle
    import workloads
    q = workloads.as_f32(inp["q"])
    k = workloads.as_f32(inp["k"])
    v = workloads.as_f32(inp["v"])
    t = workloads.as_f32(inp["table"])
    do = dout.float().cpu().numpy()
    gq, gk, gv, gt = (None if x is None else x.float().cpu().numpy() for x in grads)
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0, "dtable": 0.0}
    heads = 0
    t0 = time.perf_counter()
    elapsed = 0.0
    for h in range(w.H):
        sl = slice(h, h + 1)
        res = oracle.binary_attention_backward(q[:, sl], k[:, sl], v[:, sl], do[:, sl],
                                               None if t is None else t[sl], inp["gh"], inp["gw"])
        for name, got in (("dq", gq[:, sl]), ("dk", gk[:, sl]), ("dv", gv[:, sl]),
                          ("dtable", None if gt is None else gt[sl])):
            ref = res[name]
            if got is None or ref is None:
                continue
            worst[name] = max(worst[name], float(np.abs(got - ref).max()) / max(float(np.abs(ref).max()), 1e-300))
        heads += w.B
        elapsed = time.perf_counter() - t0
        if elapsed >= seconds:
            break
    flop = 10.0 * heads * w.N * w.N * w.d
    return {
        "value": flop / elapsed / 1e12,
        "unit": "TFLOP-eq/s",
        "cores": int(_host_threads()),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} (b,h) heads (all {w.B} batch entries of {heads // w.B} heads), "
                  f"float64 numpy on the host, oracle.binary_attention_backward ({elapsed:.1f} s)",
        "parity_max_err_over_max_ref": worst,
    }


def qk_routes(args, w, inp, lib, dev) -> int:
    """Times ba_qk_int_dot in its row-sum form for the fp4-MFMA, int8-MFMA
    and VALU xor/popcount routes on the workload's packed Q and K (the three
    ways of taking the integer dots); prints one JSON line."""
    import torch

    import bit_qk_quantisation_amd as bq
    B, H, N, d = w.B, w.H, w.N, w.d
    qb, _ = bq.pack_signs(inp["q"].to(dev))
    kb, _ = bq.pack_signs(inp["k"].to(dev))
    sums = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    res, ref = {}, None
    for name, route in (("mfma_fp4", bq.ROUTE_MFMA_FP4), ("mfma_int8", bq.ROUTE_MFMA_INT8),
                        ("valu_popcount", bq.ROUTE_VALU_POPCOUNT)):
        def run():
            bq.check(lib, lib.ba_qk_int_dot(qb.data_ptr(), kb.data_ptr(), B, H, N, d, route | bq.QK_ROWSUM,
                                            sums.data_ptr(), sp))
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        got = sums.clone()
        if ref is None:
            ref = got
        res[name] = {"us_per_launch": round(us, 2),
                     "tops_eq": round(2.0 * B * H * N * N * d / (us * 1e-6) / 1e12, 1),
                     "same_sums_as_fp4": bool(torch.equal(got, ref))}
        log(f"[qk-routes] {w.name} {name}: {us:.2f} us")
    print(json.dumps({"metric": "QK integer dots, row-sum form: time per launch by route",
                      "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d},
                      "routes": res}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--layout", choices=("bhnd", "bnhd", "qkv"), default="bhnd",
                    help="memory layout of q, k, v and o (see above)")
    ap.add_argument("--bwd", action="store_true", help="time the backward pass (see above)")
    ap.add_argument("--saved", action="store_true",
                    help="with --bwd: the backward on a saved O and log-sum-exp (see above)")
    ap.add_argument("--pv", choices=("bf16", "int8"), default="bf16",
                    help="P.V precision (see above)")
    ap.add_argument("--bias", choices=("table", "dense", "dense-batch"), default="table",
                    help="bias form (see above)")
    ap.add_argument("--qk-routes", action="store_true",
                    help="time the three QK routes against each other instead (see above)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB "
                         "(reference kernel for HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the BinaryAttention forward here is "
              "a single-GPU kernel; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import bit_qk_quantisation_amd as bq
    import workloads

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    lib = bq._lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = workloads.workload_inputs(w)
    if args.qk_routes:
        return qk_routes(args, w, inp, lib, dev)
    q = inp["q"].to(dev)
    k = inp["k"].to(dev)
    v = inp["v"].to(dev)
    table = inp["table"].to(dev) if inp["table"] is not None else None
    gh, gw = inp["gh"], inp["gw"]
    dense = None
    if args.bias != "table":
        if args.layout != "bhnd":
            log("--bias dense runs with the contiguous layout only")
            return 2
        table, gh, gw = None, 0, 0
        Bb = w.B if args.bias == "dense-batch" else 1
        dense = workloads.make_dense_bias(Bb, w.H, w.N, seed=w.seed + 100).to(dev)
        dsb = 0 if Bb == 1 else dense.stride(0)
    B, H, N, d = w.B, w.H, w.N, w.d
    scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    nbytes = lib.ba_workspace_bytes(B, H, N, d, gh, gw)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    wsp = (ws.data_ptr() + 255) // 256 * 256
    tp = None if table is None else table.data_ptr()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def prepare():
        bq.check(lib, lib.ba_attention_prepare(k.data_ptr(), v.data_ptr(), tp, gh, gw,
                                               B, H, N, d, wsp, nbytes, sp))

    def fused():
        bq.check(lib, lib.ba_attention_fwd_prepared(q.data_ptr(), tp, gh, gw, B, H, N, d, scale, out.data_ptr(),
                                                    wsp, nbytes, sp))

    if dense is not None:
        def fused():  # noqa: F811
            bq.check(lib, lib.ba_attention_fwd_dense_bias_prepared(
                q.data_ptr(), dense.data_ptr(), dsb, dense.stride(1), dense.stride(2), B, H, N, d, scale,
                out.data_ptr(), wsp, nbytes, sp))

    # Short sequences (N <= 256, d in {32, 64}, a table that is not read in
    # rows, or none) run as one launch that packs K and V in LDS: there is no
    # prologue to time apart, so the step is the whole ba_attention_fwd call.
    one_launch = (args.layout == "bhnd" and args.pv == "bf16" and not args.bwd and dense is None
                  and N <= 256 and d in (32, 64) and (table is None or gw % 32 != 0))
    split = args.layout == "bhnd" and args.pv == "bf16" and not args.bwd and not one_launch
    if args.saved and not args.bwd:
        log("--saved goes with --bwd")
        return 2
    if args.bwd:
        if args.layout != "bhnd" or dense is not None or args.pv != "bf16":
            log("--bwd runs with the contiguous layout, the table bias and bf16 P.V only")
            return 2
        nbb = lib.ba_workspace_bytes_bwd(B, H, N, d, gh, gw)
        if nbb == 0:
            log(f"the backward does not support d = {d}")
            return 2
        wsb = torch.empty(nbb + 256, dtype=torch.uint8, device=dev)
        wspb = (wsb.data_ptr() + 255) // 256 * 256
        g = torch.Generator().manual_seed(w.seed + 200)
        dout = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).to(dev)
        gq = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
        gk, gv = torch.empty_like(gq), torch.empty_like(gq)
        gt = None if table is None else torch.empty(table.shape, dtype=torch.float32, device=dev)

        def prepare():  # noqa: F811 -- one call runs the whole backward
            bq.check(lib, lib.ba_attention_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, gh, gw, B, H, N, d,
                                               scale, dout.data_ptr(), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(),
                                               None if gt is None else gt.data_ptr(), wspb, nbb, sp))

        if args.saved:
            o_sv = torch.empty_like(q)
            lse_sv = torch.empty((B, H, N), dtype=torch.float32, device=dev)
            bq.check(lib, lib.ba_attention_fwd_train(q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, gh, gw,
                                                     B, H, N, d, scale, o_sv.data_ptr(), lse_sv.data_ptr(),
                                                     wsp, nbytes, sp))

            def prepare():  # noqa: F811 -- the backward on the saved O and log-sum-exp
                bq.check(lib, lib.ba_attention_bwd_saved(
                    q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, gh, gw, B, H, N, d, scale, o_sv.data_ptr(),
                    lse_sv.data_ptr(), dout.data_ptr(), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(),
                    None if gt is None else gt.data_ptr(), wspb, nbb, sp))

        def fused():  # noqa: F811
            pass
    elif args.pv == "int8":
        if args.layout != "bhnd" or dense is not None:
            log("--pv int8 runs with the contiguous layout and the table bias only")
            return 2
        nb8 = lib.ba_workspace_bytes_int8pv(B, H, N, d, gh, gw)
        ws8 = torch.empty(nb8 + 256, dtype=torch.uint8, device=dev)
        wsp8 = (ws8.data_ptr() + 255) // 256 * 256

        def prepare():  # noqa: F811 -- one call runs all three kernels
            bq.check(lib, lib.ba_attention_fwd_int8pv(q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, gh, gw,
                                                      B, H, N, d, scale, out.data_ptr(), wsp8, nb8, sp))

        def fused():  # noqa: F811
            pass
    elif one_launch:
        def prepare():  # noqa: F811 -- the whole forward, one kernel
            bq.check(lib, lib.ba_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, gh, gw, B, H, N, d,
                                               scale, out.data_ptr(), wsp, nbytes, sp))

        def fused():  # noqa: F811
            pass
    elif not split:
        import ctypes
        if args.layout == "bnhd":
            views = [x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v)]
        else:
            qkv = torch.stack([q, k, v], dim=1).permute(0, 3, 1, 2, 4).contiguous()  # [B,N,3,H,d]
            views = [qkv[:, :, i].transpose(1, 2) for i in range(3)]
        sq, sk, sv = views
        so = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev).transpose(1, 2)
        strides = (ctypes.c_int64 * 12)(*[t.stride(i) for t in (sq, sk, sv, so) for i in range(3)])
        del q, k, v
        out = so

        def whole():
            bq.check(lib, lib.ba_attention_fwd_strided(sq.data_ptr(), sk.data_ptr(), sv.data_ptr(), tp, gh, gw,
                                                       B, H, N, d, scale, so.data_ptr(), strides, wsp, nbytes, sp))

        def prepare():  # noqa: F811 -- one call runs both kernels
            whole()

        def fused():  # noqa: F811
            pass

    if split and dense is None and pipelined(w, table is not None):
        # The step is one ba_attention_fwd call (its prologue packs K only;
        # the pipelined kernel reads V in place).  The fused kernel alone is
        # timed as ba_attention_fwd_prepared on a workspace prepared once
        # outside the timed loops: the same kernel on the same shapes, with V
        # from the workspace's contiguous copy.
        prepare()

        def step():
            bq.check(lib, lib.ba_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, gh, gw, B, H, N, d,
                                               scale, out.data_ptr(), wsp, nbytes, sp))
        whole_call = True
    else:
        def step():
            prepare()
            fused()
        whole_call = False

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # Timed region: exactly K steps between two synchronisations, nothing else
    # on the stream; `value` and ms_per_step come from it.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(K):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / K
    # Per-kernel durations: another K steps with HIP events recorded on the
    # launch stream around each kernel (the events add their own gaps, so this
    # pass is not the one `value` is taken from).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        if whole_call:
            step()
        else:
            prepare()
        ev[i][1].record(stream)
        fused()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    pro_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    fus_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    if whole_call:  # the first interval held a whole forward: its prologue is the rest
        pro_ms = max(pro_ms - fus_ms, 0.0)
    if not split:  # the "prologue" interval held the whole step
        fus_ms = pro_ms
    peak = PEAK_MFMA_FP4_INT8 if args.pv == "int8" else PEAK_MFMA_COMPOSITE
    if args.bwd:
        # S on the fp4 unit (2 flops per score and channel), dP, dV, dQ, dK on bf16 (8)
        peak = 10.0 / (2.0 / PEAK_FP4 + 8.0 / PEAK_BF16)

    if args.copy_mb:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    flop = w.flop_eq * (2.5 if args.bwd else 1.0)
    value = flop / (ms_step * 1e-3) / 1e12
    fused_tf = flop / (fus_ms * 1e-3) / 1e12
    npad = (N + 127) // 128 * 128
    dense_bytes = None if dense is None else dense.numel() * 2
    pro_bytes, fus_bytes = algorithmic_bytes(w, npad, dense_bytes)
    traffic = measured_traffic(name) if split and dense is None else None
    fused_gbs = fus_bytes / (fus_ms * 1e-3) / 1e9
    hbm_bound = dense is not None and fused_gbs / PEAK_HBM_GBS > fused_tf / peak
    # the pipelined kernel's vector work against its matrix work: the bound
    # whose minimum time is longer is the one reported
    scores = w.B * w.H * w.N * w.N
    alu_tlc = scores * VALU_LC_PER_SCORE / (fus_ms * 1e-3) / 1e12
    alu_bound = (whole_call and not hbm_bound and
                 scores * VALU_LC_PER_SCORE / PEAK_VALU_TLC > flop / peak)

    baseline = None
    if args.cpu_seconds > 0 and args.bwd:
        baseline = cpu_baseline_bwd(w, inp, dout, (gq, gk, gv, gt), args.cpu_seconds)
    elif args.cpu_seconds > 0:
        baseline = cpu_baseline(w, inp, out, args.cpu_seconds, pv=args.pv, dense=dense)

    rec = {
        "metric": METRIC if not args.bwd else
                  "binary-QK attention bwd TFLOP-eq/s (10·B·H·N²·d) + % roofline",
        "value": round(value, 2),
        "unit": "TFLOP-eq/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.pv == "bf16" else "int8",
        "data": "synthetic",
        "config": {**w.describe(), "qk": "1-bit signs as +/-1 fp4 on MFMA (exact integer dots)",
                   "pv": ("bf16 MFMA, fp32 accumulate" if args.pv == "bf16" else
                          "u8 coefficients x per-channel s8 values on int8 MFMA, int32 accumulate"),
                   "softmax": "fp32, base 2",
                   "parallelism": "single GPU", "layout": args.layout, "bias": args.bias,
                   **({"backward": "saved O and lse" if args.saved else "forward recomputed"} if args.bwd else {})},
        "roofline": {
            "bound": "mfma",
            "kernel": ("flash_fwd_kernel (fused, pipelined)" if whole_call else
                       "attn_fwd_kernel (fused)" if split else
                       "whole backward on saved O and lse (5 kernels, one call)" if args.bwd and args.saved else
                       "whole backward (6 kernels, one call; forward recomputed)" if args.bwd else
                       "whole step (3 kernels, one call; fp4 QK + int8 P.V bound)" if args.pv == "int8" else
                       "attn_fwd_small_kernel (the whole step: one launch, K and V packed in LDS)" if one_launch else
                       "whole step (prologue + fused, one strided call)"),
            "achieved": round(fused_tf, 1),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(fused_tf / peak, 4),
            "traffic": traffic,
        } if not hbm_bound and not alu_bound else {
            "bound": "alu",
            "kernel": "flash_fwd_kernel (fused, pipelined): exp2 + FMA + half a bf16 pack per score",
            "achieved": round(alu_tlc, 2),
            "peak": round(PEAK_VALU_TLC, 2),
            "unit": "T lane-cycles/s",
            "frac": round(alu_tlc / PEAK_VALU_TLC, 4),
            "traffic": traffic,
        } if alu_bound else {
            "bound": "hbm",
            "kernel": "attn_fwd_kernel (fused, dense bias)",
            "achieved": round(fused_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(fused_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": baseline,
        "detail": {
            "fused_us": round(fus_ms * 1e3, 2) if split else None,
            "prologue_us": round(pro_ms * 1e3, 2) if split else None,
            "step_us": round(ms_step * 1e3, 2),
            "frac_of_int8_bf16_mfma_roofline": round(fused_tf / PEAK_MFMA_INT8_BF16, 4),
            "fused_frac_of_valu_roofline": round(alu_tlc / PEAK_VALU_TLC, 4) if whole_call else None,
            "step_frac_of_composite_mfma_roofline": round(value / PEAK_MFMA_COMPOSITE, 4),
            "prologue_algorithmic_GBps": round(pro_bytes / (pro_ms * 1e-3) / 1e9, 1) if split else None,
            "prologue_frac_of_hbm": round(pro_bytes / (pro_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if split else None,
            "fused_algorithmic_bytes": fus_bytes,
            "fused_algorithmic_GBps": round(fused_gbs, 1),
            "fused_frac_of_composite_mfma_roofline": round(fused_tf / PEAK_MFMA_COMPOSITE, 4),
            "device": torch.cuda.get_device_name(dev),
        },
    }
    if split:
        log(f"[bench] {name}: step {ms_step * 1e3:.1f} us (prologue {pro_ms * 1e3:.1f} us, "
            f"fused {fus_ms * 1e3:.1f} us) -> {value:.1f} TFLOP-eq/s")
    else:
        log(f"[bench] {name} ({args.layout}, pv {args.pv}{', backward' if args.bwd else ''}): "
            f"step {ms_step * 1e3:.1f} us -> {value:.1f} TFLOP-eq/s")
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
