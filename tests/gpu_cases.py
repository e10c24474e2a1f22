"""Helpers shared by the GPU parity tests: seeded inputs on the device and
the oracle's answer for the same inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads


def announce(*parts):
    """Name the case before any GPU work, so a fault names it."""
    print("CASE", *parts, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def to_dev(inp):
    dev = device()
    out = dict(inp)
    for key in ("q", "k", "v", "table"):
        if out.get(key) is not None:
            out[key] = out[key].to(dev).contiguous()
    return out


def np32(t):
    return workloads.as_f32(t.cpu() if t is not None else None)


def bits_u32(t):
    return t.cpu().numpy().view(np.uint32)


def oracle_rows(inp, rows=None):
    """Oracle O (float64) for the given query rows of a CPU input dict."""
    table = inp.get("table")
    return oracle.binary_attention_rows(
        np32(inp["q"]), np32(inp["k"]), np32(inp["v"]),
        None if table is None else np32(table), inp["gh"], inp["gw"],
        rows=rows)["O"]


def sample_rows(n, count, seed):
    """Seeded sample of query rows that always includes the first and last."""
    rng = np.random.default_rng(seed)
    count = min(count, n)
    rows = set(rng.choice(n, size=count, replace=False).tolist())
    rows.update({0, n - 1})
    return np.array(sorted(rows))


def o_error(o_gpu, o_ref, v_cpu, rows=None):
    """max |dO| / max |V| (the tolerance is 1e-2)."""
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        og = og[:, :, rows, :]
    vmax = float(np.abs(np32(v_cpu)).max())
    return float(np.abs(og - o_ref).max()) / vmax
