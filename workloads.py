"""Seeded synthetic inputs for the BinaryAttention forward.

This module only draws random numbers and rounds them to bf16.  It holds none
of the method's arithmetic, and both the HIP path and the CPU oracle take
their inputs from it.

Recipe, per workload:
* numpy default_rng(seed) draws float32 standard normals in this fixed
  order: Q, K, V (each [B, H, N, d]), then the bias table ([H, 2gh-1, 2gw-1],
  multiplied by 0.02), then the outlier-channel permutation;
* for the outlier workload, the first round(frac * d) channels of that
  permutation are multiplied by 8 in Q, K and V (all heads, all tokens);
* one conversion to bf16 (torch CPU, round-to-nearest-even) produces the only
  copy of the inputs;
* a dense bias [1 or B, H, N, N] (make_dense_bias) comes from its own
  default_rng(seed): float32 normals times sigma, then one bf16 rounding.

The five named workloads stand in for the token counts of the vision and
diffusion experiments the BinaryAttention pages report.  Those are ViT at
224^2 (14x14 patches), ViT at 1024^2 (64x64), DiT-XL/2 at 512^2 (a 32x32
latent, head dim 72) and 16K-token sequences.  The datasets and trained
weights are not used.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    gh: int
    gw: int
    d: int
    seed: int
    outlier_frac: float = 0.0

    @property
    def N(self) -> int:
        return self.gh * self.gw

    @property
    def flop_eq(self) -> float:
        """4 * B * H * N^2 * d: the FLOP count of dense QK^T and P.V."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "N": self.N,
                "grid": [self.gh, self.gw], "d": self.d,
                "bias_table": [2 * self.gh - 1, 2 * self.gw - 1],
                "outlier_frac": self.outlier_frac, "seed": self.seed}


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_vit_14x14", 1, 3, 14, 14, 64, seed=1),
        Workload("vit_base_b32_14x14", 32, 12, 14, 14, 64, seed=2),
        Workload("dit512_32x32_d72", 8, 16, 32, 32, 72, seed=3,
                 outlier_frac=0.05),
        Workload("detection_64x64", 2, 12, 64, 64, 64, seed=4),
        Workload("diffusion_128x128_d128", 1, 16, 128, 128, 128, seed=5),
    )
}

HEADLINE = "detection_64x64"


def _to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        torch.bfloat16)


def make_inputs(B: int, H: int, N: int, d: int, seed: int, *,
                grid=None, outlier_frac: float = 0.0, bias: bool = True,
                q_scale: float = 1.0, k_scale: float = 1.0,
                table_sigma: float = 0.02) -> dict:
    """Draw one seeded case.  Returns CPU bf16 tensors q, k, v [B,H,N,d] and
    table [H, 2gh-1, 2gw-1] (or None), plus gh, gw.

    grid=(gh, gw) with gh*gw == N is required when bias is True.
    q_scale/k_scale multiply Q/K before rounding (large-logit cases);
    table_sigma is the table's standard deviation (0.02 for the workloads;
    tests that must see the bias use 1 or 2).
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d), dtype=np.float32)
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    gh, gw = grid if grid is not None else (0, 0)
    table = None
    if bias:
        if gh * gw != N:
            raise ValueError("bias needs grid=(gh, gw) with gh*gw == N")
        table = np.float32(table_sigma) * rng.standard_normal(
            (H, 2 * gh - 1, 2 * gw - 1), dtype=np.float32)
    perm = rng.permutation(d)
    n_out = int(round(outlier_frac * d))
    if n_out:
        ch = perm[:n_out]
        q[..., ch] *= 8.0
        k[..., ch] *= 8.0
        v[..., ch] *= 8.0
    q *= np.float32(q_scale)
    k *= np.float32(k_scale)
    return {
        "q": _to_bf16(q), "k": _to_bf16(k), "v": _to_bf16(v),
        "table": None if table is None else _to_bf16(table),
        "gh": gh, "gw": gw, "outlier_channels": np.sort(perm[:n_out]),
    }


def workload_inputs(w: Workload, **kw) -> dict:
    return make_inputs(w.B, w.H, w.N, w.d, w.seed, grid=(w.gh, w.gw),
                       outlier_frac=w.outlier_frac, **kw)


def make_dense_bias(Bb: int, H: int, N: int, seed: int, sigma: float = 0.02,
                    ld: int | None = None) -> torch.Tensor:
    """Seeded dense bias [Bb, H, N, N] in bf16: numpy default_rng(seed) draws
    float32 standard normals, times sigma, rounded once to bf16.  With ld > N
    the rows are stored ld apart (zero padding past N) and a [Bb, H, N, N]
    view of that storage is returned, so that every row starts 16-byte
    aligned when N % 8 != 0."""
    rng = np.random.default_rng(seed)
    b = np.float32(sigma) * rng.standard_normal((Bb, H, N, N), dtype=np.float32)
    t = _to_bf16(b)
    if ld is None or ld == N:
        return t
    if ld < N:
        raise ValueError("ld must be >= N")
    wide = torch.zeros((Bb, H, N, ld), dtype=torch.bfloat16)
    wide[..., :N] = t
    return wide[..., :N]


def as_f32(t):
    """bf16 tensor -> float32 numpy array (exact widening), None passes."""
    if t is None:
        return None
    return t.to(torch.float32).numpy()
