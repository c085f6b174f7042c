"""Seeded synthetic workloads for batched Newton–Schulz orthogonalization.

This module only draws random numbers (NumPy PCG64) and rounds them to the
storage dtype of a bucket.  It holds none of the orthogonalization arithmetic:
the CPU oracle and the HIP library both receive the tensors built here, bit for
bit, and neither imports the other.

Every matrix of a bucket has its own child seed (``SeedSequence(seed).spawn(G)``)
so that any single matrix can be rebuilt without drawing the others.

The shapes follow the workloads the pages discuss: a Muon momentum matrix of a
GPT-2-small MLP (768x3072), the MLP of a 7B Llama-style model (11008x4096,
bf16 momentum), square attention projections (4096x4096) and fine-grained MoE
experts (2048x512).  The seven conditioning classes are the ones the "muon"
kernel card ("Correctness" section) uses for its fp64 comparison.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional, Sequence

import numpy as np
import torch

# Quintic coefficients used at every step by the "muon" kernel card ("How it
# works" section): X <- a X + (b A + c A^2) X with A = X X^T.
COEFFS_MUON = (3.4445, -4.7750, 2.0315)
# Classic quintic with p(1) = 1, used by the Dion3 paper's stability study
# (Appendix B.1.1).  The caption of its Figure 12 prints the middle coefficient
# without its minus sign; the body text and Eq. (4) fix it as -10/8.
COEFFS_CLASSIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)

CONDITIONING_CLASSES = (
    "gaussian",
    "ill_conditioned",
    "low_rank",
    "heavy_tailed",
    "scaled_up",
    "scaled_down",
    "near_orthogonal",
)

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    """One seeded bucket [G, R, C] plus the NS parameters it is run with."""

    name: str
    G: int
    R: int
    C: int
    dtype: str  # storage dtype of the bucket: "f16", "bf16" or "f32"
    seed: int
    kind: str  # generator name, see make_matrix
    mode: str = "gram"  # "gram" (square matrices fall back to standard) or "standard"
    steps: int = 5
    coeffs: tuple = COEFFS_MUON
    restart_after: int = 2
    safety: float = 1.05
    compute: str = "f16"  # operand dtype of the GEMMs
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return min(self.R, self.C)

    @property
    def m(self) -> int:
        return max(self.R, self.C)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]


WORKLOADS = {
    # One fp32 128x512 matrix, N(0,1) from seed 0, pre-divided by its Frobenius
    # norm.  Run in both modes, fp32 and fp16 on the GPU; s = 1 so that Gram and
    # standard see the same scaled input.
    "single_1x128x512_f32": Workload(
        "single_1x128x512_f32", 1, 128, 512, "f32", 0, "gaussian_unit_fro",
        mode="gram", safety=1.0, compute="f32",
        description="single fp32 128x512 matrix, N(0,1) seed 0, Frobenius-normalised"),
    # GPT-2-small MLP momentum bucket: 42 fp16 768x3072 matrices, the seven
    # conditioning classes in blocks of six.
    "gpt2s_mlp_42x768x3072_f16": Workload(
        "gpt2s_mlp_42x768x3072_f16", 42, 768, 3072, "f16", 2, "conditioning",
        description="42 fp16 768x3072 matrices, 6 of each of 7 conditionings"),
    # 7B-style MLP bucket: 32 bf16 11008x4096 momentum matrices, N(0, 0.02^2).
    # Transposed internally to n = 4096, m = 11008; fp16 GEMM operands.
    "llama7b_mlp_32x11008x4096_bf16": Workload(
        "llama7b_mlp_32x11008x4096_bf16", 32, 11008, 4096, "bf16", 3, "gaussian_0.02",
        description="32 bf16 11008x4096 matrices, N(0, 0.02^2)"),
    # Square attention-projection bucket: standard NS fallback.
    "square_32x4096x4096_f16": Workload(
        "square_32x4096x4096_f16", 32, 4096, 4096, "f16", 4, "gaussian",
        mode="gram", safety=1.0,
        description="32 fp16 4096x4096 matrices, N(0,1); square, so standard NS"),
    # Fine-grained MoE experts: 512 fp16 2048x512 matrices with per-expert scale
    # 10^U(-2, 2).  Transposed internally to n = 512, m = 2048.
    "moe_512x2048x512_f16": Workload(
        "moe_512x2048x512_f16", 512, 2048, 512, "f16", 5, "gaussian_logscale",
        description="512 fp16 2048x512 expert matrices, N(0,1) * 10^U(-2,2)"),
}


def _rng(seed: int, G: int, g: int) -> np.random.Generator:
    if G == 1:
        return np.random.default_rng(seed)
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(G)[g])


def _orthonormal_columns(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows x cols (rows >= cols) with orthonormal columns, from QR of a Gaussian."""
    q, r = np.linalg.qr(rng.standard_normal((rows, cols)))
    return q * np.sign(np.diag(r))[None, :]


def conditioning_matrix(cls: str, rng: np.random.Generator, R: int, C: int) -> np.ndarray:
    """One R x C fp64 matrix of the given conditioning class."""
    k = min(R, C)
    if cls == "gaussian":
        return rng.standard_normal((R, C))
    if cls == "ill_conditioned":
        u = _orthonormal_columns(rng, R, k)
        v = _orthonormal_columns(rng, C, k)
        return (u * np.logspace(0.0, -6.0, k)[None, :]) @ v.T
    if cls == "low_rank":
        rank = min(64, max(1, k // 2))
        return rng.standard_normal((R, rank)) @ rng.standard_normal((rank, C))
    if cls == "heavy_tailed":
        return rng.standard_t(3.0, size=(R, C))
    if cls == "scaled_up":
        return rng.standard_normal((R, C)) * 1e3
    if cls == "scaled_down":
        return rng.standard_normal((R, C)) * 1e-3
    if cls == "near_orthogonal":
        if R <= C:
            q = _orthonormal_columns(rng, C, R).T
        else:
            q = _orthonormal_columns(rng, R, C)
        return q + 1e-3 * rng.standard_normal((R, C))
    raise ValueError(f"unknown conditioning class {cls!r}")


def make_matrix(kind: str, seed: int, G: int, g: int, R: int, C: int) -> np.ndarray:
    """Matrix g of a seeded bucket of G, as float32 (before rounding to storage)."""
    rng = _rng(seed, G, g)
    if kind == "gaussian":
        return rng.standard_normal((R, C), dtype=np.float32)
    if kind == "gaussian_0.02":
        return rng.standard_normal((R, C), dtype=np.float32) * np.float32(0.02)
    if kind == "gaussian_unit_fro":
        x = rng.standard_normal((R, C))
        return (x / np.sqrt(np.sum(x * x))).astype(np.float32)
    if kind == "gaussian_logscale":
        scale = 10.0 ** rng.uniform(-2.0, 2.0)
        return rng.standard_normal((R, C), dtype=np.float32) * np.float32(scale)
    if kind == "conditioning":
        per = max(1, G // len(CONDITIONING_CLASSES))
        cls = CONDITIONING_CLASSES[min(g // per, len(CONDITIONING_CLASSES) - 1)]
        return conditioning_matrix(cls, rng, R, C).astype(np.float32)
    if kind.startswith("class:"):
        return conditioning_matrix(kind[6:], rng, R, C).astype(np.float32)
    raise ValueError(f"unknown generator {kind!r}")


def conditioning_class_of(G: int, g: int) -> str:
    per = max(1, G // len(CONDITIONING_CLASSES))
    return CONDITIONING_CLASSES[min(g // per, len(CONDITIONING_CLASSES) - 1)]


def make(w: Workload | str, indices: Optional[Sequence[int]] = None,
         G: Optional[int] = None, R: Optional[int] = None, C: Optional[int] = None,
         dtype: Optional[str] = None, kind: Optional[str] = None,
         seed: Optional[int] = None) -> torch.Tensor:
    """Build (part of) a bucket as a CPU tensor [len(indices), R, C] in its dtype.

    Keyword overrides build a bucket of another size with the same recipe.
    Rounding: fp32 sample -> storage dtype, round-to-nearest-even (torch cast).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    G = w.G if G is None else G
    R = w.R if R is None else R
    C = w.C if C is None else C
    dtype = w.dtype if dtype is None else dtype
    kind = w.kind if kind is None else kind
    seed = w.seed if seed is None else seed
    idx = list(range(G)) if indices is None else list(indices)
    out = torch.empty((len(idx), R, C), dtype=_TORCH_DTYPES[dtype])
    for j, g in enumerate(idx):
        out[j] = torch.from_numpy(make_matrix(kind, seed, G, g, R, C)).to(out.dtype)
    return out


def custom(G: int, R: int, C: int, dtype: str = "f16", kind: str = "gaussian",
           seed: int = 11) -> torch.Tensor:
    """A seeded bucket of any shape (test cases: ragged tails, tiny and odd sizes)."""
    out = torch.empty((G, R, C), dtype=_TORCH_DTYPES[dtype])
    for g in range(G):
        out[g] = torch.from_numpy(make_matrix(kind, seed, G, g, R, C)).to(out.dtype)
    return out


Generator = Callable[..., torch.Tensor]
