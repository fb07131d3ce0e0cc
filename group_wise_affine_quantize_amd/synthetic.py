"""Seeded synthetic inputs for the quantized-product workloads.

This module draws random numbers and nothing else: it holds none of the
quantization or product arithmetic, so both the GPU path and the CPU checker
may take their inputs from it.

Recipe: one numpy PCG64 generator per workload, `default_rng(seed)`; the
weights are drawn first, then the activations, then the expert ids.  Gaussians
are drawn in float32 and scaled by a float32 sigma; bf16 tensors are the
float32 draws rounded to nearest-even (torch's conversion).  The shapes are
LLM projection and mixture-of-experts expert shapes; the examples on the
"Quantization" page of the nuvec documentation (sections "Affine" and
"Mixture of experts") use standard-normal weights and activations.
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    w_shape: tuple          # [n, k] or [e, n, k]
    x_shape: tuple          # [m, k] or [rows, l, k]
    w_sigma: float
    dtype: str              # "f32" or "bf16" for weights, activations, scales
    group_size: int
    bits: int
    n_ids: int = 0          # > 0: mixture-of-experts ids drawn in [0, e)


WORKLOADS = {
    "affine_f32_256x512": Workload("affine_f32_256x512", (256, 512), (4, 512), 1.0, "f32", 64, 4),
    "decode_gemv": Workload("decode_gemv", (14336, 4096), (1, 4096), 0.02, "bf16", 64, 4),
    "multirow_8bit": Workload("multirow_8bit", (4096, 4096), (8, 4096), 0.02, "bf16", 128, 8),
    "splitk": Workload("splitk", (1024, 14336), (4, 14336), 0.02, "bf16", 64, 4),
    "prefill": Workload("prefill", (14336, 4096), (2048, 4096), 0.02, "bf16", 64, 4),
    "moe_gather": Workload("moe_gather", (32, 1408, 2048), (512, 1, 2048), 0.02, "bf16", 64, 4,
                           n_ids=512),
}


def to_bf16_bits(a):
    """float32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal(rng, shape, sigma=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def generate(workload, seed=0):
    """Returns a dict with 'w', 'x' (float32 arrays or uint16 bf16 bits) and
    'ids' (uint32, mixture-of-experts workloads only)."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    rng = np.random.default_rng(seed)
    w = normal(rng, wl.w_shape, wl.w_sigma)
    x = normal(rng, wl.x_shape, 1.0)
    out = {}
    if wl.n_ids:
        out["ids"] = rng.integers(0, wl.w_shape[0], size=wl.n_ids, dtype=np.uint32)
    if wl.dtype == "bf16":
        w, x = to_bf16_bits(w), to_bf16_bits(x)
    out["w"], out["x"] = w, x
    return out


def random_case(seed, w_shape, x_shape, w_sigma=1.0, dtype="f32", x_dtype=None):
    """A small seeded case of any shape, same recipe as the workloads."""
    rng = np.random.default_rng(seed)
    w = normal(rng, w_shape, w_sigma)
    x = normal(rng, x_shape, 1.0)
    if dtype == "bf16":
        w = to_bf16_bits(w)
    if (x_dtype or dtype) == "bf16":
        x = to_bf16_bits(x)
    return w, x


def random_fp_matrix(seed, lead_shape, k, bits, group_size, scale_codes, finite_bytes=False):
    """Seeded uniformly random packed codes and uint8 scale codes of a
    floating-point-mode matrix [*lead_shape, k]: the code words are uniform
    random bits (every 4-bit code equally likely); with finite_bytes (8-bit
    codes) each byte is drawn from 0..0x7e with a random top bit instead, so
    no byte has its low seven bits all set.  Scale codes are drawn uniformly
    from the inclusive range scale_codes = (lo, hi)."""
    rng = np.random.default_rng(seed)
    lead = tuple(lead_shape)
    if bits == 8 and finite_bytes:
        b = rng.integers(0, 0x7F, size=lead + (k,), dtype=np.uint8)
        b |= rng.integers(0, 2, size=lead + (k,), dtype=np.uint8) << np.uint8(7)
        words = np.ascontiguousarray(b).view(np.uint32)
    else:
        words = rng.integers(0, 1 << 32, size=lead + (k * bits // 32,), dtype=np.uint32)
    lo, hi = scale_codes
    scales = rng.integers(lo, hi + 1, size=lead + (k // group_size,), dtype=np.uint8)
    return words, scales
