"""Seeded synthetic inputs for the NVFP4 decode GEMM.

This module only draws random inputs; it holds none of the GEMM's or the
format's arithmetic (no quantisation, no packing, no dequantisation).  Both
sides of every parity check -- the CPU oracle and the HIP library -- consume
what it produces.

Workload recipe (the synthetic stand-in for the real 27B artifact, which the
pages describe in "Models and artifacts" but which is not available here):

* weights: fp32 draws from N(0, 0.02), shape [N][K] (N output rows of K
  values, K contiguous), one independent stream per matrix;
* activations: fp32 draws from N(0, 1) rounded to bf16 (round to nearest
  even), shape [M][K], returned as the 16-bit patterns;
* logits for the top-k step: fp32 draws from N(0, 4), shape [M][V], or, for
  tie-heavy cases, draws from a small pool of values that includes -0.0,
  +0.0 and the infinities.

Host draws use numpy's Philox-4x32 counter-based generator keyed by
(seed, stream).  Draws for full-size workloads are made on the GPU with
torch's device generator seeded from the same pair; the host copy of a device
draw is what the oracle then reads.
"""
from __future__ import annotations

import numpy as np

WEIGHT_STD = 0.02

# Stream ids of the 27B-class round: one per (layer, projection).
PROJECTIONS = ("qkv", "o", "gate_up", "down")


def stream_id(layer: int, proj: str) -> int:
    return 1000 + 4 * int(layer) + PROJECTIONS.index(proj)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[int(seed) & 0xFFFFFFFFFFFFFFFF,
                                                     int(stream) & 0xFFFFFFFFFFFFFFFF]))


def weights(seed: int, stream: int, N: int, K: int, std: float = WEIGHT_STD) -> np.ndarray:
    """fp32 [N][K] weights drawn from N(0, std)."""
    g = _rng(seed, stream)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(seed: int, stream: int, M: int, K: int) -> np.ndarray:
    """bf16 bit patterns (uint16 [M][K]) of N(0, 1) draws."""
    g = _rng(seed, stream + (1 << 40))
    x = g.standard_normal((M, K), dtype=np.float32)
    return _to_bf16_bits(x)


# ---- device draws (full-size workloads) ----------------------------------

def _torch_gen(seed: int, stream: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(((int(seed) * 0x9E3779B97F4A7C15) ^ int(stream)) & 0x7FFFFFFFFFFFFFFF)
    return g


def weights_device(seed: int, stream: int, N: int, K: int, device="cuda",
                   std: float = WEIGHT_STD):
    """fp32 [N][K] torch tensor on ``device`` drawn from N(0, std)."""
    import torch
    w = torch.randn((N, K), generator=_torch_gen(seed, stream, device), device=device,
                    dtype=torch.float32)
    w.mul_(std)
    return w


def activations_device(seed: int, stream: int, M: int, K: int, device="cuda"):
    """bf16 [M][K] torch tensor on ``device`` of N(0, 1) draws (RNE to bf16)."""
    import torch
    x = torch.randn((M, K), generator=_torch_gen(seed, stream + (1 << 40), device),
                    device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def random_planes(seed: int, stream: int, N: int, K: int):
    """Uniformly random canonical code/scale planes (every code and every
    finite non-negative E4M3 scale byte, 0x00..0x7E, equally likely) for
    exercising the kernels beyond the quantiser's output range."""
    g = _rng(seed, stream + (2 << 40))
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = g.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    return codes, scales


LOGIT_POOL = np.array([-np.inf, -3.0, -1.0, -0.0, 0.0, 0.5, 1.0, 2.0, 2.0, 7.5, np.inf],
                      np.float32)


def logits(seed: int, stream: int, M: int, V: int, ties: bool = False) -> np.ndarray:
    """fp32 [M][V]: N(0, 4) draws, or (ties=True) draws from LOGIT_POOL."""
    rng = _rng(seed, stream)
    if ties:
        return LOGIT_POOL[rng.integers(0, len(LOGIT_POOL), (M, V))]
    return (rng.standard_normal((M, V)) * 4.0).astype(np.float32)
