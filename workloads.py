"""Seeded synthetic inputs and the named attention workloads.

This module only draws random numbers and names shapes; it holds none of the
attention arithmetic.  Both the GPU tests / bench and the fp64 oracle take
their inputs from here.

Inputs are i.i.d. N(0, sigma^2) drawn in float32 from a seeded torch
generator and rounded to bfloat16 (round-to-nearest-even), laid out
contiguous [B, H, N, d].  The same bf16 tensors feed both sides.
"""
from dataclasses import dataclass
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n_q: int
    n_k: int
    d: int
    causal: tuple          # the mask settings this workload is run with
    index: int             # 1-based workload number, part of the seed
    num_splits: int = 0    # >0: split-KV decode workload

    @property
    def scale(self) -> float:
        # 1/sqrt(d) rounded to fp32, the value a caller passes
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def flop(self, causal: bool) -> float:
        """4*B*H*N_q*N_k*d, exactly halved for causal (the headline metric's count)."""
        f = 4.0 * self.B * self.H * self.n_q * self.n_k * self.d
        return f / 2 if causal else f

    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O (bf16) and LSE (fp32) written once."""
        bh = self.B * self.H
        return bh * (2 * self.n_q * self.d + 2 * 2 * self.n_k * self.d + 2 * self.n_q * self.d + 4 * self.n_q)


# The five workloads the method is measured on.
C1 = Workload("b1_h2_n256_d64", 1, 2, 256, 256, 64, (False,), 1)
C2 = Workload("b8_h16_n2048_d64", 8, 16, 2048, 2048, 64, (False, True), 2)
C3 = Workload("b4_h16_n4096_d128", 4, 16, 4096, 4096, 128, (True, False), 3)
C4 = Workload("b1_h32_n16384_d128", 1, 32, 16384, 16384, 128, (True, False), 4)
C5 = Workload("decode_b64_h32_nq1_nk8192_d128_s16", 64, 32, 1, 8192, 128, (False,), 5, num_splits=16)
ALL = (C1, C2, C3, C4, C5)

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


def seed_for(index: int, tensor: int, chunk: int = 0) -> int:
    """seed = index * 2^20 + tensor * 2^16 + chunk (chunk = batch index when drawn per batch)."""
    return (index << 20) + (tensor << 16) + chunk


def _draw(shape, seed: int, device, sigma: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def make_tensor(index: int, tensor: int, B: int, H: int, n: int, d: int, device="cpu",
                sigma: float = 1.0, per_batch: bool = False) -> torch.Tensor:
    """One bf16 [B, H, n, d] tensor.  per_batch draws each batch slice from its own seed
    (bounds the float32 temporary for very large tensors)."""
    if not per_batch:
        return _draw((B, H, n, d), seed_for(index, tensor), device, sigma)
    out = torch.empty((B, H, n, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        out[b] = _draw((H, n, d), seed_for(index, tensor, b), device, sigma)
    return out


def make_qkv(w: Workload, device="cpu", sigma: float = 1.0):
    """Q, K, V for a named workload.  Tensors above 2^28 elements are drawn per batch."""
    per_batch = w.B * w.H * w.n_k * w.d > (1 << 28)
    q = make_tensor(w.index, TENSOR_Q, w.B, w.H, w.n_q, w.d, device, sigma)
    k = make_tensor(w.index, TENSOR_K, w.B, w.H, w.n_k, w.d, device, sigma, per_batch)
    v = make_tensor(w.index, TENSOR_V, w.B, w.H, w.n_k, w.d, device, sigma, per_batch)
    return q, k, v


def make_qkv_shape(B, H, n_q, n_k, d, seed: int, device="cpu", sigma: float = 1.0):
    """Q, K, V for an ad-hoc shape (tests): seeds seed*4 + {0, 1, 2}."""
    q = _draw((B, H, n_q, d), seed * 4 + 0, device, sigma)
    k = _draw((B, H, n_k, d), seed * 4 + 1, device, sigma)
    v = _draw((B, H, n_k, d), seed * 4 + 2, device, sigma)
    return q, k, v


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (moved to the host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a bf16 tensor."""
    return t.detach().cpu().to(torch.float64).numpy()


def make_fp8_codes(shape, seed: int, exp_lo: int = 9, exp_hi: int = 14) -> np.ndarray:
    """Random e4m3 byte codes: sign uniform, exponent field uniform in [exp_lo, exp_hi]
    (exp_hi <= 14 keeps clear of the NaN pattern), mantissa field uniform in 0..7.
    With the defaults the magnitudes are log-uniform over [4, 240]."""
    assert 0 <= exp_lo <= exp_hi <= 14
    g = np.random.default_rng(seed)
    sign = g.integers(0, 2, shape, dtype=np.uint8)
    e = g.integers(exp_lo, exp_hi + 1, shape, dtype=np.uint8)
    m = g.integers(0, 8, shape, dtype=np.uint8)
    return (sign << 7) | (e << 3) | m


def make_fp8_descales(B: int, H: int, seed: int, lo: float = 0.008, hi: float = 0.016) -> np.ndarray:
    """fp32 [B, H] descales drawn log-uniformly from [lo, hi]."""
    g = np.random.default_rng(seed)
    return np.exp(g.uniform(np.log(lo), np.log(hi), (B, H))).astype(np.float32)


# ---- block masks (input structure of the block-sparse forward) ----
BLOCK_Q, BLOCK_K = 128, 64  # rows and keys per mask entry


def dilated_block_mask(n_q: int, n_k: int, dilation: int, window: int, causal: bool,
                       block_q: int = BLOCK_Q, block_k: int = BLOCK_K) -> np.ndarray:
    """uint8 [ceil(n_q/block_q), ceil(n_k/block_k)]: a dilated sliding window at block granularity.

    Query block qb always sees the key blocks that hold its own positions, [k0, k1] with
    k0 = qb*block_q // block_k and k1 = ((qb+1)*block_q - 1) // block_k, and beyond them every
    dilation-th key block, `window` of them on each side it may look to: k0 - dilation*t (and,
    unless causal, k1 + dilation*t) for t = 1 .. window.  Key blocks past n_k are dropped."""
    assert dilation >= 1 and window >= 0
    n_qb, n_kb = -(-n_q // block_q), -(-n_k // block_k)
    m = np.zeros((n_qb, n_kb), dtype=np.uint8)
    for qb in range(n_qb):
        k0 = qb * block_q // block_k
        k1 = ((qb + 1) * block_q - 1) // block_k
        m[qb, k0:min(k1, n_kb - 1) + 1] = 1
        for t in range(1, window + 1):
            if 0 <= k0 - dilation * t < n_kb:
                m[qb, k0 - dilation * t] = 1
            if not causal and k1 + dilation * t < n_kb:
                m[qb, k1 + dilation * t] = 1
    return m


def random_block_mask(shape, density: float, seed: int) -> np.ndarray:
    """uint8 block mask of the given shape with entries 1 at probability `density` (seeded)."""
    g = np.random.default_rng(seed)
    return (g.random(shape) < density).astype(np.uint8)
