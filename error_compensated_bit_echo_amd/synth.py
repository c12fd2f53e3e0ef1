"""Seeded synthetic inputs for the Echo all-reduce (no method arithmetic here).

This module only draws random numbers and shapes them into rank partials: it
holds none of the all-reduce's own arithmetic, so both the HIP path's tests and
the CPU oracle can be fed from it without sharing any code of the method.

Recipe (host side, numpy):
  seed(id, dir, call, rank) = id*10**9 + dir*10**8 + call*10**3 + rank;
  x = Generator(PCG64(seed)).standard_normal(n, float32) * std;
  outliers: mask = rng.random(n) < p from the same generator, x[mask] *= k;
  bf16 partials are x rounded to bfloat16 (round to nearest even).

Large messages are drawn on the device instead (torch's Philox generator
seeded with the same seed formula), because drawing gigabytes on one host core
takes minutes; the checked windows are copied back for the oracle.

The workloads stand in for the pages' tensor-parallel layers (hidden size 4096,
Qwen3-8B-like prefill and decode, a training step, and a 1 GB message); no
model weights or datasets are used.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# the workloads by name: seed id, P, shape per rank, dtype, value distribution, calls per run
WORKLOADS = {
    "tiny": dict(seed_id=1, P=2, shape=(8, 256), dtype="f32", std=1.0,
                 outlier_p=0.0, outlier_mult=1.0, calls=16),
    "prefill": dict(seed_id=2, P=4, shape=(2048, 4096), dtype="bf16", std=0.02,
                    outlier_p=1e-3, outlier_mult=50.0, calls=72),
    "decode": dict(seed_id=3, P=8, shape=(64, 4096), dtype="bf16", std=0.02,
                   outlier_p=0.0, outlier_mult=1.0, calls=128),
    "training": dict(seed_id=4, P=4, shape=(4096, 4096), dtype="bf16", std=0.02,
                     std_bwd=1e-3, outlier_p=0.0, outlier_mult=1.0, calls=56),
    "headline_1GiB": dict(seed_id=5, P=8, shape=(131072, 4096), dtype="bf16",
                          std=1.0, outlier_p=1e-4, outlier_mult=100.0, calls=10),
}


def numel(workload: str) -> int:
    r, c = WORKLOADS[workload]["shape"]
    return r * c


def seed_of(workload: str, direction: int, call: int, rank: int) -> int:
    return WORKLOADS[workload]["seed_id"] * 10**9 + direction * 10**8 + call * 10**3 + rank


def normal_f32(seed: int, n: int, std: float = 1.0, outlier_p: float = 0.0,
               outlier_mult: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draws with an optional sprinkle of scaled outliers."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(n, dtype=F32)
    if std != 1.0:
        x *= F32(std)
    if outlier_p > 0.0:
        mask = rng.random(n) < outlier_p
        x[mask] *= F32(outlier_mult)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """The float32 value of bfloat16 bit patterns (a 16-bit shift)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


def host_partials(workload: str, direction: int = 0, call: int = 0, P: int | None = None,
                  n: int | None = None, dtype: str | None = None, std: float | None = None):
    """Rank partials for one call, drawn on the host.

    Returns ``(raw, values)``: ``raw`` is what is uploaded ([P, n] float32, or
    uint16 bfloat16 bit patterns), ``values`` the same numbers as float32.
    """
    c = WORKLOADS[workload]
    P = c["P"] if P is None else P
    n = numel(workload) if n is None else n
    dtype = c["dtype"] if dtype is None else dtype
    if std is None:
        std = c.get("std_bwd", c["std"]) if direction == 1 else c["std"]
    rows = [normal_f32(seed_of(workload, direction, call, r), n, std,
                       c["outlier_p"], c["outlier_mult"]) for r in range(P)]
    x = np.stack(rows) if P else np.zeros((0, n), F32)
    if dtype == "f32":
        return x, x
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_as_f32(bits)


def device_partials(workload: str, direction: int = 0, call: int = 0, P: int | None = None,
                    n: int | None = None, device: str = "cuda"):
    """Rank partials drawn on the device with torch (for messages of gigabytes).

    Returns a list of P contiguous bfloat16 (or float32) tensors of n elements.
    """
    import torch

    c = WORKLOADS[workload]
    P = c["P"] if P is None else P
    n = numel(workload) if n is None else n
    std = c.get("std_bwd", c["std"]) if direction == 1 else c["std"]
    out = []
    for r in range(P):
        g = torch.Generator(device=device)
        g.manual_seed(seed_of(workload, direction, call, r))
        x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if c["outlier_p"] > 0.0:
            mask = torch.rand(n, generator=g, device=device) < c["outlier_p"]
            # in slices: torch's masked indexing mis-sizes its buffers past 2^32 elements
            for lo in range(0, n, 1 << 30):
                xs, ms = x[lo:lo + (1 << 30)], mask[lo:lo + (1 << 30)]
                xs[ms] *= c["outlier_mult"]
            del mask
        out.append(x if c["dtype"] == "f32" else x.to(torch.bfloat16))
        del x
    return out


# ----------------------------------------------------------------------------
# decode-shaped chain: 128 layers of a synthetic residual stream
# ----------------------------------------------------------------------------
DECODE_CHAIN = dict(rows=64, hidden=4096, layers=128, h0_std=0.02)


def decode_h0(device="cuda"):
    """Initial residual stream h_0 ~ N(0, 0.02^2), [64, 4096] float32."""
    import torch

    c = DECODE_CHAIN
    g = torch.Generator(device=device)
    g.manual_seed(seed_of("decode", 0, 0, 0))
    return torch.randn(c["rows"], c["hidden"], generator=g, device=device) * c["h0_std"]


def decode_weight(layer: int, device="cuda"):
    """Layer map W_l ~ N(0, 1)/sqrt(4096) as bfloat16 [4096, 4096], seeded per layer."""
    import torch

    hd = DECODE_CHAIN["hidden"]
    g = torch.Generator(device=device)
    g.manual_seed(WORKLOADS["decode"]["seed_id"] * 10**9 + 9 * 10**8 + layer)
    w = torch.randn(hd, hd, generator=g, device=device)
    w.mul_(1.0 / hd ** 0.5)
    return w.to(torch.bfloat16)


def decode_partials(h, w, P: int):
    """The P rank partials of one layer: with a = bf16(h / rms(h)) (pre-norm, per
    row), rank r holds bf16(gamma * (a[:, S_r] @ W[S_r, :])), S_r its slice of
    4096/P input columns, gamma = 0.02 * sqrt(P).  The product is taken in fp32.
    Returns P contiguous bfloat16 vectors of rows*hidden elements."""
    import torch

    a = (h / h.pow(2).mean(dim=-1, keepdim=True).sqrt()).to(torch.bfloat16).float()
    gamma = 0.02 * P ** 0.5
    cols = h.shape[1] // P
    wf = w.float()
    return [(gamma * (a[:, r * cols:(r + 1) * cols] @ wf[r * cols:(r + 1) * cols, :]))
            .to(torch.bfloat16).reshape(-1).contiguous() for r in range(P)]
