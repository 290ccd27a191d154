"""Seeded synthetic inputs for tests, the smoke check and the benchmark.

This module holds input recipes only -- none of the codec's arithmetic -- so
that the CPU oracle and the HIP path can be fed the same bytes.  Every draw
comes from numpy's PCG64 generator with an explicit seed; bfloat16 tensors are
made by round-to-nearest-even casts (torch CPU) and returned as uint16 bit
patterns.

Workloads (shapes of the pages' setting: data-parallel gradient buckets and a
sharded GPT weight shard; the pages name no dataset for this path):
  * roundtrip: 2^20 binary32 values ~ N(0, 1), seed 0
  * gradient bucket: 64 Mi binary32 values, Student-t (3 degrees of freedom)
    times 1e-3, seed 1
  * error-feedback steps: 128 Mi bfloat16 gradients ~ N(0, 1e-4) (standard
    deviation), seed 2 + step
  * local reduce: 8 peers x 32 Mi binary32 values ~ N(0, 1), seeds 10..17,
    each quantized by its peer before the reduce
  * weight difference: 840 Mi bfloat16 weights of one 8-way shard of a
    32-layer, hidden-4096 GPT: w_prev = bf16(0.02 N(0,1)), then
    w_new = bf16(w_prev + 1e-4 N(0,1)), both from one PCG64(3) stream
"""
from __future__ import annotations

import numpy as np

MI = 1 << 20
CHUNK = 1 << 24   # draw in chunks to bound host memory

ROUNDTRIP_N = 1 << 20
BUCKET_N = 64 * MI
EF_N = 128 * MI
EF_STEPS = 5
PEER_N = 32 * MI
PEERS = 8
WEIGHT_N = 840 * MI


def _gen(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(n: int, seed: int, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2): standard normal in float32, times std in float32."""
    g = _gen(seed)
    out = np.empty(n, np.float32)
    for lo in range(0, n, CHUNK):
        hi = min(n, lo + CHUNK)
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def student_t_f32(n: int, seed: int, dof: float = 3.0, scale: float = 1e-3) -> np.ndarray:
    """float32(scale * t_dof), drawn in float64."""
    g = _gen(seed)
    out = np.empty(n, np.float32)
    for lo in range(0, n, CHUNK):
        hi = min(n, lo + CHUNK)
        out[lo:hi] = (g.standard_t(dof, hi - lo) * scale).astype(np.float32)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even) as uint16 bit patterns."""
    import torch
    out = np.empty(x.shape, np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    for lo in range(0, flat_in.size, CHUNK):
        hi = min(flat_in.size, lo + CHUNK)
        t = torch.from_numpy(np.ascontiguousarray(flat_in[lo:hi])).to(torch.bfloat16)
        flat_out[lo:hi] = t.view(torch.int16).numpy().view(np.uint16)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def random_bits(n: int, seed: int) -> np.ndarray:
    """uint32 random words (e.g. arbitrary packed codes)."""
    return _gen(seed).integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)


def random_scales_f16(n: int, seed: int, lo: float = 1e-3, hi: float = 1.0) -> np.ndarray:
    """Positive binary16 scale bit patterns, log-uniform in [lo, hi]."""
    v = np.exp(_gen(seed).uniform(np.log(lo), np.log(hi), size=n)).astype(np.float16)
    return v.view(np.uint16)


# ------------------------------------------------------------ workloads ---
def roundtrip_input(n: int = ROUNDTRIP_N) -> np.ndarray:
    return normal_f32(n, seed=0)


def bucket_input(n: int = BUCKET_N) -> np.ndarray:
    return student_t_f32(n, seed=1, dof=3.0, scale=1e-3)


def ef_gradient(step: int, n: int = EF_N) -> np.ndarray:
    """bfloat16 bits of 1e-4 * N(0, 1) for error-feedback step `step`."""
    return to_bf16_bits(normal_f32(n, seed=2 + step, std=1e-4))


def peer_input(p: int, n: int = PEER_N) -> np.ndarray:
    return normal_f32(n, seed=10 + p)


def weight_pair(n: int = WEIGHT_N):
    """(w_prev_bits, w_new_bits) bfloat16 bit patterns from one PCG64(3) stream."""
    import torch
    g = _gen(3)
    w_prev = np.empty(n, np.uint16)
    w_new = np.empty(n, np.uint16)
    # all of w_prev first, then all of the delta, from the same stream
    for lo in range(0, n, CHUNK):
        hi = min(n, lo + CHUNK)
        a = g.standard_normal(hi - lo, dtype=np.float32) * np.float32(0.02)
        w_prev[lo:hi] = to_bf16_bits(a)
    for lo in range(0, n, CHUNK):
        hi = min(n, lo + CHUNK)
        d = g.standard_normal(hi - lo, dtype=np.float32) * np.float32(1e-4)
        base = torch.from_numpy(bf16_bits_to_f32(w_prev[lo:hi]))
        w_new[lo:hi] = (base + torch.from_numpy(d)).to(torch.bfloat16).view(torch.int16) \
            .numpy().view(np.uint16)
    return w_prev, w_new
