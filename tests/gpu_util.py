"""Helpers of the GPU parity tests: moving seeded host inputs to the GPU,
viewing results as the wire format, and comparing with the oracle."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def f32_to_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bf16_to_gpu(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_gpu(a: np.ndarray) -> torch.Tensor:
    return f32_to_gpu(a) if a.dtype == np.float32 else bf16_to_gpu(a)


def codes_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def scales_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def f32_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.float32)


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_same(got: np.ndarray, want: np.ndarray, what: str):
    """Bit-exact comparison with a useful message."""
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    bad = np.nonzero(g != w)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


def assert_close_scaled(got: np.ndarray, want: np.ndarray, scale_per_elem: np.ndarray,
                        what: str, rel=1e-6):
    """|got - want| <= rel * block scale (the stated float tolerance)."""
    d = np.abs(got.astype(np.float64) - want.astype(np.float64))
    lim = rel * scale_per_elem.astype(np.float64)
    bad = np.nonzero(~(d <= lim))[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} beyond 1e-6*scale; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r} scale {scale_per_elem[i]!r}")


def scale_per_element(scales_bits: np.ndarray, n: int, block: int) -> np.ndarray:
    return np.repeat(scales_bits.view(np.float16).astype(np.float32), block)[:n]


def mixed_input(seed: int, n: int) -> np.ndarray:
    """Normal values whose magnitude changes every 32 elements (1e-9 .. 1e3),
    so that many blocks get binary16-subnormal scales; a few exact zeros,
    negative zeros and exact ties."""
    g = np.random.default_rng(seed)
    x = g.standard_normal(n)
    mag = 10.0 ** g.uniform(-9, 3, size=-(-n // 32)).repeat(32)[:n]
    x = (x * mag).astype(np.float32)
    if n > 64:
        x[g.integers(0, n, size=n // 50)] = 0.0
        x[g.integers(0, n, size=n // 50)] = -0.0
    return x


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def sample_blocks(nb: int, count: int, seed: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    k = g.choice(nb, size=min(count, nb), replace=False) if nb > count else np.arange(nb)
    return np.unique(np.concatenate([k, [0, nb - 1]]))


def word_range(k: int, block: int, bits: int, n: int):
    """Word indices [a, b) holding block k."""
    per = 32 // bits
    lo = k * block
    hi = min(n, (k + 1) * block)
    return lo // per, (hi + per - 1) // per
