"""Helpers shared by the GPU parity tests (device plumbing only)."""
import numpy as np
import pytest
import torch

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def to_dev(bits: np.ndarray, device="cuda:0") -> torch.Tensor:
    """uint16 binary16 patterns -> torch.float16 device tensor, bit for bit."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """torch.float16 tensor -> uint16 binary16 patterns, bit for bit."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_bf16(bits: np.ndarray, device="cuda:0") -> torch.Tensor:
    """uint16 bfloat16 patterns -> torch.bfloat16 device tensor, bit for bit."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)


def assert_same_bits(got: np.ndarray, ref: np.ndarray, what: str, bf16: bool = False):
    import oracle
    ok = oracle.same_bits_bf16(got, ref) if bf16 else oracle.same_bits(got, ref)
    if not ok.all():
        bad = np.flatnonzero(~ok)
        j = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} of {ok.size} values differ; first at {j}: "
                             f"got {got[j]:#06x}, oracle {ref[j]:#06x}")


def specials_mix(n: int, seed: int) -> np.ndarray:
    """Gaussian binary16 values of mixed scale with every special class planted."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n).astype(np.float32) *
         np.float32(10.0) ** rng.integers(-6, 4, n).astype(np.float32))
    bits = x.astype(np.float16).view(np.uint16).copy()
    k = max(1, n // 50)
    idx = rng.integers(0, n, k)
    bits[idx] = rng.choice(np.array([0x0000, 0x8000, 0x0001, 0x83FF, 0x0400, 0x7BFF, 0xFBFF,
                                     0x7C00, 0xFC00, 0x7E00], np.uint16), k)
    return bits


def specials_mix_bf16(n: int, seed: int) -> np.ndarray:
    """bfloat16 values over the whole exponent range with every special
    class planted (subnormals, extremes, signed zeros, infinities, NaN)."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    bits = np.where(((bits & 0x7F80) == 0x7F80), bits & 0xBFFF, bits).astype(np.uint16)  # no stray inf/NaN
    k = max(1, n // 50)
    idx = rng.integers(0, n, k)
    bits[idx] = rng.choice(np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x0080, 0x7F7F, 0xFF7F,
                                     0x7F80, 0xFF80, 0x7FC0], np.uint16), k)
    return bits
