"""Helpers shared by the GPU parity tests: host <-> device marshalling of the
numpy buffers the oracle reads (bf16 tensors are uint16 bit patterns)."""
import numpy as np
import torch

DEV = "cuda"


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def scalar(v=0.0) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def empty_codes(shape, fill=0xA5) -> torch.Tensor:
    """uint8 output filled with a sentinel so unwritten bytes show up."""
    return torch.full(shape if isinstance(shape, tuple) else (shape,), fill, dtype=torch.uint8, device=DEV)


def empty_f32(shape, fill=-7.25) -> torch.Tensor:
    return torch.full(shape if isinstance(shape, tuple) else (shape,), fill, dtype=torch.float32, device=DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def same_f32(got, want) -> bool:
    """Bitwise equal float32 arrays, NaNs compared as a class."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    if got.shape != want.shape:
        return False
    gn, wn = np.isnan(got), np.isnan(want)
    if not np.array_equal(gn, wn):
        return False
    return np.array_equal(f32_bits(got[~gn]), f32_bits(want[~wn]))


def first_mismatches(got: np.ndarray, want: np.ndarray, k: int = 8):
    idx = np.nonzero(got.ravel() != want.ravel())[0][:k]
    return [(int(i), hex(int(got.ravel()[i])), hex(int(want.ravel()[i]))) for i in idx]
