"""Helpers for the GPU parity tests: host<->device transfer of numpy arrays
(bfloat16 travels as uint16 bit patterns) and bit-exact comparison with a
report of the first difference."""
import hashlib

import numpy as np
import torch

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def sha(a) -> str:
    if isinstance(a, torch.Tensor):
        a = to_np(a)
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def assert_bitwise(gpu, want, name):
    g = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    w = np.ascontiguousarray(want)
    g = np.ascontiguousarray(g).reshape(w.shape) if g.size == w.size else g
    assert g.shape == w.shape, f"{name}: shape {g.shape} != {w.shape}"
    gb = g.view(np.uint8).reshape(-1)
    wb = w.view(np.uint8).reshape(-1)
    if gb.size == wb.size and np.array_equal(gb, wb):
        return
    it = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[w.dtype.itemsize]
    gi, wi = g.reshape(-1).view(it), w.reshape(-1).view(it)
    bad = np.nonzero(gi != wi)[0]
    i = int(bad[0])
    raise AssertionError(
        f"{name}: {bad.size} of {w.size} elements differ; first at flat index {i} "
        f"(multi-index {np.unravel_index(i, w.shape)}): gpu {g.reshape(-1)[i]!r} "
        f"[{int(gi[i]):#x}] oracle {w.reshape(-1)[i]!r} [{int(wi[i]):#x}]")


def codes(rng, shape):
    return rng.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)
