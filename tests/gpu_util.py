"""Helpers shared by the GPU tests: host <-> device copies of bf16-bit arrays,
cache allocation with a sentinel fill, and first-mismatch reports."""
import numpy as np
import torch


def dev(a, dtype=None):
    """NumPy array -> GPU tensor (uint16 arrays become bfloat16 bit-for-bit)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t):
    """GPU tensor -> NumPy (bfloat16 as uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def filled_cache(shape, fill):
    return torch.full(shape, fill, dtype=torch.uint8, device="cuda")


def assert_same(got, want, what):
    """Bit-exact comparison with a readable first mismatch."""
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    if bad.size:
        i = int(bad[0])
        idx = np.unravel_index(i, got.shape)
        raise AssertionError(f"{what}: {bad.size} of {got.size} elements differ; first at {idx}: "
                             f"got {got.reshape(-1)[i]:#x}, want {want.reshape(-1)[i]:#x}")
