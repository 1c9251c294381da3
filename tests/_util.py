"""Shared helpers for the GPU parity tests (conversion and comparison only)."""
import numpy as np
import torch

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 tensor."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits (bf16 -> uint16, fp32 -> uint32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def np_bits(a: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Storage bits of float64 values that are exactly representable in `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == torch.bfloat16:
        t2 = t.to(torch.bfloat16)
        assert torch.equal(t2.to(torch.float32), t), "value not representable in bf16"
        return bits(t2)
    return bits(t)


def meta_u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def rel_err(got, ref, floor=1e-3):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + floor)))


class Report:
    """Collects the parity error of every output, prints them all, then asserts."""

    def __init__(self, dtype):
        self.tol = TOL[dtype]
        self.errs = {}

    def add(self, name, got, ref, floor=1e-3):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        e = rel_err(got, ref, floor)
        where = None
        if got.size and e > self.tol:
            i = np.unravel_index(np.argmax(np.abs(got - ref) / (np.abs(ref) + floor)), got.shape)
            where = (tuple(int(x) for x in i), float(got[i]), float(ref[i]))
        self.errs[name] = (e, where)

    def check(self):
        print({k: f"{e:.2e}" for k, (e, _) in self.errs.items()}, flush=True)
        bad = {k: v for k, v in self.errs.items() if v[0] > self.tol}
        assert not bad, f"parity above {self.tol:.0e}: {bad}"


def assert_close(name, got, ref, dtype, floor=1e-3):
    r = Report(dtype)
    r.add(name, got, ref, floor)
    r.check()
    return r.errs[name][0]


def tie_heavy(shape, seed, dtype=torch.bfloat16):
    """Values from a small alphabet (exact in bf16), so magnitude ties are everywhere."""
    rng = np.random.default_rng(seed)
    alphabet = np.array([0.0, -0.0, 0.5, -0.5, 1.0, 2.0, -2.0, 0.25])
    return torch.from_numpy(rng.choice(alphabet, size=shape).astype(np.float32)).to(dtype)
