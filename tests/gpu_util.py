"""Helpers for the GPU parity tests: host <-> device copies and comparisons."""
import numpy as np
import torch

DEV = "cuda"


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty_bf16(*shape) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.bfloat16, device=DEV)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    bad = np.argwhere(g != w)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}"


def assert_rel(got: np.ndarray, want: np.ndarray, rel: float, floor: np.ndarray, what: str):
    """|got - want| <= rel * max(|want|, floor) elementwise."""
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    lim = rel * np.maximum(np.abs(want), floor)
    bad = np.argwhere(np.abs(got - want) > lim)
    assert bad.size == 0, f"{what}: {len(bad)} out of tolerance, first {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


GUARD = 256          # canary bytes on each side of a guarded output
CANARY = 0xA5


class Guarded:
    """A device output buffer with GUARD canary bytes (0xA5) before and after
    it, so that a kernel writing past either end of its output is caught.
    `t` is the output itself (16-byte aligned), viewed with the given dtype
    and shape; check() asserts both guards are intact."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((GUARD + n + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        inner = self.raw[GUARD:GUARD + n]
        self.t = inner.view(dtype).view(shape) if n else torch.empty(shape, dtype=dtype, device=DEV)

    def check(self, what: str) -> None:
        g = self.raw.cpu().numpy()
        lo, hi = g[:GUARD], g[GUARD + self.n:]
        assert np.all(lo == CANARY), f"{what}: {np.count_nonzero(lo != CANARY)} bytes written before the output"
        assert np.all(hi == CANARY), f"{what}: {np.count_nonzero(hi != CANARY)} bytes written after the output"
