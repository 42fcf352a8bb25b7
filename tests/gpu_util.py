"""Helpers for the GPU parity tests: host<->device copies of the formats and the comparisons."""
import numpy as np
import torch


def to_dev(a: np.ndarray, fmt: str, dev="cuda") -> torch.Tensor:
    """numpy array in an oracle format (f32 / bf16 bits / e4m3 codes / int32) -> device tensor."""
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the oracle's representation (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 codes along the number line (-0 and +0 coincide)."""
    def mono(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(mono(a) - mono(b))


def assert_close_out(got: np.ndarray, want: np.ndarray, fmt: str):
    """Combine tolerance: bf16 within one code; fp32 within 1e-5 relative (|want| = 0: |got| tiny)."""
    assert got.shape == want.shape
    if fmt == "bf16":
        d = bf16_ulp_distance(got, want)
        assert d.max() <= 1, f"max bf16 code distance {d.max()} at {np.unravel_index(d.argmax(), d.shape)}"
    else:
        g, w = got.astype(np.float64), want.astype(np.float64)
        bad = np.abs(g - w) > 1e-5 * np.abs(w) + (w == 0) * 1e-30
        assert not bad.any(), f"{bad.sum()} fp32 elements beyond 1e-5, first at {np.argwhere(bad)[0]}"
