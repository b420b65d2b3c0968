"""Test helpers: storage views and tolerance checks (no attention arithmetic)."""
import numpy as np
import torch

import oracle


def storage(t: torch.Tensor):
    """(numpy storage array, oracle dtype code) for a torch tensor."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy(), oracle.F32
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), oracle.BF16
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy(), oracle.FP8_E4M3
    if t.dtype == torch.int8:
        return t.numpy(), oracle.INT8
    if t.dtype == torch.uint8:  # packed int4 pool
        return t.numpy(), oracle.INT4
    raise TypeError(t.dtype)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def assert_close(got, want, max_abs, mean_abs=None, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    mn = float(err.mean()) if err.size else 0.0
    assert mx <= max_abs, f"{what}: max-abs error {mx:.3e} > {max_abs:.1e} (mean {mn:.3e})"
    if mean_abs is not None:
        assert mn <= mean_abs, f"{what}: mean-abs error {mn:.3e} > {mean_abs:.1e}"
    return mx, mn
