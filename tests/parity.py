"""Helpers shared by the GPU parity tests: device upload of seeded inputs and
the tolerance checks of the parity bar.

Bar (element-wise against the fp64 oracle): bfloat16 outputs max |err| <= 2e-2
and mean |err| <= 2e-3; float32 outputs max |err| <= 1e-4.  Extra guards
(not the bar, but tighter on small outputs): relative Frobenius error
<= 1e-2 (bf16) / 1e-5 (fp32), LSE max |err| <= 1e-2 (bf16) / 1e-4 (fp32).
"""
import numpy as np
import torch

BF16_MAX, BF16_MEAN, BF16_REL = 2e-2, 2e-3, 1e-2
F32_MAX, F32_REL = 1e-4, 1e-5
LSE_BF16, LSE_F32 = 1e-2, 1e-4


def log(*a):
    print(*a, flush=True)


def to_dev(t, device="cuda"):
    """workloads.Tensor (or float64 array + dtype) -> torch tensor on the GPU."""
    if t.dtype == "bf16":
        x = torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16)
    else:
        x = torch.from_numpy(np.ascontiguousarray(t.values, dtype=np.float32))
    return x.to(device)


def from_dev(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def check(got, want, dtype, what, rel=True):
    g = from_dev(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - w)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    nw = float(np.linalg.norm(w))
    rfro = float(np.linalg.norm(g - w) / nw) if nw > 0 else 0.0
    log(f"  {what}: max|err|={mx:.3e} mean|err|={mean:.3e} relF={rfro:.3e} (|ref| max {float(np.abs(w).max()) if w.size else 0:.3e})")
    if dtype == "bf16":
        assert mx <= BF16_MAX, f"{what}: max err {mx}"
        assert mean <= BF16_MEAN, f"{what}: mean err {mean}"
        if rel:
            assert rfro <= BF16_REL, f"{what}: relative Frobenius err {rfro}"
    else:
        assert mx <= F32_MAX, f"{what}: max err {mx}"
        if rel:
            assert rfro <= F32_REL, f"{what}: relative Frobenius err {rfro}"


def check_lse(got, want, dtype, what):
    g = from_dev(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    both_inf = np.isneginf(g) & np.isneginf(w)
    assert (np.isneginf(g) == np.isneginf(w)).all(), f"{what}: -inf pattern differs"
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_inf, 0.0, g - w))
    mx = float(d.max()) if d.size else 0.0
    log(f"  {what}: max|err|={mx:.3e}")
    assert mx <= (LSE_BF16 if dtype == "bf16" else LSE_F32), f"{what}: LSE err {mx}"
