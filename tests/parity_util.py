"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
reading results back, and the comparison metrics (computed in float64 on the
host over whole flattened tensors)."""
import numpy as np

# Tolerances: fp32 path (relative L2), bf16 path (relative L2 and max abs).
F32_REL_L2 = 1e-5
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 2e-2
# For bf16 outputs whose magnitude reaches past 4 (where one bf16 step is
# 2^-5 or more, so rounding alone exceeds BF16_MAX_ABS), the element bound
# is max(BF16_MAX_ABS, BF16_STEP_REL * |ref|): one bf16 step at |ref|.
BF16_STEP_REL = 2.0 ** -7


def to_device(store, dev):
    """Storage array from `workloads` (float32, or uint16 bf16 bits) -> GPU tensor."""
    import torch
    if store.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(store).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(store)).to(dev)


def to_host(t):
    """GPU tensor -> float64 numpy (bf16 widened exactly)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64))))


def assert_close(name, x, ref, rel, mabs=None):
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    r = rel_l2(x, ref)
    a = max_abs(x, ref)
    msg = f"{name}: rel_l2={r:.3e} (<= {rel:g}) max_abs={a:.3e}" + (
        f" (<= {mabs:g})" if mabs is not None else "")
    print(msg)
    assert r <= rel, msg
    if mabs is not None:
        assert a <= mabs, msg
    return r, a


def assert_close_scaled(name, x, ref, rel):
    """rel-L2 <= rel and, element by element,
    |x - ref| <= max(BF16_MAX_ABS, BF16_STEP_REL * |ref|)."""
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(x, ref)
    excess = np.abs(x - ref) - np.maximum(BF16_MAX_ABS, BF16_STEP_REL * np.abs(ref))
    msg = f"{name}: rel_l2={r:.3e} (<= {rel:g}) worst element excess={excess.max():.3e} (<= 0)"
    print(msg)
    assert r <= rel, msg
    assert excess.max() <= 0, msg
    return r
