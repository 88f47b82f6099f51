"""Test-side plumbing: move a seeded workload to the GPU, run the library, read results back."""
import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_device(arr, dtype, device="cuda"):
    """numpy storage array (uint16 bits for bf16) -> torch tensor of the element type."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_numpy_storage(t, dtype):
    """torch tensor -> numpy storage array (uint16 bits for bf16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t):
    """GPU result -> float64 (exact widening of the stored values)."""
    return t.detach().double().cpu().numpy()


class DeviceWorkload:
    """The tensors of a Workload on the GPU."""

    def __init__(self, w, device="cuda"):
        import torch
        self.w = w
        self.q = to_device(w.q, w.dtype, device)
        self.k_pool = to_device(w.k_pool, w.dtype, device)
        self.v_pool = to_device(w.v_pool, w.dtype, device)
        self.page_table = torch.from_numpy(w.page_table).to(device)
        self.context_lens = torch.from_numpy(w.context_lens).to(device)
        self.append_lens = None if w.append_lens is None else torch.from_numpy(w.append_lens).to(device)
        self.k_new = None if w.k_new is None else to_device(w.k_new, w.dtype, device)
        self.v_new = None if w.v_new is None else to_device(w.v_new, w.dtype, device)
        self.scale = float(w.scale)


TOL = {"f32": 1e-5, "bf16": 2e-3, "f16": 2e-3}
EXPLICIT_MANTISSA_BITS = {"bf16": 7, "f16": 10}
# Bound on how far the kernels' float32 result (before the final rounding to the output type)
# may lie from the exact value: the same 1e-4 that the path's other float32 results (split
# partials and log-sum-exps) are held to.
FP32_MARGIN = 1e-4


def half_ulp(ref, dtype):
    """Half a unit in the last place of the 16-bit output type at |ref| (the largest error of a
    correctly rounded result)."""
    a = np.maximum(np.abs(ref), 2.0 ** -126)   # zero: the smallest normal's half ulp
    e = np.floor(np.log2(a))
    return np.exp2(e - EXPLICIT_MANTISSA_BITS[dtype] - 1)


def elementwise_tolerance(ref, dtype):
    """The flat bar (1e-5 f32, 2e-3 bf16/f16) wherever a correctly rounded output can meet it.
    Where it cannot (half an output ulp of the exact value is itself >= the flat bar: |ref| >= 1
    for bf16, >= 8 for f16), the bar is that half ulp plus FP32_MARGIN: the rounding to the output
    type plus the float32 computation's own error, and no more."""
    base = TOL[dtype]
    if dtype == "f32":
        return np.full(ref.shape, base)
    hu = half_ulp(ref, dtype)
    return np.where(hu < base, base, hu + FP32_MARGIN)


def tolerance_note(ref, dtype):
    """The bar elementwise_tolerance enforces on `ref`, in words, for logs."""
    tol = elementwise_tolerance(ref, dtype)
    if dtype == "f32" or float(tol.max(initial=0)) <= TOL[dtype]:
        return f"flat {TOL[dtype]:.0e}"
    return (f"flat {TOL[dtype]:.0e}; {float(tol.max()):.3e} (half ulp + {FP32_MARGIN:.0e}) "
            f"on {int((tol > TOL[dtype]).sum())} element(s) with |ref| >= "
            f"{1.0 if dtype == 'bf16' else 8.0:g}")


def max_abs_err(got, want):
    both_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    d = np.where(both_inf, 0.0, np.abs(got - want))
    return float(np.nanmax(d)) if d.size else 0.0


def assert_parity(got, want, dtype, what="", strict=False):
    """strict: the flat bar (1e-5 f32, 2e-3 bf16/f16) on every element, and |ref| < 1 so that the
    flat bar is attainable by a correctly rounded 16-bit result."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    err = np.abs(got - want)
    tol = np.full(want.shape, TOL[dtype]) if strict else elementwise_tolerance(want, dtype)
    worst = float(np.max(err - tol)) if err.size else -1.0
    rel = float(np.max(err / np.maximum(np.abs(want), 1e-30))) if err.size else 0.0
    log(f"  parity {what}: max|err|={err.max(initial=0):.3e} "
        f"(bar: {'flat ' + format(TOL[dtype], '.0e') + ', strict' if strict else tolerance_note(want, dtype)}) "
        f"max|ref|={np.abs(want).max(initial=0):.3f} max rel={rel:.2e}")
    if strict:
        assert np.abs(want).max(initial=0) < 1.0, f"{what}: |ref| >= 1, flat 16-bit bar not attainable"
    assert worst <= 0, f"{what}: error exceeds tolerance by {worst:.3e}"
