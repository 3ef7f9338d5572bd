"""Parity bar: the HIP result y against the f64 oracle x, elementwise.

bf16/f16: |y - x| <= 2e-3 + 2**-8 * |x|; f32: |y - x| <= 1e-5 + 1e-5 * |x|.
An LSE of -inf must match exactly; any NaN fails.  (rocm-libraries "one K/V
resource per page on the gfx942 2D i64 path", Coverage and the author's
reply: atol 2e-3, rtol 2^-8, sized for bf16 rounding of outputs near 1.8.)
"""

import numpy as np
import torch

TOL = {
    torch.float32: (1e-5, 1e-5),
    torch.float16: (2e-3, 2.0 ** -8),
    torch.bfloat16: (2e-3, 2.0 ** -8),
}


def to_f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def assert_close(y, x, dtype, what=""):
    atol, rtol = TOL[dtype]
    y = to_f64(y)
    x = np.asarray(x, dtype=np.float64)
    assert y.shape == x.shape, f"{what}: shape {y.shape} vs {x.shape}"
    assert not np.isnan(y).any(), f"{what}: NaN in GPU result"
    assert not np.isnan(x).any(), f"{what}: NaN in oracle result"
    inf_x, inf_y = np.isinf(x), np.isinf(y)
    assert np.array_equal(inf_x, inf_y), f"{what}: -inf positions differ ({inf_x.sum()} vs {inf_y.sum()})"
    assert np.array_equal(x[inf_x], y[inf_y]), f"{what}: infinities differ in sign"
    fin = ~inf_x
    err = np.abs(y[fin] - x[fin])
    bound = atol + rtol * np.abs(x[fin])
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; "
                             f"worst |y-x|={err[i]:.3e} at |x|={abs(x[fin][i]):.3e} "
                             f"(bound {bound[i]:.3e})")
    return float(err.max()) if err.size else 0.0
